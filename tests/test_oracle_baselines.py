"""Oracle pins for the baseline policies on the same engine (the eviction
policies the gist.science summary of "Not All Thoughts Need HBM" compares
against, Results; tier rules of Method §1 and §4).

* Eviction-only (no T1, heavy hitters kept): hand-derived counts
  (tests/golden/baseline_counts.json), the order property on many tiny
  cases with ties (every kept candidate ranks above every evicted one), and
  brute force: the live set equals P plus the top floor(hN) - |P| candidates
  of a full sort.
* Sinks + recent window (hbm 0, evict 1, prompt 0 under the tiered rules):
  reduces to the textbook sliding window with attention sinks; with a
  reassignment after every step the oracle's outputs equal softmax attention
  written out over exactly the sinks and the last recent + 1 positions.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
import tkvsynth
from oracle import tiering
from oracle.tiering import T0, T1, T2, T3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "baseline_counts.json")
IMPORTANCE = {T3: 0, T2: 1, T1: 2, T0: 3}


def _rows():
    doc = json.load(open(GOLDEN))
    return [dict(zip(doc["fields"], r["case"]), why=r["why"]) for r in doc["rows"]]


@pytest.mark.parametrize("row", _rows(), ids=lambda r: r["why"][:40])
def test_no_t1_golden_counts(row):
    n = row["n"]
    prot = tiering.protected_mask(n, row["prompt"], row["sinks"], row["recent"])
    assert prot.sum() == row["expect_protected"]
    old = np.full(n, T1, np.uint8)
    unprot = np.nonzero(~prot)[0]
    old[unprot[: row["n_evicted_before"]]] = T3
    cand = (~prot) & (old != T3)
    assert cand.sum() == row["expect_candidates"]
    got = tiering.tier_counts(n, int(prot.sum()), int(cand.sum()), row["n_evicted_before"],
                              row["hbm"], 0.77, row["t2"], no_t1=True)   # the eviction ratio plays no part
    assert got == (row["expect_n3"], row["expect_n0c"], row["expect_n2"])
    new = tiering.reassign(old, np.random.default_rng(n).random(n), n, row["prompt"], row["sinks"],
                           row["recent"], row["hbm"], 0.0, row["t2"], no_t1=True)
    counts = [int((new == t).sum()) for t in (T0, T1, T2, T3)]
    assert counts == [row["expect_T0"], row["expect_T1"], row["expect_T2"], row["expect_T3"]]


def test_no_t1_order_property_tiny_cases():
    rng = np.random.default_rng(1)
    levels = np.array([0.0, 0.25, 0.5, 1.0])
    for n in range(1, 13):
        for trial in range(30):
            prompt, sinks, recent = (int(x) for x in rng.integers(0, 4, 3))
            h, t2 = (float(x) for x in rng.choice([0.0, 0.1, 0.3, 0.5, 1.0], 2))
            scores = levels[rng.integers(0, len(levels), n)]
            old = np.full(n, T1, np.uint8)
            prot = tiering.protected_mask(n, prompt, sinks, recent)
            unprot = np.nonzero(~prot)[0]
            old[rng.choice(unprot, size=int(rng.integers(0, len(unprot) + 1)), replace=False)] = T3
            new = tiering.reassign(old, scores, n, prompt, sinks, recent, h, 0.0, t2, no_t1=True)
            assert not np.any(new == T1)
            assert np.all(new[old == T3] == T3) and np.all(new[prot & (old != T3)] == T0)
            cand = np.nonzero(~prot & (old != T3))[0]
            for a, b in itertools.combinations(cand, 2):
                a_first = (scores[a] > scores[b]) or (scores[a] == scores[b] and a < b)
                hi, lo = (a, b) if a_first else (b, a)
                assert IMPORTANCE[int(new[hi])] >= IMPORTANCE[int(new[lo])]


def test_no_t1_brute_force_live_set():
    rng = np.random.default_rng(2)
    n, prompt, sinks, recent, h = 300, 20, 4, 30, 0.4
    scores = rng.random(n)
    new = tiering.reassign(np.full(n, T1, np.uint8), scores, n, prompt, sinks, recent, h, 0.0, 0.0, no_t1=True)
    prot = tiering.protected_mask(n, prompt, sinks, recent)
    cand = [i for i in range(n) if not prot[i]]
    keep = sorted(cand, key=lambda i: (-scores[i], i))[: int(np.floor(h * n)) - int(prot.sum())]
    expect = prot.copy()
    expect[keep] = True
    assert np.array_equal(new != T3, expect)


def test_no_t1_first_placement_evicts_the_t1_rows():
    t = tiering.initial_placement(100, 10, 4, 20, 0.5, no_t1=True)
    assert np.array_equal(np.nonzero(t == T0)[0], np.r_[0:30, 80:100])
    assert np.all(t[30:80] == T3) and not np.any(t == T1)


def test_sinks_plus_recent_reduces_to_the_window():
    """hbm 0, evict 1, prompt 0: after a reassignment only the sinks and the
    recent window are live, whatever the scores."""
    rng = np.random.default_rng(3)
    n, sinks, recent = 500, 4, 64
    new = tiering.reassign(np.full(n, T1, np.uint8), rng.random(n), n, 0, sinks, recent, 0.0, 1.0, 0.0)
    live = np.nonzero(new != T3)[0]
    assert np.array_equal(live, np.r_[0:sinks, n - recent:n])


def test_sinks_plus_recent_engine_equals_windowed_attention():
    w = tkvsynth.CONFIGS["tiny"].replace(prefill=40, steps=12, delta=1, hbm_ratio=0.0, evict_ratio=1.0,
                                         prompt=0, sinks=4, recent=8)
    heavy, u = w.heavy_mask(), w.unit_vector()
    K0, V0 = w.values(w.kv(0, 0, w.prefill, heavy, u)), w.values(w.kv(1, 0, w.prefill, heavy, u))
    Kn, Vn = w.values(w.kv(0, w.prefill, w.steps, heavy, u)), w.values(w.kv(1, w.prefill, w.steps, heavy, u))
    Q = w.values(w.q(0, w.steps, u))
    o = oracle.OracleTKV.for_workload(w)
    o.prefill(K0, V0)
    o.reassign()                      # the window applies from the first step on
    K = np.concatenate([K0, Kn], axis=2).astype(np.float64)
    V = np.concatenate([V0, Vn], axis=2).astype(np.float64)
    g = w.q_heads // w.kv_heads
    for t in range(w.steps):
        o.append(Kn[:, :, t], Vn[:, :, t])
        got = o.attend(Q[t])
        n = w.prefill + t + 1
        keep = np.r_[0:w.sinks, n - w.recent - 1:n]    # the window before this step's append, plus it
        for l in range(w.layers):
            for h in range(w.q_heads):
                q = Q[t][l, 0, h].astype(np.float64)
                k = K[l, 0, keep, h // g]
                v = V[l, 0, keep, h // g]
                z = k @ q / np.sqrt(w.head_dim)
                a = np.exp(z - z.max())
                ref = (a / a.sum()) @ v
                assert np.max(np.abs(got[l, 0, h] - ref)) < 1e-12
        o.reassign()
