"""Pins for the oracle's scored prefill (oracle/prefill.py): Eq. 1 of "Not
All Thoughts Need HBM" (gist.science summary, Method §2) applied to the
prompt's causal attention.

* q = 0: every query spreads its weight evenly over positions 0..t, so
  s_j = sum_{t=j}^{n-1} 1/(t+1) = H_n - H_j (harmonic numbers);
* every query adds exactly 1 in total: sum_j s_j = n;
* brute force: pure-Python loops over (t, j) on a tiny case;
* the decode engine (already pinned) fed the same tokens one at a time from
  a one-token prefill reaches the same scores, except that it never runs
  the first token's own query (which gives position 0 a weight of 1);
* a scored prefill followed by the tier rules ranks by these scores.
"""
import math

import numpy as np

import oracle
import tkvsynth
from oracle import tiering
from oracle.prefill import prefill_scores


def _draw(w, n):
    heavy, u = w.heavy_mask(), w.unit_vector()
    K = w.values(w.kv(0, 0, n, heavy, u))
    V = w.values(w.kv(1, 0, n, heavy, u))
    Q = np.ascontiguousarray(np.moveaxis(w.values(w.q(0, n, u)), 0, 2))  # [L][B][n][Hq][d]
    return K, V, Q


def test_zero_queries_give_harmonic_tails():
    w = tkvsynth.CONFIGS["tiny"].replace(q_heads=8, kv_heads=4)
    n = 50
    K, _, Q = _draw(w, n)
    s = prefill_scores(K, np.zeros_like(Q), n)
    H = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, n + 1))])
    assert np.max(np.abs(s[0] - (H[n] - H[:n]))) < 1e-12


def test_every_query_adds_one():
    w = tkvsynth.CONFIGS["tiny"]
    n = 120
    K, _, Q = _draw(w, n)
    s = prefill_scores(K, Q, n)
    assert abs(s.sum() - n) < 1e-9
    assert np.all(s > 0)


def test_brute_force_tiny():
    rng = np.random.default_rng(0)
    L, B, n, Hkv, Hq, d = 2, 1, 6, 1, 2, 4
    K = rng.standard_normal((L, B, n, Hkv, d))
    Q = rng.standard_normal((L, B, n, Hq, d))
    ref = [0.0] * n
    for l in range(L):
        for h in range(Hq):
            for t in range(n):
                z = [sum(Q[l, 0, t, h, e] * K[l, 0, j, 0, e] for e in range(d)) / math.sqrt(d) for j in range(t + 1)]
                m = max(z)
                w_ = [math.exp(x - m) for x in z]
                tot = sum(w_)
                for j in range(t + 1):
                    ref[j] += w_[j] / tot / (L * Hq)
    got = prefill_scores(K, Q, n)[0]
    assert np.max(np.abs(got - np.array(ref))) < 1e-13


def test_decode_engine_reaches_the_same_scores():
    w = tkvsynth.CONFIGS["tiny"].replace(q_heads=8, kv_heads=4, hbm_ratio=1.0, evict_ratio=0.0)
    n = 40
    K, V, Q = _draw(w, n)
    o = oracle.OracleTKV.for_workload(w, max_tokens=n)
    o.prefill(K[:, :, :1], V[:, :, :1])
    for t in range(1, n):
        o.append(K[:, :, t], V[:, :, t])
        o.attend(Q[:, :, t])
    expect = o.s[:, :n].copy()
    expect[:, 0] += 1.0            # the first token's own query, which decode never runs
    assert np.max(np.abs(prefill_scores(K, Q, n) - expect)) < 1e-12


def test_scored_prefill_places_by_the_scores():
    w = tkvsynth.CONFIGS["tiny"].replace(prefill=200, prompt=8, recent=16)   # |P| = 24 < floor(.3 * 200)
    n = w.prefill
    K, V, Q = _draw(w, n)
    o = oracle.OracleTKV.for_workload(w)
    tiers, deltas = o.prefill_scored(K, V, Q)
    s = prefill_scores(K, Q, n)
    expect = tiering.reassign(tiering.initial_placement(n, w.prompt, w.sinks, w.recent, w.hbm_ratio), s[0], n,
                              w.prompt, w.sinks, w.recent, w.hbm_ratio, w.evict_ratio, w.t2_ratio)
    assert np.array_equal(tiers[0], expect)
    # the planted heavy hitters among the candidates rank high, so T0 holds them
    prot = tiering.protected_mask(n, w.prompt, w.sinks, w.recent)
    heavy = np.nonzero(w.heavy_mask()[0, :n] & ~prot)[0]
    assert len(heavy) > 0 and np.mean(tiers[0, heavy] == 0) > 0.5
    assert np.mean(tiers[0, np.setdiff1d(np.nonzero(~prot)[0], heavy)] == 0) < 0.3
