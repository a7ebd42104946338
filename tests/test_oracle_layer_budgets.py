"""Pins for the oracle's per-layer HBM budgets (OracleLayerGroups): layer
group g keeps floor(h_g N) rows in HBM, every group ranks by the one Eq. 1
score over all layers ("Not All Thoughts Need HBM", gist.science summary,
Method §1 and §2; per-layer ratios in the spirit of the ARKV summary,
Method) and the eviction and T2 ratios are shared.

* equal ratios: exactly the one-budget oracle (tiers equal; outputs and
  scores equal up to the order of the fp64 layer sum);
* different ratios: every group evicts the same rows, and the outputs equal
  the one-budget run's (Method §3, Proposition 1: only the evicted set
  enters, and without T2 no value changes);
* a group's T0 holds the protected rows plus its n0c best candidates, with
  n0c the closed form of Method §1 for its ratio, so the T0 sets nest by
  ratio; with T2 clipped by a large HBM share, each group's T2 count is
  min(|C| - n3 - n0c_g, floor(t2 N)).
"""
import math

import numpy as np

import oracle
import tkvsynth
from oracle import T0, T2, T3, tiering


def _run(w, layer_hbm=None, steps=None):
    steps = steps or w.steps
    o = oracle.OracleTKV.for_workload(w) if layer_hbm is None else oracle.OracleLayerGroups.for_workload(w, layer_hbm)
    o.prefill(w.values(w.kv(0, 0, w.prefill)), w.values(w.kv(1, 0, w.prefill)))
    Kn = w.values(w.kv(0, w.prefill, steps))
    Vn = w.values(w.kv(1, w.prefill, steps))
    Q = w.values(w.q(0, steps))
    outs = []
    for t in range(steps):
        o.append(Kn[:, :, t], Vn[:, :, t])
        outs.append(o.attend(Q[t]))
        if (t + 1) % w.delta == 0:
            o.reassign()
    return o, outs


def _small(**kw):
    base = dict(layers=5, steps=48, prefill=96, prompt=12, sinks=4, recent=16, delta=16, evict_ratio=0.10)
    base.update(kw)
    return tkvsynth.CONFIGS["tiny"].replace(**base)


def test_groups_split():
    assert oracle.layer_groups([0.5]) == [(0, 1, 0.5)]
    assert oracle.layer_groups([0.2, 0.2, 0.7, 0.2]) == [(0, 2, 0.2), (2, 3, 0.7), (3, 4, 0.2)]


def test_equal_ratios_are_the_one_budget_oracle():
    w = _small(hbm_ratio=0.4)
    a, outs_a = _run(w)
    b, outs_b = _run(w, [0.4, 0.4, 0.4, 0.4, 0.4])
    assert len(b.parts) == 1
    for x, y in zip(outs_a, outs_b):
        assert np.array_equal(x, y)
    assert np.allclose(a.s, b.s, rtol=1e-12, atol=0)
    assert np.array_equal(a.tier, b.tier_of(0))


def test_split_groups_sum_eq1_over_all_layers():
    # groups [0,2) and [2,5) with one ratio each side of a boundary: scores
    # equal the one-budget oracle's, where the layer sum runs in one piece
    w = _small(hbm_ratio=0.4)
    a, _ = _run(w)
    b, _ = _run(w, [0.4, 0.4, 0.4000001, 0.4000001, 0.4000001])
    assert len(b.parts) == 2
    assert np.allclose(a.s, b.s, rtol=1e-12, atol=0)
    for l in range(w.layers):
        assert np.array_equal(a.tier, b.tier_of(l))  # floor(h N) is the same for both ratios here


def test_different_ratios_same_evictions_and_outputs():
    w = _small(hbm_ratio=0.5)
    ratios = [0.15, 0.15, 0.5, 0.8, 0.8]
    a, outs_a = _run(w)
    b, outs_b = _run(w, ratios)
    for x, y in zip(outs_a, outs_b):
        assert np.array_equal(x, y)
    assert np.allclose(a.s, b.s, rtol=1e-12, atol=0)
    ev = a.tier == T3
    assert ev.sum() > 0
    for l in range(w.layers):
        assert np.array_equal(b.tier_of(l) == T3, ev)
    # the T0 shares differ, and nest by ratio
    n = b.n
    t0 = [b.tier_of(l)[:, :n] == T0 for l in (0, 2, 3)]
    assert int(t0[0].sum()) < int(t0[1].sum()) < int(t0[2].sum())
    assert np.all(t0[0] <= t0[1]) and np.all(t0[1] <= t0[2])


def test_t0_counts_follow_each_ratio():
    w = _small(hbm_ratio=0.5, steps=32)
    ratios = [0.1, 0.3, 0.3, 0.6, 0.95]
    b, _ = _run(w, ratios)
    n = b.n
    prot = tiering.protected_mask(n, w.prompt, w.sinks, w.recent)
    for g, (l0, l1, h) in enumerate(b.groups):
        tier = b.parts[g].tier[:, :n]
        for s in range(w.batch):
            # the last step is a reassignment: n0c of Method §1 at this n, for this group's ratio
            ev = int((tier[s] == T3).sum())
            n0c = min(n - int(prot.sum()) - ev, max(0, math.floor(h * n) - int(prot.sum())))
            assert int((tier[s] == T0).sum()) == int(prot.sum()) + n0c


def test_t2_clipped_per_group():
    # h + e + t2 > 1 in the high-ratio group: its T2 count is clipped, the low group's is not
    w = _small(hbm_ratio=0.5, t2_ratio=0.25, evict_ratio=0.10, steps=16)
    ratios = [0.2, 0.2, 0.2, 0.85, 0.85]
    b, _ = _run(w, ratios)
    n = b.n
    prot = tiering.protected_mask(n, w.prompt, w.sinks, w.recent)
    counts = []
    for g, (l0, l1, h) in enumerate(b.groups):
        tier = b.parts[g].tier[0, :n]
        ev = int((tier == T3).sum())
        c = n - int(prot.sum()) - ev
        n0c = min(c, max(0, math.floor(h * n) - int(prot.sum())))
        assert int((tier == T2).sum()) == min(c - n0c, math.floor(0.25 * n))
        counts.append(int((tier == T2).sum()))
    assert counts[0] == math.floor(0.25 * n) and counts[1] < counts[0]


def test_scored_prefill_equal_ratios_is_the_one_budget_oracle():
    w = _small(hbm_ratio=0.4, prefill=64)
    K, V = w.values(w.kv(0, 0, w.prefill)), w.values(w.kv(1, 0, w.prefill))
    Q = w.values(w.q(0, w.prefill)).transpose(1, 2, 0, 3, 4).copy()  # [L][B][n][Hq][d]
    a = oracle.OracleTKV.for_workload(w)
    a.prefill_scored(K, V, Q)
    b = oracle.OracleLayerGroups.for_workload(w, [0.4] * 2 + [0.4000001] * 3)
    b.prefill_scored(K, V, Q)
    assert np.array_equal(a.s, b.s)
    for l in range(w.layers):
        assert np.array_equal(a.tier, b.tier_of(l))
