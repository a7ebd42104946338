"""Pins of the oracle's cumulative score, Eq. 1 of "Not All Thoughts Need HBM"
(gist.science summary, Method §2): s_i grows each step by the mean over
layers and heads of that step's attention weight on position i.

Pins: the increments of one step sum to 1 over the live rows (each alpha is
a distribution, and a mean of distributions is one); q = 0 gives 1/N_live
per live row; a weight that sits on a single (layer, head) contributes
1/(L*H); evicted rows keep a frozen score.
"""
import numpy as np

import oracle
import tkvsynth
from oracle import T3


def _engine(w, **kw):
    o = oracle.OracleTKV.for_workload(w.replace(**kw) if kw else w)
    return o


def test_increment_sums_to_one_each_step():
    w = tkvsynth.CONFIGS["tiny"].replace(steps=40)
    o = _engine(w)
    o.prefill(w.values(w.kv(0, 0, w.prefill)), w.values(w.kv(1, 0, w.prefill)))
    Kn, Vn, Q = w.kv(0, w.prefill, w.steps), w.kv(1, w.prefill, w.steps), w.q(0, w.steps)
    for t in range(w.steps):
        o.append(Kn[:, :, t], Vn[:, :, t])
        before = o.s.copy()
        o.attend(Q[t])
        inc = o.s - before
        live = o.live()
        for b in range(w.batch):
            assert abs(inc[b][live[b]].sum() - 1.0) < 1e-12
            assert np.all(inc[b][~live[b]] == 0)
            assert np.all(inc[b][live[b]] > 0)
        if (t + 1) % w.delta == 0:
            o.reassign()
    assert (o.tier[0, : o.n] == T3).sum() == int(0.03 * o.n)


def test_zero_query_increment_is_uniform():
    w = tkvsynth.CONFIGS["tiny"]
    o = _engine(w)
    o.prefill(w.kv(0, 0, 64), w.kv(1, 0, 64))
    # evict a few rows by hand through the tier table
    o.tier[0, [40, 41, 50]] = T3
    q = np.zeros((w.layers, w.batch, w.q_heads, w.head_dim))
    o.attend(q)
    live = o.live()[0, : o.n]
    assert np.allclose(o.s[0, : o.n][live], 1.0 / live.sum(), rtol=0, atol=1e-15)
    assert np.all(o.s[0, : o.n][~live] == 0)


def test_single_head_weight_counts_one_over_LH():
    L, B, H, n = 3, 2, 5, 7
    alpha = np.zeros((L, B, H, n))
    # every (l, b, h) puts all its weight on position 0, except (l=1, h=3) on position 4
    alpha[..., 0] = 1.0
    alpha[1, :, 3, 0] = 0.0
    alpha[1, :, 3, 4] = 1.0
    inc = oracle.eq1_increment(alpha)
    assert np.allclose(inc[:, 4], 1.0 / (L * H), rtol=0, atol=1e-16)
    assert np.allclose(inc[:, 0], 1.0 - 1.0 / (L * H), rtol=0, atol=1e-15)
    assert np.allclose(inc.sum(axis=1), 1.0, atol=1e-15)


def test_identical_weights_everywhere_pass_through():
    rng = np.random.default_rng(0)
    a = rng.random(9)
    a /= a.sum()
    alpha = np.broadcast_to(a, (4, 2, 6, 9)).copy()
    inc = oracle.eq1_increment(alpha)
    assert np.allclose(inc, a[None, :], rtol=1e-15, atol=0)


def test_layers_and_heads_weighted_equally():
    # layer 0 (2 heads on pos 0), layer 1 (2 heads on pos 1): each position gets 1/2.
    alpha = np.zeros((2, 1, 2, 3))
    alpha[0, 0, :, 0] = 1.0
    alpha[1, 0, :, 1] = 1.0
    inc = oracle.eq1_increment(alpha)
    assert np.allclose(inc[0], [0.5, 0.5, 0.0], atol=0, rtol=0)


def test_evicted_scores_frozen():
    w = tkvsynth.CONFIGS["tiny"].replace(steps=48)
    o = _engine(w)
    o.prefill(w.kv(0, 0, w.prefill), w.kv(1, 0, w.prefill))
    Kn, Vn, Q = w.kv(0, w.prefill, w.steps), w.kv(1, w.prefill, w.steps), w.q(0, w.steps)
    frozen = None
    for t in range(w.steps):
        o.append(Kn[:, :, t], Vn[:, :, t])
        o.attend(Q[t])
        if frozen is not None:
            mask, vals = frozen
            assert np.array_equal(o.s[:, : mask.shape[1]][mask], vals)
        if (t + 1) % w.delta == 0:
            o.reassign()
            mask = o.tier[:, : o.n] == T3
            frozen = (mask, o.s[:, : o.n][mask].copy())
    assert frozen[0].sum() > 0
