"""Whole-step pins of the oracle (CPU only).

Proposition 1 of "Not All Thoughts Need HBM" (gist.science summary, Method
§3): with the evicted set fixed, the outputs do not depend on how live rows
are split between HBM (T0) and host memory (T1).  Pins: runs at HBM ratios
30/50/70% with the same eviction ratio give identical outputs, scores and
evicted sets; with no eviction and no T2 every step equals a library softmax
attention over the whole cache; a different eviction ratio does change the
outputs (so the first pin is not vacuous).
"""
import numpy as np
import torch

import oracle
import tkvsynth
from oracle import T0, T1, T3


def _run(w, record_every=1):
    o = oracle.OracleTKV.for_workload(w)
    o.prefill(w.values(w.kv(0, 0, w.prefill)), w.values(w.kv(1, 0, w.prefill)))
    Kn = w.values(w.kv(0, w.prefill, w.steps))
    Vn = w.values(w.kv(1, w.prefill, w.steps))
    Q = w.values(w.q(0, w.steps))
    outs = []
    for t in range(w.steps):
        o.append(Kn[:, :, t], Vn[:, :, t])
        out = o.attend(Q[t])
        if t % record_every == 0:
            outs.append(out)
        if (t + 1) % w.delta == 0:
            o.reassign()
    return o, outs


def _small():
    return tkvsynth.CONFIGS["tiny"].replace(steps=64, prefill=96, prompt=16, recent=16, delta=16,
                                            evict_ratio=0.10)


def test_outputs_independent_of_hbm_split():
    base = _small()
    runs = [_run(base.replace(hbm_ratio=h)) for h in (0.3, 0.5, 0.7)]
    o0, outs0 = runs[0]
    for o, outs in runs[1:]:
        assert all(np.array_equal(a, b) for a, b in zip(outs0, outs))
        assert np.array_equal(o.s, o0.s)
        assert np.array_equal(o.tier == T3, o0.tier == T3)
    # the splits themselves differ
    t0_counts = [int((o.tier[0, : o.n] == T0).sum()) for o, _ in runs]
    assert len(set(t0_counts)) == 3


def test_eviction_changes_outputs():
    base = _small()
    _, a = _run(base.replace(evict_ratio=0.03))
    _, b = _run(base.replace(evict_ratio=0.30))
    assert not all(np.array_equal(x, y) for x, y in zip(a, b))


def test_no_eviction_equals_dense_attention():
    w = _small().replace(evict_ratio=0.0, t2_ratio=0.0, steps=20)
    o, outs = _run(w)
    # recompute the last step densely with torch SDPA in float64
    n = o.n
    Q = w.values(w.q(0, w.steps))[-1]
    for l in range(w.layers):
        k = torch.from_numpy(o.K[l, 0, :n].astype(np.float64)).transpose(0, 1).contiguous()
        v = torch.from_numpy(o.V[l, 0, :n].astype(np.float64)).transpose(0, 1).contiguous()
        q = torch.from_numpy(Q[l, 0].astype(np.float64)).unsqueeze(1)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)[:, 0].numpy()
        assert np.max(np.abs(outs[-1][l, 0] - ref)) < 1e-12
    assert (o.tier[0, :n] == T3).sum() == 0
    assert set(np.unique(o.tier[0, :n]).tolist()) <= {T0, T1}


def test_rows_entering_t2_hold_their_codec_roundtrip():
    from oracle import codec
    w = _small().replace(t2_ratio=0.2, steps=16)
    o = oracle.OracleTKV.for_workload(w)
    K0 = w.values(w.kv(0, 0, w.prefill))
    V0 = w.values(w.kv(1, 0, w.prefill))
    o.prefill(K0, V0)
    Kn = w.values(w.kv(0, w.prefill, w.steps))
    Vn = w.values(w.kv(1, w.prefill, w.steps))
    Q = w.values(w.q(0, w.steps))
    for t in range(w.steps):
        o.append(Kn[:, :, t], Vn[:, :, t])
        o.attend(Q[t])
    tiers, _ = o.reassign()                      # first reassignment: nothing was in T2 before
    t2 = np.nonzero(tiers[0] == oracle.T2)[0]
    assert len(t2) == int(0.2 * o.n)
    K_all = np.concatenate([K0, Kn], axis=2)
    V_all = np.concatenate([V0, Vn], axis=2)
    for i in t2:
        for l in range(w.layers):
            assert np.array_equal(o.K[l, 0, i], codec.roundtrip(K_all[l, 0, i], bf16=False))
            assert np.array_equal(o.V[l, 0, i], codec.roundtrip(V_all[l, 0, i], bf16=False))
    others = np.nonzero(tiers[0] != oracle.T2)[0]
    assert np.array_equal(o.K[:, 0, others], K_all[:, 0, others])
