"""tkv_decode_step: one call per decode step, the append and the pending
Eq. 1 update ("Not All Thoughts Need HBM", gist.science summary, Method §2)
carried out inside the attention launch.  It must give the same bits as
tkv_append followed by tkv_decode_attn -- outputs every step, scores, tier
labels and changed-row lists across reassignments -- on every kernel
variant (vector and matrix-core paths, head_dim 64 and 128, chunk sizes
128/256/512, resident T2 values, a batch-shared T0 budget) and in stream
staging, where it is those two calls."""
import numpy as np
import pytest
import torch

import tkvsynth
from harness import Inputs, make_oracle, max_rel, to_device

pytestmark = pytest.mark.gpu


def _drive(w, inp, fused, **kw):
    import decode_attention_tkv_amd as tkv
    c = tkv.TieredKV.for_workload(w, **kw)
    c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    outs, deltas = [], []
    for t in range(w.steps):
        k, v = inp.step_kv(t)
        kd, vd, qd = to_device(k, w.dtype), to_device(v, w.dtype), to_device(inp.q[t], w.dtype)
        if fused:
            c.decode_step(kd, vd, qd, out)
        else:
            c.append(kd, vd)
            c.decode_attn(qd, out)
        outs.append(out.cpu().numpy().copy())
        if (t + 1) % w.delta == 0:
            c.reassign()
            deltas.append(c.read_deltas())
    res = dict(outs=outs, scores=c.read_scores(), tiers=c.read_tiers(), deltas=deltas, stats=c.stats())
    c.close()
    return res


CASES = {
    # bf16, 32 query heads on 32 kv heads (vector path), resident T2 values
    "7b_t2": (tkvsynth.CONFIGS["7b"].replace(layers=4, prefill=300, steps=40, delta=16, prompt=20,
                                             recent=16, t2_ratio=0.1), {}),
    # bf16 grouped heads (G = 5, matrix cores), batch-shared T0 budget, 128-row chunks
    "14b_shared_c128": (tkvsynth.CONFIGS["14b"].replace(layers=3, batch=3, prefill=500, steps=24, delta=8,
                                                        prompt=20, recent=16, shared_hbm=True), {"chunk": 128}),
    # bf16 head_dim 64 with G = 8 (matrix-core p.V with half the columns), 512-row chunks
    "d64_g8_c512": (tkvsynth.CONFIGS["7b"].replace(layers=2, q_heads=16, kv_heads=2, head_dim=64, batch=2,
                                                   prefill=700, steps=30, delta=10, prompt=20, recent=16,
                                                   t2_ratio=0.15, t2_fp8=True), {"chunk": 512}),
    # fp32, head_dim 64, G = 1
    "tiny_f32": (tkvsynth.CONFIGS["tiny"].replace(steps=40), {}),
    # stream staging with 8-bit rows: the step is the two separate calls
    "tiny_stream_t2": (tkvsynth.CONFIGS["tiny"].replace(steps=40, t2_ratio=0.1), {"staging_layers": 2}),
    # the largest batch: 64 sequences, one new row and one fold tile each
    "batch64": (tkvsynth.CONFIGS["tiny"].replace(batch=64, prefill=90, steps=17, delta=8, prompt=8, recent=8), {}),
    # the most query heads: 256 on 32 kv heads (G = 8), bf16 head_dim 64
    "heads256": (tkvsynth.CONFIGS["tiny"].replace(dtype="bf16", head_dim=64, kv_heads=32, q_heads=256, layers=1,
                                                  prefill=300, steps=17, delta=8, prompt=8, recent=16), {}),
}


@pytest.mark.parametrize("name", list(CASES))
def test_decode_step_matches_separate_calls(name):
    w, kw = CASES[name]
    print("decode_step case", name, flush=True)
    inp = Inputs(w)
    a = _drive(w, inp, fused=False, **kw)
    b = _drive(w, inp, fused=True, **kw)
    n = w.n_final
    for t, (x, y) in enumerate(zip(a["outs"], b["outs"])):
        assert np.array_equal(x, y), "step %d output differs" % t
    assert np.array_equal(a["scores"][:, :n], b["scores"][:, :n])
    assert np.array_equal(a["tiers"][:, :n], b["tiers"][:, :n])
    assert len(a["deltas"]) == len(b["deltas"]) > 0
    for (p0, d0, c0), (p1, d1, c1) in zip(a["deltas"], b["deltas"]):
        assert np.array_equal(c0, c1)
        for s in range(w.batch):
            assert np.array_equal(p0[s][:c0[s][0]], p1[s][:c1[s][0]])
            assert np.array_equal(d0[s][:c0[s][1]], d1[s][:c1[s][1]])
    for key in ("step", "n_tokens", "promotions", "demotions", "evictions", "reassigns"):
        assert a["stats"][key] == b["stats"][key], key


def test_decode_step_against_oracle():
    """The fused step on its own against the oracle (bf16 matrix-core path)."""
    w = tkvsynth.CONFIGS["14b"].replace(layers=2, batch=2, prefill=400, steps=20, delta=8, prompt=20, recent=16)
    import decode_attention_tkv_amd as tkv
    inp = Inputs(w)
    o = make_oracle(w, inp)
    c = tkv.TieredKV.for_workload(w)
    c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    worst = 0.0
    for t in range(w.steps):
        k, v = inp.step_kv(t)
        c.decode_step(to_device(k, w.dtype), to_device(v, w.dtype), to_device(inp.q[t], w.dtype), out)
        o.append(w.values(k), w.values(v))
        ref = o.attend(w.values(inp.q[t]))
        worst = max(worst, float(np.max(np.abs(out.cpu().numpy() - ref))))
        if (t + 1) % w.delta == 0:
            g_s = c.read_scores()[:, :o.n]
            c.reassign()
            tiers, _ = o.reassign(rank_scores=g_s)     # ranked by the GPU's fp32 scores
            assert np.array_equal(c.read_tiers()[:, :o.n], tiers), "labels differ at step %d" % (t + 1)
    assert worst <= 5e-3, worst
    rel = max_rel(c.read_scores()[:, :o.n], o.s[:, :o.n])
    assert rel <= 1e-4, rel
    c.close()


def test_decode_step_state_and_arguments():
    import decode_attention_tkv_amd as tkv
    w = tkvsynth.CONFIGS["tiny"].replace(prefill=40, steps=4)
    inp = Inputs(w)
    c = tkv.TieredKV.for_workload(w)
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    k, v = inp.step_kv(0)
    kd, vd, qd = to_device(k, w.dtype), to_device(v, w.dtype), to_device(inp.q[0], w.dtype)
    lib = tkv.lib()
    c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))
    assert lib.tkv_decode_step(c.h, kd.data_ptr(), vd.data_ptr(), None, out.data_ptr(), None) == tkv.TKV_EINVAL
    assert lib.tkv_decode_step(c.h, kd.data_ptr() + 4, vd.data_ptr(), qd.data_ptr(), out.data_ptr(),
                               None) == tkv.TKV_EINVAL     # misaligned k
    assert b"aligned" in lib.tkv_last_error(c.h)
    c.append(kd, vd)
    with pytest.raises(tkv.TkvError) as e:
        c.decode_step(kd, vd, qd, out)                    # a step is open
    assert e.value.code == tkv.TKV_ESTATE
    c.decode_attn(qd, out)
    c.decode_step(kd, vd, qd, out)                        # fine again
    assert c.stats()["step"] == 2
    c.close()


def test_decode_step_capacity():
    """The append's capacity errors, through the single call: the T0 pool
    (stream staging) runs full without reassignments, then max_tokens is
    reached."""
    import decode_attention_tkv_amd as tkv
    w = tkvsynth.CONFIGS["tiny"].replace(layers=3, prefill=100, steps=60, hbm_ratio=0.3, delta=4, prompt=8,
                                         recent=8)
    inp = Inputs(w)
    c = tkv.TieredKV.for_workload(w, staging_layers=2)
    c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    full_at = None
    for t in range(w.steps):
        k, v = inp.step_kv(t)
        try:
            c.decode_step(to_device(k, w.dtype), to_device(v, w.dtype), to_device(inp.q[t], w.dtype), out)
        except tkv.TkvError as e:
            assert e.code == tkv.TKV_ECAPACITY
            full_at = t
            break
    assert full_at is not None
    assert c.stats()["step"] == full_at                 # the failed call changed nothing
    c.reassign()
    for t in range(full_at, w.steps):
        k, v = inp.step_kv(t)
        c.decode_step(to_device(k, w.dtype), to_device(v, w.dtype), to_device(inp.q[t], w.dtype), out)
        if (t + 1) % w.delta == 0:
            c.reassign()
    assert c.stats()["n_tokens"] == w.n_final
    with pytest.raises(tkv.TkvError) as e:
        c.decode_step(to_device(k, w.dtype), to_device(v, w.dtype), to_device(inp.q[0], w.dtype), out)
    assert e.value.code == tkv.TKV_ECAPACITY            # max_tokens
    assert np.isfinite(out.cpu().numpy()).all()
    c.close()
