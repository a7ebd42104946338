"""Robustness of the GPU path, through the C ABI.

"Not All Thoughts Need HBM" (gist.science summary): Method §3
(Proposition 1: outputs depend only on the evicted set, not on where a live
row is kept) and Method §4 (asynchronous prefetch; only changed rows move).

Checks:
  * stream staging with every layer's staging copy held back by a bounded
    delay kernel on the copy streams gives the same bits as without it (the
    event chain attention -> copy -> attention orders every slot reuse);
  * T0 slots handed out in a seeded random order (stream staging, and the
    batch-shared budget) give the same bits as lowest-first slots and as
    resident staging;
  * with stream staging the kernels of a reassignment compact the pinned
    arenas and file the entrants over PCIe: after every reassignment each
    live row reads back bit for bit (T0/T1 values, T2 codes and scales);
  * a memory cap turns allocations into TKV_ENOMEM: at create, and at a
    reassignment's first growth, after which the handle is unchanged and
    keeps decoding as if that reassignment had not been asked for.
All conditions are forced from the host; every kernel exits normally.
"""
import numpy as np
import pytest
import torch

import tkvsynth
from harness import Inputs, make_oracle, to_device
from oracle import codec
from test_gpu_reassign import TOL, run_parity

pytestmark = pytest.mark.gpu


def _tkv():
    import decode_attention_tkv_amd as tkv
    return tkv


def _same_runs(a, b, scores=True):
    """Outputs bit for bit, and the scores and tiers unless the two runs add
    Eq. 1's terms in different orders: bf16 grouped-query heads over
    resident staging sum a step's weights within each kv head's group in the
    next step's launch, the other paths sum the stored logits head by head,
    so those scores agree to rounding only."""
    assert len(a[0]) == len(b[0])
    assert all(np.array_equal(x, y) for x, y in zip(a[0], b[0])), "outputs differ"
    if scores:
        assert np.array_equal(a[1], b[1]), "scores differ"
        assert np.array_equal(a[2], b[2]), "tiers differ"
    else:  # the split among live tiers follows the scores' last bits; the evicted set may not differ
        assert np.array_equal(a[2] == 3, b[2] == 3), "evicted sets differ"


def _deferred(w):
    return w.dtype == "bf16" and w.q_heads >= 4 * w.kv_heads


def _tiny5():
    return tkvsynth.CONFIGS["tiny"].replace(layers=5, steps=80)


def _gqa_t2():
    return tkvsynth.CONFIGS["32b_t2"].replace(layers=4, batch=2, prefill=300, steps=96, delta=32, prompt=40,
                                              recent=32)


@pytest.mark.parametrize("which,slots", [("tiny_f32", 2), ("gqa_bf16_t2", 2), ("tiny_f32", 4), ("gqa_bf16_t2", 4)],
                         ids=["tiny_f32", "gqa_bf16_t2", "tiny_f32_S4_pairs", "gqa_bf16_t2_S4_pairs"])
def test_delayed_copies_bitwise(which, slots):
    """S = 4 copies two layers at a time (tiny: 5 layers, so the last goes
    alone; the grouped-query case then has 6 layers, so that S < layers)."""
    w = _tiny5() if which == "tiny_f32" else _gqa_t2()
    if slots >= w.layers:
        w = w.replace(layers=slots + 2)
    inp = Inputs(w)
    tkv = _tkv()
    base = run_parity(w, inp, w.steps, check_every=8, staging_layers=slots)
    slow = run_parity(w, inp, w.steps, check_every=8, staging_layers=slots,
                      extra_flags=tkv.TKV_FLAG_TEST_DELAY_COPIES)
    _same_runs(base, slow)
    res = run_parity(w, inp, w.steps, check_every=8)
    _same_runs(base, res, scores=not _deferred(w))
    assert slow[3]["h2d_bytes"] == base[3]["h2d_bytes"] > 0


@pytest.mark.parametrize("which", ["tiny_f32_stream", "gqa_bf16_t2_stream", "gqa_bf16_shared"])
def test_shuffled_slots_bitwise(which):
    tkv = _tkv()
    if which == "tiny_f32_stream":
        w, kw = _tiny5(), dict(staging_layers=2)
    elif which == "gqa_bf16_t2_stream":
        w, kw = _gqa_t2(), dict(staging_layers=2)
    else:
        w, kw = _gqa_t2().replace(t2_ratio=0.0, shared_hbm=True), {}
    inp = Inputs(w)
    plain = run_parity(w, inp, w.steps, check_every=8, **kw)
    shuf = run_parity(w, inp, w.steps, check_every=8, extra_flags=tkv.TKV_FLAG_TEST_SHUFFLE_SLOTS, **kw)
    _same_runs(plain, shuf)
    if not w.shared_hbm:
        _same_runs(plain, run_parity(w, inp, w.steps, check_every=8), scores=not _deferred(w))


def _orig_row(inp, w, l, b, pos):
    """The values a position was appended with (before any 8-bit round trip)."""
    if pos < w.prefill:
        return w.values(inp.k0[l, b, pos]), w.values(inp.v0[l, b, pos])
    t = pos - w.prefill
    return w.values(inp.kn[l, b, t]), w.values(inp.vn[l, b, t])


@pytest.mark.parametrize("which", ["tiny_f32", "gqa_bf16_t2", "gqa_bf16_t2_fp8_heads"])
def test_stream_arena_rows_exact(which):
    """Stream staging: the reassignment's kernels move rows inside the pinned
    arenas and write the entrants there.  After every reassignment each live
    row reads back bit for bit: T0 and T1 rows as the oracle holds them, T2
    rows as the oracle's codec encodes their appended values."""
    if which == "tiny_f32":
        w = _tiny5().replace(t2_ratio=0.1, steps=64)
    elif which == "gqa_bf16_t2":
        w = _gqa_t2()
    else:
        w = _gqa_t2().replace(t2_fp8=True, t2_head_scales=True)
    inp = Inputs(w)
    tkv = _tkv()
    c = tkv.TieredKV.for_workload(w, staging_layers=2)
    c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))
    o = make_oracle(w, inp)
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    if w.t2_head_scales:
        def quant(x):
            return codec.quantize_row_heads(x, w.t2_fp8)
    else:
        quant = codec.quantize_row_fp8 if w.t2_fp8 else codec.quantize_row
    ns = w.kv_heads if w.t2_head_scales else 1
    checked = {0: 0, 1: 0, 2: 0}
    worst = 0.0
    for t in range(w.steps):
        k, v = inp.step_kv(t)
        c.append(to_device(k, w.dtype), to_device(v, w.dtype))
        o.append(w.values(k), w.values(v))
        c.decode_attn(to_device(inp.q[t], w.dtype), out)
        worst = max(worst, float(np.max(np.abs(out.cpu().numpy() - o.attend(w.values(inp.q[t]))))))
        if (t + 1) % w.delta:
            continue
        g_s = c.read_scores()[:, : o.n]
        c.reassign()
        tiers, _ = o.reassign(rank_scores=g_s)
        assert np.array_equal(c.read_tiers()[:, : o.n], tiers)
        for b in range(w.batch):
            for pos in range(o.n):
                tr = int(tiers[b, pos])
                if tr > 2:
                    continue
                for l in (0, w.layers - 1):
                    if tr < 2:
                        gk, gv = c.read_kv(l, b, pos)
                        assert np.array_equal(w.values(gk), o.K[l, b, pos]), (l, b, pos, tr)
                        assert np.array_equal(w.values(gv), o.V[l, b, pos]), (l, b, pos, tr)
                    else:
                        kc, vc, sc = c.read_t2(l, b, pos)
                        xk, xv = _orig_row(inp, w, l, b, pos)
                        rk, sk = quant(xk)
                        rv, sv = quant(xv)
                        assert np.array_equal(kc.view(np.uint8).ravel(), np.asarray(rk).view(np.uint8).ravel())
                        assert np.array_equal(vc.view(np.uint8).ravel(), np.asarray(rv).view(np.uint8).ravel())
                        assert np.array_equal(sc[:ns], np.ravel(sk)) and np.array_equal(sc[ns:], np.ravel(sv))
                    checked[tr] += 1
    c.close()
    assert worst <= TOL[w.dtype]
    assert checked[0] > 0 and checked[1] > 0 and checked[2] > 0, checked


def test_mem_cap_at_create():
    tkv = _tkv()
    w = tkvsynth.CONFIGS["tiny"]
    with pytest.raises(tkv.TkvError) as e:
        tkv.TieredKV.for_workload(w, mem_cap_bytes=1 << 20)
    assert e.value.code == tkv.TKV_ENOMEM and "cap" in str(e.value)
    with pytest.raises(tkv.TkvError) as e:
        tkv.TieredKV.for_workload(w, mem_cap_bytes=-1)
    assert e.value.code == tkv.TKV_EINVAL


@pytest.mark.parametrize("staging_layers", [0, 2], ids=["resident", "stream"])
def test_mem_cap_at_reassign_leaves_handle_usable(staging_layers):
    """A cap that fits the handle as created but not a reassignment's
    buffers: the reassignment fails with TKV_ENOMEM before any state
    changes, and the handle decodes on with its old tiers (the oracle that
    never reassigned agrees) -- in stream staging for as long as its T0 pool
    has free slots, since only a reassignment frees them."""
    tkv = _tkv()
    w = _tiny5().replace(t2_ratio=0.1, steps=16 + 5)
    inp = Inputs(w)
    probe = tkv.TieredKV.for_workload(w, staging_layers=staging_layers)
    held = probe.stats()["mem_bytes"]
    probe.close()
    assert held > 0
    c = tkv.TieredKV.for_workload(w, staging_layers=staging_layers, mem_cap_bytes=held)
    c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))
    o = make_oracle(w, inp)
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    failures = 0
    for t in range(w.steps):
        k, v = inp.step_kv(t)
        c.decode_step(to_device(k, w.dtype), to_device(v, w.dtype), to_device(inp.q[t], w.dtype), out)
        o.append(w.values(k), w.values(v))
        ref = o.attend(w.values(inp.q[t]))
        assert np.max(np.abs(out.cpu().numpy() - ref)) <= TOL[w.dtype]
        if (t + 1) % w.delta == 0:
            before = c.read_tiers()
            with pytest.raises(tkv.TkvError) as e:
                c.reassign()
            assert e.value.code == tkv.TKV_ENOMEM and "cap" in str(e.value)
            failures += 1
            assert np.array_equal(c.read_tiers(), before)
            assert np.array_equal(before[:, : o.n], o.tier[:, : o.n])
    st = c.stats()
    c.close()
    assert failures == 1 and st["reassigns"] == 0 and st["mem_bytes"] <= held
