"""GPU 8-bit host tier (T2) against the oracle, through the C ABI.

"Not All Thoughts Need HBM" (gist.science summary), Method §1: T2 holds
low-importance rows on the host at 8 bits; §4: only changed rows move.  Both
8-bit formats: int8 and FP8 (OCP E4M3).

Checks:
  * every row entering T2 gets int8 codes and scales identical to the
    oracle's codec applied to the same values (integer results, bit-exact),
    and attention then reads exactly the dequantised values;
  * a whole run with T2 matches the oracle (outputs within tolerance,
    scores relative 1e-4, labels and delta lists bit-exact);
  * resident and stream staging give bitwise identical outputs.
"""
import numpy as np
import pytest
import torch

import tkvsynth
from harness import Inputs, make_oracle, max_rel, to_device
from oracle import codec
from test_gpu_reassign import TOL, _check_deltas

pytestmark = pytest.mark.gpu


def _run_t2(w, inp, staging_layers=0, check_codec=True):
    import decode_attention_tkv_amd as tkv
    c = tkv.TieredKV.for_workload(w, staging_layers=staging_layers)
    c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))
    o = make_oracle(w, inp)
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    outs, worst, entered = [], 0.0, 0
    bf16 = w.dtype == "bf16"
    for t in range(w.steps):
        k, v = inp.step_kv(t)
        c.append(to_device(k, w.dtype), to_device(v, w.dtype))
        o.append(w.values(k), w.values(v))
        c.decode_attn(to_device(inp.q[t], w.dtype), out)
        ref = o.attend(w.values(inp.q[t]))
        got = out.cpu().numpy()
        outs.append(got.copy())
        worst = max(worst, float(np.max(np.abs(got - ref))))
        if (t + 1) % w.delta == 0:
            g_s = c.read_scores()[:, : o.n]
            before_k, before_v = o.K.copy(), o.V.copy()
            c.reassign()
            tiers, deltas = o.reassign(rank_scores=g_s)
            assert np.array_equal(c.read_tiers()[:, : o.n], tiers)
            _check_deltas(c, deltas, o.n)
            if not check_codec:
                continue
            for b, (pro, dem) in enumerate(deltas):
                for (pos, old, new) in dem:
                    if new != 2:
                        continue
                    entered += 1
                    if w.t2_head_scales:
                        def quant(x):
                            return codec.quantize_row_heads(x, w.t2_fp8)

                        def deq(cd, sc_, bf):
                            return codec.dequantize_row_heads(cd, sc_, w.t2_fp8, bf)
                    else:
                        quant = codec.quantize_row_fp8 if w.t2_fp8 else codec.quantize_row
                        deq = codec.dequantize_row_fp8 if w.t2_fp8 else codec.dequantize_row
                    ns = w.kv_heads if w.t2_head_scales else 1
                    for l in range(w.layers):
                        kc, vc, sc = c.read_t2(l, b, pos)
                        rk, sk = quant(before_k[l, b, pos])
                        rv, sv = quant(before_v[l, b, pos])
                        # codes compared as bytes: int8 two's complement, or the E4M3 bit patterns
                        assert np.array_equal(kc.view(np.uint8).ravel(), np.asarray(rk).view(np.uint8).ravel())
                        assert np.array_equal(vc.view(np.uint8).ravel(), np.asarray(rv).view(np.uint8).ravel())
                        assert np.array_equal(sc[:ns], np.ravel(sk)) and np.array_equal(sc[ns:], np.ravel(sv))
                        if staging_layers == 0:
                            gk, gv = c.read_kv(l, b, pos)
                            gk, gv = w.values(gk), w.values(gv)
                            assert np.array_equal(gk, deq(rk, sk, bf16).reshape(gk.shape))
                            assert np.array_equal(gv, deq(rv, sv, bf16).reshape(gv.shape))
    s = c.read_scores()
    st = c.stats()
    c.close()
    assert worst <= TOL[w.dtype], "out max-abs %.3g" % worst
    assert max_rel(s[:, : o.n], o.s[:, : o.n]) <= 1e-4
    if check_codec:
        assert entered > 0
    return outs, st, o


def _w32(**kw):
    args = dict(layers=3, batch=2, prefill=700, steps=97, delta=32)
    args.update(kw)
    return tkvsynth.CONFIGS["32b_t2"].replace(**args)


def test_t2_resident_parity_and_codec():
    w = _w32()
    outs, st, o = _run_t2(w, Inputs(w))
    n = o.n
    assert st["tier_count"][2] == 2 * int(0.2 * n)   # floor(t2 * N) rows per sequence in T2


def test_t2_stream_equals_resident():
    w = _w32(layers=5)
    inp = Inputs(w)
    a, _, _ = _run_t2(w, inp, staging_layers=0, check_codec=False)
    b, st, _ = _run_t2(w, inp, staging_layers=2, check_codec=True)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert st["h2d_bytes"] > 0


def test_t2_fp32_cache():
    w = tkvsynth.CONFIGS["tiny"].replace(t2_ratio=0.15, steps=64)
    _run_t2(w, Inputs(w))


def test_t2_fp8_resident_parity_and_codec():
    w = _w32(t2_fp8=True)
    _run_t2(w, Inputs(w))


def test_t2_fp8_stream_equals_resident():
    w = _w32(layers=5, t2_fp8=True)
    inp = Inputs(w)
    a, _, _ = _run_t2(w, inp, staging_layers=0, check_codec=False)
    b, st, _ = _run_t2(w, inp, staging_layers=2, check_codec=True)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_t2_fp8_fp32_cache():
    w = tkvsynth.CONFIGS["tiny"].replace(t2_ratio=0.15, steps=64, t2_fp8=True)
    _run_t2(w, Inputs(w))


@pytest.mark.parametrize("fp8", [False, True], ids=["int8", "fp8"])
def test_t2_head_scales_resident_and_stream(fp8):
    w = _w32(layers=4, t2_fp8=fp8, t2_head_scales=True)
    inp = Inputs(w)
    a, _, _ = _run_t2(w, inp, staging_layers=0, check_codec=True)
    b, _, _ = _run_t2(w, inp, staging_layers=2, check_codec=True)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_t2_head_scales_fp32_cache():
    w = tkvsynth.CONFIGS["tiny"].replace(t2_ratio=0.15, steps=64, t2_head_scales=True)
    _run_t2(w, Inputs(w))
