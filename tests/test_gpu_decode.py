"""GPU parity of the decode step (append + split-K attention + Eq. 1 scores)
against the fp64 oracle, through the C ABI.

Tolerances: bf16 caches, output max-abs <= 5e-3 (fp32 accumulation of bf16
inputs); fp32 caches, <= 1e-5; scores, max relative error <= 1e-4.  Runs at
different HBM ratios (T0/T1 splits of the same rows) must agree bit for bit
(Proposition 1 of "Not All Thoughts Need HBM", Method §3).
"""
import numpy as np
import pytest
import torch

import tkvsynth
from harness import Inputs, make_oracle, max_rel, to_device

pytestmark = pytest.mark.gpu

TOL = {"bf16": 5e-3, "f32": 1e-5}


def _run(w, inputs, steps, hbm=None, chunk=0, groups=None, check=None, staging_layers=0):
    import decode_attention_tkv_amd as tkv
    kw = {} if hbm is None else {"hbm_ratio": hbm}
    c = tkv.TieredKV.for_workload(w, chunk=chunk, staging_layers=staging_layers, **kw)
    c.prefill(to_device(inputs.k0, w.dtype), to_device(inputs.v0, w.dtype))
    outs = []
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    for t in range(steps):
        k, v = inputs.step_kv(t)
        c.append(to_device(k, w.dtype), to_device(v, w.dtype))
        q = to_device(inputs.q[t], w.dtype)
        if groups is None:
            c.decode_attn(q, out)
        else:
            lb = 0
            for g in groups:
                c.decode_attn(q[lb:lb + g].contiguous(), out[lb:lb + g], layer_begin=lb, layer_count=g)
                lb += g
        outs.append(out.cpu().numpy().copy())
    torch.cuda.synchronize()
    s = c.read_scores()
    tiers = c.read_tiers()
    c.close()
    return outs, s, tiers


def _oracle(w, inputs, steps):
    o = make_oracle(w, inputs)
    outs = []
    for t in range(steps):
        k, v = inputs.step_kv(t)
        o.append(w.values(k), w.values(v))
        outs.append(o.attend(w.values(inputs.q[t])))
    return outs, o


def _compare(w, gpu, ora, steps):
    g_outs, g_s, _ = gpu
    o_outs, o = ora
    tol = TOL[w.dtype]
    for t in range(steps):
        err = np.max(np.abs(g_outs[t] - o_outs[t]))
        assert err <= tol, "step %d: out max-abs %.3g > %.3g" % (t, err, tol)
    n = o.n
    rel = max_rel(g_s[:, :n], o.s[:, :n])
    assert rel <= 1e-4, "scores max-rel %.3g" % rel


def test_tiny_all_t0_parity():
    w = tkvsynth.CONFIGS["tiny"].replace(hbm_ratio=1.0, evict_ratio=0.0)
    inp = Inputs(w)
    steps = 64
    _compare(w, _run(w, inp, steps), _oracle(w, inp, steps), steps)


def test_tiny_hbm_split_bitwise():
    w = tkvsynth.CONFIGS["tiny"]
    inp = Inputs(w)
    steps = 48
    runs = [_run(w, inp, steps, hbm=h) for h in (0.3, 0.5, 1.0)]
    for r in runs[1:]:
        assert all(np.array_equal(a, b) for a, b in zip(runs[0][0], r[0]))
        assert np.array_equal(runs[0][1], r[1])
    _compare(w, runs[0], _oracle(w, inp, steps), steps)
    # the prefill placed the two splits differently
    assert (runs[0][2][0, : w.prefill] == 1).sum() > (runs[1][2][0, : w.prefill] == 1).sum() > 0


@pytest.mark.parametrize("chunk", [128, 256, 512])
def test_chunk_sizes_and_layer_groups(chunk):
    w = tkvsynth.CONFIGS["14b"].replace(layers=6, batch=2, prefill=1000, steps=3, hbm_ratio=0.5)
    inp = Inputs(w)
    a = _run(w, inp, 3, chunk=chunk)
    b = _run(w, inp, 3, chunk=chunk, groups=[1, 2, 3])
    assert all(np.array_equal(x, y) for x, y in zip(a[0], b[0]))
    assert np.array_equal(a[1], b[1])
    _compare(w, a, _oracle(w, inp, 3), 3)


@pytest.mark.parametrize("slots,groups", [(2, [1, 2, 3]), (4, [1, 2, 3]), (4, [3, 1, 3]), (6, [2, 5])],
                         ids=["S2", "S4", "S4_odd_groups", "S6_odd_layers"])
def test_layer_groups_stream_staging(slots, groups):
    # stream staging prefetches each layer's T1 rows ahead of its attention,
    # across the caller's layer groups (with an even S >= 4, two layers per
    # copy, issued once both slots are free); outputs equal the resident
    # single call's bit for bit (the reduction follows logical position,
    # whatever the staging)
    w = tkvsynth.CONFIGS["14b"].replace(layers=sum(groups), batch=2, prefill=1000, steps=3, hbm_ratio=0.5)
    inp = Inputs(w)
    a = _run(w, inp, 3)
    b = _run(w, inp, 3, groups=groups, staging_layers=slots)
    assert all(np.array_equal(x, y) for x, y in zip(a[0], b[0]))
    _compare(w, b, _oracle(w, inp, 3), 3)


@pytest.mark.parametrize("name", ["7b", "14b", "32b", "70b"])
def test_shapes_short_run(name):
    """Head layout, GQA group and dtype of each workload, on a short cache with
    a ragged last chunk (layers and batch trimmed so the oracle stays quick)."""
    base = tkvsynth.CONFIGS[name]
    w = base.replace(layers=min(base.layers, 4), batch=min(base.batch, 2), prefill=1283, steps=4)
    inp = Inputs(w)
    _compare(w, _run(w, inp, 4), _oracle(w, inp, 4), 4)


def test_7b_full_shape_few_steps():
    steps = 3
    w = tkvsynth.CONFIGS["7b"].replace(steps=steps)
    inp = Inputs(w)
    a = _run(w, inp, steps)
    b = _run(w, inp, steps, hbm=1.0)
    assert all(np.array_equal(x, y) for x, y in zip(a[0], b[0]))
    _compare(w, a, _oracle(w, inp, steps), steps)


def test_single_row_cache():
    w = tkvsynth.CONFIGS["tiny"].replace(prefill=1, steps=2, prompt=0, recent=0, sinks=0)
    inp = Inputs(w)
    g = _run(w, inp, 2)
    o = _oracle(w, inp, 2)
    _compare(w, g, o, 2)
