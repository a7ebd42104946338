"""Scored prefill on the GPU against the oracle, through the C ABI.

The prompt's causal attention weights, averaged over layers and query heads,
become the starting scores (Eq. 1 of "Not All Thoughts Need HBM",
gist.science summary, Method §2, applied to the prompt); every row is then
re-placed by them with the full tier rules (Method §1, §4).

Checks: the scores within relative 1e-4 of the oracle's fp64 ones; the
labels and changed-row lists bit-exact against the oracle's rules applied
to the GPU's fp32 scores; decode steps after it in parity (outputs within
tolerance, scores relative 1e-4, labels bit-exact at each reassignment).
"""
import numpy as np
import pytest
import torch

import oracle
import tkvsynth
from harness import Inputs, max_rel, to_device
from test_gpu_reassign import TOL, _check_deltas

pytestmark = pytest.mark.gpu


def _prefill_q(w):
    """Queries of the prompt positions: [L][B][n][Hq][d] (drawn past the decode steps' ones)."""
    q = w.q(w.steps, w.prefill, w.unit_vector())          # [n][L][B][Hq][d]
    return np.ascontiguousarray(np.moveaxis(q, 0, 2))


def run_scored(w, steps, check_every=1, **kw):
    import decode_attention_tkv_amd as tkv
    inp = Inputs(w)
    qp = _prefill_q(w)
    c = tkv.TieredKV.for_workload(w, **kw)
    c.prefill_scored(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype), to_device(qp, w.dtype))
    n = w.prefill
    g_s = c.read_scores()[:, :n]
    o = oracle.OracleTKV.for_workload(w)
    o.prefill(w.values(inp.k0), w.values(inp.v0))
    ref_s = oracle.prefill_scores(w.values(inp.k0), w.values(qp), n)
    assert max_rel(g_s, ref_s) <= 1e-4, "prefill scores max-rel %.3g" % max_rel(g_s, ref_s)
    o.s[:, :n] = ref_s
    tiers, deltas = o.reassign(rank_scores=g_s)
    assert np.array_equal(c.read_tiers()[:, :n], tiers)
    _check_deltas(c, deltas, n)
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    worst = 0.0
    for t in range(steps):
        k, v = inp.step_kv(t)
        c.append(to_device(k, w.dtype), to_device(v, w.dtype))
        o.append(w.values(k), w.values(v))
        c.decode_attn(to_device(inp.q[t], w.dtype), out)
        ref = o.attend(w.values(inp.q[t]))
        if t % check_every == 0 or t == steps - 1:
            worst = max(worst, float(np.max(np.abs(out.cpu().numpy() - ref))))
        if (t + 1) % w.delta == 0:
            gs = c.read_scores()[:, : o.n]
            c.reassign()
            tiers, deltas = o.reassign(rank_scores=gs)
            assert np.array_equal(c.read_tiers()[:, : o.n], tiers), "labels differ at step %d" % (t + 1)
            _check_deltas(c, deltas, o.n)
    s = c.read_scores()
    st = c.stats()
    c.close()
    assert worst <= TOL[w.dtype], "out max-abs %.3g" % worst
    assert max_rel(s[:, : o.n], o.s[:, : o.n]) <= 1e-4
    return st, ref_s


def test_scored_prefill_tiny_fp32():
    w = tkvsynth.CONFIGS["tiny"].replace(steps=48, prompt=8, recent=16)
    st, s = run_scored(w, w.steps)
    assert st["reassigns"] == 1 + w.steps // w.delta
    assert abs(s.sum() - w.prefill * w.batch) < 1e-6


def test_scored_prefill_7b_shape():
    w = tkvsynth.CONFIGS["7b"].replace(layers=2, prefill=600, steps=65, prompt=40)
    run_scored(w, w.steps, check_every=8)


def test_scored_prefill_gqa_t2_stream():
    w = tkvsynth.CONFIGS["32b_t2"].replace(layers=3, batch=2, prefill=500, steps=33, delta=32, prompt=40,
                                           recent=64)
    st, _ = run_scored(w, w.steps, check_every=8, staging_layers=2)
    assert st["tier_count"][2] > 0


PCASES = [(dt, d, g) for dt in ("bf16", "f32") for d in (64, 128) for g in (1, 5, 8)]


@pytest.mark.parametrize("dtype,head_dim,group", PCASES, ids=["%s-d%d-g%d" % c for c in PCASES])
def test_scored_prefill_each_path(dtype, head_dim, group):
    # 229 positions: ragged against the 16-, 32- and 128-row tiles of the scoring passes
    w = tkvsynth.CONFIGS["tiny"].replace(dtype=dtype, head_dim=head_dim, kv_heads=2, q_heads=2 * group, layers=2,
                                         batch=2, prefill=229, steps=9, delta=8, prompt=8, recent=16)
    run_scored(w, w.steps)
