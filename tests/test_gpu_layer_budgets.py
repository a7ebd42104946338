"""Per-layer HBM budgets on the GPU against the oracle (OracleLayerGroups).

Layer l keeps floor(layer_hbm[l] N) rows in HBM.  Consecutive layers with one
ratio form a group, placed by Method §1 with its own ratio.  Every group ranks
by the one Eq. 1 score over all layers and shares the eviction and T2 ratios
("Not All Thoughts Need HBM", gist.science summary, Method §1, §2, §4;
per-layer ratios in the spirit of the ARKV summary, Method).  Checked step by
step: outputs within the dtype's tolerance, scores within relative 1e-4, at
every reassignment each group's labels bit-exact against its own rule applied
to the GPU's fp32 scores, every layer of a group with the group's labels, and
the same evicted rows in every group (so the outputs never depend on the
ratios: Method §3, Proposition 1)."""
import numpy as np
import pytest
import torch

import oracle
import tkvsynth
from harness import Inputs, max_rel, to_device
from oracle import T0, T3, tiering
from test_gpu_reassign import TOL

pytestmark = pytest.mark.gpu


def run_layers(w, layer_hbm, staging_layers=0, calls="one", groups=None, check_every=2, static=False,
               scored=False):
    import decode_attention_tkv_amd as tkv
    print("[layer budgets] %s ratios %s staging %d calls %s %s static %s scored %s"
          % (w, layer_hbm, staging_layers, calls, groups, static, scored), flush=True)
    inp = Inputs(w)
    c = tkv.TieredKV.for_workload(w, staging_layers=staging_layers, layer_hbm=layer_hbm)
    o = oracle.OracleLayerGroups.for_workload(w, layer_hbm)
    dk, dv = to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype)
    if scored:
        # the prompt's causal attention over all layers gives the shared
        # scores; every group is then re-placed by them (ranked here by the
        # GPU's fp32 scores, as the decode checks do)
        from test_gpu_prefill import _prefill_q
        qp = _prefill_q(w)
        c.prefill_scored(dk, dv, to_device(qp, w.dtype))
        o.prefill(w.values(inp.k0), w.values(inp.v0))
        n = o.n
        g_s = c.read_scores()[:, :n]
        o.s[:, :n] = oracle.prefill_scores(w.values(inp.k0), w.values(qp), n)
        assert max_rel(g_s, o.s[:, :n]) <= 1e-4
        o.reassign(rank_scores=g_s)
    else:
        c.prefill(dk, dv)
        o.prefill(w.values(inp.k0), w.values(inp.v0))
    n = o.n
    for l in range(w.layers):
        assert np.array_equal(c.read_layer_tiers(l)[:, :n], o.tier_of(l)[:, :n]), "placement of layer %d" % l
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    worst, n_reassign = 0.0, 0
    for t in range(w.steps):
        k, v = inp.step_kv(t)
        dq = to_device(inp.q[t], w.dtype)
        if calls == "one":
            c.decode_step(to_device(k, w.dtype), to_device(v, w.dtype), dq, out)
        else:
            c.append(to_device(k, w.dtype), to_device(v, w.dtype))
            lb = 0
            for g in groups or [w.layers]:
                c.decode_attn(dq[lb:lb + g].contiguous(), out[lb:lb + g], layer_begin=lb, layer_count=g)
                lb += g
        o.append(w.values(k), w.values(v))
        ref = o.attend(w.values(inp.q[t]))
        if t % check_every == 0 or t == w.steps - 1:
            worst = max(worst, float(np.max(np.abs(out.cpu().numpy() - ref))))
        if (t + 1) % w.delta == 0:
            n = o.n
            g_s = c.read_scores()[:, :n]
            rel = max_rel(g_s, o.s[:, :n])
            assert rel <= 1e-4, "scores max-rel %.3g at step %d" % (rel, t + 1)
            old = [c.read_layer_tiers(l0)[:, :n] for (l0, _, _) in o.groups]
            if static:
                tkv.tkv_reassign_static(c.h)
            else:
                c.reassign()
            new = []
            for g, (l0, l1, h) in enumerate(o.groups):
                got = c.read_layer_tiers(l0)[:, :n]
                for b in range(w.batch):
                    ref_t = tiering.reassign(old[g][b], g_s[b], n, w.prompt, w.sinks, w.recent, h,
                                             w.evict_ratio, w.t2_ratio)
                    assert np.array_equal(got[b], ref_t), "labels of group %d differ at step %d" % (g, t + 1)
                for l in range(l0, l1):
                    assert np.array_equal(c.read_layer_tiers(l)[:, :n], got)
                assert np.array_equal(got == T3, new[0] == T3) if new else True, "groups evict different rows"
                new.append(got)
            o.reassign(rank_scores=g_s, adopt=new)
            n_reassign += 1
            # the values attention reads for sampled live rows of every layer (T2 rows as their
            # dequantised values; with stream staging those exist only as codes) are the oracle's,
            # bit for bit
            rng = np.random.default_rng(t)
            for l in range(w.layers):
                g, ll = o.part_of(l)
                tier = o.parts[g].tier
                for b in range(w.batch):
                    live = np.nonzero(tier[b, :n] < (2 if staging_layers else 3))[0]
                    for pos in rng.choice(live, size=min(4, len(live)), replace=False):
                        gk, gv = c.read_kv(l, b, int(pos))
                        assert np.array_equal(w.values(gk), o.parts[g].K[ll, b, pos])
                        assert np.array_equal(w.values(gv), o.parts[g].V[ll, b, pos])
    rel = max_rel(c.read_scores()[:, : o.n], o.s[:, : o.n])
    st = c.stats()
    c.close()
    assert worst <= TOL[w.dtype], "out max-abs %.3g" % worst
    assert rel <= 1e-4, "scores max-rel %.3g" % rel
    return st, o, n_reassign


def _w(dtype, group, layers, **kw):
    base = dict(dtype=dtype, head_dim=128 if dtype == "bf16" else 64, kv_heads=2, q_heads=2 * group,
                layers=layers, batch=2, prefill=300, steps=40, delta=16, prompt=16, sinks=4, recent=24,
                evict_ratio=0.08, hbm_ratio=0.5)
    base.update(kw)
    return tkvsynth.CONFIGS["tiny"].replace(**base)


CASES = [
    # (dtype, group, layers, ratios, staging, t2, calls, groups)
    ("f32", 1, 6, [0.2, 0.2, 0.5, 0.5, 0.8, 0.8], 0, 0.0, "one", None),
    ("bf16", 5, 6, [0.8, 0.8, 0.3, 0.3, 0.3, 0.55], 0, 0.0, "one", None),
    ("bf16", 1, 9, [0.2] * 3 + [0.5] * 3 + [0.8] * 3, 2, 0.0, "one", None),
    ("bf16", 4, 8, [0.7] * 4 + [0.25] * 4, 3, 0.1, "two", [3, 2, 3]),
    ("f32", 2, 6, [0.3, 0.3, 0.6, 0.6, 0.9, 0.9], 0, 0.15, "two", [2, 3, 1]),
    ("bf16", 8, 5, [0.4, 0.1, 0.1, 0.9, 0.4], 0, 0.1, "one", None),
]


@pytest.mark.parametrize("case", CASES, ids=["%s-g%d-L%d-S%d-t2%.2f-%s" % (c[0], c[1], c[2], c[4], c[5], c[6])
                                             for c in CASES])
def test_layer_budgets_parity(case):
    dtype, group, layers, ratios, staging, t2, calls, groups = case
    w = _w(dtype, group, layers, t2_ratio=t2)
    st, o, nr = run_layers(w, ratios, staging_layers=staging, calls=calls, groups=groups)
    assert nr == w.steps // w.delta
    # the groups' T0 shares differ as their ratios do; the evicted rows are the same
    n = o.n
    t0 = {h: int((o.parts[g].tier[:, :n] == T0).sum()) for g, (_, _, h) in enumerate(o.groups)}
    hs = sorted(t0)
    assert all(t0[a] < t0[b] for a, b in zip(hs, hs[1:])), t0
    assert st["evictions"] > 0 and st["reassigns"] == nr


def test_layer_budgets_static_reassign_and_scored_prefill():
    w = _w("bf16", 4, 6, prefill=200, steps=33)
    run_layers(w, [0.25, 0.25, 0.25, 0.75, 0.75, 0.75], static=True, scored=True)


def test_layer_budgets_outputs_equal_one_budget_until_ranking_differs():
    """Before the first reassignment every row is live in both, so the
    outputs of the per-layer handle equal the one-budget handle's bit for bit
    (Proposition 1; the attention of a layer never depends on which handle or
    group holds it)."""
    import decode_attention_tkv_amd as tkv
    w = _w("bf16", 5, 6, steps=15)
    inp = Inputs(w)
    outs = []
    for lh in (None, [0.2, 0.2, 0.6, 0.6, 0.9, 0.9]):
        c = tkv.TieredKV.for_workload(w, layer_hbm=lh)
        c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))
        out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
        got = []
        for t in range(w.steps):
            k, v = inp.step_kv(t)
            c.decode_step(to_device(k, w.dtype), to_device(v, w.dtype), to_device(inp.q[t], w.dtype), out)
            got.append(out.cpu().numpy())
        c.close()
        outs.append(got)
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_layer_budgets_hbm_in_stream_staging():
    """Stream staging: each group's T0 pool is sized by its own ratio, so the
    HBM the handle holds lies between the one-budget handles at the lowest and
    the highest ratio, and is the sum over the groups (each with its own
    staging slots)."""
    import decode_attention_tkv_amd as tkv
    w = _w("bf16", 1, 12, steps=1)
    ratios = [0.2] * 4 + [0.5] * 4 + [0.8] * 4
    hb = {}
    for name, kw in (("low", dict(hbm_ratio=0.2)), ("high", dict(hbm_ratio=0.8)), ("layers", dict(layer_hbm=ratios))):
        c = tkv.TieredKV.for_workload(w, staging_layers=2, **kw)
        hb[name] = c.stats()["hbm_bytes"]
        c.close()
    parts = 0
    for h in (0.2, 0.5, 0.8):
        c = tkv.TieredKV.for_workload(w.replace(layers=4), staging_layers=2, hbm_ratio=h)
        parts += c.stats()["hbm_bytes"]
        c.close()
    assert hb["low"] < hb["layers"] < hb["high"], hb
    assert hb["layers"] == parts


def test_layer_budgets_errors():
    import decode_attention_tkv_amd as tkv
    w = _w("f32", 1, 6, steps=4)
    c = tkv.TieredKV.for_workload(w, layer_hbm=[0.2, 0.2, 0.5, 0.5, 0.8, 0.8])
    with pytest.raises(tkv.TkvError):
        c.read_layer_tiers(6)
    inp = Inputs(w)
    c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))
    k, v = inp.step_kv(0)
    c.append(to_device(k, w.dtype), to_device(v, w.dtype))
    with pytest.raises(tkv.TkvError) as e:
        c.reassign()  # between the layer groups of a step
    assert e.value.code == tkv.TKV_ESTATE
    dq = to_device(inp.q[0], w.dtype)
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    with pytest.raises(tkv.TkvError) as e:  # out of order
        c.decode_attn(dq[1:3].contiguous(), out[1:3], layer_begin=1, layer_count=2)
    assert e.value.code == tkv.TKV_ESTATE
    c.decode_attn(dq, out)
    c.reassign()
    c.close()


@pytest.mark.timeout(900)
def test_layer_budgets_14b_full_shape():
    """The 14B shape (48 layers, 40 q / 8 kv heads, bf16, 4 sequences, 4096
    prefilled positions) with three groups of 16 layers at HBM ratios 0.3,
    0.5 and 0.7, through one reassignment.  Sequences are independent (Method
    §1, §2), so an oracle over every layer of one sequence is exact for it:
    its outputs and scores are compared every 16 steps.  Every sequence's
    labels in every group are re-derived from the GPU's fp32 scores."""
    import decode_attention_tkv_amd as tkv
    w = tkvsynth.CONFIGS["14b"].replace(steps=65)
    ratios = [0.3] * 16 + [0.5] * 16 + [0.7] * 16
    seq = 1
    print("[layer budgets 14b] drawing inputs", flush=True)
    inp = Inputs(w)
    c = tkv.TieredKV.for_workload(w, layer_hbm=ratios)
    c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))
    o = oracle.OracleLayerGroups(ratios, w.q_heads, w.kv_heads, w.head_dim, 1, w.n_final, w.delta, w.evict_ratio,
                                 w.t2_ratio, w.prompt, w.sinks, w.recent, True)
    o.prefill(w.values(inp.k0[:, [seq]]), w.values(inp.v0[:, [seq]]))
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    worst = 0.0
    for t in range(w.steps):
        k, v = inp.step_kv(t)
        c.decode_step(to_device(k, w.dtype), to_device(v, w.dtype), to_device(inp.q[t], w.dtype), out)
        o.append(w.values(k[:, [seq]]), w.values(v[:, [seq]]))
        ref = o.attend(w.values(inp.q[t][:, [seq]]))
        if t % 16 == 0 or t == w.steps - 1:
            worst = max(worst, float(np.max(np.abs(out.cpu().numpy()[:, [seq]] - ref))))
            print("[layer budgets 14b] step %d: max |out - oracle| %.3g" % (t + 1, worst), flush=True)
        if (t + 1) % w.delta == 0:
            n = o.n
            g_s = c.read_scores()[:, :n]
            assert max_rel(g_s[[seq]], o.s[:, :n]) <= 1e-4
            old = [c.read_layer_tiers(l0)[:, :n] for (l0, _, _) in o.groups]
            c.reassign()
            new = []
            for g, (l0, l1, h) in enumerate(o.groups):
                got = c.read_layer_tiers(l0)[:, :n]
                for b in range(w.batch):
                    ref_t = tiering.reassign(old[g][b], g_s[b], n, w.prompt, w.sinks, w.recent, h, w.evict_ratio,
                                             w.t2_ratio)
                    assert np.array_equal(got[b], ref_t), "labels of group %d, sequence %d" % (g, b)
                new.append(got)
                assert np.array_equal(got == T3, new[0] == T3)
            o.reassign(rank_scores=g_s[[seq]], adopt=[x[[seq]] for x in new])
    rel = max_rel(c.read_scores()[[seq], : o.n], o.s[:, : o.n])
    st = c.stats()
    c.close()
    assert worst <= 5e-3 and rel <= 1e-4, (worst, rel)
    assert st["reassigns"] == 1 and st["evictions"] > 0
