"""GPU reassignment against the oracle, through the C ABI.

"Not All Thoughts Need HBM" (gist.science summary), Method §1 (tiers,
protected set), §3 (Proposition 1) and §4 (re-placement every Delta steps,
only changed rows move).

Checks:
  * tier labels and changed-row lists are bit-exact against the oracle's
    rules applied to the GPU's own fp32 scores (also for written scores full
    of ties and after earlier evictions);
  * a whole run with reassignments matches the oracle step by step
    (outputs within tolerance, scores relative 1e-4);
  * outputs, scores and evicted sets are bitwise identical across HBM
    ratios 30/50/70% at each eviction level, and between resident and
    stream staging.
"""
import numpy as np
import pytest
import torch

import oracle
import tkvsynth
from harness import Inputs, make_oracle, max_rel, to_device
from oracle import tiering

pytestmark = pytest.mark.gpu

TOL = {"bf16": 5e-3, "f32": 1e-5}


def _new(w, **kw):
    import decode_attention_tkv_amd as tkv
    return tkv.TieredKV.for_workload(w, **kw)


def _check_deltas(c, o_deltas, n):
    promote, demote, counts = c.read_deltas()
    for b, (op, od) in enumerate(o_deltas):
        gp = [(int(e["pos"]), int(e["old_tier"]), int(e["new_tier"])) for e in promote[b, : counts[b, 0]]]
        gd = [(int(e["pos"]), int(e["old_tier"]), int(e["new_tier"])) for e in demote[b, : counts[b, 1]]]
        assert gp == op, "promote list differs (seq %d)" % b
        assert gd == od, "demote list differs (seq %d)" % b


def run_parity(w, inp, steps, check_every=1, score_at=(), calls="two", groups=None, static=False, **kw):
    """Drive GPU and oracle together; at every reassignment the oracle ranks by
    the GPU's fp32 scores, its labels must equal the GPU's, then both go on.
    score_at: step counts after which the scores are also compared
    (relative 1e-4), besides the end of the run.  calls: "two" (tkv_append,
    then tkv_decode_attn over every layer), "one" (tkv_decode_step) or
    "groups" (tkv_append, then tkv_decode_attn over the layer groups of
    sizes `groups`, in order).  static: reassign with tkv_reassign_static
    (the scratch in the library's static device array) instead of
    tkv_reassign."""
    c = _new(w, **kw)
    if w.prefill:  # a workload with no prefill starts from an empty cache
        c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))
    o = make_oracle(w, inp)
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    outs = []
    worst = 0.0
    n_reassign = 0
    for t in range(steps):
        k, v = inp.step_kv(t)
        dq = to_device(inp.q[t], w.dtype)
        if calls == "one":
            c.decode_step(to_device(k, w.dtype), to_device(v, w.dtype), dq, out)
        else:
            c.append(to_device(k, w.dtype), to_device(v, w.dtype))
            if calls == "groups":
                lb = 0
                for g in groups:
                    c.decode_attn(dq[lb:lb + g], out[lb:lb + g], layer_begin=lb, layer_count=g)
                    lb += g
            else:
                c.decode_attn(dq, out)
        o.append(w.values(k), w.values(v))
        ref = o.attend(w.values(inp.q[t]))
        got = out.cpu().numpy()
        outs.append(got.copy())
        if t % check_every == 0 or t == steps - 1:
            worst = max(worst, float(np.max(np.abs(got - ref))))
        if t + 1 in score_at:
            rel = max_rel(c.read_scores()[:, : o.n], o.s[:, : o.n])
            assert rel <= 1e-4, "scores max-rel %.3g after %d steps" % (rel, t + 1)
        if (t + 1) % w.delta == 0:
            g_s = c.read_scores()[:, : o.n]
            if static:
                import decode_attention_tkv_amd as tkv
                tkv.tkv_reassign_static(c.h)
            else:
                c.reassign()
            tiers, deltas = o.reassign(rank_scores=g_s)
            assert np.array_equal(c.read_tiers()[:, : o.n], tiers), "labels differ at step %d" % (t + 1)
            _check_deltas(c, deltas, o.n)
            n_reassign += 1
    g_s = c.read_scores()
    st = c.stats()
    g_tiers = c.read_tiers()
    c.close()
    assert worst <= TOL[w.dtype], "out max-abs %.3g" % worst
    rel = max_rel(g_s[:, : o.n], o.s[:, : o.n])
    assert rel <= 1e-4, "scores max-rel %.3g" % rel
    return outs, g_s, g_tiers, st, o, n_reassign


def test_tiny_full_run_parity():
    w = tkvsynth.CONFIGS["tiny"]
    outs, s, tiers, st, o, nr = run_parity(w, Inputs(w), w.steps)
    assert nr == w.steps // w.delta
    n = o.n
    counts = [int((tiers[0, :n] == t).sum()) for t in range(4)]
    # floor(.3*544)=163 in T0, floor(.03*544)=16 evicted (Method §1 budgets)
    assert counts[0] == 163 and counts[3] == 16 and counts[2] == 0
    assert st["evictions"] == 16 and st["reassigns"] == nr


@pytest.mark.parametrize("name", ["tiny", "14b"])
def test_empty_cache_start(name):
    """No prefill: the cache grows from nothing by decode steps alone, with
    reassignments (T1 and eviction) once the protected window is outgrown."""
    if name == "tiny":
        w = tkvsynth.CONFIGS["tiny"].replace(prefill=0, prompt=0, sinks=2, recent=8, steps=64)
    else:  # bf16 grouped-query heads (matrix-core path), two sequences
        w = tkvsynth.CONFIGS["14b"].replace(layers=2, batch=2, prefill=0, prompt=0, sinks=4, recent=16,
                                            delta=32, steps=96)
    inp = Inputs(w)
    outs, s, tiers, st, o, nr = run_parity(w, inp, w.steps)
    assert nr == w.steps // w.delta
    # step 0 has one live row: its weight is exactly 1, so every query head
    # returns its kv head's v row unchanged
    v0 = w.values(inp.vn[:, :, 0])  # [L][B][Hkv][d]
    g = w.q_heads // w.kv_heads
    assert np.array_equal(outs[0].astype(np.float64), np.repeat(v0, g, axis=2))
    n = o.n
    for b in range(w.batch):
        counts = [int((tiers[b, :n] == t).sum()) for t in range(4)]
        assert counts[0] == int(w.hbm_ratio * n) and counts[3] == int(w.evict_ratio * n) and counts[1] > 0
        # each step's weights sum to 1 over the live rows; evicted scores stay frozen
        assert abs(float(np.sum(s[b, :n], dtype=np.float64)) - w.steps) <= 1e-4 * w.steps


def test_tiny_stream_staging_matches_resident():
    w = tkvsynth.CONFIGS["tiny"].replace(layers=5, steps=96)
    inp = Inputs(w)
    a = run_parity(w, inp, w.steps, check_every=4)
    b = run_parity(w, inp, w.steps, check_every=4, staging_layers=2)
    assert all(np.array_equal(x, y) for x, y in zip(a[0], b[0]))
    assert np.array_equal(a[1], b[1])
    assert b[3]["h2d_bytes"] > 0


@pytest.mark.parametrize("evict", [0.03, 0.10, 0.50])
def test_prop1_hbm_grid_bitwise(evict):
    """14B-shaped heads (40 q / 8 kv, bf16), trimmed to 3 layers x 2 sequences."""
    base = tkvsynth.CONFIGS["14b"].replace(layers=3, batch=2, prefill=700, steps=140, delta=32,
                                           evict_ratio=evict)
    inp = Inputs(base)
    runs = {}
    for h in (0.3, 0.5, 0.7):
        w = base.replace(hbm_ratio=h)
        runs[h] = run_parity(w, inp, w.steps, check_every=7)
    ref = runs[0.3]
    for h in (0.5, 0.7):
        r = runs[h]
        assert all(np.array_equal(x, y) for x, y in zip(ref[0], r[0])), "outputs differ at hbm %s" % h
        assert np.array_equal(ref[1], r[1])
        assert np.array_equal(ref[2] == 3, r[2] == 3)
    # the splits really differ
    t0 = [int((runs[h][2][:, : ref[4].n] == 0).sum()) for h in (0.3, 0.5, 0.7)]
    assert t0[0] < t0[1] <= t0[2]
    # Stream staging, where a row's HBM place does follow its tier (T0 pool
    # slot or the layer's staging slot, refilled from pinned memory each
    # step): outputs, scores and evicted sets bit for bit the same at every
    # ratio, and outputs and evicted sets the same as resident staging's (its
    # scores add Eq. 1's terms in another order, so agree to rounding only),
    # with the splits again different.
    t0s, sref = [], None
    for h in (0.3, 0.5, 0.7):
        s = run_parity(base.replace(hbm_ratio=h), inp, base.steps, check_every=7, staging_layers=2)
        assert all(np.array_equal(x, y) for x, y in zip(ref[0], s[0])), "stream outputs differ at hbm %s" % h
        assert np.array_equal(ref[2] == 3, s[2] == 3)
        if sref is None:
            sref = s
        assert np.array_equal(sref[1], s[1]) and np.array_equal(sref[2] == 3, s[2] == 3)
        assert s[3]["h2d_bytes"] > 0
        t0s.append(int((s[2][:, : ref[4].n] == 0).sum()))
    assert t0s[0] < t0s[1] <= t0s[2]


def test_labels_from_written_scores_with_ties():
    """Scores full of ties written straight into the cache, several rounds
    (so later rounds see earlier evictions)."""
    w = tkvsynth.CONFIGS["tiny"].replace(prefill=200, steps=8, hbm_ratio=0.4, evict_ratio=0.2,
                                         t2_ratio=0.0, prompt=8, sinks=4, recent=16, batch=3, delta=4)
    inp = Inputs(w)
    c = _new(w)
    c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))
    o = make_oracle(w, inp)
    rng = np.random.default_rng(7)
    levels = np.array([0.0, 1e-3, 0.5, 0.5000001, 2.0], np.float32)
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    for r in range(6):
        if r % 2 == 1:   # a decode step in between so positions and live rows move on
            t = r // 2
            k, v = inp.step_kv(t)
            c.append(to_device(k, w.dtype), to_device(v, w.dtype))
            o.append(w.values(k), w.values(v))
            c.decode_attn(to_device(inp.q[t], w.dtype), out)
            ref = o.attend(w.values(inp.q[t]))
            assert np.max(np.abs(out.cpu().numpy() - ref)) <= TOL[w.dtype]
        s = levels[rng.integers(0, len(levels), (w.batch, w.n_final))].astype(np.float32)
        if r == 4:
            s[:] = 0.25   # all equal
        c.write_scores(s)
        o.s[:, :] = s.astype(np.float64)
        c.reassign()
        tiers, deltas = o.reassign(rank_scores=s[:, : o.n].astype(np.float64))
        assert np.array_equal(c.read_tiers()[:, : o.n], tiers), "round %d" % r
        _check_deltas(c, deltas, o.n)
    c.close()


def test_7b_shape_with_reassignment():
    """7B-shaped heads (32/32, d128, bf16) with the 7B tier policy, 8 layers,
    two reassignments."""
    w = tkvsynth.CONFIGS["7b"].replace(layers=8, steps=129)
    run_parity(w, Inputs(w), w.steps, check_every=16)


@pytest.mark.parametrize("name", ["tiny", "32b_t2"])
def test_rows_keep_their_values_through_reassignments(name):
    """Resident staging keeps every live row at its own position: after each
    reassignment every live row reads back bit for bit as the oracle holds it
    (its appended values, or its dequantised values once it has entered T2)."""
    if name == "tiny":
        w = tkvsynth.CONFIGS["tiny"].replace(steps=48, delta=16)
    else:  # bf16 grouped-query heads with an 8-bit tier
        w = tkvsynth.CONFIGS["32b_t2"].replace(layers=2, batch=2, prefill=300, steps=64, delta=32, prompt=40,
                                               recent=32)
    inp = Inputs(w)
    c = _new(w)
    c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))
    o = make_oracle(w, inp)
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    checked = 0
    for t in range(w.steps):
        k, v = inp.step_kv(t)
        c.decode_step(to_device(k, w.dtype), to_device(v, w.dtype), to_device(inp.q[t], w.dtype), out)
        o.append(w.values(k), w.values(v))
        o.attend(w.values(inp.q[t]))
        if (t + 1) % w.delta:
            continue
        g_s = c.read_scores()[:, : o.n]
        c.reassign()
        tiers, _ = o.reassign(rank_scores=g_s)
        assert np.array_equal(c.read_tiers()[:, : o.n], tiers)
        for b in range(w.batch):
            for pos in range(o.n):
                if tiers[b, pos] > 2:
                    continue
                for l in range(w.layers):
                    gk, gv = c.read_kv(l, b, pos)
                    assert np.array_equal(w.values(gk), o.K[l, b, pos])
                    assert np.array_equal(w.values(gv), o.V[l, b, pos])
                    checked += 1
    c.close()
    assert checked > 0
