"""Full-size workloads on the GPU, checked against the oracle.

The 7B, 14B, 32B, 32B with the 8-bit tier, and 70B workloads run at their real
shapes and cache sizes through one reassignment; the 70B one also in its
defining mode, stream staging, where about two thirds of the rows live in
pinned host memory and every step copies each layer's T1 rows to the GPU
one layer ahead.

Sequences are independent ("Not All Thoughts Need HBM", gist.science
summary, Method §2: Eq. 1 sums over the layers and heads of one sequence;
Method §1: each sequence is ranked on its own), so an oracle that follows
every layer of one sequence is exact for that sequence: it runs every step,
and its outputs and scores (relative 1e-4) are compared with the GPU's.
Where that is too costly (70B) the oracle follows sampled layers and
sequences for the outputs, and the score increments of a step are checked
against the invariant that holds at any size: they sum to 1 over the live
rows of each sequence (Eq. 1).  Every sequence's tier labels are re-derived
from the GPU's fp32 scores and compared bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import tkvsynth
from harness import Inputs, max_rel, to_device
from oracle import tiering

pytestmark = pytest.mark.gpu


def _oracle(w, layers, seqs, inp):
    o = oracle.OracleTKV(len(layers), w.q_heads, w.kv_heads, w.head_dim, len(seqs), w.n_final, w.delta,
                         w.hbm_ratio, w.evict_ratio, w.t2_ratio, w.prompt, w.sinks, w.recent, w.dtype == "bf16",
                         t2_fp8=w.t2_fp8, t2_head_scales=w.t2_head_scales)
    o.prefill(w.values(inp.k0[layers][:, seqs]), w.values(inp.v0[layers][:, seqs]))
    return o


def run_full(w, layers, seqs, sample_every, staging_layers=0, full_seq=None):
    """layers, seqs: what the sampled oracle follows (outputs every
    sample_every steps); full_seq: a sequence followed in every layer and
    every step (outputs at the sampled steps, scores at each reassignment
    and at the end), or None."""
    import decode_attention_tkv_amd as tkv
    print("[fullsize] %s (staging %d): drawing inputs" % (w.name, staging_layers), flush=True)
    inp = Inputs(w)
    c = tkv.TieredKV.for_workload(w, staging_layers=staging_layers)
    c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))
    ls, bs = list(layers), list(seqs)
    o = _oracle(w, ls, bs, inp)
    allL = list(range(w.layers))
    of = _oracle(w, allL, [full_seq], inp) if full_seq is not None else None
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    worst, worst_full, s_rel, checked = 0.0, 0.0, 0.0, 0
    for t in range(w.steps):
        k, v = inp.step_kv(t)
        c.append(to_device(k, w.dtype), to_device(v, w.dtype))
        o.append(w.values(k[ls][:, bs]), w.values(v[ls][:, bs]))
        sample = t % sample_every == 0 or t == w.steps - 1
        if sample:
            s0 = c.read_scores().astype(np.float64)
            live0 = c.read_tiers() < 3
        c.decode_attn(to_device(inp.q[t], w.dtype), out)
        if of is not None:
            of.append(w.values(k[:, [full_seq]]), w.values(v[:, [full_seq]]))
            ref_f = of.attend(w.values(inp.q[t][:, [full_seq]]))
        if sample:
            got_all = out.cpu().numpy()
            got = got_all[ls][:, bs]
            q = w.values(inp.q[t][ls][:, bs])
            ref, _ = oracle.attend(o.K, o.V, o.live(), q, o.n)
            worst = max(worst, float(np.max(np.abs(got - ref))))
            if of is not None:
                worst_full = max(worst_full, float(np.max(np.abs(got_all[:, [full_seq]] - ref_f))))
            checked += 1
            s1 = c.read_scores().astype(np.float64)
            inc = np.where(live0, s1 - s0, 0.0)
            assert np.all(np.abs(inc.sum(axis=1) - 1.0) < 1e-3), inc.sum(axis=1)
            assert np.all(np.where(live0, 0.0, s1 - s0) == 0.0)
            print("[fullsize] %s step %d: max |out - oracle| %.3g (sampled), %.3g (sequence %s, all layers)"
                  % (w.name, t + 1, worst, worst_full, full_seq), flush=True)
        if (t + 1) % w.delta == 0:
            g_s = c.read_scores()[:, : o.n].astype(np.float64)
            if of is not None:
                s_rel = max(s_rel, max_rel(g_s[[full_seq]], of.s[:, : of.n]))
            old = c.read_tiers()[:, : o.n]
            c.reassign()
            new = c.read_tiers()[:, : o.n]
            for b in range(w.batch):
                ref_t = tiering.reassign(old[b], g_s[b], o.n, w.prompt, w.sinks, w.recent,
                                         w.hbm_ratio, w.evict_ratio, w.t2_ratio)
                assert np.array_equal(new[b], ref_t), "labels differ (seq %d)" % b
            o.reassign(rank_scores=g_s[bs], adopt=new[bs])
            if of is not None:
                of.reassign(rank_scores=g_s[[full_seq]], adopt=new[[full_seq]])
    if of is not None:
        s_rel = max(s_rel, max_rel(c.read_scores()[[full_seq], : of.n], of.s[:, : of.n]))
    st = c.stats()
    c.close()
    print("[fullsize] %s: %d sampled steps, max |out - oracle| = %.3g / %.3g, scores max-rel %.3g"
          % (w.name, checked, worst, worst_full, s_rel), flush=True)
    assert worst <= 5e-3 and worst_full <= 5e-3
    assert s_rel <= 1e-4
    return st


@pytest.mark.timeout(900)
def test_7b_full_size():
    """The 7B workload at its real shape (32 layers, 32 kv heads, one query
    head each, logits summed over 32 heads per layer), its one sequence
    followed by the oracle in every layer."""
    w = tkvsynth.CONFIGS["7b"].replace(steps=66)
    st = run_full(w, layers=(0, 31), seqs=(0,), sample_every=16, full_seq=0)
    assert st["reassigns"] == 1 and st["tier_count"][3] > 0


@pytest.mark.timeout(900)
def test_14b_full_size():
    w = tkvsynth.CONFIGS["14b"].replace(steps=65)
    st = run_full(w, layers=(0, 47), seqs=(0, 3), sample_every=16, full_seq=2)
    assert st["reassigns"] == 1 and st["tier_count"][3] > 0


@pytest.mark.timeout(900)
def test_32b_full_size():
    """The plain 32B workload: HBM 30%, eviction 5%, no 8-bit tier."""
    w = tkvsynth.CONFIGS["32b"].replace(steps=65)
    st = run_full(w, layers=(0, 63), seqs=(0, 7), sample_every=16, full_seq=5)
    n = w.prefill + 64
    assert st["reassigns"] == 1 and st["tier_count"][2] == 0
    assert st["tier_count"][3] == w.batch * int(0.05 * n)


@pytest.mark.timeout(900)
def test_32b_t2_full_size():
    w = tkvsynth.CONFIGS["32b_t2"].replace(steps=65)
    st = run_full(w, layers=(0, 63), seqs=(0, 7), sample_every=16, full_seq=3)
    assert st["tier_count"][2] == w.batch * int(0.2 * (w.prefill + 64))


@pytest.mark.timeout(1200)
def test_70b_full_size():
    w = tkvsynth.CONFIGS["70b"].replace(steps=65)
    st = run_full(w, layers=(0, 79), seqs=(0, 7), sample_every=16)
    assert st["reassigns"] == 1


@pytest.mark.timeout(1200)
def test_70b_full_size_stream_staging():
    """70B in stream staging (two HBM slots): each step copies every layer's
    T1 rows from pinned host memory one layer ahead of its attention, and the
    reassignment moves rows in and out of the pinned arenas."""
    w = tkvsynth.CONFIGS["70b"].replace(steps=66)
    st = run_full(w, layers=(0, 41, 79), seqs=(0, 5), sample_every=16, staging_layers=2)
    assert st["reassigns"] == 1 and st["h2d_bytes"] > 0
    # about two thirds of the K/V lives in pinned host memory, not in HBM
    assert st["host_bytes"] > 0.6 * st["full_cache_bytes"] and st["hbm_bytes"] < 0.4 * st["full_cache_bytes"]
