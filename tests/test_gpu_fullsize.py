"""Full-size workloads on the GPU, checked against the oracle on samples.

The 14B, 32B (with the 8-bit tier) and 70B workloads run at their real
shapes and cache sizes through one reassignment.  The oracle cannot redo
every layer of every sequence at these sizes, so it follows sampled layers
and sequences: it re-derives the tier labels of every sequence from the
GPU's fp32 scores (bit-exact check), adopts them for the sampled sequences
(applying its own codec to rows entering T2) and recomputes the sampled
outputs.  The score increments of a step are checked against the invariant
that holds at any size: they sum to 1 over the live rows of each sequence
("Not All Thoughts Need HBM", gist.science summary, Method §2, Eq. 1).
"""
import numpy as np
import pytest
import torch

import oracle
import tkvsynth
from harness import Inputs, to_device
from oracle import tiering

pytestmark = pytest.mark.gpu


def run_sampled(w, layers, seqs, sample_every, staging_layers=0):
    import decode_attention_tkv_amd as tkv
    print("[fullsize] %s: drawing inputs" % w.name, flush=True)
    inp = Inputs(w)
    c = tkv.TieredKV.for_workload(w, staging_layers=staging_layers)
    k0, v0 = to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype)
    c.prefill(k0, v0)
    ls, bs = list(layers), list(seqs)
    o = oracle.OracleTKV(len(ls), w.q_heads, w.kv_heads, w.head_dim, len(bs), w.n_final, w.delta,
                         w.hbm_ratio, w.evict_ratio, w.t2_ratio, w.prompt, w.sinks, w.recent, w.dtype == "bf16")
    o.prefill(w.values(inp.k0[ls][:, bs]), w.values(inp.v0[ls][:, bs]))
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    worst, checked = 0.0, 0
    for t in range(w.steps):
        k, v = inp.step_kv(t)
        c.append(to_device(k, w.dtype), to_device(v, w.dtype))
        o.append(w.values(k[ls][:, bs]), w.values(v[ls][:, bs]))
        sample = t % sample_every == 0 or t == w.steps - 1
        if sample:
            s0 = c.read_scores().astype(np.float64)
            live0 = c.read_tiers() < 3
        c.decode_attn(to_device(inp.q[t], w.dtype), out)
        if sample:
            got = out.cpu().numpy()[ls][:, bs]
            q = w.values(inp.q[t][ls][:, bs])
            ref, _ = oracle.attend(o.K, o.V, o.live(), q, o.n)
            worst = max(worst, float(np.max(np.abs(got - ref))))
            checked += 1
            s1 = c.read_scores().astype(np.float64)
            inc = np.where(live0, s1 - s0, 0.0)
            assert np.all(np.abs(inc.sum(axis=1) - 1.0) < 1e-3), inc.sum(axis=1)
            assert np.all(np.where(live0, 0.0, s1 - s0) == 0.0)
        if (t + 1) % w.delta == 0:
            g_s = c.read_scores()[:, : o.n].astype(np.float64)
            old = c.read_tiers()[:, : o.n]
            c.reassign()
            new = c.read_tiers()[:, : o.n]
            for b in range(w.batch):
                ref_t = tiering.reassign(old[b], g_s[b], o.n, w.prompt, w.sinks, w.recent,
                                         w.hbm_ratio, w.evict_ratio, w.t2_ratio)
                assert np.array_equal(new[b], ref_t), "labels differ (seq %d)" % b
            o.reassign(rank_scores=g_s[bs], adopt=new[bs])
    st = c.stats()
    c.close()
    print("[fullsize] %s: %d sampled steps, max |out - oracle| = %.3g" % (w.name, checked, worst), flush=True)
    assert worst <= 5e-3
    return st


@pytest.mark.timeout(900)
def test_14b_full_size():
    w = tkvsynth.CONFIGS["14b"].replace(steps=65)
    st = run_sampled(w, layers=(0, 47), seqs=(0, 3), sample_every=16)
    assert st["reassigns"] == 1 and st["tier_count"][3] > 0


@pytest.mark.timeout(900)
def test_32b_t2_full_size():
    w = tkvsynth.CONFIGS["32b_t2"].replace(steps=65)
    st = run_sampled(w, layers=(0, 63), seqs=(0, 7), sample_every=16)
    assert st["tier_count"][2] == w.batch * int(0.2 * (w.prefill + 64))


@pytest.mark.timeout(1200)
def test_70b_full_size():
    w = tkvsynth.CONFIGS["70b"].replace(steps=65)
    st = run_sampled(w, layers=(0, 79), seqs=(0, 7), sample_every=16)
    assert st["reassigns"] == 1
