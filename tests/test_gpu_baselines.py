"""Baseline policies on the same engine, GPU against the oracle through the
C ABI (the eviction policies the gist.science summary of "Not All Thoughts
Need HBM" compares against, Results; tier rules of Method §1, §4).

* Eviction-only (no T1, heavy hitters kept in T0): labels and changed-row
  lists bit-exact against the oracle's rules on the GPU's fp32 scores,
  outputs within tolerance, scores relative 1e-4; no row ever sits in T1 and
  nothing crosses PCIe.
* Sinks + recent window (hbm 0, evict 1, prompt 0): only the window stays
  live, checked the same way.
"""
import numpy as np
import pytest

import tkvsynth
from harness import Inputs
from test_gpu_reassign import run_parity

pytestmark = pytest.mark.gpu


def test_no_t1_tiny_full_run():
    w = tkvsynth.CONFIGS["tiny"].replace(no_t1=True, steps=96)
    outs, s, tiers, st, o, nr = run_parity(w, Inputs(w), w.steps)
    n = o.n
    assert not np.any(tiers[:, :n] == 1)
    assert (tiers[0, :n] == 0).sum() == int(np.floor(w.hbm_ratio * n))
    assert st["h2d_bytes"] == 0


def test_no_t1_with_t2_bf16():
    # P = 20 prompt + 64 recent, well under floor(.3 N); the first placement evicts what the
    # tiered policy would put in T1, so T2 fills from the candidates that remain
    w = tkvsynth.CONFIGS["32b_t2"].replace(layers=3, batch=2, prefill=700, steps=65, delta=32, no_t1=True,
                                           prompt=20, recent=64)
    outs, s, tiers, st, o, nr = run_parity(w, Inputs(w), w.steps)
    n = o.n
    for b in range(w.batch):
        assert (tiers[b, :n] == 2).sum() > 0
        assert not np.any(tiers[b, :n] == 1)


def test_no_t1_7b_shape_stream_staging():
    w = tkvsynth.CONFIGS["7b"].replace(layers=4, steps=129, no_t1=True)
    run_parity(w, Inputs(w), w.steps, check_every=8, staging_layers=2)


def test_sinks_plus_recent_window():
    w = tkvsynth.CONFIGS["7b"].replace(layers=4, prefill=600, steps=80, delta=16, hbm_ratio=0.0,
                                       evict_ratio=1.0, prompt=0)
    outs, s, tiers, st, o, nr = run_parity(w, Inputs(w), w.steps, check_every=4)
    n = o.n
    live = np.nonzero(tiers[0, :n] != 3)[0]
    assert np.array_equal(live, np.r_[0:w.sinks, n - w.recent:n])


def test_sinks_plus_recent_window_from_the_first_placement():
    w = tkvsynth.CONFIGS["tiny"].replace(prefill=100, steps=40, delta=8, hbm_ratio=0.0, no_t1=True,
                                         prompt=0, sinks=4, recent=16)
    import decode_attention_tkv_amd as tkv
    from harness import to_device
    inp = Inputs(w)
    c = tkv.TieredKV.for_workload(w)
    c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))
    live = np.nonzero(c.read_tiers()[0, : w.prefill] != 3)[0]
    assert np.array_equal(live, np.r_[0:4, w.prefill - 16:w.prefill])
    assert c.stats()["host_bytes"] <= 2 * w.layers * w.kv_heads * w.head_dim * 4   # one-row T1 arena
    c.close()
    run_parity(w, inp, w.steps)
