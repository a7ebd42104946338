"""Batch-shared HBM budget on the GPU against the oracle, through the C ABI
(the batch projection of "Not All Thoughts Need HBM", gist.science summary,
Results; tier rules of Method §1 with one T0 budget for the batch).

Checks: labels and changed-row lists bit-exact against the oracle's joint
ranking applied to the GPU's fp32 scores, outputs within tolerance, scores
relative 1e-4; the T0 rows of the batch fill the shared budget while the
sequences hold unequal shares; stream staging; the per-sequence mode is
unchanged by the two-pass slot handling (covered by the other suites).
"""
import math

import numpy as np
import pytest

import tkvsynth
from harness import Inputs
from test_gpu_reassign import run_parity

pytestmark = pytest.mark.gpu


def _t0_shares(tiers, w, n):
    prot = np.zeros(n, bool)
    prot[: max(w.prompt, w.sinks)] = True
    prot[n - w.recent:] = True
    return [int(((tiers[b, :n] == 0) & ~prot).sum()) for b in range(w.batch)]


def test_shared_budget_7b_shape():
    # the run ends right after a reassignment, so the protected window is the one it used
    w = tkvsynth.CONFIGS["7b"].replace(layers=3, batch=4, prefill=700, steps=64, delta=32, prompt=40,
                                       shared_hbm=True)
    outs, s, tiers, st, o, nr = run_parity(w, Inputs(w), w.steps, check_every=8)
    n = o.n
    shares = _t0_shares(tiers, w, n)
    prot = max(w.prompt, w.sinks) + w.recent
    assert sum(shares) == w.batch * (math.floor(w.hbm_ratio * n) - prot)
    assert max(shares) > min(shares)          # the joint ranking gives the sequences unequal shares


def test_shared_budget_gqa_t2_stream():
    w = tkvsynth.CONFIGS["32b_t2"].replace(layers=3, batch=3, prefill=600, steps=65, delta=32, prompt=40,
                                           recent=64, shared_hbm=True)
    run_parity(w, Inputs(w), w.steps, check_every=8, staging_layers=2)


def test_shared_budget_gqa_t2_resident():
    # bf16 grouped-query heads over resident staging: Eq. 1 is deferred to the
    # next step's launch, so each reassignment first runs the score-only pass
    # whose scores the joint ranking then reads
    w = tkvsynth.CONFIGS["32b_t2"].replace(layers=3, batch=3, prefill=600, steps=65, delta=32, prompt=40,
                                           recent=64, shared_hbm=True)
    outs, s, tiers, st, o, nr = run_parity(w, Inputs(w), w.steps, check_every=8)
    assert nr == 2
    shares = _t0_shares(tiers, w, o.n)
    assert max(shares) > min(shares)


def test_shared_budget_fp32_tiny_batch():
    w = tkvsynth.CONFIGS["tiny"].replace(batch=3, steps=48, prompt=8, recent=16, shared_hbm=True)
    run_parity(w, Inputs(w), w.steps)


def test_shared_budget_rejects_no_t1():
    import decode_attention_tkv_amd as tkv
    w = tkvsynth.CONFIGS["tiny"]
    with pytest.raises(tkv.TkvError) as e:
        tkv.TieredKV.for_workload(w, shared_hbm=True, no_t1=True)
    assert e.value.code == tkv.TKV_EINVAL
