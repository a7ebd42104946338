"""Every (cache dtype, head_dim, GQA group) the library accepts, on short
runs against the oracle through the C ABI: the vector path (fp32, and bf16
with groups below 4) and the matrix-core path (bf16, groups 4 and up), head
dims 64 and 128, ragged last chunks, one reassignment with eviction, and the
largest batch and query-head count the header allows.  Attention is "Not All
Thoughts Need HBM" Method §3 (every live row, exactly), scores Eq. 1 (§2).
"""
import numpy as np
import pytest

import tkvsynth
from harness import Inputs
from test_gpu_reassign import run_parity

pytestmark = pytest.mark.gpu

CASES = [(dt, d, g) for dt in ("bf16", "f32") for d in (64, 128) for g in (1, 2, 4, 5, 8)]


@pytest.mark.parametrize("dtype,head_dim,group", CASES, ids=["%s-d%d-g%d" % c for c in CASES])
def test_dtype_headdim_group(dtype, head_dim, group):
    kv = 2
    w = tkvsynth.CONFIGS["tiny"].replace(dtype=dtype, head_dim=head_dim, kv_heads=kv, q_heads=kv * group,
                                         layers=2, batch=2, prefill=611, steps=9, delta=8, prompt=16,
                                         recent=24, hbm_ratio=0.4, evict_ratio=0.05)
    outs, s, tiers, st, o, nr = run_parity(w, Inputs(w), w.steps)
    assert nr == 1 and st["tier_count"][3] > 0


def test_stream_staging_each_path():
    for dtype, group in (("bf16", 1), ("bf16", 8), ("f32", 4)):
        w = tkvsynth.CONFIGS["tiny"].replace(dtype=dtype, head_dim=128, kv_heads=2, q_heads=2 * group, layers=4,
                                             batch=1, prefill=700, steps=9, delta=8, prompt=16, recent=24,
                                             hbm_ratio=0.4, evict_ratio=0.05, t2_ratio=0.1)
        run_parity(w, Inputs(w), w.steps, staging_layers=2)


def test_largest_batch():
    w = tkvsynth.CONFIGS["tiny"].replace(batch=64, prefill=90, steps=9, delta=8, prompt=8, recent=8)
    run_parity(w, Inputs(w), w.steps)


def test_most_query_heads():
    w = tkvsynth.CONFIGS["tiny"].replace(dtype="bf16", head_dim=64, kv_heads=32, q_heads=256, layers=1, batch=1,
                                         prefill=300, steps=9, delta=8, prompt=8, recent=16)
    run_parity(w, Inputs(w), w.steps)


@pytest.mark.parametrize("group,delta", [(4, 5), (4, 13), (5, 7), (5, 11), (8, 5), (8, 7)])
def test_deferred_pairs_odd_delta(group, delta):
    """The matrix-core path over resident staging forms Eq. 1 of several
    pending steps together in one launch (11 at g = 4, 8 at g = 5, 5 at g = 8:
    16/g - 1 of them in the running step's logits tile, the rest in two extra
    tiles).  A Delta below that count leaves every step pending until the
    reassignment's score-only pass; a larger one prime to the cadence has
    forming launches and finds a different count pending at each
    reassignment.  The scores read at every step come from a copy; scores,
    outputs and labels still follow the oracle (Method §2 and §4)."""
    w = tkvsynth.CONFIGS["tiny"].replace(dtype="bf16", head_dim=128, kv_heads=2, q_heads=2 * group, layers=3,
                                         batch=2, prefill=400, steps=3 * delta + 2, delta=delta, prompt=16,
                                         recent=24, hbm_ratio=0.4, evict_ratio=0.05)
    outs, s, tiers, st, o, nr = run_parity(w, Inputs(w), w.steps, check_every=1)
    assert nr == 3
