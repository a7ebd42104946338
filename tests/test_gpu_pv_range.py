"""The matrix-core p.V of bf16 heads (one, five or eight query heads per kv
head) against the oracle on large values, and the vector pass of the same
heads.

Attention output is the weighted sum of the live V rows ("Not All Thoughts
Need HBM", gist.science summary, Method §3: every live row contributes at
full precision).  The matrix-core pass feeds V to v_mfma_f32_16x16x32_bf16
as its bf16 values and the weights as three bf16 terms that carry all of
their fp32 bits, so its error is fp32 rounding whatever the size of V.
Inputs: V scaled by 16, a few V entries set to +-1e3, and a few beyond the
fp16 range (+-7e4), rounded to bf16; outputs within 5e-3 of the oracle and
within 1e-6 relative to the largest |v|.
"""
import numpy as np
import pytest

import tkvsynth
from harness import Inputs
from test_gpu_reassign import run_parity

pytestmark = pytest.mark.gpu


def _bf16_bits(x):
    """float32 -> bf16 bit patterns, round to nearest even (finite values)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _loud_v(inp, w, seed=3):
    """V x 16, then 0.05% of the entries at +-1e3 and 0.005% at +-7e4."""
    rng = np.random.default_rng(seed)
    for name in ("v0", "vn"):
        a = tkvsynth.bf16_to_f32(getattr(inp, name)) * np.float32(16.0)
        flat = a.reshape(-1)
        for frac, mag in ((5e-4, 1e3), (5e-5, 7e4)):
            idx = rng.choice(flat.size, max(1, int(frac * flat.size)), replace=False)
            flat[idx] = (mag * rng.choice([-1.0, 1.0], idx.size)).astype(np.float32)
        setattr(inp, name, _bf16_bits(a))
    return float(max(np.abs(tkvsynth.bf16_to_f32(inp.v0)).max(), np.abs(tkvsynth.bf16_to_f32(inp.vn)).max()))


@pytest.mark.parametrize("heads", ["7b", "14b", "70b"])
@pytest.mark.parametrize("staging", [0, 2], ids=["resident", "stream"])
def test_matrix_core_pv_large_values(heads, staging):
    w = tkvsynth.CONFIGS[heads].replace(layers=3, batch=2, prefill=900, steps=40, delta=32, prompt=40, recent=32)
    inp = Inputs(w)
    vmax = _loud_v(inp, w)
    assert vmax > 65504  # beyond the largest fp16 value
    run_parity(w, inp, w.steps, check_every=3, staging_layers=staging)


@pytest.mark.parametrize("heads", ["7b", "14b", "70b"])
def test_vector_pass_grouped_query(heads):
    """TKV_FLAG_VECTOR_PASS: the same heads (one, five or eight query heads
    per kv head) on the vector units (stored logits, Eq. 1 not deferred) match
    the oracle, and the matrix-core pass's outputs to within rounding."""
    import decode_attention_tkv_amd as tkv
    w = tkvsynth.CONFIGS[heads].replace(layers=3, batch=2, prefill=900, steps=70, delta=32, prompt=40, recent=32)
    inp = Inputs(w)
    vec = run_parity(w, inp, w.steps, check_every=5, extra_flags=tkv.TKV_FLAG_VECTOR_PASS)
    mat = run_parity(w, inp, w.steps, check_every=5)
    assert max(float(np.max(np.abs(x - y))) for x, y in zip(vec[0], mat[0])) <= 1e-4
    assert np.array_equal(vec[2] == 3, mat[2] == 3)
