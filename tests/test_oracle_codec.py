"""Pins of the oracle's 8-bit tier codec (CPU only).

"Not All Thoughts Need HBM" (gist.science summary), Method §1: T2 holds rows
at low precision on the host, 8-bit given as the example.  Pins: the
round-trip error bound (half a quantisation step plus the bf16 rounding of
the result), exact round trips of rows that are integer multiples of a
power-of-two step, the all-zero row, round-half-even ties, and that the
largest magnitude maps to +-127.
"""
import numpy as np

from oracle import codec


def _bf16(x):
    return codec._round_f32_to_bf16(np.asarray(x, np.float32))


def test_roundtrip_error_bound():
    rng = np.random.default_rng(0)
    for scale_mag in (1e-3, 1.0, 37.0):
        x = _bf16(rng.standard_normal(1024).astype(np.float32) * scale_mag)
        codes, scale = codec.quantize_row(x)
        y = codec.dequantize_row(codes, scale, bf16=True)
        bound = 0.5 * float(scale) * (1 + 1e-6) + np.abs(y).astype(np.float64) * 2.0 ** -8
        assert np.all(np.abs(x.astype(np.float64) - y) <= bound)
        assert np.max(np.abs(codes.astype(int))) == 127


def test_integer_multiples_roundtrip_exactly():
    step = np.float32(2.0 ** -4)
    k = np.arange(-127, 128, dtype=np.float32)
    x = k * step                                   # amax = 127 * step, so scale = step
    codes, scale = codec.quantize_row(x)
    assert scale == step
    assert np.array_equal(codes.astype(np.float32), k)
    assert np.array_equal(codec.dequantize_row(codes, scale, bf16=True), x)


def test_zero_row():
    codes, scale = codec.quantize_row(np.zeros(64, np.float32))
    assert scale == 1.0 and np.all(codes == 0)
    assert np.all(codec.dequantize_row(codes, scale, bf16=True) == 0)


def test_round_half_even():
    step = np.float32(0.125)
    x = np.array([127 * step, 2.5 * step, 3.5 * step, -2.5 * step, 0.5 * step], np.float32)
    codes, scale = codec.quantize_row(x)
    assert scale == step
    assert codes.tolist() == [127, 2, 4, -2, 0]


def test_bf16_rounding_of_dequantised_values():
    # 127 * (1/3-ish scale) products are not bf16 values; the result must be the nearest bf16
    x = np.array([1.0, 0.3, -0.7], np.float32)
    codes, scale = codec.quantize_row(x)
    y32 = codes.astype(np.float32) * scale
    y = codec.dequantize_row(codes, scale, bf16=True)
    for a, b in zip(y32, y):
        bits = int(np.float32(b).view(np.uint32))
        assert bits & 0xFFFF == 0                      # a bf16 value
        up = np.uint32(bits + 0x10000).view(np.float32)
        dn = np.uint32(bits - 0x10000).view(np.float32)
        assert abs(float(a) - float(b)) <= min(abs(float(a) - float(up)), abs(float(a) - float(dn)))
