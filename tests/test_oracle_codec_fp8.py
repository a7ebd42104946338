"""Pins for the oracle's FP8 (OCP E4M3, "FN" encoding) T2 codec: values the
format's definition fixes (largest finite 448 = 0x7E, smallest normal 2^-6 =
0x08, smallest subnormal 2^-9 = 0x01, one = 0x38), ties to the even code in
the normal and subnormal ranges, saturation, signed zero, exact round trips
of every finite code, and the codec's error bound (half a unit of the
3-bit mantissa, relative, above the subnormals)."""
import numpy as np

from oracle import codec


def test_format_landmarks():
    x = np.array([448.0, 2.0 ** -6, 2.0 ** -9, 1.0, 0.5, 2.0, -1.0, 0.0, 240.0, 256.0], np.float32)
    assert codec.e4m3_encode(x).tolist() == [0x7E, 0x08, 0x01, 0x38, 0x30, 0x40, 0xB8, 0x00, 0x77, 0x78]


def test_ties_to_even_and_saturation():
    x = np.array([1.0625, 1.1875, 272.0, 1.5 * 2.0 ** -9, 2.0 ** -10, 464.0, 500.0, 1e30, -500.0], np.float32)
    # 1.0625: between 0x38 and 0x39 -> even 0x38; 1.1875: between 0x39 and 0x3A -> 0x3A;
    # 272: between 256 (0x78) and 288 (0x79) -> 0x78; 1.5*2^-9 -> 0x02; 2^-10 -> 0x00;
    # beyond 448 saturates to 0x7E / 0xFE
    assert codec.e4m3_encode(x).tolist() == [0x38, 0x3A, 0x78, 0x02, 0x00, 0x7E, 0x7E, 0x7E, 0xFE]


def test_signed_zero_and_tiny_negatives():
    assert codec.e4m3_encode(np.array([-0.0, -2.0 ** -11], np.float32)).tolist() == [0x80, 0x80]


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = codec.e4m3_decode(codes)
    assert np.all(np.isfinite(vals))
    assert np.array_equal(codec.e4m3_encode(vals), codes)
    pos = codec.e4m3_decode(np.arange(127, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0) and pos[-1] == 448.0
    assert np.isnan(codec.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()


def test_row_error_bound():
    rng = np.random.default_rng(0)
    for _ in range(50):
        row = (rng.standard_normal(1024) * rng.uniform(0.01, 10)).astype(np.float32)
        codes, scale = codec.quantize_row_fp8(row)
        back = codec.dequantize_row_fp8(codes, scale, bf16=False)
        y = np.abs(row / scale)
        # relative half-unit of a 3-bit mantissa in the normal range, absolute 2^-10 below it
        bound = np.maximum(y * 2.0 ** -4, 2.0 ** -10) * scale * (1 + 1e-6)
        assert np.all(np.abs(back - row) <= bound)
        assert np.max(np.abs(codec.e4m3_decode(codes))) == 448.0      # amax maps to the top code


def test_fp8_beats_int8_on_relative_error_of_small_values():
    # a row with one large value: int8 flattens the small ones, E4M3 keeps ~2 significant digits
    row = np.array([100.0] + [0.01 * (1 + i) for i in range(63)], np.float32)
    i8 = codec.roundtrip(row, bf16=False)
    f8 = codec.roundtrip_fp8(row, bf16=False)
    small = slice(1, None)
    assert np.max(np.abs(f8[small] - row[small]) / row[small]) < 0.07
    assert np.max(np.abs(i8[small] - row[small]) / row[small]) > 0.5


def test_head_scales_are_the_row_codec_per_head():
    rng = np.random.default_rng(3)
    row = rng.standard_normal((4, 64)).astype(np.float32)
    row[2] *= 0.01                              # a head of small values
    for fp8 in (False, True):
        codes, scales = codec.quantize_row_heads(row, fp8)
        quant = codec.quantize_row_fp8 if fp8 else codec.quantize_row
        for h in range(4):
            c, s = quant(row[h])
            assert np.array_equal(codes[h], c) and scales[h] == s
        # the small head keeps its precision, which one row scale would not give it
        per_head = codec.roundtrip_heads(row, fp8, bf16=False)
        per_row = (codec.roundtrip_fp8 if fp8 else codec.roundtrip)(row, bf16=False)
        assert np.max(np.abs(per_head[2] - row[2])) < np.max(np.abs(per_row[2] - row[2]))
