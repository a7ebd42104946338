"""ORACLE (test infrastructure): the 8-bit host tier's codec.

"Not All Thoughts Need HBM" (gist.science technical summary), Method §1:
T2 keeps low-importance tokens on the CPU at low precision, 8-bit
quantisation given as the example; results §4 reports its accuracy cost.
The pages do not fix the format.  Reading used here:

  * symmetric int8, one fp32 scale per (layer, token, K or V), taken over
    that token's whole row of kv_heads * head_dim values;
  * scale = amax / 127 in fp32 (scale = 1 when the row is all zeros);
  * code = clamp(round_half_even(x / scale), -127, 127), the division in
    fp32 (the decision that produces an integer is taken in fp32);
  * value = fp32(code * scale), then rounded to the cache element type
    (bf16 round-to-nearest-even, or kept as fp32 for fp32 caches);
  * a row that entered T2 keeps its dequantised values for good, also if it
    is later promoted (the full-precision copy is dropped on entry).
"""
from __future__ import annotations

import numpy as np


def _round_f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 value (ties to even), returned as fp32."""
    b = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


def quantize_row(row: np.ndarray):
    """row: float32 values of one (layer, token, K|V) row -> (int8 codes, fp32 scale)."""
    x = np.asarray(row, np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    scale = np.float32(amax / np.float32(127.0)) if amax > 0 else np.float32(1.0)
    codes = np.clip(np.rint(x / scale), -127, 127).astype(np.int8)
    return codes, scale


def dequantize_row(codes: np.ndarray, scale, bf16: bool) -> np.ndarray:
    """int8 codes and their fp32 scale -> cache values (as float32)."""
    v = codes.astype(np.float32) * np.float32(scale)
    return _round_f32_to_bf16(v) if bf16 else v.astype(np.float32)


def roundtrip(row: np.ndarray, bf16: bool) -> np.ndarray:
    codes, scale = quantize_row(row)
    return dequantize_row(codes, scale, bf16).reshape(np.shape(row))


# ---- FP8 variant (the "FP8 etc." the ARKV summary names for low-precision
# tiers): OCP FP8 E4M3, the "FN" encoding -- 1 sign bit, 4 exponent bits with
# bias 7, 3 mantissa bits; exponent field 0 holds the subnormals m * 2^-9;
# no infinities; exponent 15 with mantissa 7 is NaN, so the largest finite
# magnitude is 2^8 * 1.75 = 448.  Reading used here, as for int8: one fp32
# scale per (layer, token, K or V) row, scale = amax / 448 (1 for an all-zero
# row); code = nearest E4M3 value of clamp(x / scale, -448, 448), ties to the
# even code, the division in fp32; value = fp32(decode(code) * scale) rounded
# to the cache type.
def _e4m3_magnitudes() -> np.ndarray:
    vals = np.empty(127, np.float64)          # codes 0x00 .. 0x7E
    for c in range(127):
        e, m = c >> 3, c & 7
        vals[c] = m * 2.0 ** -9 if e == 0 else 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return vals


E4M3_MAGNITUDES = _e4m3_magnitudes()
E4M3_MAX = 448.0


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """fp32 values -> E4M3 codes (uint8): nearest magnitude, ties to the even
    code, saturating at 448; the sign bit follows the sign of x (also -0)."""
    x = np.asarray(x, np.float32).ravel()
    a = np.minimum(np.abs(x.astype(np.float64)), E4M3_MAX)
    dist = np.abs(a[:, None] - E4M3_MAGNITUDES[None, :])
    idx = np.argmin(dist, axis=1)                       # the lower code of a tie
    nxt = np.minimum(idx + 1, len(E4M3_MAGNITUDES) - 1)
    tie = (nxt != idx) & (dist[np.arange(len(a)), nxt] == dist[np.arange(len(a)), idx])
    idx = np.where(tie & (idx % 2 == 1), nxt, idx)     # ties go to the even code
    sign = np.signbit(x).astype(np.uint8) << 7
    return (sign | idx.astype(np.uint8)).astype(np.uint8)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes (uint8) -> values (float32); the NaN codes give NaN."""
    c = np.asarray(codes, np.uint8).ravel()
    mag = c & 0x7F
    v = np.where(mag == 0x7F, np.nan, E4M3_MAGNITUDES[np.minimum(mag, 126)])
    return np.where(c & 0x80, -v, v).astype(np.float32)


def quantize_row_fp8(row: np.ndarray):
    """row: float32 values of one (layer, token, K|V) row -> (E4M3 codes, fp32 scale)."""
    x = np.asarray(row, np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    scale = np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)
    y = np.clip(x / scale, np.float32(-E4M3_MAX), np.float32(E4M3_MAX)).astype(np.float32)
    return e4m3_encode(y).reshape(np.shape(row)), scale


def dequantize_row_fp8(codes: np.ndarray, scale, bf16: bool) -> np.ndarray:
    v = (e4m3_decode(codes) * np.float32(scale)).astype(np.float32).reshape(np.shape(codes))
    return _round_f32_to_bf16(v) if bf16 else v


def roundtrip_fp8(row: np.ndarray, bf16: bool) -> np.ndarray:
    codes, scale = quantize_row_fp8(row)
    return dequantize_row_fp8(codes, scale, bf16).reshape(np.shape(row))


# ---- per-head scales: the same formats with one fp32 scale per kv head of
# the row (Hkv scales instead of one), each from that head's own amax, so a
# head of small values keeps its precision next to a head of large ones.
def quantize_row_heads(row: np.ndarray, fp8: bool):
    """row: float32 [kv_heads][head_dim] -> (codes [kv_heads][head_dim], scales [kv_heads])."""
    x = np.asarray(row, np.float32)
    quant = quantize_row_fp8 if fp8 else quantize_row
    pairs = [quant(x[h]) for h in range(x.shape[0])]
    codes = np.stack([p[0] for p in pairs])
    return codes, np.array([p[1] for p in pairs], np.float32)


def dequantize_row_heads(codes: np.ndarray, scales: np.ndarray, fp8: bool, bf16: bool) -> np.ndarray:
    deq = dequantize_row_fp8 if fp8 else dequantize_row
    return np.stack([deq(codes[h], scales[h], bf16).reshape(-1) for h in range(codes.shape[0])])


def roundtrip_heads(row: np.ndarray, fp8: bool, bf16: bool) -> np.ndarray:
    codes, scales = quantize_row_heads(row, fp8)
    return dequantize_row_heads(codes, scales, fp8, bf16).reshape(np.shape(row))
