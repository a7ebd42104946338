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
