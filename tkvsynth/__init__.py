"""Seeded synthetic workloads for tiered-KV decode attention.

This package is shared by the CPU oracle's tests and by the GPU library's
tests and benchmark.  It holds no arithmetic of the method (attention,
scoring, tiering, codec): it only defines the workload shapes and draws
their inputs.

Input recipe (one rule for every workload):
  * q, K, V elements are i.i.d. N(0, 1) from a counter-based generator
    (splitmix64 words + Box-Muller in fp64, ``synth.c``);
  * one unit vector ``u`` (length head_dim) per seed;
  * exactly ``round(heavy_frac * n_final)`` heavy-hitter positions per
    sequence, chosen as the positions with the smallest seeded random keys
    (a seeded permutation, the same for every layer and kv head);
  * heavy positions get ``K += k_amp * u`` in every layer and kv head;
    V is untouched; every q row gets ``q += q_amp * u``;
  * values are rounded once to bf16 (round to nearest even) or to fp32.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libtkvsynth.so")
_lib = None

# tensor ids of the counter-based streams
TID_K, TID_V, TID_Q, TID_U, TID_HEAVY = 1, 2, 3, 4, 5


def build(force: bool = True) -> str:
    """Compile synth.c into libtkvsynth.so (host code only)."""
    global _lib
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        u64, i64, i32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.tkvsynth_words.argtypes = [u64, u64, u64, i64, vp]
        lib.tkvsynth_normals.argtypes = [u64, u64, u64, i64, vp]
        lib.tkvsynth_kv.argtypes = [u64, i32, i32, i32, i32, i32, i64, i64, i64, vp, vp,
                                    ctypes.c_double, i32, vp]
        lib.tkvsynth_q.argtypes = [u64, i32, i32, i32, i32, i64, i64, vp, ctypes.c_double, i32, vp]
        for f in (lib.tkvsynth_words, lib.tkvsynth_normals, lib.tkvsynth_kv, lib.tkvsynth_q):
            f.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def words(seed: int, tid: int, n0: int, count: int) -> np.ndarray:
    out = np.empty(count, np.uint64)
    _load().tkvsynth_words(seed, tid, n0, count, _ptr(out))
    return out


def normals(seed: int, tid: int, n0: int, count: int) -> np.ndarray:
    out = np.empty(count, np.float64)
    _load().tkvsynth_normals(seed, tid, n0, count, _ptr(out))
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exactly equal float32 values."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape, tier policy and input recipe of one decode workload."""
    name: str
    layers: int
    q_heads: int
    kv_heads: int
    head_dim: int
    batch: int
    dtype: str            # "bf16" or "f32"
    prefill: int          # cache positions present before the first decode step
    steps: int            # decode steps
    delta: int            # reassignment period
    hbm_ratio: float
    evict_ratio: float
    t2_ratio: float
    prompt: int
    sinks: int
    recent: int
    seed: int = 0
    no_t1: bool = False   # eviction-only baseline: rows that would go to T1 are evicted
    t2_fp8: bool = False  # T2 rows held as FP8 E4M3 codes instead of int8
    shared_hbm: bool = False  # one T0 budget for the whole batch, ranked jointly
    t2_head_scales: bool = False  # one T2 scale per kv head instead of one per row
    heavy_frac: float = 0.05
    k_amp: float = 3.0
    q_amp: float = 2.0

    @property
    def n_final(self) -> int:
        return self.prefill + self.steps

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def np_dtype(self):
        return np.uint16 if self.dtype == "bf16" else np.float32

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    # ---- drawn quantities -------------------------------------------------
    def unit_vector(self) -> np.ndarray:
        g = normals(self.seed, TID_U, 0, self.head_dim)
        return g / np.sqrt(np.dot(g, g))

    def heavy_mask(self) -> np.ndarray:
        """uint8 [batch][n_final]; 1 at the planted heavy-hitter positions."""
        n = self.n_final
        nh = int(round(self.heavy_frac * n))
        m = np.zeros((self.batch, n), np.uint8)
        for b in range(self.batch):
            key = words(self.seed, TID_HEAVY, b * (1 << 32), n)
            order = np.argsort(key, kind="stable")
            m[b, order[:nh]] = 1
        return m

    def kv(self, which: int, pos0: int, npos: int, heavy=None, u=None) -> np.ndarray:
        """K (which=0) or V (which=1) rows of positions [pos0, pos0+npos):
        array [layers][batch][npos][kv_heads][head_dim] (bf16 bits or fp32)."""
        assert 0 <= pos0 and pos0 + npos <= self.n_final
        heavy = self.heavy_mask() if heavy is None else np.ascontiguousarray(heavy, np.uint8)
        u = self.unit_vector() if u is None else np.ascontiguousarray(u, np.float64)
        out = np.empty((self.layers, self.batch, npos, self.kv_heads, self.head_dim), self.np_dtype)
        _load().tkvsynth_kv(self.seed, which, self.layers, self.batch, self.kv_heads, self.head_dim,
                            self.n_final, pos0, npos, _ptr(heavy), _ptr(u), self.k_amp,
                            1 if self.dtype == "bf16" else 0, _ptr(out))
        return out

    def q(self, t0: int, nt: int, u=None) -> np.ndarray:
        """q of decode steps [t0, t0+nt) (0-based): [nt][layers][batch][q_heads][head_dim]."""
        u = self.unit_vector() if u is None else np.ascontiguousarray(u, np.float64)
        out = np.empty((nt, self.layers, self.batch, self.q_heads, self.head_dim), self.np_dtype)
        _load().tkvsynth_q(self.seed, self.layers, self.batch, self.q_heads, self.head_dim, t0, nt,
                           _ptr(u), self.q_amp, 1 if self.dtype == "bf16" else 0, _ptr(out))
        return out

    def values(self, a: np.ndarray) -> np.ndarray:
        """Drawn array -> float32 values (bf16 bits are widened exactly)."""
        return bf16_to_f32(a) if self.dtype == "bf16" else np.asarray(a, np.float32)

    def kv_bytes_per_token(self) -> int:
        """K+V bytes of one position in all layers (one sequence)."""
        return 2 * self.layers * self.kv_heads * self.head_dim * self.elem_bytes


def _w(**kw) -> Workload:
    return Workload(**kw)


# The five decode workloads.  Where a field is not fixed by the workload
# statement (steps, delta, protected set of the larger shapes), the value
# used is stated here and in the design notes.
CONFIGS = {
    "tiny": _w(name="tiny", layers=2, q_heads=4, kv_heads=4, head_dim=64, batch=1, dtype="f32",
               prefill=288, steps=256, delta=16, hbm_ratio=0.30, evict_ratio=0.03, t2_ratio=0.0,
               prompt=32, sinks=4, recent=32),
    "7b": _w(name="7b", layers=32, q_heads=32, kv_heads=32, head_dim=128, batch=1, dtype="bf16",
             prefill=2200, steps=512, delta=64, hbm_ratio=0.50, evict_ratio=0.03, t2_ratio=0.0,
             prompt=200, sinks=4, recent=128),
    "14b": _w(name="14b", layers=48, q_heads=40, kv_heads=8, head_dim=128, batch=4, dtype="bf16",
              prefill=4096, steps=256, delta=64, hbm_ratio=0.50, evict_ratio=0.03, t2_ratio=0.0,
              prompt=200, sinks=4, recent=128),
    "32b": _w(name="32b", layers=64, q_heads=40, kv_heads=8, head_dim=128, batch=8, dtype="bf16",
              prefill=8192, steps=256, delta=64, hbm_ratio=0.30, evict_ratio=0.05, t2_ratio=0.0,
              prompt=200, sinks=4, recent=128),
    "70b": _w(name="70b", layers=80, q_heads=64, kv_heads=8, head_dim=128, batch=8, dtype="bf16",
              prefill=16384, steps=1024, delta=64, hbm_ratio=0.30, evict_ratio=0.03, t2_ratio=0.0,
              prompt=200, sinks=4, recent=128),
}
# 32B-shaped variant with the 8-bit host tier enabled (20% of positions).
CONFIGS["32b_t2"] = CONFIGS["32b"].replace(name="32b_t2", t2_ratio=0.20)
