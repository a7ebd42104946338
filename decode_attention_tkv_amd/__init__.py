"""Tiered-KV decode attention for AMD Instinct MI355X (gfx950).

Thin ctypes binding of ``libtkv.so`` (C ABI in ``include/tkv.h``).  It only
marshals arguments: torch tensors become device pointers, torch streams
become hipStream_t handles, and status codes become exceptions.  Every step
of the decode path runs in the library's HIP kernels; there is no fallback.

torch is imported before the library is loaded so that the process holds a
single HIP runtime (torch's copy carries the same soname).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtkv.so")

TKV_OK, TKV_EINVAL, TKV_ECAPACITY, TKV_ENOMEM, TKV_ESTATE, TKV_EHIP = 0, -1, -2, -3, -4, -5
TKV_BF16, TKV_F32 = 0, 1
TKV_T0, TKV_T1, TKV_T2, TKV_T3 = 0, 1, 2, 3
TKV_FLAG_TIME_KERNELS = 1
TKV_FLAG_NO_T1 = 2
TKV_FLAG_T2_FP8 = 4
TKV_FLAG_SHARED_HBM = 8
TKV_FLAG_T2_HEAD_SCALES = 16
TKV_FLAG_VECTOR_PASS = 32
TKV_FLAG_TEST_DELAY_COPIES = 256
TKV_FLAG_TEST_SHUFFLE_SLOTS = 512

_NAMES = {TKV_EINVAL: "EINVAL", TKV_ECAPACITY: "ECAPACITY", TKV_ENOMEM: "ENOMEM",
          TKV_ESTATE: "ESTATE", TKV_EHIP: "EHIP"}


class TkvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("tkv %s (%d): %s" % (_NAMES.get(code, "?"), code, msg))
        self.code = code


class tkv_shape(ctypes.Structure):
    _fields_ = [("layers", ctypes.c_int32), ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("batch", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class tkv_protect(ctypes.Structure):
    _fields_ = [("prompt", ctypes.c_int32), ("sinks", ctypes.c_int32), ("recent", ctypes.c_int32)]


class tkv_options(ctypes.Structure):
    _fields_ = [("t2_ratio", ctypes.c_double), ("staging_layers", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("flags", ctypes.c_uint64), ("mem_cap_bytes", ctypes.c_int64),
                ("layer_hbm", ctypes.POINTER(ctypes.c_double))]


class tkv_delta(ctypes.Structure):
    _fields_ = [("pos", ctypes.c_uint32), ("old_tier", ctypes.c_uint8), ("new_tier", ctypes.c_uint8),
                ("reserved", ctypes.c_uint16)]


DELTA_DTYPE = np.dtype([("pos", np.uint32), ("old_tier", np.uint8), ("new_tier", np.uint8),
                        ("reserved", np.uint16)])


class tkv_stats_t(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int64), ("n_tokens", ctypes.c_int64), ("tier_count", ctypes.c_int64 * 4),
                ("hbm_bytes", ctypes.c_int64), ("host_bytes", ctypes.c_int64),
                ("full_cache_bytes", ctypes.c_int64), ("promotions", ctypes.c_int64),
                ("demotions", ctypes.c_int64), ("evictions", ctypes.c_int64), ("reassigns", ctypes.c_int64),
                ("h2d_bytes", ctypes.c_int64), ("d2h_bytes", ctypes.c_int64),
                ("attn_kernel_ms", ctypes.c_double), ("attn_kernel_launches", ctypes.c_int64),
                ("attn_kv_bytes", ctypes.c_int64),
                ("reassign_ms", ctypes.c_double), ("mem_bytes", ctypes.c_int64)]


_lib = None
_vp, _i32, _f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_double
_SIGS = {
    "tkv_create": [ctypes.POINTER(tkv_shape), _i32, _f64, _f64, tkv_protect, ctypes.POINTER(tkv_options),
                   ctypes.POINTER(_vp)],
    "tkv_destroy": [_vp],
    "tkv_last_error": [_vp],
    "tkv_prefill": [_vp, _vp, _vp, _i32, _vp],
    "tkv_prefill_scored": [_vp, _vp, _vp, _vp, _i32, _vp],
    "tkv_append": [_vp, _vp, _vp, _vp],
    "tkv_decode_attn": [_vp, _i32, _i32, _vp, _vp, _vp],
    "tkv_decode_step": [_vp, _vp, _vp, _vp, _vp, _vp],
    "tkv_reassign": [_vp, _vp],
    "tkv_reassign_static": [_vp, _vp],
    "tkv_stats": [_vp, ctypes.POINTER(tkv_stats_t)],
    "tkv_read_scores": [_vp, _vp, _vp],
    "tkv_write_scores": [_vp, _vp, _vp],
    "tkv_read_tiers": [_vp, _vp, _vp],
    "tkv_read_layer_tiers": [_vp, _i32, _vp, _vp],
    "tkv_read_deltas": [_vp, _vp, _vp, _vp],
    "tkv_read_kv": [_vp, _i32, _i32, _i32, _vp, _vp, _vp],
    "tkv_read_t2": [_vp, _i32, _i32, _i32, _vp, _vp, _vp],
}


def lib():
    """Load libtkv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libtkv.so is not built (run __graft_entry__.build() or "
                               "python decode_attention_tkv_amd/_build.py)")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_char_p if name == "tkv_last_error" else ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int, handle=None):
    if rc != TKV_OK:
        msg = lib().tkv_last_error(handle)
        raise TkvError(rc, msg.decode() if msg else "")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev_ptr(x: torch.Tensor, shape, dtype, name):
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    if tuple(x.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(x.shape), tuple(shape)))
    if x.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, x.dtype, dtype))
    if not x.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if x.data_ptr() % 16:
        raise ValueError("%s must start on a 16-byte boundary" % name)
    return x.data_ptr()


# ---- functions named as the C ABI --------------------------------------------

def tkv_create(layers, q_heads, kv_heads, head_dim, batch, max_tokens, dtype, delta, hbm_ratio,
               evict_ratio, prompt, sinks, recent, t2_ratio=0.0, staging_layers=0, chunk=0, flags=0,
               mem_cap_bytes=0, layer_hbm=None):
    shape = tkv_shape(layers, q_heads, kv_heads, head_dim, batch, max_tokens, dtype)
    lh = None
    if layer_hbm is not None:
        if len(layer_hbm) != layers:
            raise ValueError("layer_hbm has %d ratios for %d layers" % (len(layer_hbm), layers))
        lh = (ctypes.c_double * len(layer_hbm))(*[float(x) for x in layer_hbm])
    opts = tkv_options(t2_ratio, staging_layers, chunk, flags, mem_cap_bytes,
                       ctypes.cast(lh, ctypes.POINTER(ctypes.c_double)) if lh is not None else None)
    h = _vp()
    rc = lib().tkv_create(ctypes.byref(shape), delta, hbm_ratio, evict_ratio,
                          tkv_protect(prompt, sinks, recent), ctypes.byref(opts), ctypes.byref(h))
    _check(rc, None)
    return h


def tkv_destroy(h):
    _check(lib().tkv_destroy(h), h)


def tkv_prefill(h, k_ptr, v_ptr, n_tokens, stream=None):
    _check(lib().tkv_prefill(h, k_ptr, v_ptr, n_tokens, _stream(stream)), h)


def tkv_prefill_scored(h, k_ptr, v_ptr, q_ptr, n_tokens, stream=None):
    _check(lib().tkv_prefill_scored(h, k_ptr, v_ptr, q_ptr, n_tokens, _stream(stream)), h)


def tkv_append(h, k_ptr, v_ptr, stream=None):
    _check(lib().tkv_append(h, k_ptr, v_ptr, _stream(stream)), h)


def tkv_decode_attn(h, layer_begin, layer_count, q_ptr, out_ptr, stream=None):
    _check(lib().tkv_decode_attn(h, layer_begin, layer_count, q_ptr, out_ptr, _stream(stream)), h)


def tkv_decode_step(h, k_ptr, v_ptr, q_ptr, out_ptr, stream=None):
    _check(lib().tkv_decode_step(h, k_ptr, v_ptr, q_ptr, out_ptr, _stream(stream)), h)


def tkv_reassign(h, stream=None):
    _check(lib().tkv_reassign(h, _stream(stream)), h)


def tkv_reassign_static(h, stream=None):
    _check(lib().tkv_reassign_static(h, _stream(stream)), h)


def tkv_stats(h) -> dict:
    s = tkv_stats_t()
    _check(lib().tkv_stats(h, ctypes.byref(s)), h)
    d = {f: getattr(s, f) for f, _ in tkv_stats_t._fields_}
    d["tier_count"] = list(s.tier_count)
    return d


def tkv_read_scores(h, batch, max_tokens, stream=None) -> np.ndarray:
    out = np.empty((batch, max_tokens), np.float32)
    _check(lib().tkv_read_scores(h, out.ctypes.data, _stream(stream)), h)
    return out


def tkv_write_scores(h, scores: np.ndarray, stream=None):
    s = np.ascontiguousarray(scores, np.float32)
    _check(lib().tkv_write_scores(h, s.ctypes.data, _stream(stream)), h)


def tkv_read_tiers(h, batch, max_tokens, stream=None) -> np.ndarray:
    out = np.empty((batch, max_tokens), np.uint8)
    _check(lib().tkv_read_tiers(h, out.ctypes.data, _stream(stream)), h)
    return out


def tkv_read_layer_tiers(h, layer, batch, max_tokens, stream=None) -> np.ndarray:
    out = np.empty((batch, max_tokens), np.uint8)
    _check(lib().tkv_read_layer_tiers(h, layer, out.ctypes.data, _stream(stream)), h)
    return out


def tkv_read_deltas(h, batch, max_tokens):
    promote = np.zeros((batch, max_tokens), DELTA_DTYPE)
    demote = np.zeros((batch, max_tokens), DELTA_DTYPE)
    counts = np.zeros((batch, 2), np.int32)
    _check(lib().tkv_read_deltas(h, promote.ctypes.data, demote.ctypes.data, counts.ctypes.data), h)
    return promote, demote, counts


def tkv_read_kv(h, layer, seq, pos, kv_heads, head_dim, np_dtype, stream=None):
    k = np.empty((kv_heads, head_dim), np_dtype)
    v = np.empty((kv_heads, head_dim), np_dtype)
    _check(lib().tkv_read_kv(h, layer, seq, pos, k.ctypes.data, v.ctypes.data, _stream(stream)), h)
    return k, v


def tkv_read_t2(h, layer, seq, pos, kv_heads, head_dim, n_scales=1):
    """n_scales: scales per row (kv_heads with per-head scales, else 1); returns
    codes [kv_heads][head_dim] for K and V and the scales [2 * n_scales]."""
    kc = np.empty((kv_heads, head_dim), np.int8)
    vc = np.empty((kv_heads, head_dim), np.int8)
    sc = np.empty(2 * n_scales, np.float32)
    _check(lib().tkv_read_t2(h, layer, seq, pos, kc.ctypes.data, vc.ctypes.data, sc.ctypes.data), h)
    return kc, vc, sc


# ---- a handle object over the same calls ---------------------------------------

class TieredKV:
    """One tiered KV cache for a batch of sequences (owns a tkv handle)."""

    def __init__(self, layers, q_heads, kv_heads, head_dim, batch, max_tokens, dtype="bf16", delta=64,
                 hbm_ratio=0.5, evict_ratio=0.03, prompt=0, sinks=4, recent=128, t2_ratio=0.0,
                 staging_layers=0, chunk=0, time_kernels=False, no_t1=False, t2_fp8=False, shared_hbm=False,
                 t2_head_scales=False, extra_flags=0, mem_cap_bytes=0, layer_hbm=None):
        self.L, self.Hq, self.Hkv, self.D, self.B, self.nmax = layers, q_heads, kv_heads, head_dim, batch, max_tokens
        self.dtype = dtype
        self.tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.h = tkv_create(layers, q_heads, kv_heads, head_dim, batch, max_tokens,
                            TKV_BF16 if dtype == "bf16" else TKV_F32, delta, hbm_ratio, evict_ratio,
                            prompt, sinks, recent, t2_ratio, staging_layers, chunk,
                            (TKV_FLAG_TIME_KERNELS if time_kernels else 0) | (TKV_FLAG_NO_T1 if no_t1 else 0)
                            | (TKV_FLAG_T2_FP8 if t2_fp8 else 0) | (TKV_FLAG_SHARED_HBM if shared_hbm else 0)
                            | (TKV_FLAG_T2_HEAD_SCALES if t2_head_scales else 0) | extra_flags, mem_cap_bytes,
                            layer_hbm)
        self.n_scales = kv_heads if t2_head_scales else 1

    @classmethod
    def for_workload(cls, w, **kw):
        args = dict(layers=w.layers, q_heads=w.q_heads, kv_heads=w.kv_heads, head_dim=w.head_dim,
                    batch=w.batch, max_tokens=w.n_final, dtype=w.dtype, delta=w.delta,
                    hbm_ratio=w.hbm_ratio, evict_ratio=w.evict_ratio, prompt=w.prompt, sinks=w.sinks,
                    recent=w.recent, t2_ratio=w.t2_ratio, no_t1=w.no_t1, t2_fp8=w.t2_fp8,
                    shared_hbm=w.shared_hbm, t2_head_scales=w.t2_head_scales)
        args.update(kw)
        return cls(**args)

    def close(self):
        if self.h is not None:
            tkv_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def prefill(self, k: torch.Tensor, v: torch.Tensor, stream=None):
        n = k.shape[2]
        shape = (self.L, self.B, n, self.Hkv, self.D)
        tkv_prefill(self.h, _dev_ptr(k, shape, self.tdtype, "k"), _dev_ptr(v, shape, self.tdtype, "v"), n, stream)

    def prefill_scored(self, k: torch.Tensor, v: torch.Tensor, q: torch.Tensor, stream=None):
        n = k.shape[2]
        shape = (self.L, self.B, n, self.Hkv, self.D)
        tkv_prefill_scored(self.h, _dev_ptr(k, shape, self.tdtype, "k"), _dev_ptr(v, shape, self.tdtype, "v"),
                           _dev_ptr(q, (self.L, self.B, n, self.Hq, self.D), self.tdtype, "q"), n, stream)

    def append(self, k: torch.Tensor, v: torch.Tensor, stream=None):
        shape = (self.L, self.B, self.Hkv, self.D)
        tkv_append(self.h, _dev_ptr(k, shape, self.tdtype, "k"), _dev_ptr(v, shape, self.tdtype, "v"), stream)

    def decode_attn(self, q: torch.Tensor, out: torch.Tensor, layer_begin=0, layer_count=None, stream=None):
        lc = self.L - layer_begin if layer_count is None else layer_count
        tkv_decode_attn(self.h, layer_begin, lc,
                        _dev_ptr(q, (lc, self.B, self.Hq, self.D), self.tdtype, "q"),
                        _dev_ptr(out, (lc, self.B, self.Hq, self.D), torch.float32, "out"), stream)

    def decode_step(self, k: torch.Tensor, v: torch.Tensor, q: torch.Tensor, out: torch.Tensor, stream=None):
        """append(k, v) then decode_attn(q, out) over every layer, as one call."""
        shape = (self.L, self.B, self.Hkv, self.D)
        tkv_decode_step(self.h, _dev_ptr(k, shape, self.tdtype, "k"), _dev_ptr(v, shape, self.tdtype, "v"),
                        _dev_ptr(q, (self.L, self.B, self.Hq, self.D), self.tdtype, "q"),
                        _dev_ptr(out, (self.L, self.B, self.Hq, self.D), torch.float32, "out"), stream)

    def reassign(self, stream=None):
        tkv_reassign(self.h, stream)

    def stats(self) -> dict:
        return tkv_stats(self.h)

    def read_scores(self, stream=None):
        return tkv_read_scores(self.h, self.B, self.nmax, stream)

    def write_scores(self, s, stream=None):
        tkv_write_scores(self.h, s, stream)

    def read_tiers(self, stream=None):
        return tkv_read_tiers(self.h, self.B, self.nmax, stream)

    def read_layer_tiers(self, layer, stream=None):
        return tkv_read_layer_tiers(self.h, layer, self.B, self.nmax, stream)

    def read_deltas(self):
        return tkv_read_deltas(self.h, self.B, self.nmax)

    def read_kv(self, layer, seq, pos, stream=None):
        """Values attention reads for a live row (bf16 bits as uint16, or fp32)."""
        return tkv_read_kv(self.h, layer, seq, pos, self.Hkv, self.D,
                           np.uint16 if self.dtype == "bf16" else np.float32, stream)

    def read_t2(self, layer, seq, pos):
        return tkv_read_t2(self.h, layer, seq, pos, self.Hkv, self.D, self.n_scales)
