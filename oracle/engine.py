"""ORACLE (test infrastructure): one tiered KV cache, step by step, in fp64.

"Not All Thoughts Need HBM" (gist.science technical summary) and the paper's
abstract fix what a decode step computes:
  * every generated token adds a K/V row to the cache (problem statement);
  * attention runs over every non-evicted row; T1 rows come back at full
    precision and contribute exactly what they would have from HBM (Method
    §3, Proposition 1) -- the placement of a live row does not enter;
  * Eq. 1 (Method §2): s_i += (1/|L|) sum_l (1/H) sum_h alpha_{l,h}[i];
  * every Delta steps tokens are re-placed by score (Method §1 and §4); rows
    entering T2 are quantised (codec.py).

Readings (listed in the design notes): a new token is appended before the
step's attention and attends to itself; it enters T0 with s = 0; H in Eq. 1
is the number of query heads; sequences of a batch are independent and
advance together.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import codec, prefill as _prefill, tiering
from .tiering import T0, T1, T2, T3

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attend.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None
_UNUSED = 255   # tier code of positions not appended yet


def build(force: bool = True) -> str:
    global _lib
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC",
                               "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        i32, i64, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
        lib.oracle_attend.argtypes = [i32, i32, i32, i32, i32, i64, i64, vp, vp, vp, vp, vp, vp]
        lib.oracle_attend.restype = None
        _lib = lib
    return _lib


def _p(a):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def attend(K, V, live, q, n):
    """Softmax attention of every (layer, sequence, query head) over the live rows.

    K, V: float32 [L][B][nmax][Hkv][d]; live: bool/uint8 [B][nmax];
    q: [L][B][Hq][d].  Returns out [L][B][Hq][d] and alpha [L][B][Hq][nmax]
    (fp64; alpha is 0 off the live set)."""
    K = np.ascontiguousarray(K, np.float32)
    V = np.ascontiguousarray(V, np.float32)
    live = np.ascontiguousarray(live, np.uint8)
    q = np.ascontiguousarray(q, np.float64)
    L, B, nmax, Hkv, d = K.shape
    Hq = q.shape[2]
    assert q.shape == (L, B, Hq, d) and live.shape == (B, nmax) and Hq % Hkv == 0
    out = np.empty((L, B, Hq, d), np.float64)
    alpha = np.empty((L, B, Hq, nmax), np.float64)
    _load().oracle_attend(L, B, Hq, Hkv, d, nmax, n, _p(K), _p(V), _p(live), _p(q), _p(out),
                          _p(alpha))
    return out, alpha


def eq1_increment(alpha: np.ndarray) -> np.ndarray:
    """Eq. 1 increment per (sequence, position): (1/|L|) sum_l (1/H) sum_h alpha.

    alpha: [L][B][H][n] -> [B][n]."""
    per_layer = alpha.sum(axis=2) / alpha.shape[2]      # (1/H) sum_h, [L][B][n]
    return per_layer.sum(axis=0) / alpha.shape[0]       # (1/|L|) sum_l, [B][n]


class OracleTKV:
    """Plain model of the tiered cache of a batch of sequences."""

    def __init__(self, layers, q_heads, kv_heads, head_dim, batch, max_tokens, delta,
                 hbm_ratio, evict_ratio, t2_ratio, prompt, sinks, recent, bf16, no_t1=False, t2_fp8=False,
                 shared_hbm=False, t2_head_scales=False):
        self.L, self.Hq, self.Hkv, self.d, self.B = layers, q_heads, kv_heads, head_dim, batch
        self.nmax, self.delta = max_tokens, delta
        self.hbm, self.evict, self.t2 = hbm_ratio, evict_ratio, t2_ratio
        self.no_t1 = no_t1
        self.t2_fp8 = t2_fp8
        self.shared_hbm = shared_hbm
        self.t2_head_scales = t2_head_scales
        self.prompt, self.sinks, self.recent = prompt, sinks, recent
        self.bf16 = bf16
        self.K = np.zeros((layers, batch, max_tokens, kv_heads, head_dim), np.float32)
        self.V = np.zeros_like(self.K)
        self.tier = np.full((batch, max_tokens), _UNUSED, np.uint8)
        self.s = np.zeros((batch, max_tokens), np.float64)
        self.n = 0
        self.step = 0

    @classmethod
    def for_workload(cls, w, max_tokens=None):
        return cls(w.layers, w.q_heads, w.kv_heads, w.head_dim, w.batch,
                   max_tokens or w.n_final, w.delta, w.hbm_ratio, w.evict_ratio, w.t2_ratio,
                   w.prompt, w.sinks, w.recent, w.dtype == "bf16", w.no_t1, w.t2_fp8, w.shared_hbm,
                   w.t2_head_scales)

    # -- cache contents ------------------------------------------------------
    def prefill(self, K, V):
        """K, V: float32 values [L][B][n0][Hkv][d]; first placement of the rows."""
        n0 = K.shape[2]
        assert self.n == 0 and n0 <= self.nmax
        self.K[:, :, :n0] = K
        self.V[:, :, :n0] = V
        self.n = n0
        first = tiering.initial_placement(n0, self.prompt, self.sinks, self.recent, self.hbm, self.no_t1)
        self.tier[:, :n0] = first[None, :]

    def prefill_scored(self, K, V, Q):
        """Scored prefill: the rows as prefill() places them, the prompt's
        causal attention weights added to the scores (prefill.py), then one
        re-placement by those scores with the full tier rules.  Returns what
        reassign() returns."""
        self.prefill(K, V)
        self.s[:, : self.n] = _prefill.prefill_scores(K, Q, self.n)
        return self.reassign()

    def append(self, k, v):
        """k, v: float32 values [L][B][Hkv][d] of the new token (position n)."""
        assert self.n < self.nmax
        self.K[:, :, self.n] = k
        self.V[:, :, self.n] = v
        self.tier[:, self.n] = T0
        self.s[:, self.n] = 0.0
        self.n += 1

    def live(self):
        return (self.tier != T3) & (self.tier != _UNUSED)

    # -- one decode step -----------------------------------------------------
    def attend(self, q, update_scores=True):
        """q: [L][B][Hq][d] values.  Returns out [L][B][Hq][d] fp64 and adds the
        step's Eq. 1 increment to s (evicted rows keep their frozen score)."""
        live = self.live()
        out, alpha = attend(self.K, self.V, live, q, self.n)
        if update_scores:
            inc = eq1_increment(alpha[..., : self.n])
            self.s[:, : self.n] += np.where(live[:, : self.n], inc, 0.0)
            self.step += 1
        self.last_alpha = alpha
        return out

    # -- reassignment ----------------------------------------------------------
    def reassign(self, rank_scores=None, adopt=None):
        """Re-place every sequence's rows.

        rank_scores: optional [B][n] scores to rank by (e.g. another
        implementation's fp32 scores); default is the oracle's own fp64 s.
        adopt: optional [B][n] tiers to take instead of the computed ones
        (after checking them elsewhere).  Returns (new tiers [B][n],
        [(promote, demote)] per sequence)."""
        n = self.n
        scores = self.s[:, :n] if rank_scores is None else np.asarray(rank_scores, np.float64)
        new_all = np.empty((self.B, n), np.uint8)
        deltas = []
        shared = None
        if self.shared_hbm:
            shared = tiering.reassign_shared(self.tier[:, :n].copy(), scores, n, self.prompt, self.sinks,
                                             self.recent, self.hbm, self.evict, self.t2)
        for b in range(self.B):
            old = self.tier[b, :n].copy()
            if shared is not None:
                new = shared[b]
            else:
                new = tiering.reassign(old, scores[b], n, self.prompt, self.sinks, self.recent,
                                       self.hbm, self.evict, self.t2, self.no_t1)
            if adopt is not None:
                new = np.asarray(adopt[b][:n], np.uint8)
            deltas.append(tiering.delta_lists(old, new))
            # rows entering T2 lose their full-precision values for good
            entering = np.nonzero((new == T2) & (old != T2))[0]
            for i in entering:
                for l in range(self.L):
                    for X in (self.K, self.V):
                        if self.t2_head_scales:
                            X[l, b, i] = codec.roundtrip_heads(X[l, b, i], self.t2_fp8, self.bf16)
                        else:
                            X[l, b, i] = (codec.roundtrip_fp8 if self.t2_fp8 else codec.roundtrip)(X[l, b, i],
                                                                                                   self.bf16)
            self.tier[b, :n] = new
            new_all[b] = new
        return new_all, deltas


def layer_groups(layer_hbm):
    """Consecutive layers with the same HBM ratio, as [(first layer, end, ratio)]."""
    out = []
    for l, h in enumerate(layer_hbm):
        if out and out[-1][2] == h:
            out[-1] = (out[-1][0], l + 1, h)
        else:
            out.append((l, l + 1, h))
    return out


class OracleLayerGroups:
    """Per-layer HBM budgets (the budget variant in the spirit of ARKV's
    per-layer ratios, gist.science ARKV summary, Method; tiers and Eq. 1 from
    "Not All Thoughts Need HBM", Method §1, §2 and §4).  Reading: layer l
    keeps floor(h_l N) rows in HBM.  Consecutive layers with one ratio form a
    group, and each group places its rows by the rules of Method §1 with its
    own ratio.  Every group ranks by the one Eq. 1 score, which averages over
    all layers, and shares the eviction and T2 ratios.  So every group evicts
    the same rows, and a group's T0 holds the protected rows and its best
    candidates.  Each group is an OracleTKV over its layers.  They hold one
    score array, to which each step adds the all-layer increment once."""

    def __init__(self, layer_hbm, q_heads, kv_heads, head_dim, batch, max_tokens, delta, evict_ratio, t2_ratio,
                 prompt, sinks, recent, bf16, t2_fp8=False, t2_head_scales=False):
        self.groups = layer_groups(list(layer_hbm))
        self.L, self.B, self.Hq = len(layer_hbm), batch, q_heads
        self.parts = [OracleTKV(l1 - l0, q_heads, kv_heads, head_dim, batch, max_tokens, delta, h, evict_ratio,
                                t2_ratio, prompt, sinks, recent, bf16, t2_fp8=t2_fp8, t2_head_scales=t2_head_scales)
                      for (l0, l1, h) in self.groups]
        self.s = self.parts[0].s
        for p in self.parts:
            p.s = self.s  # one score array for every group

    @classmethod
    def for_workload(cls, w, layer_hbm, max_tokens=None):
        assert len(layer_hbm) == w.layers
        return cls(layer_hbm, w.q_heads, w.kv_heads, w.head_dim, w.batch, max_tokens or w.n_final, w.delta,
                   w.evict_ratio, w.t2_ratio, w.prompt, w.sinks, w.recent, w.dtype == "bf16", w.t2_fp8,
                   w.t2_head_scales)

    @property
    def n(self):
        return self.parts[0].n

    def part_of(self, layer):
        """(group index, layer within the group) of a layer."""
        for g, (l0, l1, _) in enumerate(self.groups):
            if l0 <= layer < l1:
                return g, layer - l0
        raise IndexError(layer)

    def tier_of(self, layer):
        return self.parts[self.part_of(layer)[0]].tier

    def live(self):
        return self.parts[0].live()

    def prefill(self, K, V):
        """K, V: float32 values [L][B][n0][Hkv][d]."""
        for (l0, l1, _), p in zip(self.groups, self.parts):
            p.prefill(K[l0:l1], V[l0:l1])

    def prefill_scored(self, K, V, Q):
        """The scored prefill: each group places its rows as prefill() does,
        the prompt's causal attention weights over all layers become the shared
        scores (prefill.py), then every group is re-placed by them."""
        self.prefill(K, V)
        self.s[:, : self.n] = _prefill.prefill_scores(K, Q, self.n)
        return self.reassign()

    def append(self, k, v):
        for (l0, l1, _), p in zip(self.groups, self.parts):
            p.append(k[l0:l1], v[l0:l1])

    def attend(self, q):
        """q: [L][B][Hq][d] values.  Returns out [L][B][Hq][d] and adds the
        step's Eq. 1 increment over all L layers to the shared scores."""
        live = self.live()
        outs, inc = [], 0.0
        for (l0, l1, _), p in zip(self.groups, self.parts):
            assert np.array_equal(p.live(), live), "groups disagree on the evicted rows"
            outs.append(p.attend(q[l0:l1], update_scores=False))
            # (1/L_g) sum over the group's layers, weighted L_g / L: (1/L) sum over all layers
            inc = inc + eq1_increment(p.last_alpha[..., : self.n]) * ((l1 - l0) / self.L)
        self.s[:, : self.n] += np.where(live[:, : self.n], inc, 0.0)
        for p in self.parts:
            p.step += 1
        return np.concatenate(outs, axis=0)

    def reassign(self, rank_scores=None, adopt=None):
        """Every group re-placed by the shared scores with its own ratio.
        adopt: optional per-group tiers [G][B][n].  Returns [(tiers, deltas)]
        per group."""
        scores = self.s[:, : self.n] if rank_scores is None else rank_scores
        return [p.reassign(rank_scores=scores, adopt=None if adopt is None else adopt[g])
                for g, p in enumerate(self.parts)]
