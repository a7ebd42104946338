"""Pins of the oracle's attention (CPU only).

Method §3 of "Not All Thoughts Need HBM" (gist.science summary): every
non-evicted row contributes to the step's attention exactly as if it sat in
HBM.  The oracle's attention over the live set is pinned against:
  * torch's float64 scaled_dot_product_attention (a library routine), with a
    boolean mask for evicted rows and kv heads repeated for grouped queries;
  * closed forms: q = 0 gives uniform weights and the mean of V; one live
    row gives that row; two rows give a logistic weight;
  * the grouped-query head mapping, h -> floor(h / group).
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _case(rng, L=2, B=2, Hq=4, Hkv=2, d=16, nmax=13, n=11, evict_frac=0.0):
    K = rng.standard_normal((L, B, nmax, Hkv, d)).astype(np.float32)
    V = rng.standard_normal((L, B, nmax, Hkv, d)).astype(np.float32)
    q = rng.standard_normal((L, B, Hq, d))
    live = np.zeros((B, nmax), np.uint8)
    live[:, :n] = 1
    if evict_frac:
        for b in range(B):
            off = rng.choice(n, size=int(evict_frac * n), replace=False)
            live[b, off] = 0
    return K, V, q, live, n


def _sdpa(K, V, q, live, n):
    """Library reference: torch float64 SDPA per (layer, sequence)."""
    L, B, nmax, Hkv, d = K.shape
    Hq = q.shape[2]
    out = np.zeros((L, B, Hq, d))
    for l in range(L):
        for b in range(B):
            k = torch.from_numpy(K[l, b, :n].astype(np.float64)).transpose(0, 1)   # [Hkv, n, d]
            v = torch.from_numpy(V[l, b, :n].astype(np.float64)).transpose(0, 1)
            k = k.repeat_interleave(Hq // Hkv, dim=0).contiguous()
            v = v.repeat_interleave(Hq // Hkv, dim=0).contiguous()
            qq = torch.from_numpy(q[l, b]).unsqueeze(1)                             # [Hq, 1, d]
            mask = torch.from_numpy(live[b, :n].astype(bool)).view(1, 1, n).expand(Hq, 1, n)
            o = torch.nn.functional.scaled_dot_product_attention(qq, k, v, attn_mask=mask)
            out[l, b] = o[:, 0].numpy()
    return out


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (6, 1), (8, 2)])
def test_dense_equals_sdpa(Hq, Hkv):
    rng = np.random.default_rng(1)
    K, V, q, live, n = _case(rng, Hq=Hq, Hkv=Hkv)
    out, alpha = oracle.attend(K, V, live, q, n)
    ref = _sdpa(K, V, q, live, n)
    assert np.max(np.abs(out - ref)) < 1e-12
    assert np.allclose(alpha[..., :n].sum(-1), 1.0, atol=1e-13)
    assert np.all(alpha[..., n:] == 0)


@pytest.mark.parametrize("evict_frac", [0.2, 0.5])
def test_evicted_rows_masked_equals_sdpa(evict_frac):
    rng = np.random.default_rng(2)
    K, V, q, live, n = _case(rng, evict_frac=evict_frac)
    out, alpha = oracle.attend(K, V, live, q, n)
    ref = _sdpa(K, V, q, live, n)
    assert np.max(np.abs(out - ref)) < 1e-12
    dead = np.broadcast_to(live[None, :, None, :] == 0, alpha.shape)
    assert np.all(alpha[dead] == 0)


def test_zero_query_gives_uniform_weights_and_mean_value():
    rng = np.random.default_rng(3)
    K, V, q, live, n = _case(rng, evict_frac=0.3)
    q[:] = 0
    out, alpha = oracle.attend(K, V, live, q, n)
    L, B, nmax, Hkv, d = K.shape
    Hq = q.shape[2]
    for l in range(L):
        for b in range(B):
            idx = np.nonzero(live[b, :n])[0]
            for h in range(Hq):
                g = h // (Hq // Hkv)
                assert np.allclose(alpha[l, b, h, idx], 1.0 / len(idx), rtol=0, atol=1e-15)
                mean_v = V[l, b, idx, g].astype(np.float64).mean(axis=0)
                assert np.max(np.abs(out[l, b, h] - mean_v)) < 1e-13


def test_single_live_row_returns_it():
    rng = np.random.default_rng(4)
    K, V, q, live, n = _case(rng)
    live[:] = 0
    live[0, 5] = 1
    live[1, 0] = 1
    out, alpha = oracle.attend(K, V, live, q, n)
    for l in range(K.shape[0]):
        for h in range(q.shape[2]):
            g = h // (q.shape[2] // K.shape[3])
            assert np.array_equal(out[l, 0, h], V[l, 0, 5, g].astype(np.float64))
            assert np.array_equal(out[l, 1, h], V[l, 1, 0, g].astype(np.float64))
            assert alpha[l, 0, h, 5] == 1.0 and alpha[l, 1, h, 0] == 1.0


def test_two_rows_logistic_weight():
    # q = (1, 0), k1 = (2, 0), k2 = (0, 0), d = 2: z1 = 2/sqrt(2), z2 = 0.
    K = np.zeros((1, 1, 2, 1, 2), np.float32)
    V = np.zeros_like(K)
    K[0, 0, 0, 0] = [2.0, 0.0]
    V[0, 0, 0, 0] = [1.0, 0.0]
    V[0, 0, 1, 0] = [0.0, 1.0]
    q = np.array([[[[1.0, 0.0]]]])
    live = np.ones((1, 2), np.uint8)
    out, alpha = oracle.attend(K, V, live, q, 2)
    a1 = 1.0 / (1.0 + math.exp(-math.sqrt(2.0)))
    assert abs(alpha[0, 0, 0, 0] - a1) < 1e-15
    assert abs(alpha[0, 0, 0, 1] - (1 - a1)) < 1e-15
    assert np.allclose(out[0, 0, 0], [a1, 1 - a1], atol=1e-15, rtol=0)


def test_grouped_query_head_mapping():
    # kv head g holds the constant value row g, so out[h] reveals the kv head read.
    L, B, Hq, Hkv, d, n = 1, 1, 8, 2, 4, 5
    rng = np.random.default_rng(5)
    K = rng.standard_normal((L, B, n, Hkv, d)).astype(np.float32)
    V = np.zeros((L, B, n, Hkv, d), np.float32)
    for g in range(Hkv):
        V[:, :, :, g, :] = g
    q = rng.standard_normal((L, B, Hq, d))
    out, _ = oracle.attend(K, V, np.ones((B, n), np.uint8), q, n)
    for h in range(Hq):
        assert np.allclose(out[0, 0, h], h // (Hq // Hkv), atol=1e-14)


def test_positions_beyond_n_are_ignored():
    rng = np.random.default_rng(6)
    K, V, q, live, n = _case(rng)
    live[:] = 1                         # rows >= n are flagged live but not appended
    out, _ = oracle.attend(K, V, live, q, n)
    live2 = live.copy()
    live2[:, n:] = 0
    ref = _sdpa(K, V, q, live2, n)
    assert np.max(np.abs(out - ref)) < 1e-12
