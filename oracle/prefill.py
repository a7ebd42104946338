"""ORACLE (test infrastructure): cumulative scores of a prefilled prompt.

The step before the decode path ("Not All Thoughts Need HBM", gist.science
technical summary, Method §2): Eq. 1 accumulates each token's attention
weight, averaged over layers and heads, step after step.  A scored prefill
applies the same rule to the prompt: position t attends causally to the
positions 0..t (the usual prefill attention, softmax(q k^T / sqrt(d)) per
layer and query head, query head h reading kv head h / (Hq/Hkv)), and its
weights are added to the scores as a decode step's would be:

    s_j = sum over t >= j of (1/|L|) sum_l (1/H) sum_h alpha_{l,h,t}[j].

The first placement then ranks by these scores with the tier rules of
Method §1 (tiering.reassign) instead of the score-free placement.
"""
from __future__ import annotations

import numpy as np


def prefill_scores(K: np.ndarray, Q: np.ndarray, n: int) -> np.ndarray:
    """K: values [L][B][>=n][Hkv][d]; Q: values [L][B][>=n][Hq][d].
    Returns the scores [B][n] (fp64) after the n prompt positions."""
    L, B, _, Hkv, d = K.shape
    Hq = Q.shape[3]
    g = Hq // Hkv
    s = np.zeros((B, n), np.float64)
    sees = np.tril(np.ones((n, n), bool))           # query t sees keys 0..t
    for l in range(L):
        for b in range(B):
            for h in range(Hq):
                q = Q[l, b, :n, h].astype(np.float64)
                k = K[l, b, :n, h // g].astype(np.float64)
                z = np.where(sees, q @ k.T / np.sqrt(d), -np.inf)
                w = np.exp(z - z.max(axis=1, keepdims=True))
                alpha = w / w.sum(axis=1, keepdims=True)  # row t: weights of query t
                s[b] += alpha.sum(axis=0) / (L * Hq)      # every query's weights, added up
    return s
