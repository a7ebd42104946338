"""Pins for the oracle's batch-shared HBM budget (tiering.reassign_shared):
one T0 budget of B * floor(h N) for a batch, the candidates ranked jointly by
(score descending, sequence ascending, position ascending); eviction and T2
per sequence as in Method §1 of "Not All Thoughts Need HBM" (gist.science
summary).

* one sequence: exactly the per-sequence rules (tiering.reassign);
* a hand-derived two-sequence case (every T0 slot goes to the sequence whose
  tokens score higher);
* tiny cases with heavy ties: per-sequence T3 and T2 as the per-sequence
  rules fix them, the T0 total equal to the shared budget, and every T0
  candidate ranked jointly above every candidate left in T1 or T2.
"""
import math

import numpy as np

from oracle import tiering
from oracle.tiering import T0, T1, T2, T3


def test_one_sequence_is_the_per_sequence_rule():
    rng = np.random.default_rng(0)
    for trial in range(200):
        n = int(rng.integers(1, 40))
        prompt, sinks, recent = (int(x) for x in rng.integers(0, 5, 3))
        h, e, t2 = (float(x) for x in rng.choice([0.0, 0.1, 0.3, 0.5, 1.0], 3))
        scores = rng.choice([0.0, 0.5, 1.0], n)
        old = np.full(n, T1, np.uint8)
        prot = tiering.protected_mask(n, prompt, sinks, recent)
        unprot = np.nonzero(~prot)[0]
        old[rng.choice(unprot, size=int(rng.integers(0, len(unprot) + 1)), replace=False)] = T3
        a = tiering.reassign(old, scores, n, prompt, sinks, recent, h, e, t2)
        b = tiering.reassign_shared(old[None, :], scores[None, :], n, prompt, sinks, recent, h, e, t2)[0]
        assert np.array_equal(a, b)


def test_hand_derived_two_sequences():
    # n = 20, P = {0, 1, 18, 19}; budget 2*floor(.5*20) - 2*4 = 12; floor(.1*20) = 2 evicted and 2 in T2 each
    n = 20
    old = np.full((2, n), T1, np.uint8)
    scores = np.stack([np.ones(n), np.zeros(n)])
    new = tiering.reassign_shared(old, scores, n, 2, 2, 2, 0.5, 0.1, 0.1)
    assert np.array_equal(np.nonzero(new[0] == T0)[0], np.r_[0:14, 18:20])
    assert np.array_equal(np.nonzero(new[0] == T2)[0], [14, 15])
    assert np.array_equal(np.nonzero(new[0] == T3)[0], [16, 17])
    assert np.array_equal(np.nonzero(new[1] == T0)[0], [0, 1, 18, 19])
    assert np.array_equal(np.nonzero(new[1] == T1)[0], np.r_[2:14])
    assert np.array_equal(np.nonzero(new[1] == T2)[0], [14, 15])
    assert np.array_equal(np.nonzero(new[1] == T3)[0], [16, 17])


def test_properties_on_tiny_batches():
    rng = np.random.default_rng(1)
    for trial in range(300):
        B = int(rng.integers(1, 4))
        n = int(rng.integers(1, 14))
        prompt, sinks, recent = (int(x) for x in rng.integers(0, 4, 3))
        h, e, t2 = (float(x) for x in rng.choice([0.0, 0.1, 0.3, 0.5, 0.7], 3))
        scores = rng.choice([0.0, 0.25, 1.0], (B, n))
        prot = tiering.protected_mask(n, prompt, sinks, recent)
        old = np.full((B, n), T1, np.uint8)
        for b in range(B):
            unprot = np.nonzero(~prot)[0]
            old[b, rng.choice(unprot, size=int(rng.integers(0, len(unprot) + 1)), replace=False)] = T3
        new = tiering.reassign_shared(old, scores, n, prompt, sinks, recent, h, e, t2)
        kept, left = [], []
        n_rem = 0
        for b in range(B):
            cand = np.nonzero(~prot & (old[b] != T3))[0]
            n3, _, _ = tiering.tier_counts(n, int(prot.sum()), len(cand), int((old[b] == T3).sum()), h, e, t2)
            ranked = tiering.rank_best_first(cand, scores[b])
            assert np.array_equal(np.sort(np.nonzero((new[b] == T3) & (old[b] != T3))[0]), np.sort(ranked[len(ranked) - n3:]))
            n0c = int(((new[b] == T0) & ~prot).sum())
            n2 = min(len(cand) - n3 - n0c, math.floor(t2 * n))
            assert np.array_equal(np.sort(np.nonzero(new[b] == T2)[0]),
                                  np.sort(ranked[len(ranked) - n3 - n2:len(ranked) - n3]))
            n_rem += len(cand) - n3
            kept += [(scores[b][i], b, i) for i in cand if new[b][i] == T0]
            left += [(scores[b][i], b, i) for i in cand if new[b][i] in (T1, T2)]
        assert len(kept) == min(n_rem, max(0, B * math.floor(h * n) - B * int(prot.sum())))
        for sk, bk, ik in kept:
            for sl, bl, il in left:
                assert (-sk, bk, ik) < (-sl, bl, il)
