"""ORACLE (test infrastructure): tier placement, ranking and delta lists.

Follows "Not All Thoughts Need HBM" (gist.science technical summary):
  * Method §1, four tiers: T0 in HBM holds the protected tokens (prompt,
    attention sinks, recent window) and the most important reasoning tokens;
    T1 (host DDR, full precision) the middle; T2 (host, 8-bit) the low end;
    T3 only the least important tail, deleted for good.
  * Method §2, Eq. 1: the cumulative score s_i is what tokens are ranked by.
  * Method §4: placement is recomputed every Delta decode steps.

Readings where the pages leave a step open (each is listed in the design
notes):
  * counts are floor(ratio * N), N counting every appended position
    including evicted ones; eviction is cumulative and never undone;
    precedence T3, then T0, then T2, then T1;
  * rank order is score descending, then position ascending (unique keys);
  * the first placement (before any score exists) protects P, fills T0 with
    the lowest-index candidates, evicts nothing and uses no T2;
  * the eviction-only baseline (no T1, heavy hitters kept in T0, in the
    manner of the H2O-style policies the summary compares against) takes the
    same ranking and evicts every candidate that would have gone to T1: T0
    first, then T2, and the rest to T3 (the eviction ratio then plays no
    part).  Its first placement evicts what the tiered one puts in T1.
"""
from __future__ import annotations

import math

import numpy as np

T0, T1, T2, T3 = 0, 1, 2, 3


def protected_mask(n: int, prompt: int, sinks: int, recent: int) -> np.ndarray:
    """P = [0, prompt) U [0, sinks) U [n - recent, n): always resident in T0."""
    i = np.arange(n)
    return (i < prompt) | (i < sinks) | (i >= n - recent)


def tier_counts(n: int, n_protected: int, n_candidates: int, n_evicted: int,
                hbm_ratio: float, evict_ratio: float, t2_ratio: float, no_t1: bool = False):
    """How many candidates go to T3, T0 and T2 at one reassignment.

    n3  = min(|C|, max(0, floor(e N) - |T3|))        newly evicted
    n0c = min(|C| - n3, max(0, floor(h N) - |P|))    candidates kept in T0
    n2  = min(|C| - n3 - n0c, floor(t2 N))           candidates put in T2

    Without T1 (eviction-only baseline): n0c = min(|C|, max(0, floor(h N) -
    |P|)), n2 = min(|C| - n0c, floor(t2 N)) and n3 = |C| - n0c - n2.
    """
    if no_t1:
        n0c = min(n_candidates, max(0, math.floor(hbm_ratio * n) - n_protected))
        n2 = min(n_candidates - n0c, math.floor(t2_ratio * n))
        return n_candidates - n0c - n2, n0c, n2
    n3 = min(n_candidates, max(0, math.floor(evict_ratio * n) - n_evicted))
    n0c = min(n_candidates - n3, max(0, math.floor(hbm_ratio * n) - n_protected))
    n2 = min(n_candidates - n3 - n0c, math.floor(t2_ratio * n))
    return n3, n0c, n2


def rank_best_first(candidates, scores) -> list:
    """Candidates ordered by score descending, ties by lower position first."""
    return sorted((int(i) for i in candidates), key=lambda i: (-float(scores[i]), i))


def reassign(old_tiers: np.ndarray, scores: np.ndarray, n: int, prompt: int, sinks: int,
             recent: int, hbm_ratio: float, evict_ratio: float, t2_ratio: float,
             no_t1: bool = False) -> np.ndarray:
    """New tier of each of the n positions from the scores (Method §1, §4)."""
    old = np.asarray(old_tiers)[:n]
    new = np.empty(n, np.uint8)
    prot = protected_mask(n, prompt, sinks, recent)
    evicted = old == T3
    cand = np.nonzero(~prot & ~evicted)[0]
    n3, n0c, n2 = tier_counts(n, int(prot.sum()), len(cand), int(evicted.sum()),
                              hbm_ratio, evict_ratio, t2_ratio, no_t1)
    ranked = rank_best_first(cand, scores)          # best first
    c = len(ranked)
    new[evicted] = T3
    new[prot & ~evicted] = T0
    for r, i in enumerate(ranked):
        if r < n0c:
            new[i] = T0
        elif r >= c - n3:
            new[i] = T3
        elif r >= c - n3 - n2:
            new[i] = T2
        else:
            new[i] = T1
    return new


def initial_placement(n: int, prompt: int, sinks: int, recent: int, hbm_ratio: float,
                      no_t1: bool = False) -> np.ndarray:
    """Tiers of a freshly filled cache: every score is 0, so the rank order is
    position order; no eviction and no T2 before the first real ranking.
    Without T1, the rows that would go to T1 are evicted instead."""
    none_yet = np.full(n, T1, np.uint8)
    zero = np.zeros(n)
    first = reassign(none_yet, zero, n, prompt, sinks, recent, hbm_ratio, 0.0, 0.0)
    if no_t1:
        first[first == T1] = T3
    return first


def delta_lists(old_tiers: np.ndarray, new_tiers: np.ndarray):
    """Rows whose tier changed, ascending by position (Method §4: only changed
    rows move).  A promotion lowers the tier index (towards T0), a demotion
    raises it (towards T3).  Entries are (position, old tier, new tier)."""
    old = np.asarray(old_tiers).astype(np.int64)
    new = np.asarray(new_tiers).astype(np.int64)
    promote = [(int(i), int(old[i]), int(new[i])) for i in np.nonzero(new < old)[0]]
    demote = [(int(i), int(old[i]), int(new[i])) for i in np.nonzero(new > old)[0]]
    return promote, demote


def reassign_shared(old_tiers: np.ndarray, scores: np.ndarray, n: int, prompt: int, sinks: int, recent: int,
                    hbm_ratio: float, evict_ratio: float, t2_ratio: float) -> np.ndarray:
    """Budget variant: one HBM (T0) budget shared by the sequences of a batch
    (the batch projection of the summary's Results; Method §1 rules
    otherwise).  Per sequence, exactly as reassign(): the protected rows stay
    in T0, the n3 lowest-ranked candidates are evicted and T2 takes the next
    lowest.  T0 beyond the protected rows holds the best n0c_total of the
    batch's remaining candidates, ranked jointly by (score descending,
    sequence ascending, position ascending), with
        n0c_total = min(sum of remaining, max(0, B floor(h N) - sum |P|)).
    old_tiers, scores: [B][>= n]."""
    B = len(old_tiers)
    prot = protected_mask(n, prompt, sinks, recent)
    ranked, n3s = [], []
    for b in range(B):
        old = np.asarray(old_tiers[b])[:n]
        evicted = old == T3
        cand = np.nonzero(~prot & ~evicted)[0]
        n3, _, _ = tier_counts(n, int(prot.sum()), len(cand), int(evicted.sum()), hbm_ratio, evict_ratio, t2_ratio)
        ranked.append(rank_best_first(cand, scores[b]))
        n3s.append(n3)
    remaining = [(b, i) for b in range(B) for i in ranked[b][: len(ranked[b]) - n3s[b]]]
    budget = B * math.floor(hbm_ratio * n) - B * int(prot.sum())
    n0c_total = min(len(remaining), max(0, budget))
    joint = sorted(remaining, key=lambda bi: (-float(scores[bi[0]][bi[1]]), bi[0], bi[1]))
    in_t0 = set(joint[:n0c_total])
    new = np.empty((B, n), np.uint8)
    for b in range(B):
        old = np.asarray(old_tiers[b])[:n]
        new[b][old == T3] = T3
        new[b][prot & (old != T3)] = T0
        rb = ranked[b]
        c, n3 = len(rb), n3s[b]
        n0c = sum(1 for i in rb if (b, i) in in_t0)
        n2 = min(c - n3 - n0c, math.floor(t2_ratio * n))
        for r, i in enumerate(rb):
            if (b, i) in in_t0:
                new[b][i] = T0
            elif r >= c - n3:
                new[b][i] = T3
            elif r >= c - n3 - n2:
                new[b][i] = T2
            else:
                new[b][i] = T1
    return new
