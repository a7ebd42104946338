"""Pins of the oracle's placement rules (CPU only).

"Not All Thoughts Need HBM" (gist.science summary), Method §1 (four tiers,
protected set in T0, only the least important tail evicted) and Method §4
(score-ranked re-placement every Delta steps, only changed rows move).

Pins: hand-derived tier counts (tests/golden/tier_counts.json); on many tiny
random cases with heavy score ties, properties that together fix the one
correct labelling -- protected rows in T0, evicted rows stay evicted, tier
sizes equal the counts, and no candidate ranked above another (score
descending, position ascending) sits in a lower tier; all-equal scores put
the lowest positions in T0 and the highest in T3; the delta lists are
exactly the changed rows, split by direction, in position order.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import tiering
from oracle.tiering import T0, T1, T2, T3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tier_counts.json")
# rank of a tier in "importance" order: T3 (lowest) < T2 < T1 < T0 (highest)
IMPORTANCE = {T3: 0, T2: 1, T1: 2, T0: 3}


def _golden_rows():
    doc = json.load(open(GOLDEN))
    return [dict(zip(doc["fields"], r["case"]), why=r["why"]) for r in doc["rows"]]


@pytest.mark.parametrize("row", _golden_rows(), ids=lambda r: r["why"][:40])
def test_golden_counts(row):
    n = row["n"]
    prot = tiering.protected_mask(n, row["prompt"], row["sinks"], row["recent"])
    assert prot.sum() == row["expect_protected"]
    # place the prior evictions on the first unprotected positions
    old = np.full(n, T1, np.uint8)
    unprot = np.nonzero(~prot)[0]
    old[unprot[: row["n_evicted_before"]]] = T3
    cand = (~prot) & (old != T3)
    assert cand.sum() == row["expect_candidates"]
    n3, n0c, n2 = tiering.tier_counts(n, int(prot.sum()), int(cand.sum()), row["n_evicted_before"],
                                      row["hbm"], row["evict"], row["t2"])
    assert (n3, n0c, n2) == (row["expect_n3"], row["expect_n0c"], row["expect_n2"])
    scores = np.random.default_rng(n).random(n)
    new = tiering.reassign(old, scores, n, row["prompt"], row["sinks"], row["recent"],
                           row["hbm"], row["evict"], row["t2"])
    counts = [int((new == t).sum()) for t in (T0, T1, T2, T3)]
    assert counts == [row["expect_T0"], row["expect_T1"], row["expect_T2"], row["expect_T3"]]


def _check_labelling(old, new, scores, n, prompt, sinks, recent, h, e, t2):
    prot = tiering.protected_mask(n, prompt, sinks, recent)
    was_evicted = old == T3
    assert np.all(new[was_evicted] == T3)
    assert np.all(new[prot & ~was_evicted] == T0)
    cand = np.nonzero(~prot & ~was_evicted)[0]
    n3, n0c, n2 = tiering.tier_counts(n, int(prot.sum()), len(cand), int(was_evicted.sum()), h, e, t2)
    got = {t: int((new[cand] == t).sum()) for t in (T0, T1, T2, T3)}
    assert got[T3] == n3 and got[T0] == n0c and got[T2] == n2
    assert got[T1] == len(cand) - n3 - n0c - n2
    # order consistency over every pair of candidates
    for a, b in itertools.combinations(cand, 2):
        a_first = (scores[a] > scores[b]) or (scores[a] == scores[b] and a < b)
        hi, lo = (a, b) if a_first else (b, a)
        assert IMPORTANCE[int(new[hi])] >= IMPORTANCE[int(new[lo])], (hi, lo, new[hi], new[lo])


def test_exhaustive_tiny_cases_with_ties():
    rng = np.random.default_rng(0)
    levels = np.array([0.0, 0.25, 0.5, 1.0])
    cases = 0
    for n in range(1, 13):
        for trial in range(40):
            prompt, sinks, recent = (int(x) for x in rng.integers(0, 4, 3))
            h, e, t2 = (float(x) for x in rng.choice([0.0, 0.1, 0.3, 0.5, 0.7, 1.0], 3))
            scores = levels[rng.integers(0, len(levels), n)]
            old = np.full(n, T1, np.uint8)
            prot = tiering.protected_mask(n, prompt, sinks, recent)
            unprot = np.nonzero(~prot)[0]
            k = int(rng.integers(0, len(unprot) + 1))
            old[rng.choice(unprot, size=k, replace=False)] = T3
            new = tiering.reassign(old, scores, n, prompt, sinks, recent, h, e, t2)
            _check_labelling(old, new, scores, n, prompt, sinks, recent, h, e, t2)
            cases += 1
    assert cases == 480


def test_all_equal_scores_break_ties_by_position():
    n, prompt, sinks, recent = 40, 4, 4, 6
    new = tiering.reassign(np.full(n, T1, np.uint8), np.full(n, 0.5), n, prompt, sinks, recent,
                           0.5, 0.25, 0.25)
    prot = tiering.protected_mask(n, prompt, sinks, recent)
    cand = np.nonzero(~prot)[0]                 # 4..33
    # floor(.25*40)=10 evicted: the 10 highest candidate positions
    assert np.array_equal(np.nonzero(new == T3)[0], cand[-10:])
    # T0 budget 20 - 10 protected = 10 lowest candidates
    assert np.array_equal(np.nonzero((new == T0) & ~prot)[0], cand[:10])
    assert np.array_equal(np.nonzero(new == T2)[0], cand[-20:-10])
    assert (new == T1).sum() == 0


def test_higher_score_wins_over_position():
    n = 10
    scores = np.zeros(n)
    scores[9] = 1.0       # the last (unprotected when recent = 0) position is the best
    new = tiering.reassign(np.full(n, T1, np.uint8), scores, n, 0, 0, 0, 0.1, 0.1, 0.0)
    assert new[9] == T0 and (new == T0).sum() == 1
    assert new[8] == T3 and (new == T3).sum() == 1


def test_initial_placement():
    n, prompt, sinks, recent = 100, 10, 4, 20
    t = tiering.initial_placement(n, prompt, sinks, recent, 0.5)
    assert np.array_equal(np.nonzero(t == T0)[0], np.r_[0:30, 80:100])
    assert np.all(t[30:80] == T1)
    assert (t == T3).sum() == 0 and (t == T2).sum() == 0


def test_delta_lists():
    old = np.array([T0, T1, T2, T3, T0, T1, T1, T2, T0], np.uint8)
    new = np.array([T1, T0, T0, T3, T3, T1, T2, T1, T0], np.uint8)
    promote, demote = tiering.delta_lists(old, new)
    assert promote == [(1, T1, T0), (2, T2, T0), (7, T2, T1)]
    assert demote == [(0, T0, T1), (4, T0, T3), (6, T1, T2)]
