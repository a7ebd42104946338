"""ORACLE -- test infrastructure, not part of the product.

A plain, slow fp64 CPU model of the tiered-KV decode step of "Not All
Thoughts Need HBM: Semantics-Aware Memory Hierarchy for LLM Reasoning"
(arXiv 2605.09490): attention over the non-evicted rows, the cumulative
score of Eq. 1, score-ranked re-placement into T0..T3 every Delta steps, the
changed-row lists, the 8-bit codec of T2, the scores of a scored prefill
(causal attention weights of the prompt added up as Eq. 1 does), and the
two HBM budget variants (one budget shared by a batch; per-layer budgets).

It shares no code with the GPU library (decode_attention_tkv_amd) and never
imports it.  Only tests/, the smoke check in __graft_entry__.py and the
CPU-baseline leg of bench.py may import or run anything here.

Pins (tests/test_oracle_*.py): dense special case equals a textbook softmax
attention (torch float64 SDPA and a pure-Python loop), closed forms (q = 0,
one live row, two rows), the Eq. 1 increments summing to 1 per step,
independence from the T0/T1 split, exhaustive ranking properties on tiny
cases, hand-derived tier counts (tests/golden/), and the codec's error bound.
"""
from .engine import OracleLayerGroups, OracleTKV, attend, build, eq1_increment, layer_groups
from .prefill import prefill_scores
from .tiering import T0, T1, T2, T3

__all__ = ["OracleLayerGroups", "OracleTKV", "attend", "build", "eq1_increment", "layer_groups", "prefill_scores",
           "T0", "T1", "T2", "T3"]
