"""Shared driver for GPU-vs-oracle tests: feeds the same seeded inputs to the
HIP library (through the C ABI binding) and to the CPU oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import tkvsynth


def to_device(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Drawn array (bf16 bits or fp32) -> contiguous device tensor of that dtype."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
    return t.cuda().contiguous()


class Inputs:
    """Every input of a workload, drawn once."""

    def __init__(self, w: tkvsynth.Workload):
        self.w = w
        heavy, u = w.heavy_mask(), w.unit_vector()
        self.k0 = w.kv(0, 0, w.prefill, heavy, u)
        self.v0 = w.kv(1, 0, w.prefill, heavy, u)
        self.kn = w.kv(0, w.prefill, w.steps, heavy, u)     # [L][B][T][Hkv][d]
        self.vn = w.kv(1, w.prefill, w.steps, heavy, u)
        self.q = w.q(0, w.steps, u)                          # [T][L][B][Hq][d]

    def step_kv(self, t):
        return (np.ascontiguousarray(self.kn[:, :, t]), np.ascontiguousarray(self.vn[:, :, t]))


def make_oracle(w, inputs: Inputs):
    o = oracle.OracleTKV.for_workload(w)
    o.prefill(w.values(inputs.k0), w.values(inputs.v0))
    return o


def max_rel(a, b, floor=0.0):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.maximum(np.abs(b), floor)
    m = den > 0
    return float(np.max(np.abs(a[m] - b[m]) / den[m])) if m.any() else 0.0
