"""Seeded random configurations through the whole path, against the oracle.

Each case draws a small workload -- dtype, head_dim, kv heads and group,
layers, batch, prefill (0 to a few hundred positions, so also an empty
cache), decode steps and Delta, the HBM, eviction and 8-bit ratios
("Not All Thoughts Need HBM", gist.science summary, Method §1: the tier
budgets; HBM + eviction may exceed 1), the protected prompt, sinks and
recent window, the 8-bit codec variants, eviction-only, the batch-shared
budget, resident or stream staging with a random number of slots, and the
chunk size, and the calls of a step (append and attention, the single-call
step, or the attention in layer groups), and whether the reassignments go
through tkv_reassign or tkv_reassign_static -- and runs it step by step with
a reassignment every Delta steps
(Method §4), as the fixed tests do: outputs within the dtype's tolerance,
scores within relative 1e-4 (Method §2, Eq. 1), and every reassignment's
labels and changed-row lists bit-exact against the oracle's rules applied to
the GPU's fp32 scores.  The draws cover combinations no fixed test names.
"""
import numpy as np
import pytest

import tkvsynth
from harness import Inputs
from test_gpu_reassign import run_parity

pytestmark = pytest.mark.gpu

N_CASES = 64


def _draw(i):
    r = np.random.default_rng(1000 + i)
    dtype = "bf16" if r.random() < 0.6 else "f32"
    group = int(r.choice([1, 2, 4, 5, 8]))
    kv_heads = int(r.choice([1, 2, 4]))
    layers = int(r.integers(1, 5))
    batch = int(r.integers(1, 4))
    prefill = int(r.choice([0, int(r.integers(40, 420))]))
    delta = int(r.choice([8, 16, 32]))
    steps = int(r.integers(2, 4)) * delta + int(r.integers(0, delta))
    no_t1 = bool(r.random() < 0.15)
    shared = bool(not no_t1 and batch > 1 and r.random() < 0.25)
    t2 = float(r.choice([0.0, 0.0, 0.1, 0.25]))
    w = tkvsynth.CONFIGS["tiny"].replace(
        name="random%d" % i, dtype=dtype, head_dim=int(r.choice([64, 128])), kv_heads=kv_heads,
        q_heads=kv_heads * group, layers=layers, batch=batch, prefill=prefill, steps=steps, delta=delta,
        hbm_ratio=float(np.round(r.uniform(0.0, 1.0), 2)), evict_ratio=float(np.round(r.uniform(0.0, 0.6), 2)),
        t2_ratio=t2, prompt=int(r.integers(0, min(prefill, 48) + 1)), sinks=int(r.integers(0, 6)),
        recent=int(r.integers(0, 40)), seed=int(r.integers(0, 1 << 20)), no_t1=no_t1, shared_hbm=shared,
        t2_fp8=bool(t2 > 0 and r.random() < 0.5), t2_head_scales=bool(t2 > 0 and r.random() < 0.5))
    staging = int(r.integers(2, layers)) if layers >= 3 and r.random() < 0.4 else 0
    chunk = int(r.choice([0, 128, 256, 512]))
    # the calls of a step: append + attention, the single-call step, or layer groups
    calls = str(r.choice(["two", "one", "groups"])) if layers > 1 else str(r.choice(["two", "one"]))
    groups = None
    if calls == "groups":
        cut = sorted(r.choice(np.arange(1, layers), size=int(r.integers(1, layers)), replace=False).tolist())
        groups = [b - a for a, b in zip([0] + cut, cut + [layers])]
    static = bool(r.random() < 0.5)  # reassign through the entry point that allocates nothing
    return w, staging, chunk, calls, groups, static


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_config(i):
    w, staging, chunk, calls, groups, static = _draw(i)
    print("[random %d] %s staging %d chunk %d calls %s %s static %s" % (i, w, staging, chunk, calls, groups, static),
          flush=True)
    outs, s, tiers, st, o, n_reassign = run_parity(w, Inputs(w), w.steps, check_every=3, staging_layers=staging,
                                                   chunk=chunk, calls=calls, groups=groups, static=static)
    assert n_reassign == w.steps // w.delta
    assert st["reassigns"] == n_reassign


def _draw_long(i):
    """A long cache on few layers and heads: up to 9000 prefilled positions,
    more than 16 chunks of 128 or 256 rows, so a head's chunk list runs past the 16 pairs
    the merge pass keeps in registers and it takes its two-pass form."""
    r = np.random.default_rng(5000 + i)
    chunk = int(r.choice([128, 256]))
    dtype = "bf16" if r.random() < 0.6 else "f32"
    kv_heads = int(r.choice([1, 2]))
    group = int(r.choice([1, 2, 4, 5, 8]))
    prefill = int(r.integers(17 * chunk, 9001))  # more than 16 chunks
    delta = 16
    w = tkvsynth.CONFIGS["tiny"].replace(
        name="long%d" % i, dtype=dtype, head_dim=int(r.choice([64, 128])), kv_heads=kv_heads,
        q_heads=kv_heads * group, layers=int(r.integers(1, 3)), batch=int(r.integers(1, 3)), prefill=prefill,
        steps=delta + int(r.integers(1, delta)), delta=delta, hbm_ratio=float(np.round(r.uniform(0.1, 0.9), 2)),
        evict_ratio=float(np.round(r.uniform(0.0, 0.3), 2)), t2_ratio=float(r.choice([0.0, 0.1])),
        prompt=int(r.integers(0, 200)), sinks=4, recent=int(r.integers(16, 129)), seed=int(r.integers(0, 1 << 20)))
    return w, chunk


@pytest.mark.parametrize("i", range(8))
def test_random_long_cache(i):
    w, chunk = _draw_long(i)
    assert (w.prefill + w.steps + chunk - 1) // chunk > 16
    print("[long %d] %s chunk %d" % (i, w, chunk), flush=True)
    outs, s, tiers, st, o, n_reassign = run_parity(w, Inputs(w), w.steps, check_every=4, chunk=chunk)
    assert n_reassign == 1


@pytest.mark.parametrize("i", range(16))
def test_random_scored_prefill(i):
    """The same draws (a prompt of at least 40 positions) started with the
    scored prefill: the prompt's causal attention gives the first scores and
    one full re-placement, against the oracle's, then the decode steps."""
    from test_gpu_prefill import run_scored
    w, staging, chunk, _, _, _ = _draw(100 + i)
    if w.prefill < 40:
        w = w.replace(prefill=40 + 7 * i, prompt=min(w.prompt, 20))
    print("[scored %d] %s staging %d chunk %d" % (i, w, staging, chunk), flush=True)
    run_scored(w, w.steps, check_every=3, staging_layers=staging, chunk=chunk)


@pytest.mark.parametrize("i", range(24))
def test_random_odd_delta(i):
    """Draws with an odd Delta (5, 7, 9 or 11), so that on the paths that
    defer Eq. 1 several steps at a time (bf16, one or 4 and more query heads
    per kv head, resident staging) the reassignments find different counts of
    pending steps in turn; every other path runs them as usual (Method §4)."""
    w, staging, chunk, calls, groups, static = _draw(200 + i)
    r = np.random.default_rng(7000 + i)
    delta = int(r.choice([5, 7, 9, 11]))
    w = w.replace(delta=delta, steps=int(r.integers(3, 5)) * delta + int(r.integers(0, delta)))
    print("[odd-delta %d] %s staging %d chunk %d calls %s %s static %s" % (i, w, staging, chunk, calls, groups,
                                                                         static), flush=True)
    outs, s, tiers, st, o, n_reassign = run_parity(w, Inputs(w), w.steps, check_every=2, staging_layers=staging,
                                                   chunk=chunk, calls=calls, groups=groups, static=static)
    assert n_reassign == w.steps // w.delta


def _draw_layers(i):
    """A random workload with per-layer HBM budgets: two to four groups of
    consecutive layers, each with its own ratio (stream staging only where
    every group has more layers than staging slots)."""
    r = np.random.default_rng(9000 + i)
    dtype = "bf16" if r.random() < 0.6 else "f32"
    group = int(r.choice([1, 2, 4, 5, 8]))
    kv_heads = int(r.choice([1, 2]))
    ngroups = int(r.integers(2, 5))
    sizes = [int(x) for x in r.integers(1, 4, ngroups)]
    staging = 0
    if min(sizes) >= 3 and r.random() < 0.5:
        staging = int(r.integers(2, min(sizes)))
    layer_hbm = []
    for sz in sizes:
        layer_hbm += [float(np.round(r.uniform(0.0, 1.0), 2))] * sz
    prefill = int(r.integers(60, 400))
    delta = int(r.choice([7, 8, 16]))
    t2 = float(r.choice([0.0, 0.0, 0.1, 0.2]))
    w = tkvsynth.CONFIGS["tiny"].replace(
        name="layers%d" % i, dtype=dtype, head_dim=int(r.choice([64, 128])), kv_heads=kv_heads,
        q_heads=kv_heads * group, layers=len(layer_hbm), batch=int(r.integers(1, 4)), prefill=prefill,
        steps=int(r.integers(2, 4)) * delta + int(r.integers(0, delta)), delta=delta,
        evict_ratio=float(np.round(r.uniform(0.0, 0.4), 2)), t2_ratio=t2,
        prompt=int(r.integers(0, min(prefill, 48) + 1)), sinks=int(r.integers(0, 6)), recent=int(r.integers(0, 40)),
        seed=int(r.integers(0, 1 << 20)), t2_fp8=bool(t2 > 0 and r.random() < 0.5))
    calls = str(r.choice(["one", "two"]))
    return w, layer_hbm, staging, calls


@pytest.mark.parametrize("i", range(16))
def test_random_layer_budgets(i):
    from test_gpu_layer_budgets import run_layers
    w, layer_hbm, staging, calls = _draw_layers(i)
    st, o, n_reassign = run_layers(w, layer_hbm, staging_layers=staging, calls=calls, check_every=3)
    assert n_reassign == w.steps // w.delta


def _draw_deferral(i):
    """A bf16 workload on the matrix-core path over resident staging (one, 4, 5
    or 8 query heads per kv head), with a Delta that leaves every count of
    pending steps at some reassignment (15 formed together at g = 1, 11 at
    g = 4, 8 at g = 5, 5 at g = 8), scores read against the oracle at random
    steps between reassignments (a read folds the pending steps into a copy),
    and the calls of a step drawn as in the general draws."""
    r = np.random.default_rng(11000 + i)
    group = int(r.choice([1, 4, 5, 8]))
    kv_heads = int(r.choice([1, 2]))
    layers = int(r.integers(1, 5))
    delta = int(r.choice([6, 9, 12, 17, 20]))
    steps = int(r.integers(2, 4)) * delta + int(r.integers(0, delta))
    prefill = int(r.integers(40, 400))
    w = tkvsynth.CONFIGS["tiny"].replace(
        name="deferral%d" % i, dtype="bf16", head_dim=int(r.choice([64, 128])), kv_heads=kv_heads,
        q_heads=kv_heads * group, layers=layers, batch=int(r.integers(1, 4)), prefill=prefill, steps=steps,
        delta=delta, hbm_ratio=float(np.round(r.uniform(0.1, 0.9), 2)),
        evict_ratio=float(np.round(r.uniform(0.0, 0.4), 2)), t2_ratio=float(r.choice([0.0, 0.1])),
        prompt=int(r.integers(0, min(prefill, 48) + 1)), sinks=int(r.integers(0, 6)), recent=int(r.integers(0, 40)),
        seed=int(r.integers(0, 1 << 20)))
    calls = str(r.choice(["two", "one", "groups"])) if layers > 1 else str(r.choice(["two", "one"]))
    groups = None
    if calls == "groups":
        cut = sorted(r.choice(np.arange(1, layers), size=int(r.integers(1, layers)), replace=False).tolist())
        groups = [b - a for a, b in zip([0] + cut, cut + [layers])]
    score_at = tuple(sorted(set(int(x) for x in r.integers(1, steps + 1, 3))))
    return w, calls, groups, score_at


@pytest.mark.parametrize("i", range(24))
def test_random_deferral(i):
    w, calls, groups, score_at = _draw_deferral(i)
    print("[deferral %d] %s calls %s %s scores at %s" % (i, w, calls, groups, score_at), flush=True)
    outs, s, tiers, st, o, n_reassign = run_parity(w, Inputs(w), w.steps, check_every=2, calls=calls, groups=groups,
                                                   score_at=score_at)
    assert n_reassign == w.steps // w.delta
