"""The Eq. 1 update of a step is applied in stream order before the scores
are next read or ranked ("Not All Thoughts Need HBM", gist.science summary,
Method §2): whether it runs inside the next append's launch or is applied
for a score read, the scores are the same bits.
For bf16 heads on the matrix cores over resident staging (one query head per
kv head, or four and more) a later step's attention launch recomputes the
step's weights (no logits are stored), as many steps at a time as fit the
16-row logits tile beside the running step's queries (16/g - 1), and with
four and more query heads per kv head two more tiles of 16/g steps; a score
read then forms the pending steps in a score-only pass over K into a copy of
the scores, which changes nothing later, and a reassignment folds them into
the scores first (Delta decides how many are pending there).  With per-layer
HBM budgets every group of layers defers its own part of Eq. 1 and a read
folds all of them into one copy."""
import numpy as np
import pytest
import torch

import tkvsynth
from harness import Inputs, to_device

pytestmark = pytest.mark.gpu


def _run(w, inp, read_every_step, write_at=None, groups=None, read_mid_step=False, layer_hbm=None, **kw):
    import decode_attention_tkv_amd as tkv
    c = tkv.TieredKV.for_workload(w, layer_hbm=layer_hbm, **kw)
    c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    written = None
    for t in range(w.steps):
        k, v = inp.step_kv(t)
        c.append(to_device(k, w.dtype), to_device(v, w.dtype))
        q = to_device(inp.q[t], w.dtype)
        if groups is None:
            c.decode_attn(q, out)
        else:
            lb = 0
            for g in groups:
                c.decode_attn(q[lb:lb + g].contiguous(), out[lb:lb + g], layer_begin=lb, layer_count=g)
                lb += g
                if read_mid_step and lb < w.layers:
                    c.read_scores()
        if read_every_step:
            c.read_scores()
        if write_at == t:
            written = np.random.default_rng(5).random((w.batch, w.n_final)).astype(np.float32)
            c.write_scores(written)
            got = c.read_scores()
            assert np.array_equal(got, written)      # the pending update did not land on top
        if (t + 1) % w.delta == 0:
            c.reassign()
    s = c.read_scores()
    tiers = c.read_tiers()
    c.close()
    return s, tiers


SHAPES = {
    # one query head per kv head: up to 15 pending steps per forming launch
    # (Delta 16 forms them once between reassignments, Delta 20 leaves 4)
    "7b": dict(layers=4, prefill=300, steps=40, delta=16, prompt=20, recent=16),
    "7b-delta20": dict(layers=4, prefill=300, steps=45, delta=20, prompt=20, recent=16),
    # bf16 grouped-query heads (g = 5): eight pending steps per forming launch
    # (or a score-only pass over K does, when the scores are read first)
    "14b": dict(layers=4, batch=2, prefill=300, steps=40, delta=16, prompt=20, recent=16),
    # an odd Delta: reassignments find other counts of pending steps
    "14b-delta7": dict(layers=4, batch=2, prefill=300, steps=40, delta=7, prompt=20, recent=16),
    # g = 8: five pending steps per forming launch (one in the running step's
    # tile, two in each extra tile)
    "70b": dict(layers=3, batch=2, prefill=300, steps=40, delta=16, prompt=20, recent=16),
    # per-layer HBM budgets: three groups of layers, each deferring its part
    "7b-layers": dict(layers=6, prefill=300, steps=45, delta=20, prompt=20, recent=16),
    "14b-layers": dict(layers=5, batch=2, prefill=300, steps=40, delta=7, prompt=20, recent=16),
    # the vector pass stores logits and sums each step from them
    "7b-vector": dict(layers=4, prefill=300, steps=40, delta=16, prompt=20, recent=16),
}
LAYER_HBM = {"7b-layers": [0.2, 0.2, 0.5, 0.5, 0.9, 0.9], "14b-layers": [0.3, 0.3, 0.8, 0.8, 0.8]}


@pytest.mark.parametrize("name", list(SHAPES))
def test_fold_placement_does_not_change_scores(name):
    import decode_attention_tkv_amd as tkv
    w = tkvsynth.CONFIGS[name.split("-")[0]].replace(**SHAPES[name])
    inp = Inputs(w)
    kw = dict(layer_hbm=LAYER_HBM.get(name))
    if name.endswith("vector"):
        kw["extra_flags"] = tkv.TKV_FLAG_VECTOR_PASS
    a, ta = _run(w, inp, read_every_step=False, **kw)
    b, tb = _run(w, inp, read_every_step=True, **kw)
    n = w.n_final
    assert np.array_equal(a[:, :n], b[:, :n])
    assert np.array_equal(ta[:, :n], tb[:, :n])


@pytest.mark.parametrize("name,write_at", [("tiny", 9), ("14b", 9), ("14b", 10), ("7b", 13)])
def test_write_scores_replaces_pending_update(name, write_at):
    """Written scores replace s with every pending update (the deferred steps
    on the matrix-core path); later steps add to the written values."""
    w = tkvsynth.CONFIGS[name].replace(prefill=64, steps=20, delta=8, prompt=min(tkvsynth.CONFIGS[name].prompt, 20),
                                       recent=min(tkvsynth.CONFIGS[name].recent, 16))
    if name == "14b":
        w = w.replace(layers=3, batch=2)
    inp = Inputs(w)
    _run(w, inp, read_every_step=False, write_at=write_at)


def test_scores_read_between_layer_groups():
    """Layer groups of one step with the scores read between them: the read
    applies the last step's update on its own, and the rest of the step then
    adds nothing twice."""
    w = tkvsynth.CONFIGS["14b"].replace(**SHAPES["14b"])
    inp = Inputs(w)
    a, ta = _run(w, inp, read_every_step=False)
    b, tb = _run(w, inp, read_every_step=False, groups=[1, 2, 1], read_mid_step=True)
    n = w.n_final
    assert np.array_equal(a[:, :n], b[:, :n])
    assert np.array_equal(ta[:, :n], tb[:, :n])
