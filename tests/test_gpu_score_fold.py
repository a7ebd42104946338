"""The Eq. 1 update of a step is applied in stream order before the scores
are next read or written ("Not All Thoughts Need HBM", gist.science summary,
Method §2): whether it runs inside the next append's launch or is flushed by
a score read, a score write or a reassignment, the scores are the same bits."""
import numpy as np
import pytest
import torch

import tkvsynth
from harness import Inputs, to_device

pytestmark = pytest.mark.gpu


def _run(w, inp, read_every_step, write_at=None):
    import decode_attention_tkv_amd as tkv
    c = tkv.TieredKV.for_workload(w)
    c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    written = None
    for t in range(w.steps):
        k, v = inp.step_kv(t)
        c.append(to_device(k, w.dtype), to_device(v, w.dtype))
        c.decode_attn(to_device(inp.q[t], w.dtype), out)
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


def test_fold_placement_does_not_change_scores():
    w = tkvsynth.CONFIGS["7b"].replace(layers=4, prefill=300, steps=40, delta=16, prompt=20, recent=16)
    inp = Inputs(w)
    a, ta = _run(w, inp, read_every_step=False)
    b, tb = _run(w, inp, read_every_step=True)
    n = w.n_final
    assert np.array_equal(a[:, :n], b[:, :n])
    assert np.array_equal(ta[:, :n], tb[:, :n])


def test_write_scores_replaces_pending_update():
    w = tkvsynth.CONFIGS["tiny"].replace(prefill=64, steps=20, delta=8)
    inp = Inputs(w)
    _run(w, inp, read_every_step=False, write_at=9)
