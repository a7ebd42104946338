"""The reassignment that allocates nothing (tkv_reassign_static), through
the C ABI, against tkv_reassign on the same inputs.

For callers that cannot allocate (graph capture, tight serving loops): the
reassignment's scratch lives in the library's static device array.  Two
handles take the same steps; at every Delta one reassigns with
tkv_reassign, the other with tkv_reassign_static.  Tier labels, changed-row
lists, scores, the rows read back and every later output must be identical
bit for bit, on consecutive calls where the second moves fewer rows.  A
reassignment too large for the array is refused with TKV_ECAPACITY and
leaves the handle as it was.
"""
import numpy as np
import pytest
import torch

import tkvsynth
from harness import Inputs, to_device

pytestmark = pytest.mark.gpu


def _changed(c):
    _, _, counts = c.read_deltas()
    return int(counts.sum())


def _pair_run(w, staging):
    import decode_attention_tkv_amd as tkv
    inp = Inputs(w)
    a = tkv.TieredKV.for_workload(w, staging_layers=staging)
    b = tkv.TieredKV.for_workload(w, staging_layers=staging)
    for c in (a, b):
        c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))
    oa = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    ob = torch.empty_like(oa)
    stream = torch.cuda.current_stream().cuda_stream
    moved = []
    for t in range(w.steps):
        k, v = inp.step_kv(t)
        kd, vd, qd = to_device(k, w.dtype), to_device(v, w.dtype), to_device(inp.q[t], w.dtype)
        a.decode_step(kd, vd, qd, oa)
        b.decode_step(kd, vd, qd, ob)
        assert torch.equal(oa, ob), "outputs differ at step %d" % (t + 1)
        if (t + 1) % w.delta:
            continue
        a.reassign()
        rc = tkv.lib().tkv_reassign_static(b.h, stream)
        assert rc == 0, tkv.lib().tkv_last_error(b.h)
        n = w.prefill + t + 1
        assert np.array_equal(a.read_tiers()[:, :n], b.read_tiers()[:, :n])
        pa, da, ca = a.read_deltas()
        pb, db, cb = b.read_deltas()
        assert np.array_equal(ca, cb)
        for x in range(w.batch):
            assert np.array_equal(pa[x, : ca[x, 0]], pb[x, : cb[x, 0]])
            assert np.array_equal(da[x, : ca[x, 1]], db[x, : cb[x, 1]])
        assert np.array_equal(a.read_scores()[:, :n], b.read_scores()[:, :n])
        moved.append(_changed(b))
        tiers = b.read_tiers()
        for pos in range(0, n, 7):
            if tiers[0, pos] < 2 or (tiers[0, pos] == 2 and staging == 0):
                ka, va = a.read_kv(w.layers - 1, 0, pos)
                kb, vb = b.read_kv(w.layers - 1, 0, pos)
                assert np.array_equal(ka, kb) and np.array_equal(va, vb)
    a.close()
    b.close()
    return moved


@pytest.mark.parametrize("which", ["tiny_f32_resident", "gqa_bf16_t2_stream"])
def test_static_reassign_matches(which):
    if which == "tiny_f32_resident":
        w, staging = tkvsynth.CONFIGS["tiny"].replace(steps=48, t2_ratio=0.1), 0
    else:
        w = tkvsynth.CONFIGS["32b_t2"].replace(layers=4, batch=2, prefill=300, steps=64, delta=32, prompt=40,
                                               recent=32)
        staging = 2
    moved = _pair_run(w, staging)
    assert len(moved) >= 2 and moved[1] < moved[0], moved  # the second call moves fewer rows


def test_static_reassign_refuses_what_does_not_fit():
    """7B-shaped heads, 8 layers, stream staging: the first reassignment after
    the prefill moves ~1000 rows of 128 KB, more than the array holds."""
    import decode_attention_tkv_amd as tkv
    w = tkvsynth.CONFIGS["7b"].replace(layers=8, steps=64)
    inp = Inputs(w)
    c = tkv.TieredKV.for_workload(w, staging_layers=2)
    c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    for t in range(w.steps):
        k, v = inp.step_kv(t)
        c.decode_step(to_device(k, w.dtype), to_device(v, w.dtype), to_device(inp.q[t], w.dtype), out)
    n = w.prefill + w.steps
    before, s_before = c.read_tiers()[:, :n], c.read_scores()[:, :n]
    stream = torch.cuda.current_stream().cuda_stream
    rc = tkv.lib().tkv_reassign_static(c.h, stream)
    assert rc == tkv.TKV_ECAPACITY and b"static scratch" in tkv.lib().tkv_last_error(c.h)
    assert np.array_equal(c.read_tiers()[:, :n], before) and np.array_equal(c.read_scores()[:, :n], s_before)
    c.reassign()  # the allocating call still works on the unchanged handle
    assert c.stats()["reassigns"] == 1 and not np.array_equal(c.read_tiers()[:, :n], before)
    c.close()
