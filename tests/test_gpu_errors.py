"""Error and state paths of the C ABI on a GPU: every failure is a status
code (no exception crosses the boundary), leaves the handle usable, and is
forced from the host, so every kernel that does run exits normally."""
import numpy as np
import pytest
import torch

import tkvsynth
from harness import Inputs, to_device

pytestmark = pytest.mark.gpu


def _tiny(**kw):
    return tkvsynth.CONFIGS["tiny"].replace(**kw)


def _cache(w, **kw):
    import decode_attention_tkv_amd as tkv
    return tkv.TieredKV.for_workload(w, **kw)


def test_state_machine():
    import decode_attention_tkv_amd as tkv
    w = _tiny(prefill=40, steps=4)
    inp = Inputs(w)
    c = _cache(w)
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    q = to_device(inp.q[0], w.dtype)
    with pytest.raises(tkv.TkvError) as e:
        c.decode_attn(q, out)                          # no step started
    assert e.value.code == tkv.TKV_ESTATE
    c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))
    with pytest.raises(tkv.TkvError) as e:
        c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))   # not empty
    assert e.value.code == tkv.TKV_ESTATE
    k, v = inp.step_kv(0)
    c.append(to_device(k, w.dtype), to_device(v, w.dtype))
    with pytest.raises(tkv.TkvError) as e:
        c.append(to_device(k, w.dtype), to_device(v, w.dtype))              # step still open
    assert e.value.code == tkv.TKV_ESTATE
    with pytest.raises(tkv.TkvError) as e:
        c.reassign()                                                         # mid-step
    assert e.value.code == tkv.TKV_ESTATE
    with pytest.raises(tkv.TkvError) as e:
        c.decode_attn(q[1:].contiguous(), out[1:], layer_begin=1, layer_count=1)  # out of order
    assert e.value.code == tkv.TKV_ESTATE
    c.decode_attn(q[:1].contiguous(), out[:1], layer_begin=0, layer_count=1)
    with pytest.raises(tkv.TkvError) as e:
        c.reassign()                                                         # between layer groups
    assert e.value.code == tkv.TKV_ESTATE
    c.decode_attn(q[1:].contiguous(), out[1:], layer_begin=1, layer_count=1)
    c.reassign()                                                             # step done: fine
    assert c.stats()["step"] == 1
    c.close()


def test_max_tokens_reached():
    import decode_attention_tkv_amd as tkv
    w = _tiny(prefill=30, steps=3, hbm_ratio=1.0, evict_ratio=0.0)
    inp = Inputs(w)
    c = _cache(w)
    c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    for t in range(3):
        k, v = inp.step_kv(t)
        c.append(to_device(k, w.dtype), to_device(v, w.dtype))
        c.decode_attn(to_device(inp.q[t], w.dtype), out)
    with pytest.raises(tkv.TkvError) as e:
        c.append(to_device(k, w.dtype), to_device(v, w.dtype))
    assert e.value.code == tkv.TKV_ECAPACITY
    assert c.stats()["n_tokens"] == w.n_final
    c.close()


def test_t0_pool_full_until_reassigned():
    """Stream staging: without reassignment the T0 pool fills up (appended
    rows are T0); a reassignment frees it and the run goes on."""
    import decode_attention_tkv_amd as tkv
    w = _tiny(layers=3, prefill=100, steps=60, hbm_ratio=0.3, delta=4, prompt=8, recent=8)
    inp = Inputs(w)
    c = _cache(w, staging_layers=2)
    c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    full_at = None
    for t in range(w.steps):
        k, v = inp.step_kv(t)
        try:
            c.append(to_device(k, w.dtype), to_device(v, w.dtype))
        except tkv.TkvError as e:
            assert e.code == tkv.TKV_ECAPACITY
            full_at = t
            break
        c.decode_attn(to_device(inp.q[t], w.dtype), out)
    assert full_at is not None
    c.reassign()
    k, v = inp.step_kv(full_at)
    c.append(to_device(k, w.dtype), to_device(v, w.dtype))
    c.decode_attn(to_device(inp.q[full_at], w.dtype), out)
    assert np.isfinite(out.cpu().numpy()).all()
    c.close()


def test_resident_pool_holds_every_position():
    """Resident staging keeps every row at its own position, so appends never
    wait for a reassignment to free T0 slots."""
    w = _tiny(prefill=100, steps=60, hbm_ratio=0.3, delta=4, prompt=8, recent=8)
    inp = Inputs(w)
    c = _cache(w)
    c.prefill(to_device(inp.k0, w.dtype), to_device(inp.v0, w.dtype))
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    for t in range(w.steps):
        k, v = inp.step_kv(t)
        c.append(to_device(k, w.dtype), to_device(v, w.dtype))
        c.decode_attn(to_device(inp.q[t], w.dtype), out)
    assert c.stats()["n_tokens"] == w.n_final
    c.close()


def test_bad_arguments():
    import decode_attention_tkv_amd as tkv
    w = _tiny(prefill=20, steps=2)
    c = _cache(w)
    lib = tkv.lib()
    assert lib.tkv_append(c.h, None, None, None) == tkv.TKV_EINVAL
    assert lib.tkv_prefill(c.h, None, None, 5, None) == tkv.TKV_EINVAL
    k = torch.zeros((w.layers, w.batch, 5, w.kv_heads, w.head_dim), device="cuda")
    assert lib.tkv_prefill(c.h, k.data_ptr(), k.data_ptr(), 0, None) == tkv.TKV_EINVAL
    assert lib.tkv_prefill(c.h, k.data_ptr(), k.data_ptr(), w.n_final + 1, None) == tkv.TKV_ECAPACITY
    assert b"n_tokens" in lib.tkv_last_error(c.h)
    with pytest.raises(ValueError):
        c.append(torch.zeros(3, device="cuda"), torch.zeros(3, device="cuda"))   # binding shape check
    c.close()
