"""The C-ABI library, on the CPU: it loads, exports every call that
include/tkv.h declares, and rejects bad arguments before touching a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tkv.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tkv_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def tkv():
    import decode_attention_tkv_amd as m
    if not os.path.exists(m.LIB_PATH):
        from decode_attention_tkv_amd import _build
        _build.build()
    return m


def test_every_declared_symbol_is_exported(tkv):
    names = _declared()
    assert "tkv_create" in names and "tkv_decode_attn" in names and "tkv_reassign" in names
    lib = tkv.lib()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_every_call(tkv):
    for n in _declared():
        assert n in tkv._SIGS, n


@pytest.mark.parametrize("field,value", [("layers", 0), ("q_heads", 6), ("head_dim", 96), ("batch", 65),
                                         ("dtype", 7), ("max_tokens", 0)])
def test_create_rejects_bad_shape(tkv, field, value):
    args = dict(layers=2, q_heads=8, kv_heads=4, head_dim=64, batch=1, max_tokens=64, dtype=tkv.TKV_F32,
                delta=16, hbm_ratio=0.5, evict_ratio=0.1, prompt=4, sinks=4, recent=8)
    args[field] = value
    with pytest.raises(tkv.TkvError) as e:
        tkv.tkv_create(**args)
    assert e.value.code == tkv.TKV_EINVAL


@pytest.mark.parametrize("kw", [dict(hbm_ratio=1.5), dict(evict_ratio=-0.1), dict(delta=0),
                                dict(t2_ratio=2.0), dict(chunk=100), dict(staging_layers=1),
                                dict(prompt=-1), dict(hbm_ratio=float("nan"))])
def test_create_rejects_bad_policy(tkv, kw):
    args = dict(layers=2, q_heads=8, kv_heads=4, head_dim=64, batch=1, max_tokens=64, dtype=tkv.TKV_F32,
                delta=16, hbm_ratio=0.5, evict_ratio=0.1, prompt=4, sinks=4, recent=8)
    args.update(kw)
    with pytest.raises(tkv.TkvError) as e:
        tkv.tkv_create(**args)
    assert e.value.code == tkv.TKV_EINVAL
    assert tkv.lib().tkv_last_error(None)


@pytest.mark.parametrize("case", ["f32_g4", "bf16_g2", "bf16_g4_vector_pass"])
def test_chunk_1024_needs_the_matrix_cores(tkv, case):
    """1024-row chunks exist on the matrix-core path only (bf16, one or 4 and
    more query heads per kv head, no vector pass); elsewhere TKV_EINVAL."""
    args = dict(layers=2, q_heads=16, kv_heads=4, head_dim=64, batch=1, max_tokens=64, dtype=tkv.TKV_BF16,
                delta=16, hbm_ratio=0.5, evict_ratio=0.1, prompt=4, sinks=4, recent=8, chunk=1024)
    if case == "f32_g4":
        args["dtype"] = tkv.TKV_F32
    elif case == "bf16_g2":
        args["q_heads"] = 8
    else:
        args["flags"] = tkv.TKV_FLAG_VECTOR_PASS
    with pytest.raises(tkv.TkvError) as e:
        tkv.tkv_create(**args)
    assert e.value.code == tkv.TKV_EINVAL
    assert b"1024" in tkv.lib().tkv_last_error(None)


def test_null_handle_calls_fail_cleanly(tkv):
    lib = tkv.lib()
    assert lib.tkv_destroy(None) == tkv.TKV_OK
    assert lib.tkv_append(None, None, None, None) == tkv.TKV_EINVAL
    assert lib.tkv_decode_attn(None, 0, 1, None, None, None) == tkv.TKV_EINVAL
    assert lib.tkv_reassign(None, None) == tkv.TKV_EINVAL
    assert lib.tkv_decode_step(None, None, None, None, None, None) == tkv.TKV_EINVAL
    assert lib.tkv_prefill_scored(None, None, None, None, 1, None) == tkv.TKV_EINVAL
    assert lib.tkv_stats(None, None) == tkv.TKV_EINVAL


@pytest.mark.parametrize("layer_hbm,kw", [
    ([0.2, float("nan"), 0.5, 0.5], {}),
    ([0.2, 0.3, 1.5, 0.5], {}),
    ([0.2, 0.2, 0.5, 0.5], dict(flags=2)),       # TKV_FLAG_NO_T1
    ([0.2, 0.2, 0.5, 0.5], dict(flags=8)),       # TKV_FLAG_SHARED_HBM
    ([0.2, 0.2, 0.5, 0.5], dict(staging_layers=2)),  # stream staging: a group of 2 layers, not more than S
])
def test_create_rejects_bad_layer_budgets(tkv, layer_hbm, kw):
    """Per-layer HBM budgets: every ratio in [0, 1]; not with the eviction-only
    policy or the batch-shared budget; with stream staging every layer group
    has more layers than staging slots."""
    args = dict(layers=4, q_heads=8, kv_heads=4, head_dim=64, batch=1, max_tokens=64, dtype=tkv.TKV_F32,
                delta=16, hbm_ratio=0.5, evict_ratio=0.1, prompt=4, sinks=4, recent=8, layer_hbm=layer_hbm)
    args.update(kw)
    with pytest.raises(tkv.TkvError) as e:
        tkv.tkv_create(**args)
    assert e.value.code == tkv.TKV_EINVAL
    assert tkv.lib().tkv_last_error(None)


def test_layer_budgets_length_checked(tkv):
    with pytest.raises(ValueError):
        tkv.tkv_create(layers=4, q_heads=8, kv_heads=4, head_dim=64, batch=1, max_tokens=64, dtype=tkv.TKV_F32,
                       delta=16, hbm_ratio=0.5, evict_ratio=0.1, prompt=4, sinks=4, recent=8, layer_hbm=[0.5, 0.5])
