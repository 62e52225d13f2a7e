"""C-ABI library checks that need no GPU: it loads, exports every function
declared in include/moe.h, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^\s*(?:moe_status|const char\s*\*|size_t)\s+(\w+)\s*\(", src, flags=re.M)


def test_header_declares_the_boundary():
    names = set(_declared())
    for n in ("moe_create", "moe_destroy", "moe_set_layer", "moe_set_expert", "moe_set_router",
              "moe_layer_forward", "moe_prefill_forward", "expert_cache_lookup",
              "expert_cache_fill", "expert_cache_resize", "expert_cache_snapshot",
              "moe_get_stats", "moe_reset_stats", "moe_last_error"):
        assert n in names, n


def test_library_exports_every_declared_symbol():
    from expert_offload_serving_amd import binding as b
    for name in _declared():
        assert hasattr(b.lib, name), f"libmoe.so does not export {name}"
        assert name in b._SIGS, f"binding has no signature for {name}"


def test_expert_bytes():
    from expert_offload_serving_amd import binding as b
    assert b.moe_expert_bytes(2048, 512) == 1671168
    assert b.moe_expert_bytes(4096, 2048) == 13369344
    assert b.moe_expert_bytes(6144, 2048) == 20054016
    assert b.moe_expert_bytes(0, 512) == 0


GOOD = dict(hidden=256, inter=512, n_experts=8, top_k=2, n_layers=1, has_shared=0,
            renormalize=1, max_tokens=4, cache_slots=8, staging_slots=8, max_prefill_tokens=0)


@pytest.mark.parametrize("field,value,status", [
    ("hidden", 0, "INVALID_ARG"), ("hidden", 200, "UNSUPPORTED"), ("inter", 96, "UNSUPPORTED"),
    ("hidden", 6272, "UNSUPPORTED"), ("inter", 8192, "UNSUPPORTED"),
    ("top_k", 0, "INVALID_ARG"), ("top_k", 17, "INVALID_ARG"), ("n_experts", 1, "INVALID_ARG"),
    ("n_experts", 1025, "INVALID_ARG"), ("max_tokens", 0, "INVALID_ARG"),
    ("max_tokens", 65, "INVALID_ARG"), ("cache_slots", 9, "INVALID_ARG"),
    ("cache_slots", -1, "INVALID_ARG"), ("staging_slots", -1, "INVALID_ARG"),
    ("has_shared", 2, "INVALID_ARG"), ("n_layers", 0, "INVALID_ARG"),
])
def test_create_rejects_bad_config(field, value, status):
    from expert_offload_serving_amd import binding as b
    cfg = dict(GOOD, **{field: value})
    with pytest.raises(b.MoEError) as ei:
        b.moe_create(**cfg)
    assert ei.value.name == status
    assert b.lib.moe_last_error().decode()


def test_null_handling():
    from expert_offload_serving_amd import binding as b
    b.moe_destroy(None)
    assert b.lib.moe_create(None, None) == -1
    assert b.lib.moe_layer_forward(None, 0, None, 1, None, None, None, None, None, None) == -1
    assert b.lib.expert_cache_resize(None, 4, None) == -1
    assert b.lib.moe_probe_copy(None, None, 16, None) == -1
    assert b.lib.moe_probe_copy(ctypes.c_void_p(16), ctypes.c_void_p(32), 15, None) == -1
