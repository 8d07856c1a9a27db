"""Host-side checks of the C-ABI library that need no GPU: it loads, exports every function the
header declares, and rejects bad arguments before any HIP call."""
import ctypes as C
import os
import re

import pytest

from int4_weight_only_align_amd import w4moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4moe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(w4moe.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return w4moe.load_library()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4moe_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert sorted(w4moe.EXPORTED_SYMBOLS) == _declared()


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert w4moe.w4moe_status_string(0) == "ok"
    assert w4moe.w4moe_status_string(3) == "weights not prepacked"
    assert w4moe.w4moe_align_block(None) == -1   # the block is a property of a handle


def _create(lib, **kw):
    cfg = dict(num_experts=384, hidden=7168, inter=2048, topk=8, group_size=32, max_tokens=1024)
    cfg.update(kw)
    h = C.c_void_p()
    rc = lib.w4moe_create(C.byref(w4moe.Config(**cfg)), C.byref(h))
    return rc, h


@pytest.mark.parametrize("kw,status", [
    (dict(num_experts=0), 1), (dict(hidden=-128), 1), (dict(max_tokens=0), 1), (dict(topk=0), 1),
    (dict(group_size=48), 2), (dict(group_size=256), 2), (dict(hidden=7208), 2), (dict(inter=2000), 2), (dict(topk=400), 2),
    (dict(hidden=7200, group_size=64), 2), (dict(inter=2080, group_size=128), 2), (dict(hidden=(1 << 30) + 32), 2),
    (dict(num_experts=2048, topk=8), 2), (dict(max_tokens=1 << 20), 2), (dict(num_bits=2), 2), (dict(num_bits=16), 2),
    (dict(act_order=2), 1), (dict(act_order=1, hidden=65664), 2),
])
def test_create_rejects_bad_config_before_touching_the_device(lib, kw, status):
    rc, h = _create(lib, **kw)
    assert rc == status and not h.value
    assert w4moe.w4moe_last_error()


@pytest.mark.parametrize("kw", [dict(hidden=160, inter=96), dict(hidden=7200, inter=2016), dict(hidden=96, inter=32),
                                dict(hidden=192, inter=320, group_size=64), dict(hidden=160, inter=96, num_bits=8),
                                dict(hidden=160, inter=96, act_order=1)])
def test_create_accepts_multiples_of_the_group(lib, kw):
    """Reduction dimensions that are multiples of the scale group (32 at K2.6), not of the 128-row
    block, pass every check: without a GPU the call gets as far as asking HIP for the device."""
    rc, h = _create(lib, **kw)
    assert rc == 5 and not h.value, (rc, w4moe.w4moe_last_error())
    assert "device" in w4moe.w4moe_last_error()


def test_null_arguments_are_rejected(lib):
    assert lib.w4moe_create(None, None) == 1
    assert lib.w4moe_forward(None, None, 1, None, None, None, None) == 1
    assert lib.w4moe_prepack(None, 0, 1, None, None, None, None, None) == 1
    assert lib.w4moe_prepack_act_order(None, 0, 1, None, None, None, None, None, None, None) == 1
    assert lib.w4moe_moe_align(None, None, 1, 16, None, None, None, None, None, None, None) == 1
    assert lib.w4moe_set_plan(None, 1) == 1
    assert lib.w4moe_set_expert_range(None, 0, 8) == 1
    assert lib.w4moe_set_profiling(None, 1) == 1
    ms = (C.c_double * 4)()
    n = C.c_int64()
    assert lib.w4moe_read_profile(None, ms, C.byref(n)) == 1
    assert lib.w4moe_read_profile_calls(None, ms, 4, C.byref(n)) == 1
    assert lib.w4moe_route(None, None, 1, None, None, None) == 1
    assert lib.w4moe_forward_logits(None, None, 1, None, None, None, None, None) == 1
    f = C.c_int32()
    assert lib.w4moe_device_error(None, C.byref(f)) == 1
    assert lib.w4moe_resolved_plan(None, 1, C.byref(f)) == 1
    p, b = C.c_void_p(), C.c_int64()
    assert lib.w4moe_packed_weights(None, 1, C.byref(p), C.byref(b)) == 1
    lib.w4moe_destroy(None)   # NULL-safe


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(w4moe, "_lib", None)
    monkeypatch.setattr(w4moe, "LIB_PATH", os.path.join(ROOT, "does_not_exist", "libw4moe.so"))
    with pytest.raises(ImportError):
        w4moe.load_library()
