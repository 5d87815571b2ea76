"""Host-side checks of the C-ABI library (no GPU compute).

The library loads and exports every entry point ``include/moe.h`` declares; the
host-only calls (capacity, workspace size) and the synchronous argument checks
behave as documented.  Nothing here launches a kernel.
"""

import ctypes as C
import json
import os
import re

import pytest

from top_routing_expert_amd import binding as B, presets

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        from top_routing_expert_amd import build
        build.build()
    return B.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\s*\*)\s*(moe_\w+)\s*\(", text, re.M)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(B.ABI_FUNCTIONS)


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_capacity_matches_golden(L):
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "capacity.json")))
    for c in g["cases"]:
        p = presets.get("c1").with_(T=c["T"], E=c["E"], k=c["k"], capacity_factor=c["capacity_factor"])
        want = -1 if c["C"] is None else c["C"]
        assert B.capacity(p) == want, c


def test_status_codes_are_negative(L):
    """The header's moe_status values: 0 for success, negative codes for
    failures, each with its own text."""
    text = open(HEADER).read()
    vals = dict((n, int(v)) for n, v in re.findall(r"^\s*(MOE_(?:OK|ERR_\w+))\s*=\s*(-?\d+)", text, re.M))
    assert vals == {"MOE_OK": 0, "MOE_ERR_INVALID_ARG": -1, "MOE_ERR_UNSUPPORTED": -2,
                    "MOE_ERR_WORKSPACE": -3, "MOE_ERR_HIP": -4}
    assert (B.MOE_OK, B.MOE_ERR_INVALID_ARG, B.MOE_ERR_UNSUPPORTED, B.MOE_ERR_WORKSPACE,
            B.MOE_ERR_HIP) == (0, -1, -2, -3, -4)
    texts = [L.moe_strerror(s) for s in (0, -1, -2, -3, -4)]
    assert len(set(texts)) == 5 and b"unknown status" not in texts
    assert L.moe_strerror(99) == b"unknown status"
    assert L.moe_strerror(1) == b"unknown status"


def test_workspace_size_grows_with_tokens(L):
    for name in presets.PRESETS:
        p = presets.get(name)
        a = B.workspace_size(p, T=p.T // 2)
        b = B.workspace_size(p)
        assert 0 < a < b
        assert b % 256 == 0


def _route_status(p, **kw):
    d, o = B.dims_of(p), B.opts_of(p)
    for k, v in kw.items():
        if hasattr(d, k):
            setattr(d, k, v)
        else:
            setattr(o, k, v)
    dummy = C.c_void_p(256)
    return B.lib().moe_route(C.byref(d), C.byref(o), dummy, dummy, None, None, dummy, dummy, None,
                             None, None, None, None, dummy, 1 << 40, None)


@pytest.mark.parametrize("field,value,status", [
    ("k", 0, B.MOE_ERR_INVALID_ARG), ("k", 65, B.MOE_ERR_INVALID_ARG), ("k", 17, B.MOE_ERR_UNSUPPORTED),
    ("E", 300, B.MOE_ERR_UNSUPPORTED), ("T", -1, B.MOE_ERR_INVALID_ARG),
    ("d", 100, B.MOE_ERR_UNSUPPORTED), ("score", 7, B.MOE_ERR_INVALID_ARG),
    ("dtype", 5, B.MOE_ERR_INVALID_ARG), ("capacity_factor", float("nan"), B.MOE_ERR_INVALID_ARG),
    ("routing", 5, B.MOE_ERR_INVALID_ARG), ("routing", -1, B.MOE_ERR_INVALID_ARG),
    ("routing", 2, B.MOE_ERR_INVALID_ARG),      # noisy top-k without its inputs
    ("routing", 3, B.MOE_ERR_INVALID_ARG),      # random second expert needs k = 2
    ("routing", 4, B.MOE_ERR_INVALID_ARG),      # hash routing without token ids
    ("priority", 2, B.MOE_ERR_INVALID_ARG)])
def test_argument_errors_are_synchronous(L, field, value, status):
    p = presets.get("c4")
    assert _route_status(p, **{field: value}) == status


def test_null_and_misaligned_pointers(L):
    p = presets.get("c2")
    d, o = B.dims_of(p), B.opts_of(p)
    ok = C.c_void_p(256)
    bad = C.c_void_p(258)
    r = B.lib().moe_route
    assert r(C.byref(d), C.byref(o), None, ok, None, None, ok, ok, None, None, None, None, None, ok, 1 << 40, None) == B.MOE_ERR_INVALID_ARG
    assert r(C.byref(d), C.byref(o), bad, ok, None, None, ok, ok, None, None, None, None, None, ok, 1 << 40, None) == B.MOE_ERR_INVALID_ARG
    # workspace too small
    assert r(C.byref(d), C.byref(o), ok, ok, None, None, ok, ok, None, None, None, None, None, ok, 16, None) == B.MOE_ERR_WORKSPACE
    # workspace misaligned
    assert r(C.byref(d), C.byref(o), ok, ok, None, None, ok, ok, None, None, None, None, None, C.c_void_p(272), 1 << 40, None) == B.MOE_ERR_INVALID_ARG


def test_zero_tokens_is_a_noop(L):
    p = presets.get("c2")
    d, o = B.dims_of(p, T=0), B.opts_of(p)
    ok = C.c_void_p(256)
    assert B.lib().moe_route(C.byref(d), C.byref(o), ok, ok, None, None, ok, ok, None, None, None,
                             None, None, ok, 1 << 40, None) == B.MOE_OK
    assert B.lib().moe_combine(C.byref(d), ok, ok, ok, None, ok, None) == B.MOE_OK


def test_balance_entry_points_reject_bad_arguments(L):
    ok = C.c_void_p(256)
    h = B.lib().moe_score_histogram
    assert h(ok, 10, 4, 0.0, 1.0, 16, None, None) == B.MOE_ERR_INVALID_ARG     # no output
    assert h(ok, 10, 4, 1.0, 1.0, 16, ok, None) == B.MOE_ERR_INVALID_ARG       # lo == hi
    assert h(ok, 10, 4, 0.0, float("nan"), 16, ok, None) == B.MOE_ERR_INVALID_ARG
    assert h(ok, 10, 300, 0.0, 1.0, 16, ok, None) == B.MOE_ERR_UNSUPPORTED      # E > 256
    assert h(ok, 10, 4, 0.0, 1.0, 0, ok, None) == B.MOE_ERR_INVALID_ARG        # no bins
    s = B.lib().moe_bias_from_histogram
    assert s(ok, 4, 16, 0.0, 1.0, float("nan"), ok, None) == B.MOE_ERR_INVALID_ARG
    assert s(ok, 4, 16, 0.0, 1.0, -1.0, ok, None) == B.MOE_ERR_INVALID_ARG
    assert s(None, 4, 16, 0.0, 1.0, 3.0, ok, None) == B.MOE_ERR_INVALID_ARG
    r = B.lib().moe_router_report
    assert r(4, 8, ok, None, ok, None, ok, ok, None) == B.MOE_ERR_INVALID_ARG  # out_perm w/o offsets
    assert r(4, 8, None, None, None, None, None, ok, None) == B.MOE_ERR_INVALID_ARG
    assert r(300, 8, ok, None, None, None, None, ok, None) == B.MOE_ERR_UNSUPPORTED


def test_mx_entry_points_reject_bad_arguments(L):
    p = presets.get("c4")
    o = B.opts_of(p)
    ok, bad = C.c_void_p(256), C.c_void_p(264)
    qw = B.lib().moe_mx_quantize_weights
    assert qw(C.byref(o), ok, 2, 256, 96, ok, ok, None) == B.MOE_ERR_INVALID_ARG     # K % 64
    assert qw(C.byref(o), bad, 2, 256, 512, ok, ok, None) == B.MOE_ERR_INVALID_ARG   # misaligned w
    assert qw(C.byref(o), ok, 2, 256, 512, bad, ok, None) == B.MOE_ERR_INVALID_ARG   # misaligned codes
    qa = B.lib().moe_mx_quantize_act
    assert qa(C.byref(o), ok, 10, 512, 8, ok, ok, None) == B.MOE_ERR_INVALID_ARG     # stride < rows
    assert qa(C.byref(o), bad, 10, 512, 16, ok, ok, None) == B.MOE_ERR_INVALID_ARG   # misaligned x
    assert qa(C.byref(o), ok, 0, 512, 0, None, None, None) == B.MOE_OK              # no rows
    d = B.dims_of(p)
    f = B.lib().moe_expert_ffn_mx
    args = lambda xs_stride, a_stride, F: (C.byref(d), C.byref(o), p.E, 1000, F, ok, ok, xs_stride, ok,
                                           ok, ok, ok, ok, ok, ok, a_stride, ok, None)
    assert f(*args(1000, 1004, p.F)) == B.MOE_ERR_INVALID_ARG    # x_stride < max_rows + 4
    assert f(*args(1006, 1008, p.F)) == B.MOE_ERR_INVALID_ARG    # x_stride % 4
    assert f(*args(1004, 1004, 320)) == B.MOE_ERR_UNSUPPORTED    # F % 256


def test_noalloc_permute_limit(L):
    """moe_permute_noalloc refuses, before touching any pointer or the device,
    problems whose dispatch table exceeds its 1 MiB scratch: with 256 experts
    that is above 1024 blocks of 1024 slots (T*k > 1048576)."""
    dummy = C.c_void_p(256)

    def call(T, x):
        p = presets.get("c5", T=T)                      # E = 256, k = 8
        return L.moe_permute_noalloc(C.byref(B.dims_of(p)), C.byref(B.opts_of(p)), x, dummy,
                                     dummy, dummy, dummy, dummy, dummy, None)

    assert call(131072, None) == B.MOE_ERR_INVALID_ARG   # T*k = 1048576 fits: a null x is refused
    assert call(131073, dummy) == B.MOE_ERR_UNSUPPORTED  # one block of slots too many
    assert call(1 << 20, dummy) == B.MOE_ERR_UNSUPPORTED


def test_router_draws_argument_errors(L):
    """moe_router_draws validates before any device call: negative T or no
    experts are refused, T*E above 2^40 is unsupported, and a call with no
    output buffer (or no tokens) launches nothing and succeeds."""
    dummy = C.c_void_p(256)

    def call(T, E, noise, uniform):
        d = B.Dims(T, 0, E, 0, 0, 0)
        return L.moe_router_draws(C.byref(d), C.c_uint64(1), C.c_uint64(2), noise, uniform, None)

    assert call(-1, 8, dummy, dummy) == B.MOE_ERR_INVALID_ARG
    assert call(16, 0, dummy, dummy) == B.MOE_ERR_INVALID_ARG
    assert call(1 << 33, 256, dummy, None) == B.MOE_ERR_UNSUPPORTED
    assert call(16, 8, None, None) == B.MOE_OK
    assert call(0, 8, dummy, dummy) == B.MOE_OK
    assert L.moe_router_draws(None, C.c_uint64(1), C.c_uint64(2), dummy, dummy, None) == \
        B.MOE_ERR_INVALID_ARG
