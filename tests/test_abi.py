"""The C-ABI library: loads, exports what include/moe.h declares, and rejects
bad arguments on the host before anything is enqueued (no GPU needed)."""
import ctypes
import os
import re

import pytest

from sparse_moe_transformer_llama4_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, INVALID, UNSUPPORTED, SHAPE, WORKSPACE = 0, -1, -2, -3, -4


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    lib = moe.load_library()
    names = declared_functions()
    assert {"moe_plan", "moe_route", "moe_forward", "moe_workspace_size"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(moe.symbols)
    assert moe.moe_version().startswith("moe355")


def _cfg(**kw):
    base = dict(abi_version=moe.MOE_ABI_VERSION, d=256, n_experts=4, f=512, f_shared=512, top_k=1, x_dtype=1, w_dtype=1,
                out_dtype=0, has_router_bias=0, max_tokens=64)
    base.update(kw)
    return moe._Config(**base)


def _plan(**kw):
    lib = moe.load_library()
    h = ctypes.c_void_p()
    st = lib.moe_plan(ctypes.byref(_cfg(**kw)), ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("kw,status", [
    ({}, OK),
    ({"x_dtype": 0, "w_dtype": 0, "out_dtype": 0}, OK),
    ({"out_dtype": 1}, OK),
    ({"w_dtype": 2, "out_dtype": 1}, OK),
    ({"top_k": 2}, OK),
    ({"top_k": 4}, OK),                      # every expert
    ({"top_k": 5}, UNSUPPORTED),             # more picks than experts
    ({"top_k": 0}, UNSUPPORTED),
    ({"top_k": 9, "n_experts": 16}, UNSUPPORTED),
    ({"top_k": 8, "n_experts": 16}, OK),
    ({"top_k": 8, "n_experts": 16, "max_tokens": 1 << 28}, SHAPE),     # 2^31 routing slots
    ({"top_k": 7, "n_experts": 16, "max_tokens": 1 << 28}, OK),
    ({"top_k": 2, "n_experts": 0, "f": 0}, UNSUPPORTED),
    ({"d": 96}, UNSUPPORTED),
    ({"f": 100}, UNSUPPORTED),
    ({"f_shared": 0}, UNSUPPORTED),
    ({"n_experts": 0}, UNSUPPORTED),
    ({"n_experts": 257}, UNSUPPORTED),
    ({"x_dtype": 0}, UNSUPPORTED),
    ({"w_dtype": 2, "out_dtype": 0}, UNSUPPORTED),
    ({"w_dtype": 2, "out_dtype": 1, "d": 192}, UNSUPPORTED),
    ({"abi_version": 1}, INVALID),
    ({"abi_version": 3}, INVALID),
    ({"has_router_bias": 3}, INVALID),
    ({"max_tokens": 0}, SHAPE),
    # weight-only int8: decode sizes, widths % 128, bf16 activations
    ({"w_dtype": 3}, OK),
    ({"w_dtype": 3, "out_dtype": 1}, OK),
    ({"w_dtype": 3, "max_tokens": 65}, SHAPE),
    ({"w_dtype": 3, "d": 192}, UNSUPPORTED),
    ({"w_dtype": 3, "x_dtype": 0, "out_dtype": 0}, UNSUPPORTED),
    ({"w_dtype": 3, "n_experts": 0, "f": 0}, UNSUPPORTED),
    ({"w_dtype": 4, "d": 256, "f": 512, "f_shared": 512}, OK),   # int4: widths % 256
    ({"w_dtype": 4, "d": 384}, UNSUPPORTED),
    ({"w_dtype": 4, "max_tokens": 65}, SHAPE),
    ({"w_dtype": 5}, UNSUPPORTED),
    # the RMSNorm in front of the block
    ({"has_norm": 1, "norm_eps": 1e-5}, OK),
    ({"has_norm": 1, "norm_eps": 0.0, "x_dtype": 0, "w_dtype": 0, "out_dtype": 0}, OK),
    ({"has_norm": 1, "norm_eps": 1e-5, "w_dtype": 2, "out_dtype": 1}, OK),
    ({"has_norm": 1, "norm_eps": 1e-5, "n_experts": 0, "f": 0}, OK),
    ({"has_norm": 1, "norm_eps": -1e-5}, INVALID),
    ({"has_norm": 1, "norm_eps": float("nan")}, INVALID),
    ({"has_norm": 1, "norm_eps": float("inf")}, INVALID),
    ({"has_norm": 2, "norm_eps": 1e-5}, INVALID),
    # a dense layer (no routed experts): bf16, f == 0, no bias, widths % 128
    ({"n_experts": 0, "f": 0}, OK),
    ({"n_experts": 0, "f": 0, "out_dtype": 1}, OK),
    ({"n_experts": 0, "f": 0, "w_dtype": 2, "out_dtype": 1}, UNSUPPORTED),
    ({"n_experts": 0, "f": 0, "x_dtype": 0, "w_dtype": 0, "out_dtype": 0}, UNSUPPORTED),
    ({"n_experts": 0, "f": 0, "has_router_bias": 1}, UNSUPPORTED),
    ({"n_experts": 0, "f": 0, "d": 320}, UNSUPPORTED),
    ({"n_experts": 0, "f": 0, "f_shared": 192}, UNSUPPORTED),
    ({"n_experts": 0, "f": 0, "max_tokens": 1 << 20}, OK),
    ({"n_experts": 0, "f": 0, "max_tokens": 1 << 21}, SHAPE),
])
def test_plan_validation(kw, status):
    st, h = _plan(**kw)
    assert st == status
    if st == OK:
        assert h.value
        moe.load_library().moe_plan_destroy(h)
    else:
        assert not h.value


def test_workspace_size_grows_with_tokens():
    lib = moe.load_library()
    st, h = _plan(max_tokens=1000)
    n = ctypes.c_size_t()
    sizes = []
    for T in (0, 1, 64, 1000):
        assert lib.moe_workspace_size(h, T, ctypes.byref(n)) == OK
        sizes.append(n.value)
    assert sizes == sorted(sizes) and sizes[-1] > sizes[0]
    assert lib.moe_workspace_size(h, 1001, ctypes.byref(n)) == SHAPE
    assert lib.moe_workspace_size(h, -1, ctypes.byref(n)) == SHAPE
    lib.moe_plan_destroy(h)


def _weights(p=0x10000):
    return moe._Weights(p, None, p, None, p, None, p, None, p, None, None)


def test_forward_rejects_before_enqueue():
    """Every failing check returns before any HIP call, so this runs without a GPU."""
    lib = moe.load_library()
    st, h = _plan(max_tokens=64)
    n = ctypes.c_size_t()
    lib.moe_workspace_size(h, 64, ctypes.byref(n))
    P = 0x10000
    w = _weights(P)
    fwd = lambda x, T, w_, out, ws, wsb: lib.moe_forward(h, x, T, ctypes.byref(w_) if w_ else None, out, None,
                                                         ws, wsb, None)
    assert fwd(P, 65, w, P, P, n.value) == SHAPE
    assert fwd(P, -1, w, P, P, n.value) == SHAPE
    assert fwd(P, 64, w, P, P, n.value - 1) == WORKSPACE
    assert fwd(None, 64, w, P, P, n.value) == INVALID
    assert fwd(P + 4, 64, w, P, P, n.value) == INVALID          # misaligned x
    assert fwd(P, 64, None, P, P, n.value) == INVALID
    assert fwd(P, 64, w, None, P, n.value) == INVALID            # no output
    bad = _weights(P); bad.w_down = None
    assert fwd(P, 64, bad, P, P, n.value) == INVALID
    r = moe._Routing(P, P, P, None, P)
    assert lib.moe_route(h, P, 64, ctypes.byref(w), ctypes.byref(r), P, n.value, None) == INVALID
    assert lib.moe_route(h, P, 64, ctypes.byref(w), None, P, n.value, None) == INVALID
    lib.moe_plan_destroy(h)


def test_traced_forward_rejects_before_enqueue():
    """moe_forward_traced: too few event slots, missing events or records,
    and every check of moe_forward, all before any HIP call."""
    lib = moe.load_library()
    st, h = _plan(max_tokens=64)
    n = ctypes.c_size_t()
    lib.moe_workspace_size(h, 64, ctypes.byref(n))
    P = 0x10000
    w = _weights(P)
    M = moe.MOE_MAX_LAUNCHES
    ev = (ctypes.c_void_p * (2 * M))(*([P] * (2 * M)))
    rec = (moe._LaunchRecord * M)()
    cnt = ctypes.c_int32(-1)

    def trc(T, evs, m, recs, count):
        return lib.moe_forward_traced(h, P, T, ctypes.byref(w), P, None, P, n.value, None, evs, m, recs, count)
    assert trc(64, ev, M - 1, rec, ctypes.byref(cnt)) == INVALID
    assert trc(64, None, M, rec, ctypes.byref(cnt)) == INVALID
    assert trc(64, ev, M, None, ctypes.byref(cnt)) == INVALID
    assert trc(64, ev, M, rec, None) == INVALID
    ev_null = (ctypes.c_void_p * (2 * M))(*([P] * (2 * M - 1) + [None]))
    assert trc(64, ev_null, M, rec, ctypes.byref(cnt)) == INVALID
    assert trc(65, ev, M, rec, ctypes.byref(cnt)) == SHAPE
    assert cnt.value == 0                       # nothing was launched
    lib.moe_plan_destroy(h)


def test_dense_layer_rejects_before_enqueue():
    """A dense plan (n_experts == 0): no routing entry point, no routing record,
    the shared weights required, the router and routed weights not."""
    lib = moe.load_library()
    st, h = _plan(n_experts=0, f=0, max_tokens=64)
    assert st == OK
    n = ctypes.c_size_t()
    assert lib.moe_workspace_size(h, 64, ctypes.byref(n)) == OK
    P = 0x10000
    w = moe._Weights(None, None, None, None, None, None, P, None, P, None)   # shared weights only
    r = moe._Routing(P, P, P, P, P)
    assert lib.moe_route(h, P, 64, ctypes.byref(w), ctypes.byref(r), P, n.value, None) == UNSUPPORTED
    assert lib.moe_forward(h, P, 64, ctypes.byref(w), P, ctypes.byref(r), P, n.value, None) == INVALID
    bad = moe._Weights(None, None, None, None, None, None, P, None, None, None)
    assert lib.moe_forward(h, P, 64, ctypes.byref(bad), P, None, P, n.value, None) == INVALID
    assert lib.moe_forward(h, P, 65, ctypes.byref(w), P, None, P, n.value, None) == SHAPE
    lib.moe_plan_destroy(h)


@pytest.mark.parametrize("wdt,odt", [(2, 1), (3, 0), (4, 0)])
def test_scaled_weights_require_scales(wdt, odt):
    lib = moe.load_library()
    st, h = _plan(w_dtype=wdt, out_dtype=odt, max_tokens=8)
    assert st == OK
    n = ctypes.c_size_t()
    lib.moe_workspace_size(h, 8, ctypes.byref(n))
    P = 0x10000
    w = _weights(P)
    assert lib.moe_forward(h, P, 8, ctypes.byref(w), P, None, P, n.value, None) == INVALID
    lib.moe_plan_destroy(h)


def test_fp8_requires_scales_and_bias_when_declared():
    lib = moe.load_library()
    st, h = _plan(w_dtype=2, out_dtype=1, max_tokens=8)
    n = ctypes.c_size_t()
    lib.moe_workspace_size(h, 8, ctypes.byref(n))
    P = 0x10000
    w = _weights(P)
    assert lib.moe_forward(h, P, 8, ctypes.byref(w), P, None, P, n.value, None) == INVALID
    lib.moe_plan_destroy(h)
    st, h = _plan(has_router_bias=1, max_tokens=8)
    lib.moe_workspace_size(h, 8, ctypes.byref(n))
    assert lib.moe_forward(h, P, 8, ctypes.byref(w), P, None, P, n.value, None) == INVALID
    lib.moe_plan_destroy(h)


def test_status_strings():
    for s in (OK, INVALID, UNSUPPORTED, SHAPE, WORKSPACE, -5, moe.MOE_ERR_CHECK):
        assert moe.moe_status_string(s) != "unknown status"


def test_release_build_has_no_debug_checks():
    """moe_debug_flags answers -1 in a release build without touching a GPU."""
    assert moe.moe_debug_flags() == -1
    assert moe.moe_debug_flags(clear=True) == -1
    assert "debug" not in moe.moe_version()


@pytest.mark.skipif(not os.path.exists(moe.DEBUG_LIB_PATH), reason="debug library not built (build.py --debug)")
def test_debug_library_exports_the_same_entry_points():
    """The -DMOE_DEBUG build is the same ABI: every declared symbol, the same
    host-side argument checks (made before any enqueue, so no GPU is needed)."""
    with moe.using_library(moe.DEBUG_LIB_PATH) as lib:
        for n in declared_functions():
            assert hasattr(lib, n), n
        assert moe.moe_version().endswith("debug")
        st, h = _plan(top_k=5)
        assert st == UNSUPPORTED
        st, h = _plan()
        assert st == OK
        n = ctypes.c_size_t()
        assert lib.moe_workspace_size(h, 64, ctypes.byref(n)) == OK
        P = 0x10000
        w = _weights(P)
        fwd = lambda x, T, w_, out, ws, wsb: lib.moe_forward(h, x, T, ctypes.byref(w_) if w_ else None, out, None,
                                                             ws, wsb, None)
        assert fwd(P, 65, w, P, P, n.value) == SHAPE
        assert fwd(P, 64, w, P, P, n.value - 1) == WORKSPACE
        assert fwd(P + 4, 64, w, P, P, n.value) == INVALID
        assert fwd(P, 64, None, P, P, n.value) == INVALID
        lib.moe_plan_destroy(h)
    assert "debug" not in moe.moe_version()


def test_norm_requires_its_weight():
    """A plan with the RMSNorm needs norm_weight (16-byte aligned) in every
    entry point that reads x, and room for the normalised rows."""
    lib = moe.load_library()
    n0, n1 = ctypes.c_size_t(), ctypes.c_size_t()
    st, h0 = _plan(max_tokens=64)
    st1, h = _plan(max_tokens=64, has_norm=1, norm_eps=1e-5)
    assert st == OK and st1 == OK
    lib.moe_workspace_size(h0, 64, ctypes.byref(n0))
    lib.moe_workspace_size(h, 64, ctypes.byref(n1))
    assert n1.value >= n0.value + 64 * 256 * 2        # + T x d bf16 rows
    P = 0x10000
    r = moe._Routing(P, P, P, P, P)
    for nw, want in ((None, INVALID), (P + 2, INVALID)):
        w = _weights(P)
        w.norm_weight = nw
        assert lib.moe_forward(h, P, 64, ctypes.byref(w), P, None, P, n1.value, None) == want
        assert lib.moe_route(h, P, 64, ctypes.byref(w), ctypes.byref(r), P, n1.value, None) == want
    w = _weights(P)
    w.norm_weight = P
    assert lib.moe_forward(h, P, 64, ctypes.byref(w), P, None, P, n0.value, None) == WORKSPACE
    lib.moe_plan_destroy(h0)
    lib.moe_plan_destroy(h)


def test_workspace_grows_with_top_k():
    lib = moe.load_library()
    sizes = []
    for k in (1, 2, 4):
        st, h = _plan(max_tokens=100, top_k=k)
        n = ctypes.c_size_t()
        assert lib.moe_workspace_size(h, 100, ctypes.byref(n)) == OK
        sizes.append(n.value)
        lib.moe_plan_destroy(h)
    assert sizes[0] < sizes[1] < sizes[2]
