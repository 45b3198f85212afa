"""C-ABI library checks that need no GPU: the library loads, exports every function
include/moe.h declares, sizes its workspace on the host, and rejects bad arguments with
the documented status codes before anything is enqueued."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
LIB = os.path.join(ROOT, "mixture_experts_layer_logits_amd", "libmoe_mi355x.so")

MOE_OK, MOE_EINVAL, MOE_ENULL, MOE_EALIGN, MOE_EWORKSPACE, MOE_EUNSUPPORTED = 0, -1, -2, -3, -4, -5


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "d", "f", "E", "k", "act", "gemm", "mx_scope")]


def header_defines():
    return {m.group(1): m.group(2) for m in re.finditer(r"#define\s+(MOE_\w+)\s+(.+?)\s*(?:/\*.*)?$",
                                                          open(HEADER).read(), flags=re.M)}


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libmoe_mi355x.so is not built (run `python -m mixture_experts_layer_logits_amd.build`)")
    return ctypes.CDLL(LIB)


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ["moe_route", "moe_route_given", "moe_permute", "moe_grouped_ffn_fwd", "moe_grouped_ffn_bwd",
                     "moe_combine", "moe_combine_bwd", "moe_router_fwd", "moe_router_bwd", "moe_route_bwd",
                     "moe_permute_bwd", "moe_mx_quantize", "moe_workspace_size"]:
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_names_match_header():
    import mixture_experts_layer_logits_amd as m
    assert sorted(m.EXPORTED) == declared_functions()
    for n in declared_functions():
        assert callable(getattr(m, n))


def test_workspace_size_is_host_only(lib):
    lib.moe_workspace_size.restype = ctypes.c_size_t
    s = Shape(8192, 2048, 1024, 128, 4, 1, 1)
    n = lib.moe_workspace_size(ctypes.byref(s))
    assert n >= (8192 // 32 * 128 + 8192 * 4) * 4
    bad = Shape(8192, 2048, 1024, 128, 200, 1, 1)
    assert lib.moe_workspace_size(ctypes.byref(bad)) == 0


def _route(lib, s, ptr=0x1000, ws_bytes=1 << 30):
    P = ctypes.c_void_p
    return lib.moe_route(ctypes.byref(s), P(ptr), P(ptr), P(ptr), P(ptr), P(ptr), P(ptr), P(ptr),
                         ctypes.c_size_t(ws_bytes), P(0))


@pytest.mark.parametrize("shape,code", [
    ((64, 128, 128, 8, 9, 1, 1), MOE_EINVAL),       # k > E
    ((64, 128, 128, 8, 0, 1, 1), MOE_EINVAL),       # k < 1
    ((64, 128, 128, 2000, 4, 1, 1), MOE_EINVAL),    # E > 1024
    ((64, 100, 128, 8, 2, 1, 1), MOE_EINVAL),       # d not a multiple of 64
    ((-1, 128, 128, 8, 2, 1, 1), MOE_EINVAL),       # negative T
    ((1 << 29, 128, 128, 8, 4, 1, 1), MOE_EINVAL),  # T*k >= 2^31
    ((64, 128, 128, 8, 2, 1, 0), MOE_EUNSUPPORTED),  # bf16 activations with fp32 GEMMs
    ((64, 128, 128, 8, 2, 0, 1), MOE_EUNSUPPORTED),  # fp32 activations with bf16 GEMMs
    ((64, 192, 128, 8, 2, 1, 2), MOE_EINVAL),       # MXFP8 needs multiples of 128
    ((64, 128, 128, 8, 2, 1, 2, 64), MOE_EINVAL),   # MXFP8 scope bit beyond the six GEMMs
    ((64, 128, 128, 8, 2, 1, 2, -1), MOE_EINVAL),   # negative scope
    ((64, 128, 128, 8, 2, 1, 1, 2), MOE_EINVAL),    # a scope on bf16 GEMMs
])
def test_bad_shapes_rejected_before_launch(lib, shape, code):
    assert _route(lib, Shape(*shape)) == code


def test_null_misaligned_and_workspace(lib):
    s = Shape(64, 128, 128, 8, 2, 1, 1)
    assert _route(lib, s, ptr=0) == MOE_ENULL
    assert _route(lib, s, ws_bytes=16) == MOE_EWORKSPACE
    P = ctypes.c_void_p
    # permute checks 16-byte alignment of the row buffers
    st = lib.moe_permute(ctypes.byref(s), P(0x1008), P(0x2000), P(0x3000), P(0x4000), P(0))
    assert st == MOE_EALIGN
    st = lib.moe_permute(ctypes.byref(s), P(0x1000), P(0), P(0x3000), P(0x4000), P(0))
    assert st == MOE_ENULL
    assert lib.moe_mx_quantize(4, 33, 0, P(0), 0, P(0x1000), P(0x1000), P(0x1000), P(0)) == MOE_EINVAL
    lib.moe_status_str.restype = ctypes.c_char_p
    assert lib.moe_status_str(MOE_EWORKSPACE) == b"workspace too small"


def test_mx_scope_constants_agree():
    """The scope bits of the header, the binding's copies and the oracle's default scope
    name the same GEMMs."""
    import mixture_experts_layer_logits_amd as m
    from oracle import mx_ref
    h = header_defines()
    names = {"gemm1": "MOE_MX_GEMM1", "gemm2": "MOE_MX_GEMM2", "dgrad2": "MOE_MX_DGRAD2",
             "wgrad2": "MOE_MX_WGRAD2", "dgrad1": "MOE_MX_DGRAD1", "wgrad1": "MOE_MX_WGRAD1"}
    for n, c in names.items():
        assert int(h[c]) == m.MX_BITS[n] == getattr(m, c)
    assert set(names) == set(mx_ref.GEMMS)
    assert {n for n, b in m.MX_BITS.items() if b & m.MOE_MX_DEFAULT} == set(mx_ref.DEFAULT_SCOPE)
    assert int(h["MOE_MX_ALL"]) == m.MOE_MX_ALL == sum(m.MX_BITS.values())


def test_mx_scope_gates_the_mx_operand_entry_points(lib):
    """An entry point that takes dispatched E4M3 rows refuses a shape whose scope leaves
    its GEMM in bf16 (before touching any pointer)."""
    P = ctypes.c_void_p
    s = Shape(64, 128, 128, 8, 2, 1, 2, 0)          # default scope: GEMM2 and dgrad1
    st = lib.moe_ffn_gemm1_fwd_mx(ctypes.byref(s), P(0x1000), P(0x1000), P(0x1000), P(0x1000), P(0x1000), P(0x1000),
                                  P(0x1000), P(0x1000), ctypes.c_size_t(1 << 30), P(0))
    assert st == MOE_EUNSUPPORTED


def test_mx_scope_gates_the_fused_quantisation_entry_points(lib):
    """The calls that write MXFP8 rows from a bf16 GEMM's epilogue need the consumer GEMM in
    the scope and the producer outside it; the calls that read them need the consumer in the
    scope.  Every refusal comes before any pointer is touched."""
    P = ctypes.c_void_p
    a = P(0x1000)
    ws = ctypes.c_size_t(1 << 30)
    calls = {
        "moe_ffn_gemm1_fwd_q": lambda s: lib.moe_ffn_gemm1_fwd_q(ctypes.byref(s), a, a, a, a, a, a, a, a, P(0)),
        "moe_ffn_gemm2_fwd_mx": lambda s: lib.moe_ffn_gemm2_fwd_mx(ctypes.byref(s), a, a, a, a, a, a, ws, P(0)),
        "moe_ffn_dgrad2_q": lambda s: lib.moe_ffn_dgrad2_q(ctypes.byref(s), a, a, a, a, a, a, a, P(0)),
        "moe_ffn_dgrad1_mx": lambda s: lib.moe_ffn_dgrad1_mx(ctypes.byref(s), a, a, a, a, a, a, a, ws, P(0)),
    }
    bf16 = Shape(64, 128, 128, 8, 2, 1, 1, 0)
    all6 = Shape(64, 128, 128, 8, 2, 1, 2, 63)      # producers in scope: nothing to fuse
    producers = Shape(64, 128, 128, 8, 2, 1, 2, 1 | 4)  # GEMM1 and dgrad2 only: no consumer in scope
    for name, call in calls.items():
        assert call(bf16) == MOE_EUNSUPPORTED, name
        assert call(producers) == MOE_EUNSUPPORTED, name
    assert calls["moe_ffn_gemm1_fwd_q"](all6) == MOE_EUNSUPPORTED
    assert calls["moe_ffn_dgrad2_q"](all6) == MOE_EUNSUPPORTED
    # the default scope passes the scope check and fails on the missing offsets (no launch)
    dflt = Shape(64, 128, 128, 8, 2, 1, 2, 0)
    assert lib.moe_ffn_gemm1_fwd_q(ctypes.byref(dflt), a, a, a, P(0), a, a, a, a, P(0)) == MOE_ENULL
    assert lib.moe_ffn_dgrad2_q(ctypes.byref(dflt), a, a, a, P(0), a, a, a, P(0)) == MOE_ENULL


def test_route_noalloc_refuses_oversized_shapes_on_the_host(lib):
    """The allocation-free routing call refuses a shape whose histograms and ranks exceed its
    fixed 4 MiB scratch, before any HIP call (so this runs without a GPU)."""
    P = ctypes.c_void_p
    s = Shape(200000, 64, 64, 128, 4, 1, 1, 0)      # 6250 * 128 + 800000 int32 > 2^20
    st = lib.moe_route_noalloc(ctypes.byref(s), P(0x1000), P(0x1000), P(0x1000), P(0x1000), P(0x1000), P(0x1000), P(0))
    assert st == -7
    lib.moe_status_str.restype = ctypes.c_char_p
    assert b"scratch" in lib.moe_status_str(-7)
