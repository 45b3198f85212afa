"""Python binding of libmoe_mi355x.so (the MI355X MoE expert-layer library).

Argument marshalling only: every function here takes torch tensors that live on the
GPU, checks dtypes/shapes cheaply, and calls the C-ABI entry point of the same name
(declared in include/moe.h) on the current HIP stream.  Every step of the layer runs in
the library's HIP kernels; there is no CPU or PyTorch fallback, and importing this
package fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

MOE_F32, MOE_BF16, MOE_MXFP8 = 0, 1, 2
MOE_DEVERR_EXPERT_RANGE, MOE_DEVERR_DUPLICATE = 1, 2
# expert GEMMs as bits of moe_shape.mx_scope (include/moe.h)
MOE_MX_GEMM1, MOE_MX_GEMM2, MOE_MX_DGRAD2, MOE_MX_WGRAD2, MOE_MX_DGRAD1, MOE_MX_WGRAD1 = 1, 2, 4, 8, 16, 32
MOE_MX_ALL = 63
MOE_MX_DEFAULT = MOE_MX_GEMM2 | MOE_MX_DGRAD1
MX_BITS = {"gemm1": MOE_MX_GEMM1, "gemm2": MOE_MX_GEMM2, "dgrad2": MOE_MX_DGRAD2, "wgrad2": MOE_MX_WGRAD2,
           "dgrad1": MOE_MX_DGRAD1, "wgrad1": MOE_MX_WGRAD1}


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


class moe_shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("f", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("act", ctypes.c_int32),
                ("gemm", ctypes.c_int32), ("mx_scope", ctypes.c_int32)]

    def __repr__(self):
        return (f"moe_shape(T={self.T}, d={self.d}, f={self.f}, E={self.E}, k={self.k}, "
                f"act={self.act}, gemm={self.gemm}, mx_scope={self.mx_scope})")


def make_shape(T, d, f, E, k, act=MOE_BF16, gemm=None, mx_scope=0) -> moe_shape:
    """mx_scope: MOE_MX_* bits of the expert GEMMs that run MXFP8 when gemm is MOE_MXFP8
    (0: MOE_MX_DEFAULT); must be 0 otherwise."""
    if gemm is None:
        gemm = MOE_F32 if act == MOE_F32 else MOE_BF16
    return moe_shape(T, d, f, E, k, act, gemm, mx_scope)


def mx_scope_bits(shape: moe_shape) -> int:
    """The expert GEMMs that run MXFP8 under `shape`, as MOE_MX_* bits (0 if none)."""
    if shape.gemm != MOE_MXFP8:
        return 0
    return shape.mx_scope or MOE_MX_DEFAULT


_VP = ctypes.c_void_p
_SZ = ctypes.c_size_t
_SHP = ctypes.POINTER(moe_shape)

# entry point -> argument types after the shape pointer (None = no shape argument)
_SIGS = {
    "moe_router_fwd": [_VP, _VP, _VP, _VP, _VP],
    "moe_route": [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    "moe_route_given": [_VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    "moe_route_noalloc": [_VP, _VP, _VP, _VP, _VP, _VP, _VP],
    "moe_permute": [_VP, _VP, _VP, _VP, _VP],
    "moe_grouped_ffn_fwd": [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    "moe_ffn_gemm1_fwd": [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    "moe_ffn_gemm2_fwd": [_VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    "moe_combine": [_VP, _VP, _VP, _VP, _VP, _VP],
    "moe_combine_bwd": [_VP, _VP, _VP, _VP, _VP, _VP, _VP],
    "moe_grouped_ffn_bwd": [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    "moe_ffn_dgrad2": [_VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    "moe_ffn_wgrad2": [_VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    "moe_ffn_dgrad1": [_VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    "moe_ffn_wgrad1": [_VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    "moe_route_bwd": [_VP, _VP, _VP, _VP, _VP],
    "moe_router_bwd": [_VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    "moe_permute_bwd": [_VP, _VP, _VP, _VP, _VP, _VP],
    "moe_permute_bwd_router": [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
    # MXFP8 dispatch and the GEMMs that read its quantised rows
    "moe_permute_mx": [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
    "moe_combine_bwd_mx": [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
    "moe_ffn_gemm1_fwd_mx": [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    "moe_ffn_dgrad2_mx": [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    "moe_ffn_wgrad2_mx": [_VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    "moe_ffn_wgrad1_mx": [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    # MXFP8 operands written by the producing bf16 GEMM's epilogue
    "moe_ffn_gemm1_fwd_q": [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
    "moe_ffn_gemm2_fwd_mx": [_VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    "moe_ffn_dgrad2_q": [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
    "moe_ffn_dgrad1_mx": [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
}
EXPORTED = sorted(list(_SIGS) + ["moe_mx_quantize", "moe_workspace_size", "moe_mx_cols_ld", "moe_status_str",
                                  "moe_tuning_reload"])

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built library (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m mixture_experts_layer_logits_amd.build`")
    lib = ctypes.CDLL(path)
    for name, args in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = [_SHP] + args
        fn.restype = ctypes.c_int
    lib.moe_mx_quantize.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _VP, ctypes.c_int32, _VP, _VP,
                                    _VP, _VP]
    lib.moe_mx_quantize.restype = ctypes.c_int
    lib.moe_workspace_size.argtypes = [_SHP]
    lib.moe_workspace_size.restype = ctypes.c_size_t
    lib.moe_mx_cols_ld.argtypes = [_SHP]
    lib.moe_mx_cols_ld.restype = ctypes.c_size_t
    lib.moe_status_str.argtypes = [ctypes.c_int]
    lib.moe_status_str.restype = ctypes.c_char_p
    lib.moe_tuning_reload.argtypes = []
    lib.moe_tuning_reload.restype = None
    _lib = lib
    return lib


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor arguments must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return t.data_ptr()


def _stream(stream=None):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _call(name, shape, *args, stream=None):
    lib = load_library()
    st = getattr(lib, name)(ctypes.byref(shape), *[_p(a) if not isinstance(a, ctypes.c_size_t) else a for a in args],
                            _stream(stream))
    if st != 0:
        raise MoeError(name, st, lib.moe_status_str(st).decode())


def moe_workspace_size(shape: moe_shape) -> int:
    return int(load_library().moe_workspace_size(ctypes.byref(shape)))


def moe_mx_cols_ld(shape: moe_shape) -> int:
    return int(load_library().moe_mx_cols_ld(ctypes.byref(shape)))


def moe_status_str(status: int) -> str:
    return load_library().moe_status_str(status).decode()


def _ws(ws):
    return ctypes.c_size_t(ws.numel() * ws.element_size())


# ------------------------------------------------------------------ forward
def moe_router_fwd(shape, x, Wr, bias, logits, stream=None):
    _call("moe_router_fwd", shape, x, Wr, bias, logits, stream=stream)


def moe_route(shape, logits, topk_idx, gates, counts, offsets, slot_row, ws, stream=None):
    _call("moe_route", shape, logits, topk_idx, gates, counts, offsets, slot_row, ws, _ws(ws), stream=stream)


def moe_route_noalloc(shape, logits, topk_idx, gates, counts, offsets, slot_row, stream=None):
    _call("moe_route_noalloc", shape, logits, topk_idx, gates, counts, offsets, slot_row, stream=stream)


def moe_route_given(shape, topk_idx, counts, offsets, slot_row, dev_err, ws, stream=None):
    _call("moe_route_given", shape, topk_idx, counts, offsets, slot_row, dev_err, ws, _ws(ws), stream=stream)


def moe_permute(shape, x, slot_row, row_src, x_perm, stream=None):
    _call("moe_permute", shape, x, slot_row, row_src, x_perm, stream=stream)


def moe_grouped_ffn_fwd(shape, x_perm, W1, W3, W2, offsets, ab, h, y_perm, ws, stream=None):
    _call("moe_grouped_ffn_fwd", shape, x_perm, W1, W3, W2, offsets, ab, h, y_perm, ws, _ws(ws), stream=stream)


def moe_ffn_gemm1_fwd(shape, x_perm, W1, W3, offsets, ab, h, ws, stream=None):
    _call("moe_ffn_gemm1_fwd", shape, x_perm, W1, W3, offsets, ab, h, ws, _ws(ws), stream=stream)


def moe_ffn_gemm2_fwd(shape, h, W2, offsets, y_perm, ws, stream=None):
    _call("moe_ffn_gemm2_fwd", shape, h, W2, offsets, y_perm, ws, _ws(ws), stream=stream)


def moe_combine(shape, y_perm, gates, slot_row, y_add, y, stream=None):
    _call("moe_combine", shape, y_perm, gates, slot_row, y_add, y, stream=stream)


# ------------------------------------------------------------------ backward
def moe_combine_bwd(shape, dy, y_perm, gates, slot_row, dy_perm, dgates, stream=None):
    _call("moe_combine_bwd", shape, dy, y_perm, gates, slot_row, dy_perm, dgates, stream=stream)


def moe_grouped_ffn_bwd(shape, dy_perm, x_perm, ab, h, W1, W3, W2, offsets, dab, dx_perm, dW1, dW3, dW2, ws,
                        stream=None):
    _call("moe_grouped_ffn_bwd", shape, dy_perm, x_perm, ab, h, W1, W3, W2, offsets, dab, dx_perm, dW1, dW3, dW2,
          ws, _ws(ws), stream=stream)


def moe_ffn_dgrad2(shape, dy_perm, W2, ab, offsets, dab, ws, stream=None):
    _call("moe_ffn_dgrad2", shape, dy_perm, W2, ab, offsets, dab, ws, _ws(ws), stream=stream)


def moe_ffn_wgrad2(shape, h, dy_perm, offsets, dW2, ws, stream=None):
    _call("moe_ffn_wgrad2", shape, h, dy_perm, offsets, dW2, ws, _ws(ws), stream=stream)


def moe_ffn_dgrad1(shape, dab, W1, W3, offsets, dx_perm, ws, stream=None):
    _call("moe_ffn_dgrad1", shape, dab, W1, W3, offsets, dx_perm, ws, _ws(ws), stream=stream)


def moe_ffn_wgrad1(shape, x_perm, dab, offsets, dW1, dW3, ws, stream=None):
    _call("moe_ffn_wgrad1", shape, x_perm, dab, offsets, dW1, dW3, ws, _ws(ws), stream=stream)


def moe_route_bwd(shape, dgates, gates, topk_idx, dlogits, stream=None):
    _call("moe_route_bwd", shape, dgates, gates, topk_idx, dlogits, stream=stream)


def moe_router_bwd(shape, x, Wr, dlogits, dx_r, dWr, ws, stream=None):
    _call("moe_router_bwd", shape, x, Wr, dlogits, dx_r, dWr, ws, _ws(ws), stream=stream)


def moe_permute_bwd(shape, dx_perm, slot_row, dx_r, dx_add, dx, stream=None):
    _call("moe_permute_bwd", shape, dx_perm, slot_row, dx_r, dx_add, dx, stream=stream)


def moe_permute_bwd_router(shape, dx_perm, slot_row, topk_idx, dlogits, Wr, dx_add, dx, stream=None):
    _call("moe_permute_bwd_router", shape, dx_perm, slot_row, topk_idx, dlogits, Wr, dx_add, dx, stream=stream)


def moe_tuning_reload():
    """Forget the MOE_TILE_* / MOE_GEMM_* / MOE_MX_TILE overrides read so far; each is read
    from the environment again at its next use."""
    load_library().moe_tuning_reload()


# ------------------------------------------------------------------ MXFP8
def moe_mx_quantize(rows, cols, axis, seg_offsets, nseg, src, q, scales, stream=None):
    lib = load_library()
    st = lib.moe_mx_quantize(rows, cols, axis, _p(seg_offsets), nseg, _p(src), _p(q), _p(scales), _stream(stream))
    if st != 0:
        raise MoeError("moe_mx_quantize", st, lib.moe_status_str(st).decode())


def moe_permute_mx(shape, x, slot_row, offsets, row_src, q_rows, s_rows, q_cols, s_cols, stream=None):
    _call("moe_permute_mx", shape, x, slot_row, offsets, row_src, q_rows, s_rows, q_cols, s_cols, stream=stream)


def moe_combine_bwd_mx(shape, dy, y_perm, gates, slot_row, row_src, offsets, dgates, q_rows, s_rows, q_cols, s_cols,
                       stream=None):
    _call("moe_combine_bwd_mx", shape, dy, y_perm, gates, slot_row, row_src, offsets, dgates, q_rows, s_rows, q_cols,
          s_cols, stream=stream)


def moe_ffn_gemm1_fwd_mx(shape, xq_rows, xs_rows, W1, W3, offsets, ab, h, ws, stream=None):
    _call("moe_ffn_gemm1_fwd_mx", shape, xq_rows, xs_rows, W1, W3, offsets, ab, h, ws, _ws(ws), stream=stream)


def moe_ffn_dgrad2_mx(shape, dyq_rows, dys_rows, W2, ab, offsets, dab, ws, stream=None):
    _call("moe_ffn_dgrad2_mx", shape, dyq_rows, dys_rows, W2, ab, offsets, dab, ws, _ws(ws), stream=stream)


def moe_ffn_wgrad2_mx(shape, h, dyq_cols, dys_cols, offsets, dW2, ws, stream=None):
    _call("moe_ffn_wgrad2_mx", shape, h, dyq_cols, dys_cols, offsets, dW2, ws, _ws(ws), stream=stream)


def moe_ffn_wgrad1_mx(shape, xq_cols, xs_cols, dab, offsets, dW1, dW3, ws, stream=None):
    _call("moe_ffn_wgrad1_mx", shape, xq_cols, xs_cols, dab, offsets, dW1, dW3, ws, _ws(ws), stream=stream)


def moe_ffn_gemm1_fwd_q(shape, x_perm, W1, W3, offsets, ab, h, hq_rows, hs_rows, stream=None):
    _call("moe_ffn_gemm1_fwd_q", shape, x_perm, W1, W3, offsets, ab, h, hq_rows, hs_rows, stream=stream)


def moe_ffn_gemm2_fwd_mx(shape, hq_rows, hs_rows, W2, offsets, y_perm, ws, stream=None):
    _call("moe_ffn_gemm2_fwd_mx", shape, hq_rows, hs_rows, W2, offsets, y_perm, ws, _ws(ws), stream=stream)


def moe_ffn_dgrad2_q(shape, dy_perm, W2, ab, offsets, dab, dabq_rows, dabs_rows, stream=None):
    _call("moe_ffn_dgrad2_q", shape, dy_perm, W2, ab, offsets, dab, dabq_rows, dabs_rows, stream=stream)


def moe_ffn_dgrad1_mx(shape, dabq_rows, dabs_rows, W1, W3, offsets, dx_perm, ws, stream=None):
    _call("moe_ffn_dgrad1_mx", shape, dabq_rows, dabs_rows, W1, W3, offsets, dx_perm, ws, _ws(ws), stream=stream)


from .layer import MoEExpertLayer  # noqa: E402  (re-export)
