"""Helpers shared by the GPU parity tests: run the HIP path through the C-ABI binding
and compare with the CPU oracle under the tolerances of the method.

Tolerances (normwise: max|got - ref| / max|ref|, per tensor), every one against the
unquantised fp64 oracle (the plain layer):
  bf16 path   2e-2
  fp32 path   1e-4
  MXFP8 path  6e-2   (the layer with its default MXFP8 scope, GEMM2 and dgrad1)
A diagnostic for MXFP8 layers compares with the emulated oracle of the MXFP8 method
(operands quantised along each GEMM's reduction axis, dequantised, multiplied in fp64,
bf16 stores modelled) at TOL_MX_EMULATED; it is the only check of a layer whose scope
reaches beyond the default (such a layer is outside the 6e-2 bound).
Integers (expert ids, counts, offsets, packed rows, row sources, E4M3/E8M0 bytes) must
match bit for bit.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

TOL = {"bf16": 2e-2, "f32": 1e-4, "mxfp8": 6e-2}
# GPU against the emulated MXFP8 oracle.  Both take every E4M3 decision on bf16 values;
# they part only where fp32 and fp64 accumulation round a stored value to different bf16
# neighbours (about one element in 10^4-10^5).  Such a flip moves that element by a bf16 ulp
# (2^-8 relative) and, one time in 16, its E4M3 code by one step (2^-4 to 2^-3 of the
# element).  In a reduction over the model or hidden width (K >= 256 here) one term is a
# small share of the result: the outputs h, y, dgates, dx stay within about 1% (1.5e-2).  A
# weight gradient reduces over one expert's rows, about 100 at the small cases, where the
# largest term carries up to a third of the largest output; one flipped code on it moves the
# result by up to 2^-3 / 3, about 4% (5e-2).
TOL_MX_EMULATED = {"h": 1.5e-2, "y": 1.5e-2, "dgates": 1.5e-2, "dx": 1.5e-2, "wgrad": 5e-2}


def tol_mx_emulated(key: str) -> float:
    return TOL_MX_EMULATED.get(key, TOL_MX_EMULATED["wgrad"] if key.startswith("dW") else 1.5e-2)


def mx_scope_names(w) -> frozenset:
    """Names of the expert GEMMs an MXFP8 workload runs in MXFP8."""
    from oracle import mx_ref
    return frozenset(w.mx_scope) if w.mx_scope else mx_ref.DEFAULT_SCOPE


def mx_scope_bits(w) -> int:
    """moe_shape.mx_scope of a workload (0: the library's default scope)."""
    import mixture_experts_layer_logits_amd as m
    if w.gemm != "mxfp8" or not w.mx_scope:
        return 0
    return sum(m.MX_BITS[n] for n in w.mx_scope)


def normwise_err(got, ref) -> float:
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    den = np.abs(r).max()
    if den == 0:
        return float(np.abs(g).max())
    return float(np.abs(g - r).max() / den)


def host(t) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.numpy()


def to_dev(inp: dict) -> dict:
    def dev(v):
        if isinstance(v, torch.Tensor):
            return v.cuda()
        if isinstance(v, tuple):
            return tuple(dev(u) for u in v)
        return v
    return {k: dev(v) for k, v in inp.items()}


def say(msg: str):
    """Name the case before each GPU step (flushed, so a failing run still shows it)."""
    print(msg, flush=True)
    sys.stdout.flush()


def make_layer(w, mx_dispatch=None, recompute=False, mx_fused_quant=True, router_dx_fused=True):
    import mixture_experts_layer_logits_amd as m
    act = m.MOE_F32 if w.dtype == "f32" else m.MOE_BF16
    gemm = {"f32": m.MOE_F32, "bf16": m.MOE_BF16, "mxfp8": m.MOE_MXFP8}[w.gemm]
    return m.MoEExpertLayer(w.T, w.d, w.f, w.E, w.k, act=act, gemm=gemm, shared_f=w.shared_f,
                            mx_dispatch=mx_dispatch, mx_scope=mx_scope_bits(w), recompute=recompute,
                            mx_fused_quant=mx_fused_quant, router_dx_fused=router_dx_fused)


def run_layer(w, inp: dict, layer=None, mx_dispatch=None, recompute=False, mx_fused_quant=True,
              router_dx_fused=True):
    """Forward + backward of the whole layer on the GPU; returns the layer object
    (mx_dispatch: None = the layer's default, on when the MXFP8 scope covers every GEMM
    that reads the dispatched rows; mx_fused_quant: MXFP8 operands written by the
    producing bf16 GEMM's epilogue where the scope allows; router_dx_fused: the router's input
    gradient folded into the un-permute rather than a dense GEMM into dx_r)."""
    if layer is None:
        layer = make_layer(w, mx_dispatch, recompute, mx_fused_quant, router_dx_fused)
    d = to_dev(inp)
    sh = d.get("shared")
    if w.routing == "given_uniform":
        layer.forward(d["x"], d["W1"], d["W3"], d["W2"], topk_idx=d["topk_idx"], gates=d["gates"], shared=sh)
    else:
        layer.forward(d["x"], d["W1"], d["W3"], d["W2"], Wr=d["Wr"], bias=d["router_bias"], shared=sh)
    layer.backward(d["dy"])
    torch.cuda.synchronize()
    return layer


def oracle_for(w, inp: dict, gpu_logits=None, emulate_mx=False):
    """Oracle forward+backward on the same inputs; learned routing selects on the GPU's
    fp32 scores (the selection is an integer decision taken in fp32 on both sides).
    The plain fp64 layer, unless emulate_mx asks for the emulated MXFP8 method."""
    from oracle import moe_ref as ref
    learned = w.routing != "given_uniform"
    if w.gemm == "mxfp8" and emulate_mx:
        # the MXFP8 method: the operands of every GEMM in the scope block-quantised along
        # its reduction axis, dequantised exactly, multiplied in fp64 (tokens arrive routed)
        from oracle import mx_ref
        assert not learned, "the MXFP8 workloads take pre-routed tokens"
        out = mx_ref.mx_layer(inp["x"], inp["W1"], inp["W3"], inp["W2"], w.k, inp["topk_idx"].numpy(), inp["gates"],
                              inp["dy"], shared=inp.get("shared"), scope=mx_scope_names(w))
        fw = {k: out[k] for k in ("counts", "offsets", "slot_row", "x_perm", "a", "b", "h", "y_perm", "y")}
        fw["topk_idx"] = inp["topk_idx"].numpy()
        fw["row_src"] = ref.dispatch(fw["topk_idx"], w.E)[3]
        bw = {k: out[k] for k in ("dgates", "dx_perm", "dW1", "dW3", "dW2", "dx") + (
            ("dW1s", "dW3s", "dW2s") if inp.get("shared") is not None else ())}
        return fw, bw
    sh = inp.get("shared")
    if learned:
        fw = ref.layer_forward(inp["x"], inp["W1"], inp["W3"], inp["W2"], w.k, Wr=inp["Wr"],
                               bias=inp["router_bias"], select_logits=gpu_logits, shared=sh)
    else:
        fw = ref.layer_forward(inp["x"], inp["W1"], inp["W3"], inp["W2"], w.k,
                               topk_idx=inp["topk_idx"].numpy(), gates=inp["gates"], shared=sh)
    bw = ref.layer_backward(fw, inp["dy"], inp["x"], inp["W1"], inp["W3"], inp["W2"], Wr=inp["Wr"],
                            learned=learned, shared=sh)
    return fw, bw
