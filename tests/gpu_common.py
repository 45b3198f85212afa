"""Helpers shared by the GPU parity tests: run the HIP path through the C-ABI binding
and compare with the CPU oracle under the tolerances of the method.

Tolerances (normwise: max|got - ref| / max|ref|, per tensor):
  bf16 path   2e-2   (values and gradients against the fp64 oracle)
  fp32 path   1e-4
  MXFP8 path  6e-2   (against the fp64 oracle of the MXFP8 method: operands quantised
                     along each GEMM's reduction axis, dequantised, multiplied in fp64)
Integers (expert ids, counts, offsets, packed rows, row sources, E4M3/E8M0 bytes) must
match bit for bit.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

TOL = {"bf16": 2e-2, "f32": 1e-4, "mxfp8": 6e-2}


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


def run_layer(w, inp: dict, layer=None, mx_dispatch=None):
    """Forward + backward of the whole layer on the GPU; returns the layer object
    (mx_dispatch: None = the layer's default, on for MXFP8 GEMMs)."""
    import mixture_experts_layer_logits_amd as m
    act = m.MOE_F32 if w.dtype == "f32" else m.MOE_BF16
    gemm = {"f32": m.MOE_F32, "bf16": m.MOE_BF16, "mxfp8": m.MOE_MXFP8}[w.gemm]
    if layer is None:
        layer = m.MoEExpertLayer(w.T, w.d, w.f, w.E, w.k, act=act, gemm=gemm, shared_f=w.shared_f,
                                 mx_dispatch=mx_dispatch)
    d = to_dev(inp)
    sh = d.get("shared")
    if w.routing == "given_uniform":
        layer.forward(d["x"], d["W1"], d["W3"], d["W2"], topk_idx=d["topk_idx"], gates=d["gates"], shared=sh)
    else:
        layer.forward(d["x"], d["W1"], d["W3"], d["W2"], Wr=d["Wr"], bias=d["router_bias"], shared=sh)
    layer.backward(d["dy"])
    torch.cuda.synchronize()
    return layer


def oracle_for(w, inp: dict, gpu_logits=None):
    """Oracle forward+backward on the same inputs; learned routing selects on the GPU's
    fp32 scores (the selection is an integer decision taken in fp32 on both sides)."""
    from oracle import moe_ref as ref
    learned = w.routing != "given_uniform"
    if w.gemm == "mxfp8":
        # the MXFP8 method: every expert GEMM operand block-quantised along its reduction
        # axis, dequantised exactly, multiplied in fp64 (tokens arrive routed)
        from oracle import mx_ref
        assert not learned, "the MXFP8 workloads take pre-routed tokens"
        out = mx_ref.mx_layer(inp["x"], inp["W1"], inp["W3"], inp["W2"], w.k, inp["topk_idx"].numpy(), inp["gates"],
                              inp["dy"], shared=inp.get("shared"))
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
