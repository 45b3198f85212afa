"""The MoE expert layer as a sequence of C-ABI calls.

``MoEExpertLayer`` owns the device buffers of one layer shape (allocated once with
torch, which is used only for device memory and the stream) and runs the forward and
backward passes as the library's calls, in order, on the current stream:

  forward   moe_router_fwd -> moe_route        (learned routing)
            or moe_route_given                 (tokens arrive routed)
            -> moe_permute -> moe_grouped_ffn_fwd -> moe_combine
  backward  moe_combine_bwd -> moe_grouped_ffn_bwd
            -> moe_route_bwd -> moe_router_bwd (learned routing)
            -> moe_permute_bwd

Nothing is copied back to the host between calls; routing counts and offsets stay on
the GPU (unite.ai, "Ai2 κυκλοφορεί το Olmo-Core 3…", section "Παραλληλισμός, Ακρίβεια
και Τεχνικές Μνήμης").  ``MoEExpertFunction`` wraps the same calls as a
torch.autograd.Function.
"""
from __future__ import annotations

import torch

from . import (MOE_BF16, MOE_F32, make_shape, moe_combine, moe_combine_bwd, moe_ffn_dgrad1, moe_ffn_dgrad2,
               moe_ffn_gemm1_fwd, moe_ffn_gemm2_fwd, moe_ffn_wgrad1, moe_ffn_wgrad2, moe_permute, moe_permute_bwd,
               moe_route, moe_route_bwd, moe_route_given, moe_router_bwd, moe_router_fwd, moe_workspace_size)


class MoEExpertLayer:
    def __init__(self, T, d, f, E, k, act=MOE_BF16, gemm=None, device="cuda"):
        self.shape = make_shape(T, d, f, E, k, act, gemm)
        self.T, self.d, self.f, self.E, self.k = T, d, f, E, k
        self.R = T * k
        dt = torch.float32 if act == MOE_F32 else torch.bfloat16
        self.dtype = dt
        dev = torch.device(device)
        e = lambda *s, dtype=dt: torch.empty(*s, dtype=dtype, device=dev)  # noqa: E731
        R = self.R
        i32, f32 = torch.int32, torch.float32
        # forward buffers
        self.logits = e(T, E, dtype=f32)
        self.topk_idx = e(T, k, dtype=i32)
        self.gates = e(T, k, dtype=f32)
        self.counts = e(E, dtype=i32)
        self.offsets = e(E + 1, dtype=i32)
        self.slot_row = e(T, k, dtype=i32)
        self.row_src = e(R, dtype=i32)
        self.dev_err = torch.zeros(1, dtype=i32, device=dev)
        self.x_perm = e(R, d)
        self.ab = e(R, 2 * f)
        self.h = e(R, f)
        self.y_perm = e(R, d)
        self.y = e(T, d)
        # backward buffers
        self.dy_perm = e(R, d)
        self.dgates = e(T, k, dtype=f32)
        self.dab = e(R, 2 * f)
        self.dx_perm = e(R, d)
        self.dW1 = e(E, f, d)
        self.dW3 = e(E, f, d)
        self.dW2 = e(E, d, f)
        self.dlogits = e(T, E, dtype=f32)
        self.dx_r = e(T, d)
        self.dWr = e(E, d, dtype=f32)
        self.dx = e(T, d)
        self.ws = torch.empty(moe_workspace_size(self.shape), dtype=torch.uint8, device=dev)
        self.learned = True
        self._params = None

    # -------------------------------------------------------------- forward
    def route(self, x=None, Wr=None, bias=None, topk_idx=None):
        s = self.shape
        if topk_idx is None:
            self.learned = True
            moe_router_fwd(s, x, Wr, bias, self.logits)
            moe_route(s, self.logits, self.topk_idx, self.gates, self.counts, self.offsets, self.slot_row, self.ws)
        else:
            self.learned = False
            self.topk_idx = topk_idx
            moe_route_given(s, topk_idx, self.counts, self.offsets, self.slot_row, self.dev_err, self.ws)

    def forward(self, x, W1, W3, W2, Wr=None, bias=None, topk_idx=None, gates=None):
        s = self.shape
        self.route(x, Wr, bias, topk_idx)
        g = self.gates if topk_idx is None else gates
        self._params = (x, W1, W3, W2, Wr, g)
        moe_permute(s, x, self.slot_row, self.row_src, self.x_perm)
        moe_ffn_gemm1_fwd(s, self.x_perm, W1, W3, self.offsets, self.ab, self.h, self.ws)
        moe_ffn_gemm2_fwd(s, self.h, W2, self.offsets, self.y_perm, self.ws)
        moe_combine(s, self.y_perm, g, self.slot_row, self.y)
        return self.y

    # -------------------------------------------------------------- backward
    def backward(self, dy):
        s = self.shape
        x, W1, W3, W2, Wr, g = self._params
        moe_combine_bwd(s, dy, self.y_perm, g, self.slot_row, self.dy_perm, self.dgates)
        moe_ffn_dgrad2(s, self.dy_perm, W2, self.ab, self.offsets, self.dab, self.ws)
        moe_ffn_wgrad2(s, self.h, self.dy_perm, self.offsets, self.dW2, self.ws)
        moe_ffn_dgrad1(s, self.dab, W1, W3, self.offsets, self.dx_perm, self.ws)
        moe_ffn_wgrad1(s, self.x_perm, self.dab, self.offsets, self.dW1, self.dW3, self.ws)
        dx_r = None
        if self.learned:
            moe_route_bwd(s, self.dgates, g, self.topk_idx, self.dlogits)
            moe_router_bwd(s, x, Wr, self.dlogits, self.dx_r, self.dWr, self.ws)
            dx_r = self.dx_r
        moe_permute_bwd(s, self.dx_perm, self.slot_row, dx_r, self.dx)
        return self.dx


class MoEExpertFunction(torch.autograd.Function):
    """y = MoE(x) with learned routing; gradients for x, Wr, W1, W3, W2."""

    @staticmethod
    def forward(ctx, x, Wr, W1, W3, W2, layer: MoEExpertLayer):
        y = layer.forward(x.contiguous(), W1.contiguous(), W3.contiguous(), W2.contiguous(), Wr=Wr.contiguous())
        ctx.layer = layer
        return y.clone()

    @staticmethod
    def backward(ctx, dy):
        L = ctx.layer
        L.backward(dy.contiguous())
        return L.dx.clone(), L.dWr.to(L.dtype), L.dW1.clone(), L.dW3.clone(), L.dW2.clone(), None
