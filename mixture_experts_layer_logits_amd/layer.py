"""The MoE expert layer as a sequence of C-ABI calls.

``MoEExpertLayer`` owns the device buffers of one layer shape (allocated once with
torch, which is used only for device memory and the stream) and runs the forward and
backward passes as the library's calls, in order, on the current stream:

  forward   moe_router_fwd -> moe_route        (learned routing)
            or moe_route_given                 (tokens arrive routed)
            -> moe_permute -> moe_grouped_ffn_fwd -> moe_combine
  backward  moe_combine_bwd -> the expert GEMMs' dgrad2, wgrad2, dgrad1
            -> moe_route_bwd -> moe_router_bwd (learned routing; dWr only)
            -> moe_permute_bwd_router (learned routing) or moe_permute_bwd
            -> wgrad1 (last, after the un-permute has read dx_perm)

Router input gradient (``router_dx_fused``, on by default): the gates are a softmax over
each token's k chosen scores, so dlogits is zero outside them and dx_r = dlogits Wr is k
rows of Wr per token.  moe_permute_bwd_router adds those rows while it gathers the token's
routed rows of dx_perm, so no dense dlogits Wr GEMM runs and no dx_r is written or read
(bigchange.ai, section "Что инженер может попробовать на практике", for the learned
router).  ``router_dx_fused=False`` keeps the dense GEMM into ``dx_r`` and the plain
un-permute.

Nothing is copied back to the host between calls; routing counts and offsets stay on
the GPU (unite.ai, "Ai2 κυκλοφορεί το Olmo-Core 3…", section "Παραλληλισμός, Ακρίβεια
και Τεχνικές Μνήμης").  ``MoEExpertFunction`` wraps the same calls as a
torch.autograd.Function.

Shared expert (``shared_f > 0``): one always-on SwiGLU expert of width ``shared_f`` sees
every token (bigchange.ai, "Olmo-core 3 открывает стек обучения MoE…", section "Что
инженер может попробовать на практике": the production rows use top-four routing and
one shared expert).  It runs as a one-group call of the same grouped GEMMs over the T
token rows (E = 1, k = 1, offsets [0, T]); its output enters through moe_combine's
``y_add`` and its input gradient through moe_permute_bwd's ``dx_add``.

MXFP8 scope (``mx_scope``, MOE_MX_* bits; MOE_MX_DEFAULT = GEMM2 and dgrad1): the expert
GEMMs that take E4M3 operands when ``gemm`` is MOE_MXFP8; the others run bf16.

MXFP8 operands from the producing epilogue (``mx_fused_quant``, on by default where it
applies): when GEMM2 runs MXFP8 and GEMM1 bf16 (the default scope), GEMM1's epilogue also
writes h as MXFP8 row blocks and GEMM2 reads those; likewise dgrad2's epilogue writes
[da | db] for an MXFP8 dgrad1.  The bytes are the ones the GEMM would quantise itself, so the
results are bit-identical and two standalone quantiser passes over h and [da | db] go away.

MXFP8 dispatch (``mx_dispatch``; on by default when the scope holds all four GEMMs that
read the dispatched rows: GEMM1 and wgrad1 read x's, dgrad2 and wgrad2 the output
gradient's): moe_permute_mx and moe_combine_bwd_mx write the routed rows of x and of the
output gradient only as E4M3 codes with their block scales, in the row layout (forward /
data-gradient GEMMs) and the per-expert column layout (weight-gradient GEMMs), so no bf16
x_perm or dy_perm exists and the GEMMs quantise neither (MXFP8 for the data moved to the
experts: unite.ai, section "Παραλληλισμός, Ακρίβεια και Τεχνικές Μνήμης").  The results
are bit-identical with the bf16 dispatch.

Activation recompute (``recompute=True``): the forward keeps only ``x_perm`` of the
expert FFN; ``ab = [a | b]`` and ``h`` live in buffers allocated for the forward's GEMM1 /
GEMM2 and released right after, and the backward runs GEMM1 again (same kernel, same
inputs, so bit-identical ``ab`` and ``h``) before the gradient GEMMs.  This trades one
extra GEMM1 per step for R * 3f activation elements held between the passes, the
memory / throughput trade the pages report for recomputing activations (unite.ai,
section "Παραλληλισμός, Ακρίβεια και Τεχνικές Μνήμης").
"""
from __future__ import annotations

import torch

from . import (MOE_BF16, MOE_F32, MOE_MX_DGRAD1, MOE_MX_DGRAD2, MOE_MX_GEMM1, MOE_MX_GEMM2, MOE_MX_WGRAD1,
               MOE_MX_WGRAD2, MOE_MXFP8, make_shape, moe_combine, moe_ffn_dgrad1_mx, moe_ffn_dgrad2_q,
               moe_ffn_gemm1_fwd_q, moe_ffn_gemm2_fwd_mx, moe_combine_bwd, moe_combine_bwd_mx,
               moe_ffn_dgrad1, moe_ffn_dgrad2, moe_ffn_dgrad2_mx, moe_ffn_gemm1_fwd, moe_ffn_gemm1_fwd_mx,
               moe_ffn_gemm2_fwd, moe_ffn_wgrad1, moe_ffn_wgrad1_mx, moe_ffn_wgrad2, moe_ffn_wgrad2_mx, moe_mx_cols_ld,
               moe_permute, moe_permute_bwd, moe_permute_bwd_router, moe_permute_mx, moe_route, moe_route_bwd,
               moe_route_given, moe_router_bwd,
               moe_router_fwd, moe_workspace_size, mx_scope_bits)

# the GEMMs that read the dispatched rows: all four must run MXFP8 for the MXFP8 dispatch
_DISPATCH_READERS = MOE_MX_GEMM1 | MOE_MX_WGRAD1 | MOE_MX_DGRAD2 | MOE_MX_WGRAD2


class MoEExpertLayer:
    def __init__(self, T, d, f, E, k, act=MOE_BF16, gemm=None, device="cuda", recompute=False, shared_f=0,
                 mx_dispatch=None, mx_scope=0, mx_fused_quant=True, router_dx_fused=True):
        self.shape = make_shape(T, d, f, E, k, act, gemm, mx_scope)
        self.recompute = recompute
        # the router's input gradient folded into the un-permute (k rows of Wr per token)
        # instead of a dense dlogits Wr GEMM written to dx_r and read back
        self.router_dx_fused = bool(router_dx_fused)
        bits = mx_scope_bits(self.shape)
        # MXFP8 operands written by the producing bf16 GEMM's epilogue
        self.fq_h = bool(mx_fused_quant) and bool(bits & MOE_MX_GEMM2) and not bits & MOE_MX_GEMM1
        self.fq_dab = bool(mx_fused_quant) and bool(bits & MOE_MX_DGRAD1) and not bits & MOE_MX_DGRAD2
        covers = (bits & _DISPATCH_READERS) == _DISPATCH_READERS
        self.mx_dispatch = covers if mx_dispatch is None else bool(mx_dispatch)
        if self.mx_dispatch and not covers:
            raise ValueError("the MXFP8 dispatch needs GEMM1, wgrad1, dgrad2 and wgrad2 in the MXFP8 scope")
        self.steps = 0   # forwards run so far: the autograd wrapper checks its backward sees its own
        self.shared_f = shared_f
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
        self._e = e
        u8 = torch.uint8
        if self.mx_dispatch:  # routed rows exist only as E4M3 codes, in the row and column layouts
            L = moe_mx_cols_ld(self.shape)
            self.x_perm = self.dy_perm = None
            self.xq_rows, self.xs_rows = e(R, d, dtype=u8), e(R, d // 32, dtype=u8)
            self.xq_cols, self.xs_cols = e(d, L, dtype=u8), e(d, L // 32, dtype=u8)
            self.dyq_rows, self.dys_rows = e(R, d, dtype=u8), e(R, d // 32, dtype=u8)
            self.dyq_cols, self.dys_cols = e(d, L, dtype=u8), e(d, L // 32, dtype=u8)
        else:
            self.x_perm = e(R, d)
            self.dy_perm = e(R, d)
        self.ab = None if recompute else e(R, 2 * f)
        self.h = None if recompute else e(R, f)
        self.hq_rows = self.hs_rows = self.dabq_rows = self.dabs_rows = None
        if self.fq_h:
            self.hq_rows, self.hs_rows = e(R, f, dtype=u8), e(R, f // 32, dtype=u8)
        if self.fq_dab:
            self.dabq_rows, self.dabs_rows = e(R, 2 * f, dtype=u8), e(R, 2 * f // 32, dtype=u8)
        self.y_perm = e(R, d)
        self.y = e(T, d)
        # backward buffers
        self.dgates = e(T, k, dtype=f32)
        self.dab = e(R, 2 * f)
        self.dx_perm = e(R, d)
        self.dW1 = e(E, f, d)
        self.dW3 = e(E, f, d)
        self.dW2 = e(E, d, f)
        self.dlogits = e(T, E, dtype=f32)
        self.dx_r = None if self.router_dx_fused else e(T, d)
        self.dWr = e(E, d, dtype=f32)
        self.dx = e(T, d)
        self.ws = torch.empty(moe_workspace_size(self.shape), dtype=torch.uint8, device=dev)
        self.learned = True
        self._params = None
        self._shared = None
        if shared_f:
            fs = shared_f
            self.shape_s = make_shape(T, d, fs, 1, 1, act, gemm, mx_scope)
            self.offsets_s = torch.tensor([0, T], dtype=i32, device=dev)
            self.ab_s, self.h_s, self.y_s = e(T, 2 * fs), e(T, fs), e(T, d)
            self.dab_s, self.dx_s = e(T, 2 * fs), e(T, d)
            if self.fq_h:
                self.hq_s, self.hs_s = e(T, fs, dtype=u8), e(T, fs // 32, dtype=u8)
            if self.fq_dab:
                self.dabq_s, self.dabs_s = e(T, 2 * fs, dtype=u8), e(T, 2 * fs // 32, dtype=u8)
            self.dW1s, self.dW3s, self.dW2s = e(1, fs, d), e(1, fs, d), e(1, d, fs)
            self.ws_s = torch.empty(moe_workspace_size(self.shape_s), dtype=torch.uint8, device=dev)

    # -------------------------------------------------------------- forward
    def route(self, x=None, Wr=None, bias=None, topk_idx=None):
        s = self.shape
        if topk_idx is None:
            self.learned = True
            moe_router_fwd(s, x, Wr, bias, self.logits)
            moe_route(s, self.logits, self.topk_idx, self.gates, self.counts, self.offsets, self.slot_row, self.ws)
        else:  # the caller's ids are only read; the layer's own topk_idx buffer is left alone
            self.learned = False
            moe_route_given(s, topk_idx, self.counts, self.offsets, self.slot_row, self.dev_err, self.ws)

    def forward(self, x, W1, W3, W2, Wr=None, bias=None, topk_idx=None, gates=None, shared=None):
        """shared: (W1s [1, fs, d], W3s [1, fs, d], W2s [1, d, fs]) of the shared expert."""
        s = self.shape
        self.steps += 1
        self.route(x, Wr, bias, topk_idx)
        g = self.gates if topk_idx is None else gates
        self._params = (x, W1, W3, W2, Wr, g)
        self._shared = shared
        y_add = None
        if shared is not None:
            W1s, W3s, W2s = shared
            ss = self.shape_s
            if self.fq_h:
                moe_ffn_gemm1_fwd_q(ss, x, W1s, W3s, self.offsets_s, self.ab_s, self.h_s, self.hq_s, self.hs_s)
                moe_ffn_gemm2_fwd_mx(ss, self.hq_s, self.hs_s, W2s, self.offsets_s, self.y_s, self.ws_s)
            else:
                moe_ffn_gemm1_fwd(ss, x, W1s, W3s, self.offsets_s, self.ab_s, self.h_s, self.ws_s)
                moe_ffn_gemm2_fwd(ss, self.h_s, W2s, self.offsets_s, self.y_s, self.ws_s)
            y_add = self.y_s
        if self.mx_dispatch:
            moe_permute_mx(s, x, self.slot_row, self.offsets, self.row_src, self.xq_rows, self.xs_rows, self.xq_cols,
                           self.xs_cols)
        else:
            moe_permute(s, x, self.slot_row, self.row_src, self.x_perm)
        if self.recompute:
            self.ab, self.h = self._e(self.R, 2 * self.f), self._e(self.R, self.f)
        self._gemm1(W1, W3, with_q=True)
        if self.fq_h:
            moe_ffn_gemm2_fwd_mx(s, self.hq_rows, self.hs_rows, W2, self.offsets, self.y_perm, self.ws)
        else:
            moe_ffn_gemm2_fwd(s, self.h, W2, self.offsets, self.y_perm, self.ws)
        if self.recompute:  # the SwiGLU activations are not kept for the backward
            self.ab = self.h = None
        moe_combine(s, self.y_perm, g, self.slot_row, y_add, self.y)
        return self.y

    # -------------------------------------------------------------- backward
    def backward(self, dy):
        s = self.shape
        x, W1, W3, W2, Wr, g = self._params
        if self.mx_dispatch:
            moe_combine_bwd_mx(s, dy, self.y_perm, g, self.slot_row, self.row_src, self.offsets, self.dgates,
                               self.dyq_rows, self.dys_rows, self.dyq_cols, self.dys_cols)
        else:
            moe_combine_bwd(s, dy, self.y_perm, g, self.slot_row, self.dy_perm, self.dgates)
        if self.recompute:  # regenerate a, b and h from the kept routed rows
            self.ab, self.h = self._e(self.R, 2 * self.f), self._e(self.R, self.f)
            self._gemm1(W1, W3)
        if self.mx_dispatch:
            moe_ffn_dgrad2_mx(s, self.dyq_rows, self.dys_rows, W2, self.ab, self.offsets, self.dab, self.ws)
            moe_ffn_wgrad2_mx(s, self.h, self.dyq_cols, self.dys_cols, self.offsets, self.dW2, self.ws)
            moe_ffn_dgrad1(s, self.dab, W1, W3, self.offsets, self.dx_perm, self.ws)
        else:
            if self.fq_dab:
                moe_ffn_dgrad2_q(s, self.dy_perm, W2, self.ab, self.offsets, self.dab, self.dabq_rows,
                                 self.dabs_rows)
            else:
                moe_ffn_dgrad2(s, self.dy_perm, W2, self.ab, self.offsets, self.dab, self.ws)
            moe_ffn_wgrad2(s, self.h, self.dy_perm, self.offsets, self.dW2, self.ws)
            if self.fq_dab:
                moe_ffn_dgrad1_mx(s, self.dabq_rows, self.dabs_rows, W1, W3, self.offsets, self.dx_perm, self.ws)
            else:
                moe_ffn_dgrad1(s, self.dab, W1, W3, self.offsets, self.dx_perm, self.ws)
        dx_r = None
        if self.learned:
            moe_route_bwd(s, self.dgates, g, self.topk_idx, self.dlogits)
            moe_router_bwd(s, x, Wr, self.dlogits, self.dx_r, self.dWr, self.ws)
            dx_r = self.dx_r
        dx_add = None
        if self._shared is not None:
            W1s, W3s, W2s = self._shared
            ss, off = self.shape_s, self.offsets_s
            if self.fq_dab:
                moe_ffn_dgrad2_q(ss, dy, W2s, self.ab_s, off, self.dab_s, self.dabq_s, self.dabs_s)
            else:
                moe_ffn_dgrad2(ss, dy, W2s, self.ab_s, off, self.dab_s, self.ws_s)
            moe_ffn_wgrad2(ss, self.h_s, dy, off, self.dW2s, self.ws_s)
            if self.fq_dab:
                moe_ffn_dgrad1_mx(ss, self.dabq_s, self.dabs_s, W1s, W3s, off, self.dx_s, self.ws_s)
            else:
                moe_ffn_dgrad1(ss, self.dab_s, W1s, W3s, off, self.dx_s, self.ws_s)
            moe_ffn_wgrad1(ss, x, self.dab_s, off, self.dW1s, self.dW3s, self.ws_s)
            dx_add = self.dx_s
        if self.learned and self.router_dx_fused:
            moe_permute_bwd_router(s, self.dx_perm, self.slot_row, self.topk_idx, self.dlogits, Wr, dx_add, self.dx)
        else:
            moe_permute_bwd(s, self.dx_perm, self.slot_row, dx_r, dx_add, self.dx)
        # wgrad1 goes last: its gradient writes, the largest output of the step, would
        # otherwise push dx_perm out of the memory-side cache before the un-permute reads it
        if self.mx_dispatch:
            moe_ffn_wgrad1_mx(s, self.xq_cols, self.xs_cols, self.dab, self.offsets, self.dW1, self.dW3, self.ws)
        else:
            moe_ffn_wgrad1(s, self.x_perm, self.dab, self.offsets, self.dW1, self.dW3, self.ws)
        if self.recompute:
            self.ab = self.h = None
        return self.dx

    def _gemm1(self, W1, W3, with_q=False):
        """GEMM1 (with_q: also h's MXFP8 rows, for the forward's MXFP8 GEMM2)."""
        s = self.shape
        if with_q and self.fq_h:
            moe_ffn_gemm1_fwd_q(s, self.x_perm, W1, W3, self.offsets, self.ab, self.h, self.hq_rows, self.hs_rows)
        elif self.mx_dispatch:
            moe_ffn_gemm1_fwd_mx(s, self.xq_rows, self.xs_rows, W1, W3, self.offsets, self.ab, self.h, self.ws)
        else:
            moe_ffn_gemm1_fwd(s, self.x_perm, W1, W3, self.offsets, self.ab, self.h, self.ws)

    def activation_bytes(self):
        """Bytes of expert-FFN activations held from the forward to the backward: the
        routed rows (x_perm, or with the MXFP8 dispatch their two E4M3 layouts with
        scales), y_perm, and ab and h unless they are recomputed."""
        eb = self.y_perm.element_size()
        n = self.R * self.d * eb
        if self.mx_dispatch:
            n += sum(t.numel() for t in (self.xq_rows, self.xs_rows, self.xq_cols, self.xs_cols))
        else:
            n += self.R * self.d * eb
        if not self.recompute:
            n += self.R * 3 * self.f * eb
        return n


class MoEExpertFunction(torch.autograd.Function):
    """y = MoE(x) with learned routing (optional constant per-expert router bias);
    gradients for x, Wr, W1, W3, W2.  The layer's buffers hold one forward at a time, so
    each backward must follow its own forward: a second forward through the same layer
    before the first one's backward makes that backward raise instead of returning the
    second forward's gradients."""

    @staticmethod
    def forward(ctx, x, Wr, W1, W3, W2, layer: MoEExpertLayer, bias=None):
        y = layer.forward(x.contiguous(), W1.contiguous(), W3.contiguous(), W2.contiguous(), Wr=Wr.contiguous(),
                          bias=None if bias is None else bias.contiguous())
        ctx.layer = layer
        ctx.step = layer.steps
        return y.clone()

    @staticmethod
    def backward(ctx, dy):
        L = ctx.layer
        if L.steps != ctx.step:
            raise RuntimeError("MoEExpertFunction: the layer ran another forward since this one; its saved "
                               "activations are gone (one layer object per in-flight forward)")
        L.backward(dy.contiguous())
        return L.dx.clone(), L.dWr.to(L.dtype), L.dW1.clone(), L.dW3.clone(), L.dW2.clone(), None, None
