"""Seeded synthetic workloads for the MoE expert layer.

This module only draws random inputs; it holds none of the layer's arithmetic
(no routing, no gating, no GEMM).  Both the CPU oracle (under ``oracle/``) and
the GPU path consume exactly the tensors it returns, so the two sides see the
same bits.

Shapes mirror the pages' workloads: top-4 routing, an expert pool grown from 8
to 128 at fixed active compute, random routing for the large rows, and uniform
expert load for the MXFP8 comparison (bigchange.ai, "Olmo-core 3 открывает стек
обучения MoE от Ai2…", section "Три числа, три знаменателя"; unite.ai,
"Ai2 κυκλοφορεί το Olmo-Core 3…", section "Δοκιμές τρισεκατομμυρίων
παραμέτρων").  The pages' training data is not available; synthetic Gaussian
tensors of the same shapes stand in for it.

Layout conventions (all row-major, weights stored [out, in] per expert):
  x   [T, d]        activations
  Wr  [E, d]        router weight (logits = x @ Wr^T + router_bias)
  W1  [E, f, d]     gate projection of each expert
  W3  [E, f, d]     up projection of each expert
  W2  [E, d, f]     down projection of each expert
  dy  [T, d]        upstream gradient of the layer output
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

# Zipf bias scale for the load-imbalance workload: chosen so that the hottest
# expert receives about 10x the mean number of routed rows.  The value was
# produced by oracle/calibrate_zipf.py (which routes with the CPU oracle); it
# is stored here so that input generation itself never routes anything.
ZIPF_S = 1.1

# beta calibrated per (seed, T, d, E, k); see oracle/calibrate_zipf.py.  With one scale for
# the whole rank profile the two halves of the load-imbalance description do not meet:
# hottest/mean = 10 leaves every expert some rows, and the first beta on a 0.05 grid that
# empties an expert (0.8) makes the hottest 27x the mean.  Both are workloads.
_ZIPF_BETA_TABLE = {
    (1004, 16384, 2048, 128, 4): 0.3241,   # hottest/mean = 9.996, no empty expert
}
ZIPF_BETA_STEEP = 0.8                      # hottest/mean = 26.8, three empty experts (seed 1004)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    T: int
    d: int
    f: int
    E: int
    k: int
    dtype: str            # "f32" or "bf16": activations, weights and outputs
    gemm: str             # "f32", "bf16" or "mxfp8": grouped expert GEMM arithmetic
    routing: str          # "learned", "learned_zipf" or "given_uniform"
    note: str = ""
    shared_f: int = 0     # width of an always-on shared expert (0: none)
    zipf_beta: Optional[float] = None      # learned_zipf: bias scale (None: the calibrated table)
    mx_scope: Optional[tuple] = None       # mxfp8: names of the expert GEMMs run in MXFP8 (None: the default)

    @property
    def R(self) -> int:
        return self.T * self.k

    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32", 1001, 256, 128, 256, 8, 2, "f32", "f32", "learned",
                 "fp32 end to end; oracle finishes in well under a second"),
        Workload("e8_k4_t8192", 1002, 8192, 2048, 1024, 8, 4, "bf16", "bf16", "learned",
                 "batch 2 x seq 4096; about 4096 rows per expert"),
        Workload("e128_k4_t8192", 1003, 8192, 2048, 1024, 128, 4, "bf16", "bf16", "learned",
                 "expert pool grown 8 -> 128 at fixed active compute; uneven learned-style load"),
        Workload("e128_k4_t8192_shared", 1003, 8192, 2048, 1024, 128, 4, "bf16", "bf16", "learned",
                 "the E=128 k=4 layer plus one always-on shared expert of width f (production rows' layout)",
                 shared_f=1024),
        Workload("e128_k4_t16384_zipf", 1004, 16384, 2048, 1024, 128, 4, "bf16", "bf16", "learned_zipf",
                 "router logits get a Zipf(1.1) per-expert bias: hottest expert 10x the mean, none empty"),
        Workload("e128_k4_t16384_zipf_steep", 1004, 16384, 2048, 1024, 128, 4, "bf16", "bf16", "learned_zipf",
                 "the Zipf(1.1) bias at beta 0.8: three experts receive no rows, the hottest 27x the mean",
                 zipf_beta=ZIPF_BETA_STEEP),
        Workload("e128_k4_t16384_random", 1005, 16384, 2048, 1024, 128, 4, "bf16", "bf16", "given_uniform",
                 "top-4 sampled uniformly without replacement, gates Dirichlet(1)"),
        Workload("e32_k4_t16384_d4096_mxfp8", 1006, 16384, 4096, 1536, 32, 4, "bf16", "mxfp8", "given_uniform",
                 "one GPU's resident share: 32 local experts, tokens arrive routed; GEMM2 and dgrad1 in MXFP8"),
        Workload("e32_k4_t16384_d4096_mxfp8_all", 1006, 16384, 4096, 1536, 32, 4, "bf16", "mxfp8", "given_uniform",
                 "the same inputs with all six expert GEMMs in MXFP8 and the MXFP8 dispatch (outside the 6e-2 "
                 "error bound; for the throughput comparison)",
                 mx_scope=("gemm1", "gemm2", "dgrad2", "wgrad2", "dgrad1", "wgrad1")),
        Workload("e32_k4_t16384_d4096_bf16", 1006, 16384, 4096, 1536, 32, 4, "bf16", "bf16", "given_uniform",
                 "same inputs as the MXFP8 run, bf16 GEMMs, for the throughput/error comparison"),
    ]
}


def scaled(w: Workload, T: Optional[int] = None, d: Optional[int] = None, f: Optional[int] = None,
           E: Optional[int] = None, k: Optional[int] = None, seed: Optional[int] = None,
           name: Optional[str] = None, shared_f: Optional[int] = None, mx_scope: Optional[tuple] = None) -> Workload:
    """A smaller copy of a workload (same routing mode and dtype) for oracle-sized tests."""
    return dataclasses.replace(
        w, T=T if T is not None else w.T, d=d or w.d, f=f or w.f, E=E or w.E, k=k or w.k,
        seed=w.seed if seed is None else seed, name=name or (w.name + "_scaled"),
        shared_f=w.shared_f if shared_f is None else shared_f,
        mx_scope=w.mx_scope if mx_scope is None else tuple(mx_scope))


def _round(t: torch.Tensor, dtype) -> torch.Tensor:
    # fp32 draw rounded to nearest-even in the target dtype (torch's cast is RNE)
    return t.to(dtype).contiguous()


def zipf_bias(w: Workload, gen: torch.Generator, beta: float) -> torch.Tensor:
    """Per-expert additive router bias with a Zipf(s) rank profile.

    bias_e = -beta * s * ln(r_e), r_e a seeded random permutation of 1..E.
    """
    ranks = torch.randperm(w.E, generator=gen).to(torch.float64) + 1.0
    return (-beta * ZIPF_S * torch.log(ranks)).to(torch.float32)


def zipf_beta(w: Workload) -> float:
    if w.zipf_beta is not None:
        return w.zipf_beta
    key = (w.seed, w.T, w.d, w.E, w.k)
    if key in _ZIPF_BETA_TABLE:
        return _ZIPF_BETA_TABLE[key]
    return _ZIPF_BETA_TABLE[(1004, 16384, 2048, 128, 4)]


def make_inputs(w: Workload, zipf_beta_override: Optional[float] = None) -> dict:
    """Draw the workload's tensors on the CPU.

    Draw order is fixed: x, Wr, W1, W3, W2, dy, then routing-mode extras, then the
    shared expert's W1s, W3s, W2s ([1, fs, d], [1, fs, d], [1, d, fs]) when the
    workload has one.  x ~ N(0,1); weights ~ N(0, 0.02^2) (0.02 is the standard
    deviation); dy ~ N(0,1).  Values are drawn in fp32 and rounded to the workload dtype.
    """
    gen = torch.Generator("cpu").manual_seed(w.seed)
    dt = w.torch_dtype()
    out = {}
    out["x"] = _round(torch.randn(w.T, w.d, generator=gen), dt)
    out["Wr"] = _round(torch.randn(w.E, w.d, generator=gen) * 0.02, dt)
    out["W1"] = _round(torch.randn(w.E, w.f, w.d, generator=gen) * 0.02, dt)
    out["W3"] = _round(torch.randn(w.E, w.f, w.d, generator=gen) * 0.02, dt)
    out["W2"] = _round(torch.randn(w.E, w.d, w.f, generator=gen) * 0.02, dt)
    out["dy"] = _round(torch.randn(w.T, w.d, generator=gen), dt)
    out["router_bias"] = None
    out["topk_idx"] = None
    out["gates"] = None
    if w.routing == "learned_zipf":
        beta = zipf_beta(w) if zipf_beta_override is None else zipf_beta_override
        out["router_bias"] = zipf_bias(w, gen, beta)
    elif w.routing == "given_uniform":
        # k distinct experts per token, uniformly without replacement: the first
        # k entries of a uniformly random permutation of the E experts.
        keys = torch.rand(w.T, w.E, generator=gen)
        out["topk_idx"] = torch.argsort(keys, dim=1)[:, : w.k].to(torch.int32).contiguous()
        # Dirichlet(1) gates: iid Exp(1) draws normalised to sum 1.
        u = torch.rand(w.T, w.k, generator=gen, dtype=torch.float64)
        ex = -torch.log1p(-u)
        out["gates"] = (ex / ex.sum(dim=1, keepdim=True)).to(torch.float32).contiguous()
    out["shared"] = None
    if w.shared_f:
        fs = w.shared_f
        out["shared"] = (_round(torch.randn(1, fs, w.d, generator=gen) * 0.02, dt),
                         _round(torch.randn(1, fs, w.d, generator=gen) * 0.02, dt),
                         _round(torch.randn(1, w.d, fs, generator=gen) * 0.02, dt))
    return out
