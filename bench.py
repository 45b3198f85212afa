"""Throughput of the MoE expert layer (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --profile-kernel NAME [--steps K] [--workload NAME]   # one call, K times
    python bench.py --copy-mib N [--steps K]                              # plain copy, K times
    python bench.py --profile-steps K [--workload NAME]                   # K eager steps, nothing else
    python bench.py --pmc-summary CSV [CSV ...]                           # counter medians per call

The last two forms run under rocprofv3 counter passes: one layer call (after one full
step to set up its inputs) or a plain device copy of N MiB (the reference against which
FETCH_SIZE / WRITE_SIZE are scaled).

A step is one pass of the whole layer over one batch of synthetic, seeded input that is
already resident in HBM: router scores, top-k routing, dispatch into per-expert buffers,
the two grouped SwiGLU GEMMs, combine, and the full backward (combine, four grouped
GEMMs, gate and router gradients, un-permute).  Every step runs through the C-ABI of
libmoe_mi355x.so on one stream.  The timed steps are replays of one step captured as a
HIP graph (--no-graph: eager launches); the per-call breakdown and the roofline come from
events around each call of eager steps.  Prints ONE JSON line on stdout.

The default workload is the expert pool of 128 with top-4 routing at 8192 tokens
(d=2048, f=1024, bf16), the layer-level counterpart of the pages' 8 -> 128 expert-pool
comparison (bigchange.ai, "Olmo-core 3 открывает стек обучения MoE от Ai2…", section
"Три числа, три знаменателя").
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s fwd+bwd at E=128,k=4 on 1 GPU; grouped-GEMM MFMA % of peak"
PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")
SQ_PASS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F8 "
           "SQ_WAIT_INST_ANY SQ_WAVE_CYCLES SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE GRBM_COUNT")
N_XCC, N_SIMD = 8, 1024          # MI355X: 8 XCDs, 256 CUs x 4 SIMDs


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="e128_k4_t8192")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="tokens in the oracle's timed sample (0: sized for about 12 s of CPU work)")
    ap.add_argument("--profile-kernel", default=None, help="run only this call of the step, --steps times")
    ap.add_argument("--copy-mib", type=int, default=0, help="run a plain device copy of this many MiB, --steps times")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="run this many eager steps of the whole layer and nothing else (for counter passes)")
    ap.add_argument("--pmc-summary", nargs="+", default=None,
                    help="rocprofv3 counter_collection.csv files: print per-call medians of each counter as JSON")
    ap.add_argument("--vendor-calibration", action="store_true",
                    help="time torch.bmm (the vendor BLAS) on uniform batched GEMMs of the workload's six expert "
                         "GEMM shapes and a dense 8192^3 GEMM: the practical MFMA ceiling of this box, for reference")
    ap.add_argument("--pmc-record", default=None, metavar="DIR",
                    help="record the counter passes under DIR (pmc_sq_W, pmc_fetch_W, pmc_write_W for --workload W, "
                         "pmc_fetch_copy, pmc_write_copy) into profiles/counters.json; prints the summary table")
    ap.add_argument("--trace-summary", default=None, metavar="DIR",
                    help="turn a rocprofv3 --kernel-trace csv run under DIR into a markdown table per kernel "
                         "(calls, mean, median, min, max, share of kernel time)")
    ap.add_argument("--recompute", action="store_true",
                    help="activation recompute: keep only x_perm and run GEMM1 again in the backward")
    ap.add_argument("--seed-offset", type=int, default=0,
                    help="draw the workload's inputs at its seed + this offset (the time spread over seeds)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the step as eager launches (default: replays of the step captured as a HIP graph)")
    ap.add_argument("--bf16-dispatch", action="store_true",
                    help="MXFP8 workloads: dispatch bf16 rows and let each GEMM quantise them (default: the "
                         "MXFP8 dispatch writes E4M3 rows)")
    ap.add_argument("--unfused-quant", action="store_true",
                    help="MXFP8 workloads: GEMM2 / dgrad1 quantise their bf16 operand themselves (default: GEMM1 / "
                         "dgrad2 write it as MXFP8 rows from their epilogues)")
    return ap.parse_args()


def kernel_sources_digest():
    """Digest of every kernel source: stored traffic counters count only for the kernels
    they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_layer_logits_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def step_calls(m, L, d_inp, learned, recompute=False):
    """The layer as (name, callable) pairs, in execution order (with recompute, GEMM1 runs
    again at the start of the backward to regenerate a, b and h from x_perm)."""
    s = L.shape
    x, W1, W3, W2 = d_inp["x"], d_inp["W1"], d_inp["W3"], d_inp["W2"]
    Wr, bias, dy = d_inp["Wr"], d_inp["router_bias"], d_inp["dy"]
    g = L.gates if learned else d_inp["gates"]
    calls = []
    if learned:
        calls += [("router_fwd", lambda: m.moe_router_fwd(s, x, Wr, bias, L.logits)),
                  ("route", lambda: m.moe_route(s, L.logits, L.topk_idx, L.gates, L.counts, L.offsets, L.slot_row,
                                                L.ws))]
    else:
        calls += [("route_given", lambda: m.moe_route_given(s, d_inp["topk_idx"], L.counts, L.offsets, L.slot_row,
                                                            L.dev_err, L.ws))]
    sh = d_inp.get("shared")
    if sh is not None:  # the shared expert: one-group GEMMs over the T token rows
        ss, so = L.shape_s, L.offsets_s
        W1s, W3s, W2s = sh
        if L.fq_h:  # h's MXFP8 rows from GEMM1's epilogue feed the MXFP8 GEMM2
            calls += [("shared_gemm1", lambda: m.moe_ffn_gemm1_fwd_q(ss, x, W1s, W3s, so, L.ab_s, L.h_s, L.hq_s,
                                                                      L.hs_s)),
                      ("shared_gemm2", lambda: m.moe_ffn_gemm2_fwd_mx(ss, L.hq_s, L.hs_s, W2s, so, L.y_s, L.ws_s))]
        else:
            calls += [("shared_gemm1", lambda: m.moe_ffn_gemm1_fwd(ss, x, W1s, W3s, so, L.ab_s, L.h_s, L.ws_s)),
                      ("shared_gemm2", lambda: m.moe_ffn_gemm2_fwd(ss, L.h_s, W2s, so, L.y_s, L.ws_s))]
    y_add = L.y_s if sh is not None else None
    if L.mx_dispatch:  # routed rows of x and dy exist only as E4M3 codes (row and column layouts)
        gemm1 = lambda: m.moe_ffn_gemm1_fwd_mx(s, L.xq_rows, L.xs_rows, W1, W3, L.offsets, L.ab, L.h, L.ws)  # noqa: E731
        calls += [
            ("permute", lambda: m.moe_permute_mx(s, x, L.slot_row, L.offsets, L.row_src, L.xq_rows, L.xs_rows,
                                                 L.xq_cols, L.xs_cols)),
            ("gemm1_fwd", gemm1),
            ("gemm2_fwd", lambda: m.moe_ffn_gemm2_fwd(s, L.h, W2, L.offsets, L.y_perm, L.ws)),
            ("combine", lambda: m.moe_combine(s, L.y_perm, g, L.slot_row, y_add, L.y)),
            ("combine_bwd", lambda: m.moe_combine_bwd_mx(s, dy, L.y_perm, g, L.slot_row, L.row_src, L.offsets,
                                                         L.dgates, L.dyq_rows, L.dys_rows, L.dyq_cols, L.dys_cols)),
        ]
        if recompute:
            calls += [("gemm1_recompute", gemm1)]
        calls += [
            ("dgrad2", lambda: m.moe_ffn_dgrad2_mx(s, L.dyq_rows, L.dys_rows, W2, L.ab, L.offsets, L.dab, L.ws)),
            ("wgrad2", lambda: m.moe_ffn_wgrad2_mx(s, L.h, L.dyq_cols, L.dys_cols, L.offsets, L.dW2, L.ws)),
            ("dgrad1", lambda: m.moe_ffn_dgrad1(s, L.dab, W1, W3, L.offsets, L.dx_perm, L.ws)),
        ]
        wgrad1 = ("wgrad1", lambda: m.moe_ffn_wgrad1_mx(s, L.xq_cols, L.xs_cols, L.dab, L.offsets, L.dW1, L.dW3,
                                                          L.ws))
    else:
        calls += [("permute", lambda: m.moe_permute(s, x, L.slot_row, L.row_src, L.x_perm))]
        if L.fq_h:
            calls += [
                ("gemm1_fwd", lambda: m.moe_ffn_gemm1_fwd_q(s, L.x_perm, W1, W3, L.offsets, L.ab, L.h, L.hq_rows,
                                                            L.hs_rows)),
                ("gemm2_fwd", lambda: m.moe_ffn_gemm2_fwd_mx(s, L.hq_rows, L.hs_rows, W2, L.offsets, L.y_perm,
                                                             L.ws))]
        else:
            calls += [
                ("gemm1_fwd", lambda: m.moe_ffn_gemm1_fwd(s, L.x_perm, W1, W3, L.offsets, L.ab, L.h, L.ws)),
                ("gemm2_fwd", lambda: m.moe_ffn_gemm2_fwd(s, L.h, W2, L.offsets, L.y_perm, L.ws))]
        calls += [
            ("combine", lambda: m.moe_combine(s, L.y_perm, g, L.slot_row, y_add, L.y)),
            ("combine_bwd", lambda: m.moe_combine_bwd(s, dy, L.y_perm, g, L.slot_row, L.dy_perm, L.dgates)),
        ]
        if recompute:
            calls += [("gemm1_recompute",
                       lambda: m.moe_ffn_gemm1_fwd(s, L.x_perm, W1, W3, L.offsets, L.ab, L.h, L.ws))]
        if L.fq_dab:  # [da | db]'s MXFP8 rows from dgrad2's epilogue feed the MXFP8 dgrad1
            calls += [
                ("dgrad2", lambda: m.moe_ffn_dgrad2_q(s, L.dy_perm, W2, L.ab, L.offsets, L.dab, L.dabq_rows,
                                                      L.dabs_rows)),
                ("wgrad2", lambda: m.moe_ffn_wgrad2(s, L.h, L.dy_perm, L.offsets, L.dW2, L.ws)),
                ("dgrad1", lambda: m.moe_ffn_dgrad1_mx(s, L.dabq_rows, L.dabs_rows, W1, W3, L.offsets, L.dx_perm,
                                                       L.ws))]
        else:
            calls += [
                ("dgrad2", lambda: m.moe_ffn_dgrad2(s, L.dy_perm, W2, L.ab, L.offsets, L.dab, L.ws)),
                ("wgrad2", lambda: m.moe_ffn_wgrad2(s, L.h, L.dy_perm, L.offsets, L.dW2, L.ws)),
                ("dgrad1", lambda: m.moe_ffn_dgrad1(s, L.dab, W1, W3, L.offsets, L.dx_perm, L.ws))]
        wgrad1 = ("wgrad1", lambda: m.moe_ffn_wgrad1(s, L.x_perm, L.dab, L.offsets, L.dW1, L.dW3, L.ws))
    if learned:
        calls += [("route_bwd", lambda: m.moe_route_bwd(s, L.dgates, g, L.topk_idx, L.dlogits)),
                  ("router_bwd", lambda: m.moe_router_bwd(s, x, Wr, L.dlogits, L.dx_r, L.dWr, L.ws))]
    if sh is not None:
        if L.fq_dab:
            calls += [("shared_dgrad2", lambda: m.moe_ffn_dgrad2_q(ss, dy, W2s, L.ab_s, so, L.dab_s, L.dabq_s,
                                                                    L.dabs_s)),
                      ("shared_wgrad2", lambda: m.moe_ffn_wgrad2(ss, L.h_s, dy, so, L.dW2s, L.ws_s)),
                      ("shared_dgrad1", lambda: m.moe_ffn_dgrad1_mx(ss, L.dabq_s, L.dabs_s, W1s, W3s, so, L.dx_s,
                                                                     L.ws_s))]
        else:
            calls += [("shared_dgrad2", lambda: m.moe_ffn_dgrad2(ss, dy, W2s, L.ab_s, so, L.dab_s, L.ws_s)),
                      ("shared_wgrad2", lambda: m.moe_ffn_wgrad2(ss, L.h_s, dy, so, L.dW2s, L.ws_s)),
                      ("shared_dgrad1", lambda: m.moe_ffn_dgrad1(ss, L.dab_s, W1s, W3s, so, L.dx_s, L.ws_s))]
        calls += [("shared_wgrad1", lambda: m.moe_ffn_wgrad1(ss, x, L.dab_s, so, L.dW1s, L.dW3s, L.ws_s))]
    dx_add = L.dx_s if sh is not None else None
    if learned and L.router_dx_fused:  # the router's dx_r folded into the un-permute
        calls += [("permute_bwd", lambda: m.moe_permute_bwd_router(s, L.dx_perm, L.slot_row, L.topk_idx, L.dlogits,
                                                                   Wr, dx_add, L.dx))]
    else:
        calls += [("permute_bwd", lambda: m.moe_permute_bwd(s, L.dx_perm, L.slot_row, L.dx_r if learned else None,
                                                            dx_add, L.dx))]
    # wgrad1 last, as in the layer's backward: its gradient writes would otherwise push
    # dx_perm out of the memory-side cache before the un-permute reads it
    calls += [wgrad1]
    return calls


def fused_quant_flags(w):
    """(fq_h, fq_dab) of a workload as the layer sets them by default: GEMM1 / dgrad2 write
    MXFP8 rows when their consumer GEMM runs MXFP8 and they do not."""
    if w.gemm != "mxfp8":
        return False, False
    sc = set(w.mx_scope) if w.mx_scope else {"gemm2", "dgrad1"}
    return ("gemm2" in sc and "gemm1" not in sc), ("dgrad1" in sc and "dgrad2" not in sc)


def algorithmic_work(w, eb, mx_dispatch=False, fq_h=False, fq_dab=False):  # noqa: C901
    """Per-launch algorithmic flops (GEMMs) and HBM bytes (everything) of each call.  With
    the MXFP8 dispatch the routed rows of x and dy are written once in each of two E4M3
    layouts (1 + 1/32 bytes per element with the scales) and read in that form.  fq_h /
    fq_dab: GEMM1 / dgrad2 also write h / [da | db] as MXFP8 rows, which GEMM2 / dgrad1 read
    in place of the bf16 copy."""
    T, d, f, E, k = w.T, w.d, w.f, w.E, w.k
    R = T * k
    gem = {"gemm1_fwd": 2.0 * R * d * 2 * f, "gemm2_fwd": 2.0 * R * f * d, "dgrad2": 2.0 * R * d * f,
           "wgrad2": 2.0 * R * d * f, "dgrad1": 2.0 * R * 2 * f * d, "wgrad1": 2.0 * R * 2 * f * d}
    wbytes = E * f * d * eb
    byt = {
        "router_fwd": T * d * eb + E * d * eb + T * E * 4,
        "route": T * E * 4 + R * 12,
        "route_given": R * 8,
        "permute": T * d * eb + R * d * eb + R * 8,
        "gemm1_fwd": R * d * eb + 2 * wbytes + R * 3 * f * eb,
        "gemm2_fwd": R * f * eb + wbytes + R * d * eb,
        "combine": R * d * eb + T * d * eb + R * 8,
        "combine_bwd": T * d * eb + 2 * R * d * eb + R * 12,
        "dgrad2": R * d * eb + wbytes + R * 2 * f * eb * 2,
        "wgrad2": R * d * eb + R * f * eb + wbytes,
        "dgrad1": R * 2 * f * eb + 2 * wbytes + R * d * eb,
        "wgrad1": R * 2 * f * eb + R * d * eb + 2 * wbytes,
        "route_bwd": R * 12 + T * E * 4,
        # dlogits in, x in, dWr out (the router's dx_r is folded into the un-permute)
        "router_bwd": T * E * 4 + T * d * eb + E * d * 4,
        # dx_perm rows in, dx out; with learned routing also the k ids and dlogits of each
        # token and Wr (read once; its rows are gathered from L2)
        "permute_bwd": R * d * eb + T * d * eb + R * 4 + (R * 8 + E * d * eb if w.routing != "given_uniform" else 0),
    }
    if fq_h:
        qh = R * f * 33 // 32
        byt["gemm1_fwd"] += qh
        byt["gemm2_fwd"] = qh + wbytes + R * d * eb
    if fq_dab:
        qd = R * 2 * f * 33 // 32
        byt["dgrad2"] += qd
        byt["dgrad1"] = qd + 2 * wbytes + R * d * eb
    if mx_dispatch:
        q = R * d * 33 // 32  # one E4M3 layout of the routed rows with its scales
        byt.update({
            "permute": T * d * eb + 2 * q + R * 8,
            "combine_bwd": T * d * eb + R * d * eb + 2 * q + R * 12 + T * k * 4,
            "gemm1_fwd": q + 2 * wbytes + R * 3 * f * eb,
            "dgrad2": q + wbytes + R * 2 * f * eb * 2,
            "wgrad2": q + R * f * eb + wbytes,
            "wgrad1": R * 2 * f * eb + q + 2 * wbytes,
        })
    return gem, byt


def cpu_baseline(w, inp, ntok=0, target_s=12.0):
    """The oracle as it stands, timed on the host cores on the first `ntok` tokens of the
    same batch (all experts' weights), forward + backward.  ntok = 0 sizes the sample for
    about target_s seconds from two short calibration runs (256 and 1024 tokens); when the
    whole batch takes less, it is run again until about target_s seconds have passed."""
    import numpy as np
    from oracle import moe_ref as ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    learned = w.routing != "given_uniform"

    def run(n):
        x, dy = inp["x"][:n], inp["dy"][:n]
        t0 = time.perf_counter()
        if learned:
            fw = ref.layer_forward(x, inp["W1"], inp["W3"], inp["W2"], w.k, Wr=inp["Wr"], bias=inp["router_bias"])
        else:
            fw = ref.layer_forward(x, inp["W1"], inp["W3"], inp["W2"], w.k, topk_idx=inp["topk_idx"][:n].numpy(),
                                   gates=inp["gates"][:n])
        ref.layer_backward(fw, dy, x, inp["W1"], inp["W3"], inp["W2"], Wr=inp["Wr"], learned=learned)
        return time.perf_counter() - t0

    if not ntok:  # per-token and fixed cost from two short runs, then a run of about target_s
        n0, n1 = min(256, w.T), min(1024, w.T)
        t0, t1 = run(n0), run(n1)
        per_tok = max((t1 - t0) / max(n1 - n0, 1), 1e-6)
        ntok = int(min(w.T, max(n1, (target_s - max(t1 - per_tok * n1, 0.0)) / per_tok)))
    dt, reps = run(ntok), 1
    while ntok == w.T and dt < target_s and reps < 8:  # the whole batch is short: repeat it
        dt += run(ntok)
        reps += 1
    what = f"first {ntok} of {w.T} tokens" if ntok < w.T else f"all {w.T} tokens" + (f", {reps} runs" if reps > 1 else "")
    return {"value": reps * ntok / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{what}, all {w.E} experts' weights, fwd+bwd in fp64 NumPy ({dt:.1f} s)"}


# kernel-name fragments -> the layer call that launches them (every bf16 GEMM call is one
# launch of the pipelined kernel with its problem type; MXFP8 GEMM calls add quantiser launches)
KERNEL_CALLS = [("ProbGemm1", "gemm1_fwd"), ("ProbGemm2", "gemm2_fwd"), ("ProbDgrad2", "dgrad2"),
                ("ProbWgrad2", "wgrad2"), ("ProbDgrad1", "dgrad1"), ("ProbWgrad1", "wgrad1"),
                ("MxGemm1", "gemm1_fwd"), ("MxDgrad2", "dgrad2"), ("ProbRouterFwd", "router_fwd"),
                ("ProbRouterDx", "router_bwd"), ("ProbRouterDw", "router_bwd"), ("route_chunk", "route"),
                ("route_scan", "route"), ("route_finalize", "route"), ("route_bwd", "route_bwd"),
                ("permute_kernel", "permute"), ("combine_kernel", "combine"), ("combine_bwd_kernel", "combine_bwd"),
                ("unpermute_sum", "permute_bwd"), ("unpermute_router", "permute_bwd"), ("mx_dispatch", "mx_dispatch"), ("dgates_kernel", "combine_bwd"),
                ("row_src_kernel", "permute"), ("copyBuffer", "copy"), ("elementwise_kernel", "copy")]


def trace_summary(d, workload):
    """Per-kernel statistics of a rocprofv3 --kernel-trace csv run under d, durations in us:
    calls, mean, median, min, max and share of the summed kernel time."""
    import csv
    import glob
    path = sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True))
    if not path:
        raise SystemExit(f"no *kernel_trace.csv under {d}")
    per = {}
    for r in csv.DictReader(open(path[0])):
        per.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total = sum(sum(v) for v in per.values())
    rows = sorted(((sum(v), name, sorted(v)) for name, v in per.items()), reverse=True)
    out = [f"# rocprofv3 kernel trace: {workload}", "",
           "Per-kernel statistics over every dispatch of the run (durations in microseconds).", "",
           "| kernel | calls | mean us | median us | min us | max us | share % |", "|---|---|---|---|---|---|---|"]
    for tot, name, v in rows:
        nm = name if len(name) <= 110 else name[:107] + "..."
        out.append(f"| `{nm}` | {len(v)} | {tot / len(v):.1f} | {v[len(v) // 2]:.1f} | {v[0]:.1f} | {v[-1]:.1f} | "
                   f"{100 * tot / total:.2f} |")
    return "\n".join(out)


def pmc_summary(paths):
    """Median over dispatches of every counter, per kernel (rocprofv3 --pmc csv output)."""
    import csv
    import statistics
    vals = {}
    for path in paths:
        with open(path) as fh:
            for row in csv.DictReader(fh):
                name = row["Kernel_Name"]
                key = (name, row["Counter_Name"])
                vals.setdefault(key, {}).setdefault(row.get("Dispatch_Id", len(vals)), 0.0)
                vals[key][row.get("Dispatch_Id")] += float(row["Counter_Value"])
    out = {}
    for (name, ctr), per in vals.items():
        call = next((c for frag, c in KERNEL_CALLS if frag in name), None)
        short = name if len(name) < 110 else name[:107] + "..."
        e = out.setdefault(short, {"call": call, "dispatches": len(per)})
        e[ctr] = statistics.median(per.values())
    return out


def _csv(d, name):
    return os.path.join(d, "pmc_" + name, "p_counter_collection.csv")


def pmc_record(wname, d):
    """Per call of the step: MFMA utilisation (rocprofv3's MfmaUtil: MFMA-busy cycles over
    GUI-active cycles of one XCD times the SIMD count; GRBM_GUI_ACTIVE comes summed over the
    8 XCDs), MFMA flops counted, and HBM-side traffic from FETCH_SIZE / WRITE_SIZE scaled by
    what the same counters read for a plain 256 MiB device copy.  Writes the entries into
    COUNTERS_FILE (with the kernel-source digest) and returns the markdown summary."""
    import workloads
    w = workloads.WORKLOADS[wname]
    sq = pmc_summary([_csv(d, f"sq_{wname}")])
    fe = pmc_summary([_csv(d, f"fetch_{wname}")])
    wr = pmc_summary([_csv(d, f"write_{wname}")])
    cf = pmc_summary([_csv(d, "fetch_copy")])
    cw = pmc_summary([_csv(d, "write_copy")])
    copy_bytes = 256 << 20
    fetch_f = next(v["FETCH_SIZE"] for k, v in cf.items() if "copyBuffer" in k) * 1024 / copy_bytes
    write_f = next(v["WRITE_SIZE"] for k, v in cw.items() if "copyBuffer" in k) * 1024 / copy_bytes
    eb = 4 if w.dtype == "f32" else 2
    mx_dispatch = w.gemm == "mxfp8" and bool(w.mx_scope) and len(w.mx_scope) == 6
    gem, byt = algorithmic_work(w, eb, mx_dispatch, *fused_quant_flags(w))
    calls = {}
    for table, keys in ((sq, ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                              "SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS")),
                        (fe, ("FETCH_SIZE",)), (wr, ("WRITE_SIZE",))):
        for kname, v in table.items():
            c = v.get("call")
            if not c or c == "copy":
                continue
            if c == "route" and w.routing == "given_uniform":  # the same kernels read the given ids
                c = "route_given"
            e = calls.setdefault(c, {"kernels": set()})
            e["kernels"].add(kname)
            for key in keys:
                e[key] = e.get(key, 0.0) + v.get(key, 0.0)
    digest = kernel_sources_digest()
    rec = json.load(open(COUNTERS_FILE)) if os.path.exists(COUNTERS_FILE) else {}
    rows = []
    for c, e in calls.items():
        gui = e.get("GRBM_GUI_ACTIVE", 0.0) / N_XCC
        util = 100.0 * e.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (gui * N_SIMD) if gui else 0.0
        flops = 512.0 * (e.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + e.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0))
        reads = e.get("FETCH_SIZE", 0.0) * 1024 / fetch_f
        writes = e.get("WRITE_SIZE", 0.0) * 1024 / write_f
        entry = {"source_digest": digest, "kernels": sorted(e["kernels"]), "gui_cycles_per_xcd": round(gui),
                 "mfma_util_pct": round(util, 2), "mfma_flops_counted": flops,
                 "algorithmic_flops_per_launch": gem.get(c), "read_bytes": round(reads), "write_bytes": round(writes),
                 "bytes_per_launch": round(reads + writes), "algorithmic_bytes_per_launch": byt.get(c),
                 "copy_fetch_factor": round(fetch_f, 5), "copy_write_factor": round(write_f, 5),
                 "lds_bank_conflicts": e.get("SQ_LDS_BANK_CONFLICT", 0.0)}
        rec[f"{wname}:{c}"] = entry
        rows.append((c, entry))
    with open(COUNTERS_FILE, "w") as fh:
        json.dump(rec, fh, indent=1, sort_keys=True)
    order = ["router_fwd", "route", "permute", "gemm1_fwd", "gemm2_fwd", "combine", "combine_bwd", "dgrad2", "wgrad2",
             "dgrad1", "route_bwd", "router_bwd", "permute_bwd", "wgrad1", "mx_dispatch"]
    rows.sort(key=lambda r: order.index(r[0]) if r[0] in order else 99)
    md = [f"| call | GUI cycles / XCD | MFMA util % | MFMA flops counted / algorithmic | HBM reads | HBM writes | "
          f"traffic / algorithmic bytes |", "|---|---|---|---|---|---|---|"]
    for c, e in rows:
        fl = (f"{e['mfma_flops_counted'] / e['algorithmic_flops_per_launch']:.3f}"
              if e["algorithmic_flops_per_launch"] and e["mfma_flops_counted"] else "")
        tb = (f"{e['bytes_per_launch'] / e['algorithmic_bytes_per_launch']:.2f}"
              if e["algorithmic_bytes_per_launch"] else "")
        md.append(f"| {c} | {e['gui_cycles_per_xcd']:,} | {e['mfma_util_pct'] if fl else ''} | {fl} | "
                  f"{e['read_bytes']:,} | {e['write_bytes']:,} | {tb} |")
    md.append("")
    md.append(f"Copy calibration: FETCH_SIZE reads {fetch_f:.4f} and WRITE_SIZE {write_f:.4f} of a 256 MiB copy's "
              f"bytes; kernel sources digest {digest}.")
    return "\n".join(md)


def counter_entry(wname, call):
    """The recorded counters of one call, if they were taken on the current kernel sources."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    try:
        e = json.load(open(COUNTERS_FILE)).get(f"{wname}:{call}")
    except Exception:
        return None
    return e if e and e.get("source_digest") == kernel_sources_digest() else None


def vendor_calibration(w):
    """The vendor BLAS (torch.bmm, bf16, contiguous operands) on batched GEMMs with the shapes
    of the workload's six expert GEMMs, every expert given the mean row count R/E: what a
    tuned library reaches on these shapes without ragged experts or fused epilogues.  A
    reference point for the MFMA fractions; nothing of the layer runs through it."""
    import torch
    n = w.T * w.k // w.E
    d, f, E = w.d, w.f, w.E
    shapes = {"gemm1_fwd": (E, n, d, 2 * f), "gemm2_fwd": (E, n, f, d), "dgrad2": (E, n, d, f),
              "wgrad2": (E, d, n, f), "dgrad1": (E, n, 2 * f, d), "wgrad1": (E, 2 * f, n, d),
              "dense_8192": (1, 8192, 8192, 8192)}
    out = {}
    g = torch.Generator(device="cuda").manual_seed(0)
    for name, (B, M, K, N) in shapes.items():
        a = torch.randn(B, M, K, device="cuda", generator=g).to(torch.bfloat16).contiguous()
        b = torch.randn(B, K, N, device="cuda", generator=g).to(torch.bfloat16).contiguous()
        for _ in range(3):
            torch.bmm(a, b)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            torch.bmm(a, b)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 20
        fl = 2.0 * B * M * K * N
        out[name] = {"batch_m_k_n": [B, M, K, N], "ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 1),
                     "frac_of_2.5pf": round(fl / ms / 1e9 / PEAK_TFLOPS["bf16"], 4)}
        del a, b
    return {"workload": w.name, "rows_per_expert": n, "vendor_bmm": out}


def main():
    args = parse()
    if args.vendor_calibration:
        import workloads
        print(json.dumps(vendor_calibration(workloads.WORKLOADS[args.workload])), flush=True)
        return
    if args.pmc_summary:
        print(json.dumps(pmc_summary(args.pmc_summary), indent=1))
        return
    if args.trace_summary:
        print(trace_summary(args.trace_summary, args.workload))
        return
    if args.pmc_record:
        print(pmc_record(args.workload, args.pmc_record))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the layer runs on one GPU's resident experts and this build has no "
              f"multi-GPU path (asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_mib:
        n = args.copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "steps": args.steps}), flush=True)
        return

    import mixture_experts_layer_logits_amd as m
    import workloads

    w = workloads.WORKLOADS[args.workload]
    if args.seed_offset:
        w = dataclasses.replace(w, seed=w.seed + args.seed_offset)
    inp = workloads.make_inputs(w)
    learned = w.routing != "given_uniform"
    act = m.MOE_F32 if w.dtype == "f32" else m.MOE_BF16
    gemm = {"f32": m.MOE_F32, "bf16": m.MOE_BF16, "mxfp8": m.MOE_MXFP8}[w.gemm]
    torch.cuda.set_device(0)
    mx_scope = sum(m.MX_BITS[n] for n in w.mx_scope) if (gemm == m.MOE_MXFP8 and w.mx_scope) else 0
    mx_dispatch = False if args.bf16_dispatch else None   # None: on when the scope covers the dispatch readers
    L = m.MoEExpertLayer(w.T, w.d, w.f, w.E, w.k, act=act, gemm=gemm, shared_f=w.shared_f, mx_dispatch=mx_dispatch,
                         mx_scope=mx_scope, mx_fused_quant=not args.unfused_quant)
    mx_bits = m.mx_scope_bits(L.shape)
    gemm_peak = {n: (PEAK_TFLOPS["mxfp8"] if mx_bits & b else PEAK_TFLOPS["bf16" if w.gemm == "mxfp8" else w.gemm])
                 for n, b in (("gemm1_fwd", m.MOE_MX_GEMM1), ("gemm2_fwd", m.MOE_MX_GEMM2),
                              ("dgrad2", m.MOE_MX_DGRAD2), ("wgrad2", m.MOE_MX_WGRAD2),
                              ("dgrad1", m.MOE_MX_DGRAD1), ("wgrad1", m.MOE_MX_WGRAD1))}
    gemm_peak["gemm1_recompute"] = gemm_peak["gemm1_fwd"]
    dev = lambda v: v.cuda() if isinstance(v, torch.Tensor) else (tuple(u.cuda() for u in v)  # noqa: E731
                                                                 if isinstance(v, tuple) else v)
    d_inp = {k: dev(v) for k, v in inp.items()}
    L.forward(d_inp["x"], d_inp["W1"], d_inp["W3"], d_inp["W2"], Wr=d_inp["Wr"], bias=d_inp["router_bias"],
              topk_idx=d_inp["topk_idx"], gates=d_inp["gates"], shared=d_inp["shared"])
    calls = step_calls(m, L, d_inp, learned, args.recompute)

    if args.profile_steps:
        for _ in range(args.profile_steps):
            for _, fn in calls:
                fn()
        torch.cuda.synchronize()
        print(json.dumps({"workload": w.name, "profile_steps": args.profile_steps}), flush=True)
        return

    if args.profile_kernel:
        for _, fn in calls:  # one whole step sets up every call's inputs
            fn()
        fn = dict(calls)[args.profile_kernel]
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        print(json.dumps({"workload": w.name, "kernel": args.profile_kernel, "steps": args.steps}), flush=True)
        return

    for _ in range(args.warmup):
        for _, fn in calls:
            fn()
    torch.cuda.synchronize()

    ev = {name: [] for name, _ in calls}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for name, fn in calls:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            ev[name].append((a, b))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    per_call_ms = {name: sum(a.elapsed_time(b) for a, b in pairs) / len(pairs) for name, pairs in ev.items()}
    ms_per_step_eager = elapsed * 1e3 / args.steps

    if not args.no_graph:
        # the whole step captured once as a HIP graph (every call is kernel launches only),
        # then replayed: the step without the host's launch gaps
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _, fn in calls:
                fn()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _, fn in calls:
                fn()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        # the spread of single steps: each of K more replays between two events
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b in evs:
            a.record()
            graph.replay()
            b.record()
        torch.cuda.synchronize()
        step_ms = sorted(a.elapsed_time(b) for a, b in evs)
    else:
        step_ms = sorted(sum(ev[name][i][0].elapsed_time(ev[name][i][1]) for name, _ in calls)
                         for i in range(args.steps))
    ms_per_step = elapsed * 1e3 / args.steps
    pct = lambda q: round(step_ms[min(len(step_ms) - 1, int(q * len(step_ms)))], 4)  # noqa: E731

    # the HBM-bound row movement cold: L2 and the 256 MiB MALL flushed by reading 512 MiB
    # before every launch (the routed buffers of these workloads fit in the MALL; a read
    # evicts them without leaving dirty lines to drain during the timed launch)
    flush = torch.ones(128 << 20, dtype=torch.int32, device="cuda")
    cold_ms = {}
    for name, fn in calls:
        if name not in ("permute", "combine", "combine_bwd", "permute_bwd"):
            continue
        ts = []
        for _ in range(5):
            flush.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        cold_ms[name] = sorted(ts)[len(ts) // 2]
    del flush
    tokens_per_s = w.T * args.steps / elapsed

    eb = 4 if w.dtype == "f32" else 2
    gem, byt = algorithmic_work(w, eb, L.mx_dispatch, L.fq_h, L.fq_dab)
    if w.shared_f:  # the shared expert's GEMMs: the routed ones with R = T, f = fs, one expert
        ws_ = dataclasses.replace(w, k=1, E=1, f=w.shared_f)
        gs, bs = algorithmic_work(ws_, eb, False, L.fq_h, L.fq_dab)
        for n in ("gemm1_fwd", "gemm2_fwd", "dgrad2", "wgrad2", "dgrad1", "wgrad1"):
            key = "shared_" + n.replace("_fwd", "")
            gem[key], byt[key] = gs[n], bs[n]
    if args.recompute:
        gem["gemm1_recompute"], byt["gemm1_recompute"] = gem["gemm1_fwd"], byt["gemm1_fwd"]
    kernels = {}
    for name, ms in per_call_ms.items():
        e = {"ms": round(ms, 4)}
        if name in gem:
            e["tflops"] = round(gem[name] / (ms * 1e-3) / 1e12, 1)
        if name in byt:
            e["gbs"] = round(byt[name] / (ms * 1e-3) / 1e9, 1)
        kernels[name] = e
    # dominant kernel: the GEMM taking the most time; its roof is whichever of MFMA peak and
    # HBM bandwidth bounds its algorithmic work from below
    dom = max(gem, key=lambda n: per_call_ms[n])
    # each GEMM against the peak of its own arithmetic (fp8 for the GEMMs in the MXFP8 scope)
    peak_of = lambda n: gemm_peak.get(n, PEAK_TFLOPS["bf16" if w.gemm == "mxfp8" else w.gemm])  # noqa: E731
    peak = peak_of(dom)
    t_mfma = gem[dom] / (peak * 1e12)
    t_hbm = byt[dom] / (PEAK_HBM_GBS * 1e9)
    sec = per_call_ms[dom] * 1e-3
    # counter evidence (rocprofv3 passes recorded in profiles/counters.json on these kernel
    # sources): HBM-side traffic and MFMA utilisation per call, next to the algorithmic figures
    for name, e in kernels.items():
        ce = counter_entry(w.name, name)
        if ce:
            e["counter_traffic_bytes"] = ce["bytes_per_launch"]
            e["counter_gbs"] = round(ce["bytes_per_launch"] / (e["ms"] * 1e-3) / 1e9, 1)
            if ce.get("algorithmic_flops_per_launch"):
                e["counter_mfma_util_pct"] = ce["mfma_util_pct"]
    ce = counter_entry(w.name, dom)
    traffic = ce["bytes_per_launch"] if ce else None
    if t_hbm >= t_mfma:
        achieved = byt[dom] / sec / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic}
    else:
        achieved = gem[dom] / sec / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(achieved / peak, 4), "traffic": traffic}
    roofline.update({"kernel": dom, "ms_per_launch": round(per_call_ms[dom], 4),
                     "algorithmic_bytes_per_launch": byt[dom], "algorithmic_flops_per_launch": gem[dom],
                     "mfma_frac": round(gem[dom] / sec / 1e12 / peak, 4),
                     "hbm_frac": round(byt[dom] / sec / 1e9 / PEAK_HBM_GBS, 4)})
    gemm_ms = sum(per_call_ms[n] for n in gem)
    ideal_ms = sum(gem[n] / (peak_of(n) * 1e12) * 1e3 for n in gem)   # every GEMM at its peak
    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "ms_per_step_eager": round(ms_per_step_eager, 4),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.gemm, "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "f": w.f, "E": w.E, "k": w.k, "routing": w.routing,
                   "gemm": w.gemm, "recompute": bool(args.recompute), "shared_f": w.shared_f,
                   "mx_dispatch": L.mx_dispatch, "hip_graph": not args.no_graph, "seed": w.seed,
                   "mx_scope": [n for n, b in m.MX_BITS.items() if mx_bits & b]},
        "step_ms_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
        "roofline": roofline,
        # time all grouped GEMMs would take at their peaks over the time they took
        "grouped_gemm_mfma_frac_all6": round(ideal_ms / gemm_ms, 4),
        "kernels": kernels,
        # median of 5 launches, each after a 512 MiB read that flushes L2 and the MALL
        "kernels_cold": {n: {"ms": round(v, 4), "gbs": round(byt[n] / (v * 1e-3) / 1e9, 1)} for n, v in cold_ms.items()},
        "expert_load": {"max": int(L.counts.max().item()), "mean": w.T * w.k / w.E,
                        "empty": int((L.counts == 0).sum().item())},
        # expert-FFN activations held from the forward to the backward (the routed rows of x,
        # y_perm, and ab, h unless recomputed)
        "activation_bytes_held": L.activation_bytes() - (w.R * 3 * w.f * eb if args.recompute else 0),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp, min(args.cpu_sample_tokens, w.T))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
