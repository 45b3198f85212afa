"""Host-side logic of bench.py (no GPU): the algorithmic byte and flop model each roofline
figure divides by, the MXFP8 epilogue-quantisation flags, and the rocprofv3 kernel-trace
summary."""
import csv
import dataclasses
import importlib.util
import os

import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_algorithmic_work_counts_each_operand_once(bench):
    w = workloads.WORKLOADS["e128_k4_t8192"]
    T, d, f, E, k = w.T, w.d, w.f, w.E, w.k
    R, eb = T * k, 2
    gem, byt = bench.algorithmic_work(w, eb)
    # flops: 2 per multiply-add; GEMM1 and the GEMM1-side gradients reduce over 2f outputs
    assert gem["gemm1_fwd"] == 2.0 * R * d * 2 * f == gem["dgrad1"] == gem["wgrad1"]
    assert gem["gemm2_fwd"] == 2.0 * R * f * d == gem["dgrad2"] == gem["wgrad2"]
    # row movement: x read once, k routed copies written, 8 bytes of indices per routed row
    assert byt["permute"] == T * d * eb + R * d * eb + R * 8
    # wgrad1: dab and x_perm read once, dW1 and dW3 written once
    assert byt["wgrad1"] == R * 2 * f * eb + R * d * eb + 2 * E * f * d * eb
    # learned routing: the un-permute also folds in the router's dx_r, reading each token's k
    # ids and dlogits and Wr once; given routing does not
    assert byt["permute_bwd"] == R * d * eb + T * d * eb + R * 4 + R * 8 + E * d * eb
    # the router backward then reads dlogits and x and writes dWr only
    assert byt["router_bwd"] == T * E * 4 + T * d * eb + E * d * 4
    wg = workloads.WORKLOADS["e128_k4_t16384_random"]
    _, bg = bench.algorithmic_work(wg, eb)
    assert bg["permute_bwd"] == wg.R * wg.d * eb + wg.T * wg.d * eb + wg.R * 4


def test_epilogue_quantisation_moves_the_activation_bytes(bench):
    w = workloads.WORKLOADS["e32_k4_t16384_d4096_mxfp8"]
    R, d, f, E, eb = w.R, w.d, w.f, w.E, 2
    assert bench.fused_quant_flags(w) == (True, True)            # the default scope
    assert bench.fused_quant_flags(workloads.WORKLOADS["e32_k4_t16384_d4096_mxfp8_all"]) == (False, False)
    assert bench.fused_quant_flags(workloads.WORKLOADS["e32_k4_t16384_d4096_bf16"]) == (False, False)
    _, plain = bench.algorithmic_work(w, eb)
    _, fused = bench.algorithmic_work(w, eb, False, True, True)
    qh, qd = R * f * 33 // 32, R * 2 * f * 33 // 32              # E4M3 codes + one scale per 32
    assert fused["gemm1_fwd"] == plain["gemm1_fwd"] + qh
    assert fused["gemm2_fwd"] == qh + E * f * d * eb + R * d * eb
    assert fused["dgrad2"] == plain["dgrad2"] + qd
    assert fused["dgrad1"] == qd + 2 * E * f * d * eb + R * d * eb


def test_trace_summary_statistics(bench, tmp_path):
    rows = [("kern_a", 0, 10_000), ("kern_a", 20_000, 40_000), ("kern_a", 50_000, 56_000), ("kern_b", 60_000, 61_000)]
    path = tmp_path / "run" / "t_kernel_trace.csv"
    path.parent.mkdir()
    with open(path, "w", newline="") as fh:
        wr = csv.writer(fh)
        wr.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for n, a, b in rows:
            wr.writerow([n, a, b])
    out = bench.trace_summary(str(tmp_path), "toy")
    lines = [ln for ln in out.splitlines() if ln.startswith("| `")]
    assert lines[0].startswith("| `kern_a` | 3 | 12.0 | 10.0 | 6.0 | 20.0 | 97.30 |")
    assert lines[1].startswith("| `kern_b` | 1 | 1.0 | 1.0 | 1.0 | 1.0 | 2.70 |")


def test_workloads_are_frozen_and_scaled_copies_keep_the_routing_mode():
    w = workloads.WORKLOADS["e128_k4_t16384_zipf_steep"]
    s = workloads.scaled(w, T=64, d=128, f=128, E=16)
    assert s.routing == w.routing and s.zipf_beta == w.zipf_beta and s.name.endswith("_scaled")
    with pytest.raises(dataclasses.FrozenInstanceError):
        w.T = 1
