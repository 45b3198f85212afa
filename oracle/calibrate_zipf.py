"""Find the Zipf bias scale beta for the load-imbalance workload.

Routes the workload's tokens with the CPU oracle (fp64 router scores plus the
Zipf(1.1) per-expert bias, top-k) and bisects beta until the hottest expert
receives about 10x the mean number of rows.  The printed beta is stored in
workloads.py; input generation itself never routes anything.

Run: python -m oracle.calibrate_zipf
"""
import numpy as np

import workloads
from oracle import moe_ref as ref


def hot_ratio(w, beta):
    inp = workloads.make_inputs(w, zipf_beta_override=beta)
    L = ref.router_logits(inp["x"], inp["Wr"], inp["router_bias"])
    idx, _ = ref.topk_gates(L, w.k)
    counts = np.bincount(idx.reshape(-1), minlength=w.E)
    return counts.max() / (w.T * w.k / w.E), int((counts == 0).sum())


def main():
    w = workloads.WORKLOADS["e128_k4_t16384_zipf"]
    lo, hi = 0.0, 4.0
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        r, _ = hot_ratio(w, mid)
        if r < 10.0:
            lo = mid
        else:
            hi = mid
    beta = round(0.5 * (lo + hi), 4)
    r, zeros = hot_ratio(w, beta)
    print(f"beta={beta} hottest/mean={r:.3f} empty_experts={zeros}")


if __name__ == "__main__":
    main()
