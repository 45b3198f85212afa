"""Grouped GEMMs with loader waves against the same GEMMs without them.

On 128 x 256 tiles (and on the 256 x 256 weight-gradient tiles), four extra waves may issue
every operand load while the eight compute waves only multiply and store. That changes
which wave loads a stage, not what is summed or in which order. A layer step with loader
waves on every GEMM that can take them (MOE_GEMM_LOADERS=4: GEMM1, GEMM2, dgrad2, dgrad1
with its W1 / W3 split, the router's dx, wgrad2, wgrad1) must therefore equal the step with
them off (MOE_GEMM_LOADERS=0) bit for bit. The overrides are read once per process, so the
test asks the library to read them again after each change (moe_tuning_reload). The cases
have ragged expert ends, ragged N edges, several tiles per expert, and (given routing, 80
slots over 64 experts) empty experts.
"""
import os

import pytest
import torch

import workloads
from gpu_common import run_layer, say

pytestmark = pytest.mark.gpu

OUTS = ["logits", "ab", "h", "y_perm", "y", "dgates", "dab", "dx_perm", "dW1", "dW3", "dW2", "dlogits", "dWr", "dx_r",
        "dx"]


@pytest.mark.parametrize("wname,over", [
    ("e128_k4_t8192", dict(T=600, d=256, f=192, E=16, k=4)),
    ("e128_k4_t16384_random", dict(T=40, d=128, f=128, E=64, k=2)),
], ids=["learned_ragged", "given_empty_experts"])
def test_loader_waves_match_plain_kernel_bitwise(wname, over):
    w = workloads.scaled(workloads.WORKLOADS[wname], **over)
    inp = workloads.make_inputs(w)
    import mixture_experts_layer_logits_amd as m
    old = os.environ.get("MOE_GEMM_LOADERS")
    try:
        say(f"[gpu] layer step with loader waves {w}")
        os.environ["MOE_GEMM_LOADERS"] = "4"
        m.moe_tuning_reload()
        A = run_layer(w, inp)
        names = [n for n in OUTS if getattr(A, n, None) is not None
                 and not (w.routing == "given_uniform" and n in ("logits", "dlogits", "dWr", "dx_r"))]
        ref = {n: getattr(A, n).clone() for n in names}
        say(f"[gpu] layer step without loader waves {w}")
        os.environ["MOE_GEMM_LOADERS"] = "0"
        m.moe_tuning_reload()
        B = run_layer(w, inp)
    finally:
        if old is None:
            os.environ.pop("MOE_GEMM_LOADERS", None)
        else:
            os.environ["MOE_GEMM_LOADERS"] = old
        m.moe_tuning_reload()
    bad = [n for n in names if not torch.equal(getattr(B, n), ref[n])]
    assert not bad, bad
