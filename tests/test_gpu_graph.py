"""The layer step captured as a HIP graph.

Every library call enqueues kernel launches only (no memset, copy, allocation or host
synchronisation), so a whole forward + backward step can be captured once and replayed.
Each replay here follows eager work on the same buffers (fills that clobber every output)
and a synchronisation, and must reproduce the eager step bit for bit.
"""
import pytest
import torch

import workloads
from gpu_common import run_layer, say, to_dev

pytestmark = pytest.mark.gpu

OUTS = ["logits", "gates", "topk_idx", "counts", "offsets", "slot_row", "row_src", "h", "y_perm", "y", "dgates",
        "dab", "dx_perm", "dW1", "dW3", "dW2", "dlogits", "dWr", "dx",
        "xq_rows", "xs_rows", "dyq_rows", "dys_rows"]  # (column layouts leave unwritten tails)
ROUTER = ("logits", "dlogits", "dWr", "gates", "topk_idx")  # absent or caller inputs with given routing


@pytest.mark.parametrize("wname,over", [
    ("e128_k4_t8192", dict(T=512, d=256, f=192)),
    ("e32_k4_t16384_d4096_mxfp8", dict(T=300, d=256, f=256, E=8, k=4)),
    ("e32_k4_t16384_d4096_mxfp8_all", dict(T=300, d=256, f=256, E=8, k=4)),
], ids=["bf16_learned", "mxfp8_given", "mxfp8_all_six_dispatch"])
def test_layer_step_graph_replays_match_eager(wname, over):
    w = workloads.scaled(workloads.WORKLOADS[wname], **over)
    inp = workloads.make_inputs(w)
    say(f"[gpu] layer step in a HIP graph {w}")
    L = run_layer(w, inp)  # eager step (also sets up every launch configuration)
    names = [n for n in OUTS
             if getattr(L, n, None) is not None and not (n in ROUTER and w.routing == "given_uniform")]
    ref = {n: getattr(L, n).clone() for n in names}
    d = to_dev(inp)

    def step():
        if w.routing == "given_uniform":
            L.forward(d["x"], d["W1"], d["W3"], d["W2"], topk_idx=d["topk_idx"], gates=d["gates"])
        else:
            L.forward(d["x"], d["W1"], d["W3"], d["W2"], Wr=d["Wr"], bias=d["router_bias"])
        L.backward(d["dy"])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for n in names:  # eager work between replays: clobber every output
            getattr(L, n).fill_(7 if getattr(L, n).is_floating_point() else -1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        bad = [n for n in names if not torch.equal(getattr(L, n), ref[n])]
        assert not bad, (rep, bad)
