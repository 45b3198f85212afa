"""GPU parity of the HIP path (through the C-ABI) against the CPU oracle.

Sizes here are ones the oracle finishes in seconds but that still span several GEMM
tiles, ragged expert segments, empty experts and partial routing chunks.  Integer
outputs must match bit for bit; values within the method's tolerances.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_common import TOL, host, normwise_err, oracle_for, run_layer, say, to_dev

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS

# (workload, overrides) -- scaled copies keep dtype and routing mode
CASES = [
    ("tiny_fp32", {}),
    ("e8_k4_t8192", dict(T=512, d=256, f=128)),
    ("e128_k4_t8192", dict(T=512, d=256, f=192)),
    ("e128_k4_t16384_zipf", dict(T=600, d=128, f=128)),
    ("e128_k4_t16384_random", dict(T=333, d=192, f=128)),
    ("e8_k4_t8192", dict(T=77, d=64, f=64, E=1, k=1, name="single_expert")),
    ("e8_k4_t8192", dict(T=130, d=128, f=64, E=4, k=4, name="k_equals_E")),
    ("e128_k4_t8192_shared", dict(T=300, d=256, f=192, shared_f=128, name="shared_expert")),
    # >= 1024 rows per expert: the 256 x 256 two-stage tiles of the M-grouped GEMMs, ragged in N
    ("e8_k4_t8192", dict(T=1300, d=256, f=192, E=2, k=2, name="long_segments")),
]


def _case(name, over):
    w = W[name]
    return workloads.scaled(w, **over) if over else w


def _check_layer(w, inp, layer):
    tol = TOL[w.gemm]
    learned = w.routing != "given_uniform"
    gl = host(layer.logits) if learned else None
    fw, bw = oracle_for(w, inp, gpu_logits=gl)
    # integers: bit-exact
    assert np.array_equal(host(layer.topk_idx), fw["topk_idx"]) if learned else True
    assert np.array_equal(host(layer.counts), fw["counts"])
    assert np.array_equal(host(layer.offsets), fw["offsets"])
    assert np.array_equal(host(layer.slot_row), fw["slot_row"])
    assert np.array_equal(host(layer.row_src), fw["row_src"])
    # permute is a pure copy: bit-exact
    assert np.array_equal(host(layer.x_perm), np.asarray(fw["x_perm"], dtype=np.float64))
    errs = {}
    if learned:
        errs["logits"] = normwise_err(gl, fw["logits"])
        errs["gates"] = normwise_err(host(layer.gates), fw["gates"])
    if layer.h is not None:  # a recompute layer drops a, b and h after the backward
        errs["h"] = normwise_err(host(layer.h), fw["h"])
    errs["y_perm"] = normwise_err(host(layer.y_perm), fw["y_perm"])
    errs["y"] = normwise_err(host(layer.y), fw["y"])
    errs["dgates"] = normwise_err(host(layer.dgates), bw["dgates"])
    errs["dx_perm"] = normwise_err(host(layer.dx_perm), bw["dx_perm"])
    errs["dW1"] = normwise_err(host(layer.dW1), bw["dW1"])
    errs["dW3"] = normwise_err(host(layer.dW3), bw["dW3"])
    errs["dW2"] = normwise_err(host(layer.dW2), bw["dW2"])
    errs["dx"] = normwise_err(host(layer.dx), bw["dx"])
    if w.shared_f:
        errs["dW1s"] = normwise_err(host(layer.dW1s), bw["dW1s"])
        errs["dW3s"] = normwise_err(host(layer.dW3s), bw["dW3s"])
        errs["dW2s"] = normwise_err(host(layer.dW2s), bw["dW2s"])
    if learned:
        errs["dlogits"] = normwise_err(host(layer.dlogits), bw["dlogits"])
        errs["dWr"] = normwise_err(host(layer.dWr), bw["dWr"])
    print(w.name, {k: f"{v:.2e}" for k, v in errs.items()})
    bad = {k: v for k, v in errs.items() if v > tol}
    assert not bad, (w.name, bad)
    # experts without rows get exactly zero weight gradients
    empty = np.nonzero(fw["counts"] == 0)[0]
    for e in empty:
        assert not host(layer.dW1[e]).any() and not host(layer.dW2[e]).any()


@pytest.mark.parametrize("name,over", CASES, ids=[c[1].get("name", c[0]) for c in CASES])
def test_layer_parity(name, over):
    w = _case(name, over)
    inp = workloads.make_inputs(w)
    say(f"[gpu] layer parity {w}")
    layer = run_layer(w, inp)
    _check_layer(w, inp, layer)


RECOMPUTE_CASES = [("e128_k4_t8192", dict(T=512, d=256, f=192)),
                   ("e128_k4_t8192_shared", dict(T=300, d=256, f=192, shared_f=128, name="shared_expert")),
                   ("e128_k4_t16384_random", dict(T=333, d=192, f=128))]


@pytest.mark.parametrize("name,over", RECOMPUTE_CASES, ids=[c[1].get("name", c[0]) + "_recompute"
                                                            for c in RECOMPUTE_CASES])
def test_recompute_layer_parity(name, over):
    """The layer that recomputes GEMM1 in the backward, against the oracle."""
    w = _case(name, over)
    inp = workloads.make_inputs(w)
    say(f"[gpu] recompute layer parity {w}")
    layer = run_layer(w, inp, recompute=True)
    assert layer.ab is None and layer.h is None
    _check_layer(w, inp, layer)


ROUTER_DX_CASES = [("e128_k4_t8192", dict(T=300, d=256, f=128, E=16, k=4)),
                   ("e128_k4_t8192", dict(T=200, d=192, f=128, E=16, k=6, name="k6")),
                   ("tiny_fp32", {})]


@pytest.mark.parametrize("name,over", ROUTER_DX_CASES, ids=[c[1].get("name", c[0]) for c in ROUTER_DX_CASES])
def test_router_dx_folded_into_unpermute(name, over):
    """The un-permute with the router's input gradient folded in (k rows of Wr per token,
    the layer's default) and the dense dlogits Wr GEMM into dx_r followed by the plain
    un-permute: both against the oracle, the same dlogits and dWr bit for bit, and dx of
    the two within the tolerance of each other."""
    w = _case(name, over)
    inp = workloads.make_inputs(w)
    say(f"[gpu] router dx folded {w}")
    A = run_layer(w, inp, router_dx_fused=True)
    assert A.dx_r is None
    _check_layer(w, inp, A)
    keep = {n: getattr(A, n).clone() for n in ("dlogits", "dWr", "dx")}
    say(f"[gpu] router dx as a GEMM {w}")
    B = run_layer(w, inp, router_dx_fused=False)
    _check_layer(w, inp, B)
    assert torch.equal(B.dlogits, keep["dlogits"]) and torch.equal(B.dWr, keep["dWr"])
    assert normwise_err(host(B.dx), host(keep["dx"])) < TOL[w.gemm]


def test_folded_router_dx_clamps_expert_ids():
    """moe_permute_bwd_router reads a row of Wr per routed slot; an expert id outside [0, E)
    is clamped into it, never used as an address.  Against the oracle's un-permute and
    router backward with those clamped ids (each token's ids stay distinct after clamping)."""
    import mixture_experts_layer_logits_amd as m
    from oracle import moe_ref as ref
    T, E, k, d = 24, 8, 2, 64
    g = torch.Generator().manual_seed(5)
    idx = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).int()
    s = m.make_shape(T, d, 64, E, k)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    slot = torch.empty(T, k, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(m.moe_workspace_size(s), dtype=torch.uint8, device="cuda")
    m.moe_route_given(s, idx.cuda(), counts, offsets, slot, err, ws)
    bad = idx.clone()
    # ids that clamp to 0 or E - 1, on tokens that do not already hold that expert
    for t in range(T):
        if t % 3 == 0 and 0 not in idx[t].tolist():
            bad[t, 0] = -3
        elif t % 3 == 1 and E - 1 not in idx[t].tolist():
            bad[t, 1] = E + 5
    assert (bad < 0).any() and (bad >= E).any()
    dx_perm = torch.randn(T * k, d, generator=g).to(torch.bfloat16)
    dL = torch.randn(T, E, generator=g)
    Wr = (0.02 * torch.randn(E, d, generator=g)).to(torch.bfloat16)
    dx = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
    say("[gpu] folded router dx with clamped ids")
    m.moe_permute_bwd_router(s, dx_perm.cuda(), slot, bad.cuda(), dL.cuda(), Wr.cuda(), None, dx)
    torch.cuda.synchronize()
    used = bad.clamp(0, E - 1).numpy()
    dLs = np.zeros((T, E))
    for t in range(T):
        dLs[t, used[t]] = dL[t, used[t]].numpy()
    dx_r, _ = ref.router_bwd(np.zeros((T, d)), Wr.float().numpy(), dLs)
    want = ref.unpermute_sum(dx_perm.float().numpy(), host(slot), dx_r)
    assert normwise_err(host(dx), want) < 1e-2


def test_autograd_function_against_the_oracle():
    """MoEExpertFunction (learned routing with a router bias): torch autograd gradients of
    x, Wr, W1, W3, W2 against the oracle's; a second forward through the same layer before
    the first one's backward makes that backward raise."""
    import mixture_experts_layer_logits_amd as m
    from mixture_experts_layer_logits_amd.layer import MoEExpertFunction
    from oracle import moe_ref as ref
    w = workloads.scaled(W["e128_k4_t16384_zipf"], T=256, d=128, f=128, E=16, name="autograd")
    inp = workloads.make_inputs(w)
    say(f"[gpu] autograd function {w}")
    d = to_dev(inp)
    layer = m.MoEExpertLayer(w.T, w.d, w.f, w.E, w.k)
    leaves = {k: d[k].clone().requires_grad_(True) for k in ("x", "Wr", "W1", "W3", "W2")}
    y = MoEExpertFunction.apply(leaves["x"], leaves["Wr"], leaves["W1"], leaves["W3"], leaves["W2"], layer,
                                d["router_bias"])
    y.backward(d["dy"])
    torch.cuda.synchronize()
    fw = ref.layer_forward(inp["x"], inp["W1"], inp["W3"], inp["W2"], w.k, Wr=inp["Wr"], bias=inp["router_bias"],
                           select_logits=host(layer.logits))
    bw = ref.layer_backward(fw, inp["dy"], inp["x"], inp["W1"], inp["W3"], inp["W2"], Wr=inp["Wr"])
    errs = {"y": normwise_err(host(y), fw["y"]), "dx": normwise_err(host(leaves["x"].grad), bw["dx"]),
            "dWr": normwise_err(host(leaves["Wr"].grad), bw["dWr"]),
            "dW1": normwise_err(host(leaves["W1"].grad), bw["dW1"]),
            "dW3": normwise_err(host(leaves["W3"].grad), bw["dW3"]),
            "dW2": normwise_err(host(leaves["W2"].grad), bw["dW2"])}
    print("autograd", {k: f"{v:.2e}" for k, v in errs.items()})
    assert max(errs.values()) < TOL["bf16"], errs
    # two forwards, then the first one's backward: refused
    y1 = MoEExpertFunction.apply(leaves["x"], leaves["Wr"], leaves["W1"], leaves["W3"], leaves["W2"], layer)
    y2 = MoEExpertFunction.apply(leaves["x"], leaves["Wr"], leaves["W1"], leaves["W3"], leaves["W2"], layer)
    with pytest.raises(RuntimeError, match="another forward"):
        y1.backward(d["dy"])
    y2.backward(d["dy"])
    torch.cuda.synchronize()


def test_given_routing_leaves_the_layer_ids_alone():
    """A forward with caller-given expert ids only reads them: a later learned-routing
    forward writes its ids into the layer's own buffer, never into the caller's tensor."""
    import mixture_experts_layer_logits_amd as m
    w = workloads.scaled(W["e128_k4_t16384_random"], T=64, d=128, f=128, E=8, name="given_then_learned")
    inp = workloads.make_inputs(w)
    say("[gpu] given routing then learned routing")
    d = to_dev(inp)
    layer = m.MoEExpertLayer(w.T, w.d, w.f, w.E, w.k)
    given = d["topk_idx"].clone()
    layer.forward(d["x"], d["W1"], d["W3"], d["W2"], topk_idx=given, gates=d["gates"])
    Wr = (torch.randn(w.E, w.d, generator=torch.Generator().manual_seed(3)) * 0.02).to(torch.bfloat16).cuda()
    layer.forward(d["x"], d["W1"], d["W3"], d["W2"], Wr=Wr)
    torch.cuda.synchronize()
    assert torch.equal(given, d["topk_idx"])
    assert layer.topk_idx.data_ptr() != given.data_ptr()


def test_layer_deterministic():
    w = workloads.scaled(W["e128_k4_t8192"], T=512, d=256, f=128)
    inp = workloads.make_inputs(w)
    say("[gpu] determinism")
    a = run_layer(w, inp)
    outs = [t.clone() for t in (a.y, a.dx, a.dW1, a.dW2, a.dW3, a.dWr, a.slot_row)]
    b = run_layer(w, inp, layer=a)
    for t0, t1 in zip(outs, (b.y, b.dx, b.dW1, b.dW2, b.dW3, b.dWr, b.slot_row)):
        assert torch.equal(t0, t1)


@pytest.mark.parametrize("wname", ["e128_k4_t8192", "e32_k4_t16384_d4096_mxfp8"])
def test_activation_recompute_bitwise(wname):
    """Recomputing GEMM1 in the backward (keeping only x_perm) gives the same outputs and
    gradients bit for bit as keeping a, b and h: GEMM1 is deterministic, so the
    regenerated activations are identical."""
    import mixture_experts_layer_logits_amd as m
    over = dict(T=300, d=256, f=192) if wname == "e128_k4_t8192" else dict(T=300, d=256, f=256, E=8)
    w = workloads.scaled(W[wname], **over)
    inp = workloads.make_inputs(w)
    say(f"[gpu] activation recompute {w}")
    kept = run_layer(w, inp)
    gemm = {"bf16": m.MOE_BF16, "mxfp8": m.MOE_MXFP8}[w.gemm]
    rec = run_layer(w, inp, layer=m.MoEExpertLayer(w.T, w.d, w.f, w.E, w.k, gemm=gemm, recompute=True))
    names = ["y", "dgates", "dx_perm", "dW1", "dW3", "dW2", "dx"] + (["dWr"] if kept.learned else [])
    for n in names:
        assert torch.equal(getattr(kept, n), getattr(rec, n)), n
    assert rec.ab is None and rec.h is None
    assert rec.activation_bytes() == kept.activation_bytes() - w.R * 3 * w.f * 2


def test_empty_batch():
    import mixture_experts_layer_logits_amd as m
    w = workloads.scaled(W["e8_k4_t8192"], T=0, d=64, f=64)
    say("[gpu] T = 0")
    L = m.MoEExpertLayer(0, 64, 64, 8, 4)
    inp = workloads.make_inputs(workloads.scaled(W["e8_k4_t8192"], T=1, d=64, f=64))
    d = to_dev(inp)
    x = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    L.forward(x, d["W1"], d["W3"], d["W2"], Wr=d["Wr"])
    L.backward(x)
    torch.cuda.synchronize()
    assert not host(L.counts).any() and not host(L.offsets).any()
    assert not host(L.dW1).any() and not host(L.dW2).any() and not host(L.dWr).any()


def test_route_ties_and_limits():
    """Constructed ties (equal scores, +-0), the largest E and k the kernels support."""
    import mixture_experts_layer_logits_amd as m
    from oracle import moe_ref as ref
    for (T, E, k) in [(96, 16, 4), (64, 1024, 8), (70, 64, 32), (33, 1, 1)]:
        say(f"[gpu] route ties T={T} E={E} k={k}")
        g = torch.Generator().manual_seed(T * E + k)
        L = torch.randint(-2, 3, (T, E), generator=g).float()
        L[0] = 0.0
        L[1, ::2] = -0.0
        s = m.make_shape(T, 64, 64, E, k)
        out = dict(idx=torch.empty(T, k, dtype=torch.int32, device="cuda"),
                   gates=torch.empty(T, k, device="cuda"),
                   counts=torch.empty(E, dtype=torch.int32, device="cuda"),
                   offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
                   slot=torch.empty(T, k, dtype=torch.int32, device="cuda"))
        ws = torch.empty(m.moe_workspace_size(s), dtype=torch.uint8, device="cuda")
        m.moe_route(s, L.cuda(), out["idx"], out["gates"], out["counts"], out["offsets"], out["slot"], ws)
        torch.cuda.synchronize()
        idx, gates = ref.topk_gates(L.numpy(), k)
        counts, offsets, slot_row, _ = ref.dispatch(idx, E)
        assert np.array_equal(host(out["idx"]), idx)
        assert np.array_equal(host(out["counts"]), counts)
        assert np.array_equal(host(out["offsets"]), offsets)
        assert np.array_equal(host(out["slot"]), slot_row)
        assert normwise_err(host(out["gates"]), gates) < 1e-6
        assert np.abs(host(out["gates"]).sum(axis=1) - 1).max() < 1e-6


def test_route_given_errors():
    """Out-of-range and duplicate pre-routed ids set the device error word and are
    clamped, so the dispatch stays a bijection."""
    import mixture_experts_layer_logits_amd as m
    from oracle import moe_ref as ref
    T, E, k = 40, 8, 2
    idx = torch.stack([torch.randperm(E)[:k] for _ in range(T)]).int()
    idx[3, 1] = 9
    idx[5, 0] = -2
    idx[7] = torch.tensor([4, 4])
    s = m.make_shape(T, 64, 64, E, k)
    say("[gpu] route_given errors")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    slot = torch.empty(T, k, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(m.moe_workspace_size(s), dtype=torch.uint8, device="cuda")
    m.moe_route_given(s, idx.cuda(), counts, offsets, slot, err, ws)
    torch.cuda.synchronize()
    assert int(err.item()) == (m.MOE_DEVERR_EXPERT_RANGE | m.MOE_DEVERR_DUPLICATE)
    flags = ref.validate_given_routing(idx.numpy(), E)
    assert flags[3] & 1 and flags[5] & 1 and flags[7] & 2
    clamped = idx.clamp(0, E - 1).numpy()
    c, o, sr, _ = ref.dispatch(clamped, E)
    assert np.array_equal(host(counts), c) and np.array_equal(host(offsets), o) and np.array_equal(host(slot), sr)
