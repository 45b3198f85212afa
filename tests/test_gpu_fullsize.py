"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

The oracle cannot run whole layers of these sizes in seconds, so:
  * routing (top-k ids, counts, offsets, packed rows) is checked in full, bit for bit,
    with the selection taken on the GPU's fp32 scores; the oracle's own fp64 scores are
    also routed in full, and every token they route differently is reported with its
    margin (the gap between the k-th and (k+1)-th fp64 score), which must be a rounding
    difference's size;
  * the dispatch copy is checked bit for bit on sampled packed rows;
  * values are checked on sampled tokens (forward output, input gradient, gate and score
    gradients) and on sampled experts (weight gradients, which sum over all of an
    expert's rows), each recomputed by the oracle from that token's or expert's inputs;
  * the gate gradient of the scores (dlogits) and the router weight gradient are checked in
    full against the oracle's fp64 route and router backward applied to the GPU's dgates
    (which are checked against the oracle on the sampled tokens).
Tolerance: 2e-2 normwise against the fp64 oracle for bf16, 6e-2 for the MXFP8 layer (its
default scope), both against the unquantised layer, as for the small cases.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_common import TOL, host, normwise_err, run_layer, say

pytestmark = pytest.mark.gpu

FULL = [("e8_k4_t8192", False), ("e128_k4_t8192", False), ("e128_k4_t8192", True), ("e128_k4_t8192_shared", False),
        ("e128_k4_t16384_zipf", False), ("e128_k4_t16384_zipf_steep", False), ("e128_k4_t16384_random", False),
        ("e32_k4_t16384_d4096_bf16", False), ("e32_k4_t16384_d4096_mxfp8", False)]


def _f64(t):
    return np.asarray(t.float().numpy() if t.dtype == torch.bfloat16 else t.numpy(), dtype=np.float64)


def _ffn_fwd(inp, X, e):
    from oracle import moe_ref as ref
    return ref.expert_ffn_fwd(X, [0, len(X)], inp["W1"][e:e + 1], inp["W3"][e:e + 1], inp["W2"][e:e + 1])


def _ffn_bwd(inp, dY, X, a, b, h, e):
    """(dX, dW1_e, dW3_e, dW2_e) of one expert's rows."""
    from oracle import moe_ref as ref
    dx, dW1, dW3, dW2, _, _ = ref.expert_ffn_bwd(dY, X, a, b, [0, len(X)], inp["W1"][e:e + 1], inp["W3"][e:e + 1],
                                                 inp["W2"][e:e + 1])
    return dx, dW1[0], dW3[0], dW2[0]


def _token_reference(inp, w, t, idx_t, learned):
    """Forward and backward of one token through its chosen experts (oracle primitives,
    fp64, unquantised)."""
    from oracle import moe_ref as ref
    x = _f64(inp["x"][t:t + 1])
    dy = _f64(inp["dy"][t:t + 1])
    ys, rows = [], []
    for e in idx_t:
        a, b, h, y = _ffn_fwd(inp, x, e)
        ys.append(y[0])
        rows.append((a, b, h))
    if learned:
        L = ref.router_logits(x, inp["Wr"], inp["router_bias"])[0]
        sel = L[np.asarray(idx_t)]
        g = np.exp(sel - sel.max())
        g = g / g.sum()
    else:
        g = _f64(inp["gates"][t])
    y = sum(g[j] * ys[j] for j in range(len(idx_t)))
    dg = np.array([float(dy[0] @ ys[j]) for j in range(len(idx_t))])
    dx = np.zeros(w.d)
    if inp.get("shared") is not None:  # the shared expert sees every token
        sh = [_f64(u) for u in inp["shared"]]
        a_s, b_s, h_s, y_s = ref.shared_expert_fwd(x, *sh)
        y = y + y_s[0]
        dx += ref.expert_ffn_bwd(dy, x, a_s, b_s, [0, 1], *sh)[0][0]
    for j, e in enumerate(idx_t):
        a, b, h = rows[j]
        dxp, *_ = _ffn_bwd(inp, g[j] * dy, x, a, b, h, e)
        dx += dxp[0]
    out = {"y": y, "dgates": dg}
    if learned:
        dL = ref.route_bwd(dg[None], g[None], np.asarray(idx_t)[None], w.E)[0]
        out["dlogits"] = dL
        dx += dL @ _f64(inp["Wr"])
    out["dx"] = dx
    return out


def _expert_reference(inp, w, e, idx, gates_f64):
    """Weight gradients of expert e from all of its routed rows (oracle primitives)."""
    from oracle import moe_ref as ref
    tt, jj = np.nonzero(idx == e)
    if len(tt) == 0:
        z = np.zeros
        return z((w.f, w.d)), z((w.f, w.d)), z((w.d, w.f))
    X = _f64(inp["x"][torch.from_numpy(tt)])
    dY = gates_f64[tt, jj][:, None] * _f64(inp["dy"][torch.from_numpy(tt)])
    a, b, h, y = _ffn_fwd(inp, X, e)
    _, dW1, dW3, dW2 = _ffn_bwd(inp, dY, X, a, b, h, e)
    return dW1, dW3, dW2


def fp64_routing_disagreements(inp, w, gpu_idx):
    """Tokens whose top-k set under the oracle's own fp64 scores differs from the GPU's
    (selected on fp32 scores), with each one's fp64 margin between the k-th and (k+1)-th
    score: (count, margins)."""
    from oracle import moe_ref as ref
    L64 = ref.router_logits(inp["x"], inp["Wr"], inp["router_bias"])
    idx64, _ = ref.topk_gates(L64, w.k)
    differ = np.nonzero((np.sort(idx64, axis=1) != np.sort(gpu_idx, axis=1)).any(axis=1))[0]
    srt = -np.sort(-L64[differ], axis=1)
    margins = srt[:, w.k - 1] - srt[:, w.k] if w.k < w.E else np.zeros(len(differ))
    return len(differ), margins


@pytest.mark.parametrize("name,recompute", FULL, ids=[n + ("_recompute" if r else "") for n, r in FULL])
def test_full_size_layer(name, recompute):
    from oracle import moe_ref as ref
    w = workloads.WORKLOADS[name]
    inp = workloads.make_inputs(w)
    learned = w.routing != "given_uniform"
    say(f"[gpu] full-size layer {w} recompute={recompute}")
    L = run_layer(w, inp, recompute=recompute)
    tol = TOL[w.gemm]
    rng = np.random.default_rng(7)

    # routing in full, bit for bit (selection on the GPU's fp32 scores)
    if learned:
        gl = host(L.logits)
        idx, _ = ref.topk_gates(gl, w.k)
        assert np.array_equal(host(L.topk_idx), idx)
        n_diff, margins = fp64_routing_disagreements(inp, w, idx)
        print(f"{name}: fp64 scores route {n_diff} of {w.T} tokens differently; margins "
              f"{np.array2string(margins, precision=2)}")
        # fp32 accumulation of |x||Wr| ~ sqrt(d) terms: a flip needs a margin of a few ulps
        assert n_diff <= max(1, w.T // 1000) and (margins < 1e-5).all()
    else:
        idx = inp["topk_idx"].numpy()
    counts, offsets, slot_row, row_src = ref.dispatch(idx, w.E)
    assert np.array_equal(host(L.counts), counts)
    assert np.array_equal(host(L.offsets), offsets)
    assert np.array_equal(host(L.slot_row), slot_row)
    assert np.array_equal(host(L.row_src), row_src)
    rows = rng.choice(w.R, 64, replace=False)
    if L.mx_dispatch:  # the routed rows exist only as E4M3 codes: sampled rows, two experts' column segments
        from test_gpu_mxfp8 import check_mx_layouts, routed_dy_rows
        order = np.argsort(counts, kind="stable")
        keep = sorted({int(order[len(order) // 2]), int(order[0])})
        say("  [oracle] quantising sampled dispatched rows and two experts' column segments")
        check_mx_layouts(L.xq_rows, L.xs_rows, L.xq_cols, L.xs_cols,
                         lambda i: _f64(inp["x"][torch.from_numpy(row_src[i]).long()]), offsets, rows, keep)
        check_mx_layouts(L.dyq_rows, L.dys_rows, L.dyq_cols, L.dys_cols,
                         lambda i: routed_dy_rows(inp, slot_row, row_src, i), offsets, rows, keep)
    else:
        assert torch.equal(L.x_perm[torch.from_numpy(rows).cuda()].cpu(),
                           inp["x"][torch.from_numpy(row_src[rows]).long()])
    # MXFP8 rows written by the bf16 producer GEMMs' epilogues: on sampled rows, the oracle's
    # row quantiser applied to the bf16 values the same kernels stored, byte for byte
    from oracle import mx_ref
    sel = torch.from_numpy(rows).cuda()
    for on, q, sc, v in ((L.fq_h, L.hq_rows, L.hs_rows, L.h), (L.fq_dab, L.dabq_rows, L.dabs_rows, L.dab)):
        if on:
            codes, scales = mx_ref.quantize_rows(host(v[sel]).astype(np.float64))
            assert np.array_equal(host(q[sel]), codes) and np.array_equal(host(sc[sel]), scales)

    # sampled tokens: forward output and gradients
    toks = rng.choice(w.T, 8 if w.d >= 4096 else 24, replace=False)
    got = {"y": host(L.y[toks]), "dx": host(L.dx[toks]), "dgates": host(L.dgates[toks])}
    if learned:
        got["dlogits"] = host(L.dlogits[toks])
        L64 = ref.router_logits(inp["x"][toks], inp["Wr"], inp["router_bias"])
        got_logits = host(L.logits[toks])
        assert normwise_err(got_logits, L64) < 1e-5
    refs = {k: [] for k in got}
    for t in toks:
        r = _token_reference(inp, w, int(t), idx[t], learned)
        for k in got:
            refs[k].append(r[k])
    errs = {k: normwise_err(got[k], np.stack(refs[k])) for k in got}

    # sampled experts: weight gradients (a median-load and the lightest expert)
    if learned:
        g_sel = np.take_along_axis(ref.router_logits(inp["x"], inp["Wr"], inp["router_bias"]), idx.astype(np.int64), 1)
        gw = np.exp(g_sel - g_sel[:, :1])
        gates64 = gw / gw.sum(axis=1, keepdims=True)
    else:
        gates64 = _f64(inp["gates"])
    order = np.argsort(counts, kind="stable")
    for e in {int(order[len(order) // 2]), int(order[0])}:
        dW1, dW3, dW2 = _expert_reference(inp, w, e, idx, gates64)
        errs[f"dW1[{e}]"] = normwise_err(host(L.dW1[e]), dW1)
        errs[f"dW3[{e}]"] = normwise_err(host(L.dW3[e]), dW3)
        errs[f"dW2[{e}]"] = normwise_err(host(L.dW2[e]), dW2)
    if learned:
        # the oracle's gate gradient (fp64, its own gates) from the GPU's dgates, which are
        # checked against the oracle on the sampled tokens above, then the oracle's router
        # backward over every token
        dL64 = ref.route_bwd(host(L.dgates), gates64, idx, w.E)
        errs["dlogits_all"] = normwise_err(host(L.dlogits), dL64)
        errs["dWr"] = normwise_err(host(L.dWr), ref.router_bwd(inp["x"], inp["Wr"], dL64)[1])
    if inp.get("shared") is not None:  # shared expert weight gradients over all T tokens
        sh = [_f64(u) for u in inp["shared"]]
        X = _f64(inp["x"])
        a_s, b_s, _, _ = ref.shared_expert_fwd(X, *sh)
        _, dW1s, dW3s, dW2s, _, _ = ref.expert_ffn_bwd(_f64(inp["dy"]), X, a_s, b_s, [0, w.T], *sh)
        errs["dW1s"] = normwise_err(host(L.dW1s), dW1s)
        errs["dW3s"] = normwise_err(host(L.dW3s), dW3s)
        errs["dW2s"] = normwise_err(host(L.dW2s), dW2s)
    print(name, {k: f"{v:.2e}" for k, v in errs.items()})
    bad = {k: v for k, v in errs.items() if v > tol}
    assert not bad, (name, bad)

    # experts that receive no rows get exactly zero weight gradients
    for e in np.nonzero(counts == 0)[0]:
        assert not host(L.dW1[e]).any() and not host(L.dW3[e]).any() and not host(L.dW2[e]).any()
    if name == "e128_k4_t16384_zipf_steep":
        assert (counts == 0).sum() >= 1

    # bitwise reproducible at full size
    y0, dx0, dW10 = L.y.clone(), L.dx.clone(), L.dW1.clone()
    run_layer(w, inp, layer=L)
    assert torch.equal(y0, L.y) and torch.equal(dx0, L.dx) and torch.equal(dW10, L.dW1)
