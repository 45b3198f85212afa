"""MXFP8 path on the GPU: quantiser bytes bit-exact against the oracle; each MXFP8
grouped GEMM against fp64 GEMMs of its dequantised operands; the MXFP8 layer with its
default scope (GEMM2 and dgrad1 on E4M3 operands with E8M0 block scales) within 6e-2
normwise of the unquantised fp64 oracle, and every scope (all six GEMMs included) against
the emulated fp64 oracle of the MXFP8 method as a diagnostic."""
import numpy as np
import pytest
import torch

import workloads
from gpu_common import TOL, host, normwise_err, oracle_for, run_layer, say, tol_mx_emulated

pytestmark = pytest.mark.gpu


def _bf16_sample(rows, cols, seed):
    """bf16 values over a wide exponent range: zero rows, bf16 subnormals, huge values,
    negative zeros, and ordinary Gaussians."""
    g = torch.Generator().manual_seed(seed)
    v = torch.randn(rows, cols, generator=g) * torch.exp2(torch.randint(-30, 30, (rows, 1), generator=g).float())
    if rows >= 5:
        v[0] = 0.0
        v[1] = -0.0
        v[2, :8] = torch.tensor([1e-39, -2e-39, 3e-40, 0.0, 5e-41, -1e-38, 2e-38, 1e-45])  # fp32/bf16 subnormals
        v[3] = torch.randn(cols, generator=g) * 1e30
        v[4, ::3] = 0.0
    return v.to(torch.bfloat16)


def test_mx_quantize_rows_bit_exact():
    import mixture_experts_layer_logits_amd as m
    from oracle import mx_ref
    for (rows, cols, seed) in [(1, 32, 1), (77, 96, 2), (256, 2048, 3)]:
        say(f"[gpu] mx quantize rows {rows}x{cols}")
        src = _bf16_sample(rows, cols, seed)
        q = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
        s = torch.empty(rows, cols // 32, dtype=torch.uint8, device="cuda")
        m.moe_mx_quantize(rows, cols, 0, None, 0, src.cuda(), q, s)
        torch.cuda.synchronize()
        codes, scales = mx_ref.quantize_rows(src.float().numpy().astype(np.float64))
        assert np.array_equal(host(q), codes)
        assert np.array_equal(host(s), scales)


def test_mx_quantize_every_bf16_value():
    """Every bf16 value of magnitude <= 448 (zeros, subnormals and both signs included) in
    blocks whose maximum is 448, so the block scale is 2^0 and each code is the element's
    own E4M3 encoding: both quantisers (blocks along rows, and down segment columns) against
    the oracle's encoder, byte for byte."""
    import mixture_experts_layer_logits_amd as m
    from oracle import mx_ref
    pat = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()
    vals = pat[pat.abs() <= 448]                                   # NaN compares false: dropped
    nrow = -(-len(vals) // 31)
    blocks = torch.zeros(nrow * 31)
    blocks[:len(vals)] = vals
    src = torch.cat([torch.full((nrow, 1), 448.0), blocks.view(nrow, 31)], dim=1).to(torch.bfloat16)  # [nrow, 32]
    say(f"[gpu] mx quantize every bf16 value: {len(vals)} values")
    q = torch.empty(nrow, 32, dtype=torch.uint8, device="cuda")
    sc = torch.empty(nrow, 1, dtype=torch.uint8, device="cuda")
    m.moe_mx_quantize(nrow, 32, 0, None, 0, src.cuda(), q, sc)
    # the same blocks as columns of one 32-row segment (columns padded to a multiple of 32)
    ncol = -(-nrow // 32) * 32
    srcT = torch.zeros(32, ncol, dtype=torch.bfloat16)
    srcT[:, :nrow] = src.T
    qT = torch.empty(ncol, 32 + 128, dtype=torch.uint8, device="cuda")
    sT = torch.empty(ncol, (32 + 128) // 32, dtype=torch.uint8, device="cuda")
    m.moe_mx_quantize(32, ncol, 1, torch.tensor([0, 32], dtype=torch.int32).cuda(), 1, srcT.contiguous().cuda(), qT,
                      sT)
    torch.cuda.synchronize()
    ref = mx_ref.e4m3_encode(src.float().numpy().astype(np.float64))
    assert (host(sc) == 127).all()                                  # scale 2^0 everywhere
    assert np.array_equal(host(q), ref)
    assert np.array_equal(host(qT)[:nrow, :32], ref)
    assert (host(sT)[:nrow, 0] == 127).all()


def test_mx_quantize_segment_cols_bit_exact():
    import mixture_experts_layer_logits_amd as m
    from oracle import mx_ref
    for (offsets, cols, seed) in [([0, 5, 5, 45, 200, 333], 96, 4), ([0, 0, 128, 129, 400], 64, 5),
                                  ([0, 300], 32, 6)]:
        offsets = np.asarray(offsets, dtype=np.int32)
        rows, nseg = int(offsets[-1]), len(offsets) - 1
        say(f"[gpu] mx quantize segment cols {offsets.tolist()} x {cols}")
        src = _bf16_sample(rows, cols, seed)
        rows_pad = rows + 128 * nseg
        q = torch.full((cols, rows_pad), 0xAB, dtype=torch.uint8, device="cuda")
        s = torch.full((cols, rows_pad // 32), 0xAB, dtype=torch.uint8, device="cuda")
        m.moe_mx_quantize(rows, cols, 1, torch.from_numpy(offsets).cuda(), nseg, src.cuda(), q, s)
        torch.cuda.synchronize()
        codes, scales = mx_ref.quantize_segment_cols(src.float().numpy().astype(np.float64), offsets)
        gq, gs = host(q), host(s)
        P = 0
        for e in range(nseg):
            lo, hi = offsets[e], offsets[e + 1]
            n = hi - lo
            npad = -(-n // 128) * 128
            assert np.array_equal(gq[:, P:P + n], codes[lo:hi].T)
            assert not gq[:, P + n:P + npad].any()                  # padding rows: zero codes
            nb = -(-n // 32)
            assert np.array_equal(gs[:, P // 32:P // 32 + nb], scales[e].T)
            assert not gs[:, P // 32 + nb:(P + npad) // 32].any()   # all-padding blocks: zero scale byte
            P += npad


MX = workloads.WORKLOADS["e32_k4_t16384_d4096_mxfp8"]          # default scope: GEMM2, dgrad1
MX_ALL = workloads.WORKLOADS["e32_k4_t16384_d4096_mxfp8_all"]  # all six GEMMs, MXFP8 dispatch

MX_CASES = [
    dict(T=256, d=256, f=256, E=8, k=4, name="mx_small"),
    dict(T=300, d=384, f=256, E=32, k=4, name="mx_ragged_e32"),
    dict(T=200, d=256, f=384, E=16, k=2, name="mx_k2"),
    dict(T=260, d=256, f=256, E=8, k=4, shared_f=256, name="mx_shared_expert"),
    # >= 1024 rows per expert: 256 x 256 tiles in two stages for the M-grouped GEMMs
    dict(T=1100, d=256, f=384, E=2, k=2, name="mx_long_segments"),
    dict(T=150, d=256, f=128, E=64, k=2, name="mx_sparse_e64"),    # many tiny and empty experts
]


def _layer_errors(w, inp, L):
    keys = ["h", "y", "dgates", "dx", "dW1", "dW3", "dW2"] + (["dW1s", "dW3s", "dW2s"] if w.shared_f else [])
    plain = oracle_for(w, inp)                         # the unquantised fp64 layer: the gate
    emu = oracle_for(w, inp, emulate_mx=True)          # the emulated MXFP8 method: a diagnostic
    def pick(fb, k):
        fw, bw = fb
        return fw[k] if k in fw else bw[k]
    got = {k: host(getattr(L, k)) for k in keys}
    e_plain = {k: normwise_err(got[k], pick(plain, k)) for k in keys}
    e_emu = {k: normwise_err(got[k], pick(emu, k)) for k in keys}
    print(w.name, "| vs unquantised", {k: f"{v:.2e}" for k, v in e_plain.items()},
          "| vs emulated MXFP8", {k: f"{v:.2e}" for k, v in e_emu.items()})
    return plain, e_plain, e_emu


@pytest.mark.parametrize("over", MX_CASES, ids=[c["name"] for c in MX_CASES])
def test_mxfp8_layer_parity(over):
    """The default-scope MXFP8 layer against the unquantised fp64 oracle at 6e-2."""
    w = workloads.scaled(MX, **over)
    inp = workloads.make_inputs(w)
    say(f"[gpu] mxfp8 layer {w}")
    L = run_layer(w, inp)
    assert not L.mx_dispatch
    (fw, bw), e_plain, e_emu = _layer_errors(w, inp, L)
    assert np.array_equal(host(L.slot_row), fw["slot_row"])
    bad = {k: v for k, v in e_plain.items() if v > TOL["mxfp8"]}
    assert not bad, (w.name, bad)
    bad = {k: v for k, v in e_emu.items() if v > tol_mx_emulated(k)}
    assert not bad, (w.name, "emulated", bad)
    for e in np.nonzero(fw["counts"] == 0)[0]:
        assert not host(L.dW1[e]).any() and not host(L.dW2[e]).any()


@pytest.mark.parametrize("over", MX_CASES[:4], ids=[c["name"] + "_all6" for c in MX_CASES[:4]])
def test_mxfp8_all_six_against_the_emulated_method(over):
    """All six expert GEMMs in MXFP8 with the MXFP8 dispatch: outside the 6e-2 bound (two
    or three quantised GEMMs in series), so checked against the emulated MXFP8 oracle only;
    the unquantised error is printed."""
    w = workloads.scaled(MX_ALL, **over)
    inp = workloads.make_inputs(w)
    say(f"[gpu] mxfp8 layer, all six GEMMs {w}")
    L = run_layer(w, inp)
    assert L.mx_dispatch
    _, e_plain, e_emu = _layer_errors(w, inp, L)
    bad = {k: v for k, v in e_emu.items() if v > tol_mx_emulated(k)}
    assert not bad, (w.name, "emulated", bad)
    assert max(e_plain.values()) < 0.25


def check_mx_layouts(q_rows, s_rows, q_cols, s_cols, vrows, offsets, rows=None, experts=None):
    """The two MXFP8 layouts of a routed row set against the oracle's quantisers, byte for
    byte.  vrows(idx) gives the fp64 rows idx of the set; the row layout is checked on
    `rows` (all rows if None), the column layout on the padded segments of `experts` (all
    if None), padding included (zero codes, zero scale bytes)."""
    from oracle import mx_ref
    offsets = np.asarray(offsets, dtype=np.int64)
    R = int(offsets[-1])
    sel = np.arange(R) if rows is None else np.asarray(rows, dtype=np.int64)
    codes, scales = mx_ref.quantize_rows(vrows(sel))
    idx = torch.from_numpy(sel).cuda()
    assert np.array_equal(host(q_rows[idx]), codes)
    assert np.array_equal(host(s_rows[idx]), scales)
    npad = -(-np.diff(offsets) // 128) * 128
    starts = np.concatenate([[0], np.cumsum(npad)])
    for e in (range(len(offsets) - 1) if experts is None else experts):
        lo, hi, P, n = int(offsets[e]), int(offsets[e + 1]), int(starts[e]), int(offsets[e + 1] - offsets[e])
        if n == 0:
            continue
        gq, gs = host(q_cols[:, P:P + npad[e]]), host(s_cols[:, P // 32:(P + npad[e]) // 32])
        ccodes, cscales = mx_ref.quantize_segment_cols(vrows(np.arange(lo, hi)), [0, n])
        nb = -(-n // 32)
        assert np.array_equal(gq[:, :n], ccodes.T), e
        assert np.array_equal(gs[:, :nb], cscales[0].T), e
        assert not gq[:, n:].any() and not gs[:, nb:].any(), e


def routed_dy_rows(inp, slot_row, row_src, idx):
    """Packed rows idx of bf16(gates[t, j] * dy[t]), the product taken in fp32 and rounded
    once to bf16 (the precision the routed gradient is stored in), in fp64."""
    gate_of_row = np.empty(slot_row.size, dtype=np.float32)
    gate_of_row[slot_row.reshape(-1)] = inp["gates"].numpy().reshape(-1)
    t = torch.from_numpy(row_src[idx].astype(np.int64))
    v = torch.from_numpy(gate_of_row[idx])[:, None] * inp["dy"].float()[t]
    return v.to(torch.bfloat16).float().numpy().astype(np.float64)


MX_DISPATCH_CASES = [
    dict(T=300, d=384, f=256, E=32, k=4, name="mxd_ragged_e32"),
    dict(T=200, d=256, f=128, E=16, k=2, name="mxd_k2"),
    dict(T=150, d=256, f=128, E=64, k=2, name="mxd_sparse_e64"),   # many tiny and empty experts
    dict(T=700, d=128, f=128, E=2, k=2, name="mxd_long_segments"),  # several 128-row tiles per expert
]


@pytest.mark.parametrize("over", MX_DISPATCH_CASES, ids=[c["name"] for c in MX_DISPATCH_CASES])
def test_mx_dispatch_bytes_bit_exact(over):
    """moe_permute_mx and moe_combine_bwd_mx write, for the routed rows of x and of the
    gated output gradient, exactly the E4M3 codes and E8M0 scales the oracle's quantisers
    give for those rows, in both layouts."""
    from oracle import moe_ref as ref
    w = workloads.scaled(MX_ALL, **over)
    inp = workloads.make_inputs(w)
    say(f"[gpu] mxfp8 dispatch bytes {w}")
    L = run_layer(w, inp, mx_dispatch=True)
    counts, offsets, slot_row, row_src = ref.dispatch(inp["topk_idx"].numpy(), w.E)
    assert np.array_equal(host(L.offsets), offsets)
    assert np.array_equal(host(L.row_src), row_src)
    x = inp["x"].float().numpy().astype(np.float64)
    check_mx_layouts(L.xq_rows, L.xs_rows, L.xq_cols, L.xs_cols, lambda i: x[row_src[i]], offsets)
    check_mx_layouts(L.dyq_rows, L.dys_rows, L.dyq_cols, L.dys_cols,
                     lambda i: routed_dy_rows(inp, slot_row, row_src, i), offsets)


@pytest.mark.parametrize("over", MX_CASES[:2] + MX_CASES[3:5], ids=[c["name"] for c in MX_CASES[:2] + MX_CASES[3:5]])
def test_mx_dispatch_equals_bf16_dispatch_bitwise(over):
    """The layer with the MXFP8 dispatch gives bit for bit the outputs of the layer that
    dispatches bf16 rows and quantises them inside each GEMM (the same bytes reach the
    same GEMM kernels; dgates keeps its summation order)."""
    w = workloads.scaled(MX_ALL, **over)
    inp = workloads.make_inputs(w)
    say(f"[gpu] mxfp8 dispatch vs bf16 dispatch {w}")
    A = run_layer(w, inp, mx_dispatch=True)
    B = run_layer(w, inp, mx_dispatch=False)
    names = ["ab", "h", "y_perm", "y", "dgates", "dab", "dx_perm", "dW1", "dW3", "dW2", "dx"]
    if w.shared_f:
        names += ["dW1s", "dW3s", "dW2s"]
    diff = [n for n in names if not torch.equal(getattr(A, n), getattr(B, n))]
    assert not diff, diff


@pytest.mark.parametrize("over,recompute", [(c, False) for c in MX_CASES] + [(MX_CASES[1], True)],
                         ids=[c["name"] for c in MX_CASES] + [MX_CASES[1]["name"] + "_recompute"])
def test_fused_quantisation_bytes_and_layer_bitwise(over, recompute):
    """With the default scope, GEMM1's epilogue writes h and dgrad2's writes [da | db] also as
    MXFP8 row blocks: those bytes equal the oracle's row quantiser applied to the bf16 h and
    [da | db] the same kernels store, and the layer's outputs equal, bit for bit, those of the
    layer whose MXFP8 GEMM2 and dgrad1 quantise their bf16 operands themselves."""
    from oracle import mx_ref
    w = workloads.scaled(MX, **over)
    inp = workloads.make_inputs(w)
    say(f"[gpu] fused MXFP8 quantisation {w} recompute={recompute}")
    A = run_layer(w, inp, recompute=recompute, mx_fused_quant=True)
    assert A.fq_h and A.fq_dab and not A.mx_dispatch
    if not recompute:
        for q, sc, v in ((A.hq_rows, A.hs_rows, A.h), (A.dabq_rows, A.dabs_rows, A.dab)):
            codes, scales = mx_ref.quantize_rows(host(v).astype(np.float64))
            assert np.array_equal(host(q), codes)
            assert np.array_equal(host(sc), scales)
        if w.shared_f:
            for q, sc, v in ((A.hq_s, A.hs_s, A.h_s), (A.dabq_s, A.dabs_s, A.dab_s)):
                codes, scales = mx_ref.quantize_rows(host(v).astype(np.float64))
                assert np.array_equal(host(q), codes) and np.array_equal(host(sc), scales)
    say(f"[gpu] unfused MXFP8 layer {w} recompute={recompute}")
    B = run_layer(w, inp, recompute=recompute, mx_fused_quant=False)
    assert not B.fq_h and not B.fq_dab
    names = ["y_perm", "y", "dgates", "dab", "dx_perm", "dW1", "dW3", "dW2", "dx"]
    if not recompute:
        names += ["ab", "h"]
    if w.shared_f:
        names += ["y_s", "dW1s", "dW3s", "dW2s"]
    diff = [n for n in names if not torch.equal(getattr(A, n), getattr(B, n))]
    assert not diff, diff


def test_mx_gemms_match_dequantized_operands():
    """Each MXFP8 grouped GEMM equals the fp64 GEMM of its dequantised operands (the
    oracle's quantiser is bit-exact with the GPU's), up to fp32 accumulation and the bf16
    rounding of the outputs: a check of the scaled-MFMA operand and scale layouts."""
    from oracle import moe_ref as ref
    from oracle import mx_ref as mx
    w = workloads.scaled(MX_ALL, T=300, d=256, f=384, E=8, k=4, name="mx_emulated")
    inp = workloads.make_inputs(w)
    say(f"[gpu] mxfp8 GEMMs vs dequantised operands {w}")
    L = run_layer(w, inp, mx_dispatch=False)  # keeps bf16 x_perm and dy_perm to quantise here
    off = host(L.offsets).astype(np.int64)
    E, d, f = w.E, w.d, w.f

    def deq_rows(t):
        c, s = mx.quantize_rows(np.asarray(t, dtype=np.float64))
        return mx.dequantize_rows(c, s)

    def deq_cols(t, offsets):
        c, s = mx.quantize_segment_cols(np.asarray(t, dtype=np.float64), offsets)
        return mx.dequantize_segment_cols(c, s, offsets)

    X, H, dY, dAB = host(L.x_perm), host(L.h), host(L.dy_perm), host(L.dab)
    W1 = host(inp["W1"]).reshape(E * f, d)
    W3 = host(inp["W3"]).reshape(E * f, d)
    W2 = host(inp["W2"]).reshape(E * d, f)
    Xq, Hq, dYq, dABq = deq_rows(X), deq_rows(H), deq_rows(dY), deq_rows(dAB)
    W1q, W3q, W2q = deq_rows(W1).reshape(E, f, d), deq_rows(W3).reshape(E, f, d), deq_rows(W2).reshape(E, d, f)
    # backward weights: blocks along the other axis, one segment per expert
    W2t = deq_cols(W2, np.arange(E + 1) * d).reshape(E, d, f)
    W1t = deq_cols(W1, np.arange(E + 1) * f).reshape(E, f, d)
    W3t = deq_cols(W3, np.arange(E + 1) * f).reshape(E, f, d)
    # weight-gradient operands: blocks along the rows of each expert
    dYc, Hc, dABc, Xc = deq_cols(dY, off), deq_cols(H, off), deq_cols(dAB, off), deq_cols(X, off)
    R = w.R
    a = np.zeros((R, f)); b = np.zeros((R, f)); y = np.zeros((R, d)); dh = np.zeros((R, f)); dx = np.zeros((R, d))
    dW1 = np.zeros((E, f, d)); dW3 = np.zeros((E, f, d)); dW2 = np.zeros((E, d, f))
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        a[lo:hi] = Xq[lo:hi] @ W1q[e].T
        b[lo:hi] = Xq[lo:hi] @ W3q[e].T
        y[lo:hi] = Hq[lo:hi] @ W2q[e].T
        dh[lo:hi] = dYq[lo:hi] @ W2t[e]
        dx[lo:hi] = dABq[lo:hi, :f] @ W1t[e] + dABq[lo:hi, f:] @ W3t[e]
        dW2[e] = dYc[lo:hi].T @ Hc[lo:hi]
        dW1[e] = dABc[lo:hi, :f].T @ Xc[lo:hi]
        dW3[e] = dABc[lo:hi, f:].T @ Xc[lo:hi]
    AB = host(L.ab)
    ga, gb = AB[:, :f].astype(np.float64), AB[:, f:].astype(np.float64)
    s_ = ref.sigmoid(ga)
    errs = {
        "a": normwise_err(AB[:, :f], a), "b": normwise_err(AB[:, f:], b),
        "y_perm": normwise_err(host(L.y_perm), y),
        "da": normwise_err(dAB[:, :f], dh * gb * s_ * (1 + ga * (1 - s_))),
        "db": normwise_err(dAB[:, f:], dh * ga * s_),
        "dx_perm": normwise_err(host(L.dx_perm), dx),
        "dW1": normwise_err(host(L.dW1), dW1), "dW3": normwise_err(host(L.dW3), dW3),
        "dW2": normwise_err(host(L.dW2), dW2),
    }
    print({k: f"{v:.2e}" for k, v in errs.items()})
    bad = {k: v for k, v in errs.items() if v > 1e-2}
    assert not bad, bad
