"""Pins for the MXFP8 quantisation oracle (no GPU).

The E4M3 table is checked against torch's float8_e4m3fn dtype (an independent
library definition of the same format), the rounding against torch's cast and
against hand-derived cases under tests/golden/, and the block quantiser
against the error bound that follows from a 3-bit mantissa.
"""
import os

import numpy as np
import pytest
import torch

from oracle import mx_ref as mx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_rne_cases.txt")


def test_decode_table_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    t = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    o = mx.e4m3_decode(np.arange(256))
    assert np.array_equal(np.isnan(t), np.isnan(o))
    ok = ~np.isnan(t)
    assert np.array_equal(t[ok], o[ok])
    assert np.nanmax(o) == 448.0 and o[1] == 2.0 ** -9 and np.isnan(o[0x7F]) and np.isnan(o[0xFF])


def test_encode_matches_torch_rne_inside_range():
    rng = np.random.default_rng(5)
    grid = mx.e4m3_decode(np.arange(0x7F))
    mids = (grid[1:] + grid[:-1]) / 2                     # every exact halfway point
    v = np.concatenate([rng.uniform(-448, 448, 20000), rng.uniform(-1, 1, 20000) * 2.0 ** -6,
                        mids, -mids, grid, -grid])
    v32 = v.astype(np.float32)
    want = torch.tensor(v32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = mx.e4m3_encode(v32.astype(np.float64))
    assert np.array_equal(got, want)


def test_encode_golden_cases():
    rows = [ln.split() for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    vals = np.array([float(r[0]) for r in rows])
    want = np.array([int(r[1], 16) for r in rows], dtype=np.uint8)
    assert np.array_equal(mx.e4m3_encode(vals), want)


def test_grid_roundtrip():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    assert np.array_equal(mx.e4m3_encode(mx.e4m3_decode(codes)), codes.astype(np.uint8))


@pytest.mark.parametrize("K", [32, 96, 70])
def test_quantize_rows_bounds(K):
    rng = np.random.default_rng(K)
    v = rng.standard_normal((64, K)) * np.exp2(rng.integers(-20, 20, size=(64, 1)))
    v[3] = 0.0                                   # an all-zero row: scale byte 0, codes 0
    v[5, :7] = 0.0
    codes, scales = mx.quantize_rows(v)
    assert scales.shape == (64, -(-K // 32))
    assert (scales[3] == 0).all() and (codes[3] == 0).all()
    s = scales.astype(np.int64) - 127
    for r in range(64):
        for b in range(scales.shape[1]):
            blk = v[r, 32 * b: 32 * b + 32]
            amax = np.abs(blk).max()
            if amax == 0:
                continue
            scaled_max = amax * 2.0 ** -s[r, b]
            assert 224 < scaled_max <= 448                    # smallest scale with no saturation
    deq = mx.dequantize_rows(codes, scales)
    rep = np.repeat(s, 32, axis=1)[:, :K].astype(np.float64)
    sv = v * np.exp2(-rep)                                    # value in units of the block scale
    normal = (np.abs(sv) >= 2.0 ** -6) & (np.abs(sv) <= 448)
    ulp = np.exp2(np.floor(np.log2(np.where(normal, np.abs(v), 1.0))) - 3)
    assert (np.abs(deq - v)[normal] <= 0.5 * ulp[normal]).all()    # RNE: half a 3-bit-mantissa ulp
    sub = np.abs(sv) < 2.0 ** -6
    assert (np.abs(deq - v)[sub] <= 2.0 ** -10 * np.exp2(rep)[sub]).all()
    assert not (np.abs(sv) > 448).any()                     # nothing saturates


def test_segment_cols_equals_rows_of_transposed_segments():
    rng = np.random.default_rng(9)
    offsets = np.array([0, 5, 5, 45, 110, 111])
    v = rng.standard_normal((111, 40))
    codes, scales = mx.quantize_segment_cols(v, offsets)
    for e in range(5):
        lo, hi = offsets[e], offsets[e + 1]
        if hi == lo:
            assert scales[e].shape == (0, 40)
            continue
        c2, s2 = mx.quantize_rows(v[lo:hi].T)          # blocks along the segment's rows
        assert np.array_equal(codes[lo:hi], c2.T) and np.array_equal(scales[e], s2.T)
    deq = mx.dequantize_segment_cols(codes, scales, offsets)
    assert np.abs(deq - v).max() <= np.abs(v).max() * 2.0 ** -4   # half-ulp of a 3-bit mantissa


def _mx_case(seed, T=40, d=64, f=96, E=4, k=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    W1 = rng.standard_normal((E, f, d)) * 0.3
    W3 = rng.standard_normal((E, f, d)) * 0.3
    W2 = rng.standard_normal((E, d, f)) * 0.3
    dy = rng.standard_normal((T, d))
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    g = rng.dirichlet(np.ones(k), size=T)
    return x, W1, W3, W2, dy, idx, g


def test_mx_layer_without_quantisation_is_the_plain_layer():
    from oracle import moe_ref as ref
    x, W1, W3, W2, dy, idx, g = _mx_case(1)
    out = mx.mx_layer(x, W1, W3, W2, 2, idx, g, dy, quant=False, bf16=False)
    fw = ref.layer_forward(x, W1, W3, W2, 2, topk_idx=idx, gates=g)
    bw = ref.layer_backward(fw, dy, x, W1, W3, W2, learned=False)
    for key, want in [("y", fw["y"]), ("dx", bw["dx"]), ("dW1", bw["dW1"]), ("dW3", bw["dW3"]),
                      ("dW2", bw["dW2"]), ("dgates", bw["dgates"])]:
        assert np.allclose(out[key], want, rtol=1e-12, atol=1e-12), key


# ------------------------------------------------------------------ per-GEMM quantisation axes
# Operands snapped onto the MXFP8 grid along one GEMM's reduction axis quantise to
# themselves, so that GEMM must return the exact fp64 product.  Each operand also spans a
# range of 2^+-12 across the other axis, so blocking it along the wrong axis pushes the
# small entries of a block into E4M3's subnormal range, moves them off the grid and
# changes the product; every test checks that the wrong axis does change it.

def _wide(rng, shape, axis):
    """Gaussian entries, each slice along `axis` scaled by its own power of two in 2^[-12, 12]."""
    v = rng.standard_normal(shape)
    sc_shape = [1] * len(shape)
    sc_shape[axis] = shape[axis]
    return v * np.exp2(rng.integers(-12, 13, size=sc_shape).astype(np.float64))


def test_gemm_fwd_blocks_along_the_shared_width():
    rng = np.random.default_rng(31)
    off = [0, 40, 40, 97]                              # three experts, one empty, ragged
    K, N = 96, 64
    A = mx.q_along_rows(_wide(rng, (97, K), 0))        # rows of A: 2^+-12 apart
    W = np.stack([mx.q_along_rows(_wide(rng, (N, K), 0)) for _ in range(3)])
    exact = np.zeros((97, N))
    for e in range(3):
        exact[off[e]:off[e + 1]] = A[off[e]:off[e + 1]] @ W[e].T
    assert np.array_equal(mx.mx_gemm_fwd(A, W, off), exact)
    wrong = mx.q_down_cols(A[:40]) @ mx.q_down_cols(W[0]).T
    assert not np.array_equal(wrong, exact[:40])


def test_gemm_dgrad_blocks_weights_down_their_columns():
    rng = np.random.default_rng(32)
    off = [0, 33, 90]
    K, N = 128, 64
    A = mx.q_along_rows(_wide(rng, (90, K), 0))
    W = np.stack([mx.q_down_cols(_wide(rng, (K, N), 1)) for _ in range(2)])   # [E, K, N]
    exact = np.zeros((90, N))
    for e in range(2):
        exact[off[e]:off[e + 1]] = A[off[e]:off[e + 1]] @ W[e]
    assert np.array_equal(mx.mx_gemm_dgrad(A, W, off), exact)
    wrong = A[:33] @ mx.q_along_rows(W[0])              # weights blocked along their rows
    assert not np.array_equal(wrong, exact[:33])
    assert np.array_equal(mx.q_down_cols(W[0]), W[0])
    assert not np.array_equal(mx.q_along_rows(W[0]), W[0])


def test_gemm_wgrad_blocks_down_each_experts_rows():
    """Blocks of 32 rows restart at every expert: experts of 45, 0, 70 and 13 rows whose
    magnitudes differ by 2^20 are each on the grid in their own blocks; blocking the packed
    rows across the expert boundaries (or along the columns) changes dW."""
    rng = np.random.default_rng(33)
    counts = [45, 0, 70, 13]
    off = np.concatenate([[0], np.cumsum(counts)])
    R, M, N = int(off[-1]), 64, 96
    mag = np.exp2(np.array([10.0, 0.0, -10.0, 6.0]))
    A = np.zeros((R, M)); B = np.zeros((R, N))
    for e in range(4):
        lo, hi = off[e], off[e + 1]
        A[lo:hi] = _wide(rng, (hi - lo, M), 1) * mag[e]
        B[lo:hi] = _wide(rng, (hi - lo, N), 1) / mag[e]
    A = mx.q_down_cols(A, off)
    B = mx.q_down_cols(B, off)
    exact = np.zeros((4, M, N))
    for e in range(4):
        exact[e] = A[off[e]:off[e + 1]].T @ B[off[e]:off[e + 1]]
    got = mx.mx_gemm_wgrad(A, B, off)
    assert np.array_equal(got, exact)
    assert not got[1].any()                                     # the empty expert
    # the same operands blocked as one segment over all packed rows: the blocks that
    # straddle an expert boundary take the larger expert's scale
    A1, B1 = mx.q_down_cols(A), mx.q_down_cols(B)
    across = [A1[off[e]:off[e + 1]].T @ B1[off[e]:off[e + 1]] for e in range(4)]
    assert not all(np.array_equal(across[e], exact[e]) for e in range(4))
    wrong = mx.q_along_rows(A[:45]).T @ mx.q_along_rows(B[:45])
    assert not np.array_equal(wrong, exact[0])


# ------------------------------------------------------------------ the layer's MXFP8 scope
# Which outputs each GEMM reaches: a quantised GEMM may change exactly these, and must
# leave every other output bit-identical with the layer that quantises nothing.
_REACH = {
    "gemm1": {"a", "b", "h", "y_perm", "y", "dgates", "dab", "dx_perm", "dx", "dW1", "dW3", "dW2"},
    "gemm2": {"y_perm", "y", "dgates"},
    "dgrad2": {"dab", "dx_perm", "dx", "dW1", "dW3"},
    "wgrad2": {"dW2"},
    "dgrad1": {"dx_perm", "dx"},
    "wgrad1": {"dW1", "dW3"},
}


@pytest.mark.parametrize("gemm", mx.GEMMS)
def test_scope_reaches_only_the_gemms_outputs(gemm):
    x, W1, W3, W2, dy, idx, g = _mx_case(4, T=48, d=64, f=64, E=4, k=2)
    base = mx.mx_layer(x, W1, W3, W2, 2, idx, g, dy, scope=frozenset())
    one = mx.mx_layer(x, W1, W3, W2, 2, idx, g, dy, scope=frozenset([gemm]))
    keys = set(_REACH["gemm1"])
    changed = {k for k in keys if not np.array_equal(one[k], base[k])}
    assert changed == _REACH[gemm], (gemm, changed ^ _REACH[gemm])


def test_default_scope_passes_each_output_through_one_quantised_gemm():
    reach = [_REACH[gm] for gm in mx.DEFAULT_SCOPE]
    for i, r in enumerate(reach):
        for r2 in reach[i + 1:]:
            assert not (r & r2)


@pytest.mark.parametrize("scope", [frozenset(), mx.DEFAULT_SCOPE, mx.ALL_GEMMS], ids=["none", "default", "all"])
def test_stored_tensors_are_bf16(scope):
    """Every activation and gradient the device stores in bf16 is a bf16 value in the
    oracle too (the next GEMM quantises exactly those values)."""
    x, W1, W3, W2, dy, idx, g = _mx_case(5, T=40, d=64, f=64, E=4, k=2)
    out = mx.mx_layer(x, W1, W3, W2, 2, idx, g, dy, scope=scope)
    for key in ("a", "b", "h", "y_perm", "y", "dab", "dx_perm", "dx", "dW1", "dW3", "dW2"):
        assert np.array_equal(mx.bf16_round(out[key]), out[key]), key
        assert np.abs(out[key]).max() > 0, key


def test_mx_layer_error_is_the_formats():
    """A quantised GEMM changes what it reaches by a few percent (a 3-bit mantissa): more
    than bf16 rounding alone, far less than the values themselves."""
    x, W1, W3, W2, dy, idx, g = _mx_case(3, T=64, d=128, f=128)
    p = mx.mx_layer(x, W1, W3, W2, 2, idx, g, dy, quant=False, bf16=False)
    for scope in (mx.DEFAULT_SCOPE, mx.ALL_GEMMS):
        q = mx.mx_layer(x, W1, W3, W2, 2, idx, g, dy, scope=scope)
        reached = set().union(*(_REACH[gm] for gm in scope))
        for key in ("y", "dx", "dW1", "dW3", "dW2"):
            rel = np.abs(q[key] - p[key]).max() / np.abs(p[key]).max()
            if key in reached:
                assert 1e-2 < rel < 0.25, (key, rel)
            else:
                assert rel < 1e-2, (key, rel)


def test_bf16_round_matches_torch():
    import torch
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.standard_normal(5000) * np.exp2(rng.integers(-40, 40, 5000)), [0.0, -0.0, 1.0, 3.0]])
    want = torch.tensor(v, dtype=torch.float64).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(mx.bf16_round(v), want)
