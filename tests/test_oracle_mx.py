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


def test_mx_layer_on_grid_operands_forward_gemm_exact():
    """Operands already on the MXFP8 grid quantise to themselves: the first forward GEMM
    of the MXFP8 layer then equals the unquantised one exactly."""
    x, W1, W3, W2, dy, idx, g = _mx_case(2)
    # snap x and W1/W3 onto the grid (quantise once); a second quantisation is the identity
    xg = mx.dequantize_rows(*mx.quantize_rows(x))
    W1g = mx.dequantize_rows(*mx.quantize_rows(W1.reshape(-1, 64))).reshape(W1.shape)
    W3g = mx.dequantize_rows(*mx.quantize_rows(W3.reshape(-1, 64))).reshape(W3.shape)
    assert np.array_equal(mx.dequantize_rows(*mx.quantize_rows(xg)), xg)
    Wq = mx.mx_expert_weights(W1g[0], W3g[0], W2[0])
    a_q, b_q, _, _ = mx.mx_expert_fwd(xg[:10], Wq, quant=True, bf16=False)
    assert np.array_equal(a_q, xg[:10] @ W1g[0].T) and np.array_equal(b_q, xg[:10] @ W3g[0].T)


def test_mx_layer_error_is_the_formats():
    """Quantisation changes the layer by a few percent (a 3-bit mantissa), not by more."""
    x, W1, W3, W2, dy, idx, g = _mx_case(3, T=64, d=128, f=128)
    q = mx.mx_layer(x, W1, W3, W2, 2, idx, g, dy, quant=True)
    p = mx.mx_layer(x, W1, W3, W2, 2, idx, g, dy, quant=False, bf16=False)
    for key in ("y", "dx", "dW1", "dW3", "dW2"):
        rel = np.abs(q[key] - p[key]).max() / np.abs(p[key]).max()
        assert 1e-3 < rel < 0.25, (key, rel)


def test_bf16_round_matches_torch():
    import torch
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.standard_normal(5000) * np.exp2(rng.integers(-40, 40, 5000)), [0.0, -0.0, 1.0, 3.0]])
    want = torch.tensor(v, dtype=torch.float64).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(mx.bf16_round(v), want)
