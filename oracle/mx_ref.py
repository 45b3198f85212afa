"""CPU oracle for MXFP8 block quantisation -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module; the product path never does.

MXFP8 is the reduced-precision format the pages report for the expert
feed-forward compute and for moving data between experts (unite.ai, "Ai2
κυκλοφορεί το Olmo-Core 3…", section "Παραλληλισμός, Ακρίβεια και Τεχνικές
Μνήμης"; ettayeb.fr, "Olmo-core 3 ouvre l'entraînement des MoE…", section
"Trois parallélismes, trois optimisations de routage", where it is described as
storing some values in fewer bits).  The pages give no bit layout; the reading
taken is the OCP microscaling one: blocks of 32 consecutive elements along the
GEMM's reduction axis share one power-of-two scale stored as an E8M0 byte, and
each element is an FP8 E4M3 code.

Definitions written out here:
  E4M3  sign | 4-bit exponent (bias 7) | 3-bit mantissa; exponent field 0 is
        subnormal (m/8 * 2^-6); codes 0x7F and 0xFF are NaN; no infinities;
        largest finite magnitude 1.75 * 2^8 = 448.
  E8M0  byte b encodes 2^(b-127); b = 255 is NaN (never produced here).
  block scale   s = the smallest integer with amax * 2^-s <= 448, clamped to
                [-127, 127]; amax = 0 -> -127.  Computed exactly as
                s0 = floor(log2(amax)) - 8 (8 = exponent of E4M3's largest
                normal), plus one when amax * 2^-s0 > 448.  No element of a block
                saturates, so amax * 2^-s lies in (224, 448].  (The other common
                reading, s0 alone with saturation at 448, clips up to 12.5% off
                the largest element of about a fifth of all blocks.)
  element       code = RNE(v * 2^-s) on the E4M3 grid; the encoder still
                saturates at 448 as a guard.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
BLOCK = 32


def e4m3_decode(codes) -> np.ndarray:
    """Value of every E4M3 code (float64; NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    v = np.where(s == 1, -mag, mag)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def _positive_grid():
    codes = np.arange(0x7F, dtype=np.int64)      # 0x00 .. 0x7E: the finite non-negative codes
    return codes, e4m3_decode(codes)              # ascending in value


def e4m3_encode(v) -> np.ndarray:
    """Round-to-nearest-even onto the E4M3 grid, saturating at +-448.

    Nearest grid point by magnitude; on an exact tie the code with an even
    mantissa (even code) wins.  The sign bit follows the input's sign bit, so
    -0.0 and negative values that round to zero give 0x80.
    """
    x = np.asarray(v, dtype=np.float64)
    assert not np.isnan(x).any()
    codes, grid = _positive_grid()
    mag = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(grid, mag, side="left")          # grid[hi] >= mag
    hi = np.minimum(hi, len(grid) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = mag - grid[lo]
    dhi = grid[hi] - mag
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (codes[hi] % 2 == 0))
    out = np.where(pick_hi, codes[hi], codes[lo])
    out = np.where(grid[hi] == mag, codes[hi], out)        # exact grid hit
    sign = np.signbit(x).astype(np.int64) << 7
    return (out | sign).astype(np.uint8)


def block_scale_exponent(amax) -> np.ndarray:
    """Shared exponent s of a block with largest magnitude amax (exact, via frexp)."""
    a = np.asarray(amax, dtype=np.float64)
    mant, ex = np.frexp(a)                 # a = mant * 2^ex, mant in [0.5, 1)
    fl = ex.astype(np.int64) - 1           # floor(log2 a) for a > 0
    s = fl - 8
    s = s + (a * np.exp2(-s.astype(np.float64)) > E4M3_MAX)   # exact: power-of-two scaling
    s = np.clip(s, -127, 127)
    return np.where(a == 0, -127, s).astype(np.int64)


def quantize_rows(v, block: int = BLOCK):
    """Quantise a [R, K] matrix in blocks of ``block`` consecutive elements along
    each row (the reduction axis when rows are contiguous in K).  A partial last
    block is zero-padded (zeros do not change amax).
    Returns codes uint8 [R, K] and scale bytes uint8 [R, ceil(K / block)]."""
    x = np.asarray(v, dtype=np.float64)
    R, K = x.shape
    nb = -(-K // block)
    pad = np.zeros((R, nb * block))
    pad[:, :K] = x
    blocks = pad.reshape(R, nb, block)
    amax = np.abs(blocks).max(axis=2)
    s = block_scale_exponent(amax)                         # [R, nb]
    scaled = blocks * np.exp2(-s.astype(np.float64))[:, :, None]
    codes = e4m3_encode(scaled).reshape(R, nb * block)[:, :K]
    return codes, (s + 127).astype(np.uint8)


def quantize_segment_cols(v, offsets, block: int = BLOCK):
    """Quantise a [R, K] matrix in blocks of ``block`` consecutive ROWS, restarting
    at every segment start offsets[e] (rows of one expert form one segment; the
    reduction of a weight-gradient GEMM runs over them).  A segment's last block
    is zero-padded.
    Returns codes uint8 [R, K] (in place of the values) and a list, one entry per
    segment, of scale bytes uint8 [ceil(count_e / block), K]."""
    x = np.asarray(v, dtype=np.float64)
    off = np.asarray(offsets).astype(np.int64)
    R, K = x.shape
    codes = np.zeros((R, K), dtype=np.uint8)
    scales = []
    for e in range(len(off) - 1):
        lo, hi = off[e], off[e + 1]
        n = hi - lo
        nb = -(-n // block)
        if n == 0:
            scales.append(np.zeros((0, K), dtype=np.uint8))
            continue
        pad = np.zeros((nb * block, K))
        pad[:n] = x[lo:hi]
        blocks = pad.reshape(nb, block, K)
        amax = np.abs(blocks).max(axis=1)                  # [nb, K]
        s = block_scale_exponent(amax)
        scaled = blocks * np.exp2(-s.astype(np.float64))[:, None, :]
        codes[lo:hi] = e4m3_encode(scaled).reshape(nb * block, K)[:n]
        scales.append((s + 127).astype(np.uint8))
    return codes, scales


def dequantize_rows(codes, scales, block: int = BLOCK) -> np.ndarray:
    c = np.asarray(codes)
    R, K = c.shape
    s = np.asarray(scales).astype(np.float64) - 127.0
    rep = np.repeat(s, block, axis=1)[:, :K]
    return e4m3_decode(c) * np.exp2(rep)


def dequantize_segment_cols(codes, scales, offsets, block: int = BLOCK) -> np.ndarray:
    c = np.asarray(codes)
    off = np.asarray(offsets).astype(np.int64)
    out = np.zeros(c.shape)
    for e in range(len(off) - 1):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        s = np.asarray(scales[e]).astype(np.float64) - 127.0
        rep = np.repeat(s, block, axis=0)[: hi - lo]
        out[lo:hi] = e4m3_decode(c[lo:hi]) * np.exp2(rep)
    return out


# ----------------------------------------------------------------------------- MXFP8 layer
# The expert FFN with MXFP8 GEMMs: every GEMM operand is block-quantised along that
# GEMM's reduction axis (forward: activations and weights along the model / hidden
# width; data gradient: the upstream gradient along its width and the weights along the
# other axis; weight gradient: both operands along the expert's rows), dequantised
# exactly, and multiplied in fp64.  The GEMMs produce bf16 (round to nearest even at each
# stored activation and gradient), and it is those bf16 values that the next GEMM
# quantises: the E4M3 code of a value depends on its bf16 rounding, so the oracle takes
# that decision on the same bf16 values as the device.  Everything else (routing,
# dispatch, gates, combine, SwiGLU and its gradient) is the plain layer of moe_ref.
# quant=False and bf16=False recover the unquantised, unrounded layer exactly.

def bf16_round(v) -> np.ndarray:
    """Round to bfloat16 (nearest, ties to even) through fp32, returned as float64."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    out = u.astype(np.uint32).view(np.float32).astype(np.float64)
    return np.where(nan, np.nan, out)


def _q_rows(v, quant=True):
    if not quant:
        return np.asarray(v, dtype=np.float64)
    c, s = quantize_rows(v)
    return dequantize_rows(c, s)


def _q_cols(v, quant=True):
    """Blocks down the columns of one segment (all rows of v)."""
    if not quant:
        return np.asarray(v, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    c, s = quantize_segment_cols(v, [0, v.shape[0]])
    return dequantize_segment_cols(c, s, [0, v.shape[0]])


def mx_expert_weights(W1e, W3e, W2e, quant=True) -> dict:
    """The dequantised weight operands of one expert for the three GEMMs that read it:
    forward (W1, W3 along d; W2 along f) and data gradient (W2 along d; W1, W3 along f)."""
    W1e, W3e, W2e = (np.asarray(w, dtype=np.float64) for w in (W1e, W3e, W2e))
    return {"W1": _q_rows(W1e, quant), "W3": _q_rows(W3e, quant), "W2": _q_rows(W2e, quant),
            "W2t": _q_cols(W2e, quant),
            "W13t": np.concatenate([_q_cols(W1e, quant), _q_cols(W3e, quant)], axis=0)}


def mx_expert_fwd(X, Wq: dict, quant=True, bf16=True):
    """One expert's rows X [n, d]: a = q(X) q(W1)^T, b likewise (stored bf16),
    h = silu(a) b from the unrounded a, b (stored bf16), y = q(h) q(W2)^T (stored bf16)."""
    from oracle import moe_ref as ref
    rnd = bf16_round if bf16 else (lambda z: z)
    Xq = _q_rows(X, quant)
    a = Xq @ Wq["W1"].T
    b = Xq @ Wq["W3"].T
    h = rnd(ref.silu(a) * b)
    y = rnd(_q_rows(h, quant) @ Wq["W2"].T)
    return rnd(a), rnd(b), h, y


def mx_expert_bwd(dY, X, a, b, h, Wq: dict, quant=True, bf16=True):
    """Backward of mx_expert_fwd for one expert's rows (a, b, h as stored): returns dX,
    dW1, dW3, dW2.  dh = q(dY) q_d(W2); dW2 = q_r(dY)^T q_r(h); [da|db] from dh and the
    stored a, b (stored bf16); dX = q([da|db]) q_f([W1; W3]); [dW1; dW3] =
    q_r([da|db])^T q_r(X)  (q_r: blocks along the expert's rows)."""
    from oracle import moe_ref as ref
    rnd = bf16_round if bf16 else (lambda z: z)
    f = Wq["W1"].shape[0]
    dh = _q_rows(dY, quant) @ Wq["W2t"]
    dW2 = rnd(_q_cols(dY, quant).T @ _q_cols(h, quant))
    s = ref.sigmoid(a)
    dab = rnd(np.concatenate([dh * b * s * (1.0 + a * (1.0 - s)), dh * a * s], axis=1))
    dX = rnd(_q_rows(dab, quant) @ Wq["W13t"])
    dW13 = rnd(_q_cols(dab, quant).T @ _q_cols(X, quant))
    return dX, dW13[:f], dW13[f:], dW2


def mx_layer(x, W1, W3, W2, k, topk_idx, gates, dy, quant=True, bf16=True, shared=None):
    """Whole layer forward + backward with MXFP8 expert GEMMs, for tokens that arrive
    routed (topk_idx, gates given).  Returns a dict like moe_ref's forward/backward.
    shared: (W1s, W3s, W2s) of a shared expert run with the same MXFP8 GEMMs on every
    token; its output (bf16, as stored) joins the combine and its input gradient the
    un-permute sum."""
    from oracle import moe_ref as ref
    rnd = bf16_round if bf16 else (lambda z: z)
    W1, W3, W2 = ref.f64(W1), ref.f64(W3), ref.f64(W2)
    E = W1.shape[0]
    idx = np.asarray(topk_idx).astype(np.int32)
    g = ref.f64(gates)
    counts, offsets, slot_row, row_src = ref.dispatch(idx, E)
    xp = ref.permute(x, row_src)
    R, d = xp.shape
    f = W1.shape[1]
    Wq = [mx_expert_weights(W1[e], W3[e], W2[e], quant) if counts[e] else None for e in range(E)]
    a = np.zeros((R, f)); b = np.zeros((R, f)); h = np.zeros((R, f)); yp = np.zeros((R, d))
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            a[lo:hi], b[lo:hi], h[lo:hi], yp[lo:hi] = mx_expert_fwd(xp[lo:hi], Wq[e], quant, bf16)
    ys = None
    if shared is not None:
        Wq_s = mx_expert_weights(ref.f64(shared[0])[0], ref.f64(shared[1])[0], ref.f64(shared[2])[0], quant)
        xs = ref.f64(x)
        a_s, b_s, h_s, ys = mx_expert_fwd(xs, Wq_s, quant, bf16)
    y = ref.combine(yp, g, slot_row)
    y = rnd(y if ys is None else ys + y)
    dyp, dgates = ref.combine_bwd(dy, yp, g, slot_row)
    dyp = rnd(dyp)
    dxp = np.zeros((R, d)); dW1 = np.zeros_like(W1); dW3 = np.zeros_like(W3); dW2 = np.zeros_like(W2)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            dxp[lo:hi], dW1[e], dW3[e], dW2[e] = mx_expert_bwd(dyp[lo:hi], xp[lo:hi], a[lo:hi], b[lo:hi], h[lo:hi],
                                                               Wq[e], quant, bf16)
    out = {}
    dx_add = None
    if shared is not None:
        dx_s, dW1s, dW3s, dW2s = mx_expert_bwd(bf16_round(ref.f64(dy)) if bf16 else ref.f64(dy), xs, a_s, b_s, h_s,
                                               Wq_s, quant, bf16)
        dx_add = rnd(dx_s)
        out.update(dW1s=dW1s[None], dW3s=dW3s[None], dW2s=dW2s[None], dx_s=dx_add, y_s=ys)
    dx = rnd(ref.unpermute_sum(dxp, slot_row, dx_add))
    out.update(dict(counts=counts, offsets=offsets, slot_row=slot_row, x_perm=xp, a=a, b=b, h=h, y_perm=yp, y=y,
                    dgates=dgates, dx_perm=dxp, dW1=dW1, dW3=dW3, dW2=dW2, dx=dx))
    return out
