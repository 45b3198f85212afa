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
# The expert FFN with MXFP8 GEMMs.  A GEMM in the layer's MXFP8 scope takes both operands
# block-quantised along that GEMM's reduction axis, dequantised exactly and multiplied in
# fp64; a GEMM outside the scope multiplies its operands as stored.  The three kinds of
# expert GEMM differ in where their reduction axis lies:
#   forward        out_e = A_e W_e^T    K = columns of A and of W  (blocks along rows of both)
#   data gradient  out_e = A_e W_e      K = columns of A, rows of W (blocks down W's columns)
#   weight grad.   out_e = A_e^T B_e    K = the expert's rows       (blocks down the columns of
#                                       A_e and B_e, restarting at the expert's first row)
# The GEMMs produce bf16 (round to nearest even at each stored activation and gradient),
# and it is those bf16 values that the next GEMM quantises: the E4M3 code of a value
# depends on its bf16 rounding, so the oracle takes that decision on the same bf16 values
# as the device.  Everything else (routing, dispatch, gates, combine, SwiGLU and its
# gradient) is the plain layer of moe_ref.  quant=False and bf16=False recover the
# unquantised, unrounded layer exactly.
#
# Which GEMMs are in the scope is a reading: the pages put MXFP8 on selected operations,
# where it helped most, with most of the gain in the feed-forward compute and in moving
# data between experts (bigchange.ai, "Olmo-core 3 открывает стек обучения MoE от Ai2…",
# section "Главное изменение"; ettayeb.fr, "Olmo-core 3 ouvre l'entraînement des MoE…",
# section "Trois parallélismes, trois optimisations de routage").  DEFAULT_SCOPE holds
# the two GEMMs that reduce over the hidden width and produce the d-wide rows returned to
# the tokens: GEMM2 (y_perm) and the input-gradient GEMM dgrad1 (dx_perm).  Every output
# and gradient of the layer then passes through at most one quantised GEMM.

# The six expert GEMMs by name.
GEMMS = ("gemm1", "gemm2", "dgrad2", "wgrad2", "dgrad1", "wgrad1")
ALL_GEMMS = frozenset(GEMMS)
DEFAULT_SCOPE = frozenset(("gemm2", "dgrad1"))


def bf16_round(v) -> np.ndarray:
    """Round to bfloat16 (nearest, ties to even) through fp32, returned as float64."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    out = u.astype(np.uint32).view(np.float32).astype(np.float64)
    return np.where(nan, np.nan, out)


def q_along_rows(v, on=True) -> np.ndarray:
    """v dequantised after blocking along each row (32 consecutive columns)."""
    v = np.asarray(v, dtype=np.float64)
    if not on:
        return v
    return dequantize_rows(*quantize_rows(v))


def q_down_cols(v, offsets=None, on=True) -> np.ndarray:
    """v dequantised after blocking down each column (32 consecutive rows), the blocks
    restarting at every offsets[e] (one segment spanning all rows if offsets is None)."""
    v = np.asarray(v, dtype=np.float64)
    if not on:
        return v
    off = [0, v.shape[0]] if offsets is None else offsets
    c, s = quantize_segment_cols(v, off)
    return dequantize_segment_cols(c, s, off)


def _groups(offsets):
    off = np.asarray(offsets).astype(np.int64)
    return [(e, off[e], off[e + 1]) for e in range(len(off) - 1)]


def mx_gemm_fwd(A, W, offsets, on=True) -> np.ndarray:
    """Grouped forward GEMM: out[rows of e] = q(A_e) q(W_e)^T with A [R, K], W [E, N, K];
    K (the columns of both) is the reduction axis."""
    A = np.asarray(A, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    out = np.zeros((A.shape[0], W.shape[1]))
    Aq = q_along_rows(A, on)
    for e, lo, hi in _groups(offsets):
        if hi > lo:
            out[lo:hi] = Aq[lo:hi] @ q_along_rows(W[e], on).T
    return out


def mx_gemm_dgrad(A, W, offsets, on=True) -> np.ndarray:
    """Grouped data-gradient GEMM: out[rows of e] = q(A_e) q(W_e) with A [R, K], W [E, K, N];
    the reduction runs over A's columns and W's rows, so W is blocked down its columns."""
    A = np.asarray(A, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    out = np.zeros((A.shape[0], W.shape[2]))
    Aq = q_along_rows(A, on)
    for e, lo, hi in _groups(offsets):
        if hi > lo:
            out[lo:hi] = Aq[lo:hi] @ q_down_cols(W[e], None, on)
    return out


def mx_gemm_wgrad(A, B, offsets, on=True) -> np.ndarray:
    """Grouped weight-gradient GEMM: out[e] = q(A_e)^T q(B_e) with A [R, M], B [R, N]; the
    reduction runs over the expert's rows, blocked down each column and restarting at
    every offsets[e] so no block mixes two experts.  Experts with no rows get zeros."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    Aq = q_down_cols(A, offsets, on)
    Bq = q_down_cols(B, offsets, on)
    groups = _groups(offsets)
    out = np.zeros((len(groups), A.shape[1], B.shape[1]))
    for e, lo, hi in groups:
        if hi > lo:
            out[e] = Aq[lo:hi].T @ Bq[lo:hi]
    return out


def mx_ffn_fwd(xp, W1, W3, W2, offsets, quant=True, bf16=True, scope=DEFAULT_SCOPE):
    """Grouped SwiGLU FFN on the packed rows xp [R, d]: a = X W1^T, b = X W3^T (GEMM1,
    stored bf16), h = silu(a) b from the unrounded a, b (stored bf16), y_perm = h W2^T
    (GEMM2, stored bf16).  Returns a, b, h, y_perm as stored."""
    from oracle import moe_ref as ref
    rnd = bf16_round if bf16 else (lambda z: z)
    q = lambda name: quant and name in scope  # noqa: E731
    a = mx_gemm_fwd(xp, W1, offsets, q("gemm1"))
    b = mx_gemm_fwd(xp, W3, offsets, q("gemm1"))
    h = rnd(ref.silu(a) * b)
    y = rnd(mx_gemm_fwd(h, W2, offsets, q("gemm2")))
    return rnd(a), rnd(b), h, y


def mx_ffn_bwd(dyp, xp, a, b, h, W1, W3, W2, offsets, quant=True, bf16=True, scope=DEFAULT_SCOPE):
    """Backward of mx_ffn_fwd from the stored a, b, h and the routed gradient dyp [R, d]:
    dh = dY W2 (dgrad2); dW2 = dY^T h (wgrad2); [da | db] from dh and a, b (stored bf16);
    dx_perm = [da | db] [W1; W3] (dgrad1, one reduction over 2f); [dW1; dW3] =
    [da | db]^T X (wgrad1).  Returns dx_perm, dW1, dW3, dW2, dab as stored."""
    from oracle import moe_ref as ref
    rnd = bf16_round if bf16 else (lambda z: z)
    q = lambda name: quant and name in scope  # noqa: E731
    f = np.asarray(W1).shape[1]
    dh = mx_gemm_dgrad(dyp, W2, offsets, q("dgrad2"))
    dW2 = rnd(mx_gemm_wgrad(dyp, h, offsets, q("wgrad2")))
    s = ref.sigmoid(a)
    dab = rnd(np.concatenate([dh * b * s * (1.0 + a * (1.0 - s)), dh * a * s], axis=1))
    W13 = np.concatenate([np.asarray(W1, dtype=np.float64), np.asarray(W3, dtype=np.float64)], axis=1)
    dxp = rnd(mx_gemm_dgrad(dab, W13, offsets, q("dgrad1")))
    dW13 = rnd(mx_gemm_wgrad(dab, xp, offsets, q("wgrad1")))
    return dxp, dW13[:, :f], dW13[:, f:], dW2, dab


def mx_layer(x, W1, W3, W2, k, topk_idx, gates, dy, quant=True, bf16=True, shared=None, scope=DEFAULT_SCOPE):
    """Whole layer forward + backward with the expert GEMMs of `scope` in MXFP8, for tokens
    that arrive routed (topk_idx, gates given).  Returns a dict like moe_ref's
    forward/backward.  shared: (W1s, W3s, W2s) of a shared expert run with the same GEMMs
    on every token (one group of T rows); its output (bf16, as stored) joins the combine
    and its input gradient the un-permute sum."""
    from oracle import moe_ref as ref
    rnd = bf16_round if bf16 else (lambda z: z)
    W1, W3, W2 = ref.f64(W1), ref.f64(W3), ref.f64(W2)
    E = W1.shape[0]
    idx = np.asarray(topk_idx).astype(np.int32)
    g = ref.f64(gates)
    counts, offsets, slot_row, row_src = ref.dispatch(idx, E)
    xp = ref.permute(x, row_src)
    a, b, h, yp = mx_ffn_fwd(xp, W1, W3, W2, offsets, quant, bf16, scope)
    ys = None
    if shared is not None:
        xs = ref.f64(x)
        Ws = [ref.f64(w) for w in shared]
        off_s = [0, xs.shape[0]]
        a_s, b_s, h_s, ys = mx_ffn_fwd(xs, *Ws, off_s, quant, bf16, scope)
    y = ref.combine(yp, g, slot_row)
    y = rnd(y if ys is None else ys + y)
    dyp, dgates = ref.combine_bwd(dy, yp, g, slot_row)
    dyp = rnd(dyp)
    dxp, dW1, dW3, dW2, dab = mx_ffn_bwd(dyp, xp, a, b, h, W1, W3, W2, offsets, quant, bf16, scope)
    out = {}
    dx_add = None
    if shared is not None:
        dys = bf16_round(ref.f64(dy)) if bf16 else ref.f64(dy)
        dx_s, dW1s, dW3s, dW2s, _ = mx_ffn_bwd(dys, xs, a_s, b_s, h_s, *Ws, off_s, quant, bf16, scope)
        dx_add = dx_s
        out.update(dW1s=dW1s, dW3s=dW3s, dW2s=dW2s, dx_s=dx_add, y_s=ys)
    dx = rnd(ref.unpermute_sum(dxp, slot_row, dx_add))
    out.update(dict(counts=counts, offsets=offsets, slot_row=slot_row, x_perm=xp, a=a, b=b, h=h, y_perm=yp, y=y,
                    dgates=dgates, dab=dab, dx_perm=dxp, dW1=dW1, dW3=dW3, dW2=dW2, dx=dx))
    return out
