"""CPU oracle for the MoE expert layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library and its
Python binding) never imports, links or calls it, and this module imports
nothing from the product path.

What it computes: one MoE expert layer, forward and backward, written out as
its plain definition in NumPy float64:

  router      L = x Wr^T (+ bias)                       [T, E]
  top-k       S_t = the k largest L[t, :], ties -> lower expert index
  gates       g[t, j] = softmax over the k selected logits
  dispatch    stable counting sort of the T*k routed slots by expert
  permute     x_perm[slot_row[t, j]] = x[t]
  experts     a = X_e W1_e^T, b = X_e W3_e^T, h = silu(a) * b, y_e = h W2_e^T
  combine     y[t] = sum_j g[t, j] y_perm[slot_row[t, j]]

Passages followed (the pages describe the structure, not the formulas):
  * routing into per-expert input buffers, metadata kept on the GPU, grouped
    GEMM over many small expert computations: unite.ai, "Ai2 κυκλοφορεί το
    Olmo-Core 3…", section "Παραλληλισμός, Ακρίβεια και Τεχνικές Μνήμης";
    ettayeb.fr, "Olmo-core 3 ouvre l'entraînement des MoE…", section
    "Trois parallélismes, trois optimisations de routage".
  * E experts with k (= 4) chosen per token, expert pool 8 vs 128: unite.ai,
    opening section; ettayeb.fr, section "Le problème que les MoE n'ont jamais
    tout à fait résolu"; bigchange.ai, section "Три числа, три знаменателя".
  * random routing as a measured mode: bigchange.ai, section "Три числа, три
    знаменателя"; unite.ai, section "Δοκιμές τρισεκατομμυρίων παραμέτρων".
The gate function (softmax renormalised over the chosen k), the SwiGLU expert
form, the tie rule and the row order inside an expert buffer are not on the
pages; the readings taken are the plainest ones and are listed in the design
notes.  Weights are stored [out, in] per expert: W1, W3 [E, f, d], W2 [E, d, f],
Wr [E, d].

Every array argument may be any real dtype; it is widened to float64 first.
bf16 and fp32 inputs widen exactly.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "f64", "router_logits", "topk_gates", "dispatch", "validate_given_routing",
    "permute", "expert_ffn_fwd", "combine", "combine_bwd", "expert_ffn_bwd",
    "route_bwd", "router_bwd", "unpermute_sum", "sigmoid", "silu",
    "layer_forward", "layer_backward",
]


def f64(a) -> np.ndarray:
    """Widen to a float64 ndarray (exact for fp32/bf16 sources)."""
    if hasattr(a, "detach"):  # torch tensor: go through fp32, which holds bf16 exactly
        import torch
        a = a.detach().cpu()
        if a.dtype in (torch.bfloat16, torch.float16):
            a = a.to(torch.float32)
        a = a.numpy()
    return np.asarray(a, dtype=np.float64)


def sigmoid(z: np.ndarray) -> np.ndarray:
    # 1 / (1 + e^-z), written through tanh so it cannot overflow
    return 0.5 * (1.0 + np.tanh(0.5 * z))


def silu(z: np.ndarray) -> np.ndarray:
    return z * sigmoid(z)


# ----------------------------------------------------------------------------- router
def router_logits(x, Wr, bias=None) -> np.ndarray:
    """Router scores L[t, e] = <x[t], Wr[e]> (+ bias[e]).  Router of the
    learned-routing rows (bigchange.ai, section "Что инженер может попробовать
    на практике": learned routing for the small scripts)."""
    L = f64(x) @ f64(Wr).T
    if bias is not None:
        L = L + f64(bias)[None, :]
    return L


def topk_gates(logits, k: int):
    """Top-k expert choice and gate weights per token.

    Selection: the k largest scores, ordered by value descending, equal values
    broken toward the lower expert index (a stable sort on -score).  Gates:
    softmax over the k selected scores, i.e. the softmax over all E renormalised
    over the chosen k.  Returns (topk_idx int32 [T, k], gates float64 [T, k]).
    """
    L = f64(logits)
    T, E = L.shape
    assert 1 <= k <= E
    # -0.0 and +0.0 compare equal, so they tie and fall back to index order
    order = np.argsort(-L, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(L, order, axis=1)
    m = sel[:, :1]
    w = np.exp(sel - m)
    gates = w / w.sum(axis=1, keepdims=True)
    return order.astype(np.int32), gates


# ----------------------------------------------------------------------------- dispatch
def dispatch(topk_idx, E: int):
    """Routing metadata for writing routed rows into per-expert buffers.

    The T*k routed slots s = t*k + j are counting-sorted by expert, stably, so
    inside an expert's buffer the rows keep ascending slot order.
      counts[e]        rows routed to expert e
      offsets[e]       start of expert e's buffer; offsets[E] = T*k
      slot_row[t, j]   row of the packed buffer that slot (t, j) occupies
      row_src[r]       source token of packed row r
    """
    idx = np.asarray(topk_idx).astype(np.int64)
    T, k = idx.shape
    flat = idx.reshape(-1)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(flat, kind="stable")          # packed row -> slot
    slot_row = np.empty(T * k, dtype=np.int32)
    slot_row[order] = np.arange(T * k, dtype=np.int32)
    row_src = (order // k).astype(np.int32)
    return counts, offsets, slot_row.reshape(T, k), row_src


def validate_given_routing(topk_idx, E: int) -> np.ndarray:
    """Per-token flags for pre-routed input: bit 0 = an expert id outside
    [0, E), bit 1 = the same expert chosen twice for one token."""
    idx = np.asarray(topk_idx).astype(np.int64)
    T, k = idx.shape
    flags = np.zeros(T, dtype=np.int32)
    oob = (idx < 0) | (idx >= E)
    flags |= oob.any(axis=1).astype(np.int32)
    for t in range(T):
        row = idx[t]
        if len(set(row.tolist())) != k:
            flags[t] |= 2
    return flags


def permute(x, row_src) -> np.ndarray:
    """x_perm[r] = x[row_src[r]] (rows written straight into expert buffers)."""
    return f64(x)[np.asarray(row_src)]


# ----------------------------------------------------------------------------- experts
def expert_ffn_fwd(x_perm, offsets, W1, W3, W2):
    """Grouped SwiGLU expert FFN over the packed per-expert buffers.

    For each expert e and its rows X_e = x_perm[offsets[e]:offsets[e+1]]:
    a = X_e W1_e^T, b = X_e W3_e^T, h = silu(a) * b, y_e = h W2_e^T.
    Grouped GEMM over many small expert computations: unite.ai, section
    "Παραλληλισμός, Ακρίβεια και Τεχνικές Μνήμης".
    Returns a, b, h [R, f] and y_perm [R, d].
    """
    X = f64(x_perm)
    W1, W3, W2 = f64(W1), f64(W3), f64(W2)
    off = np.asarray(offsets).astype(np.int64)
    E, f, d = W1.shape
    R = X.shape[0]
    a = np.zeros((R, f)); b = np.zeros((R, f)); h = np.zeros((R, f)); y = np.zeros((R, d))
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        Xe = X[lo:hi]
        a[lo:hi] = Xe @ W1[e].T
        b[lo:hi] = Xe @ W3[e].T
        h[lo:hi] = silu(a[lo:hi]) * b[lo:hi]
        y[lo:hi] = h[lo:hi] @ W2[e].T
    return a, b, h, y


def combine(y_perm, gates, slot_row) -> np.ndarray:
    """y[t] = sum_j gates[t, j] * y_perm[slot_row[t, j]]."""
    Y = f64(y_perm)
    g = f64(gates)
    sr = np.asarray(slot_row)
    T, k = sr.shape
    y = np.zeros((T, Y.shape[1]))
    for j in range(k):
        y += g[:, j:j + 1] * Y[sr[:, j]]
    return y


# ----------------------------------------------------------------------------- backward
def combine_bwd(dy, y_perm, gates, slot_row):
    """dgates[t, j] = <dy[t], y_perm[slot_row[t, j]]>;
    dy_perm[slot_row[t, j]] = gates[t, j] * dy[t]."""
    dY = f64(dy)
    Y = f64(y_perm)
    g = f64(gates)
    sr = np.asarray(slot_row)
    T, k = sr.shape
    dgates = np.zeros((T, k))
    dy_perm = np.zeros_like(Y)
    for j in range(k):
        dgates[:, j] = np.einsum("td,td->t", dY, Y[sr[:, j]])
        dy_perm[sr[:, j]] = g[:, j:j + 1] * dY
    return dy_perm, dgates


def expert_ffn_bwd(dy_perm, x_perm, a, b, offsets, W1, W3, W2):
    """Backward of the grouped SwiGLU FFN.

    dh = dy_e W2_e, dW2_e = dy_e^T h_e, da = dh * b * s (1 + a (1 - s)) with
    s = sigmoid(a), db = dh * silu(a), dx_e = da W1_e + db W3_e,
    dW1_e = da^T X_e, dW3_e = db^T X_e.  Experts with no rows get zero weight
    gradients.  Returns dx_perm [R, d], dW1, dW3 [E, f, d], dW2 [E, d, f], and
    da, db [R, f].
    """
    dY = f64(dy_perm)
    X = f64(x_perm)
    A, B = f64(a), f64(b)
    W1, W3, W2 = f64(W1), f64(W3), f64(W2)
    off = np.asarray(offsets).astype(np.int64)
    E, f, d = W1.shape
    R = X.shape[0]
    dx = np.zeros((R, d)); da = np.zeros((R, f)); db = np.zeros((R, f))
    dW1 = np.zeros_like(W1); dW3 = np.zeros_like(W3); dW2 = np.zeros_like(W2)
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        ae, be = A[lo:hi], B[lo:hi]
        s = sigmoid(ae)
        h = ae * s * be
        dh = dY[lo:hi] @ W2[e]
        dW2[e] = dY[lo:hi].T @ h
        da[lo:hi] = dh * be * s * (1.0 + ae * (1.0 - s))
        db[lo:hi] = dh * ae * s
        dx[lo:hi] = da[lo:hi] @ W1[e] + db[lo:hi] @ W3[e]
        dW1[e] = da[lo:hi].T @ X[lo:hi]
        dW3[e] = db[lo:hi].T @ X[lo:hi]
    return dx, dW1, dW3, dW2, da, db


def route_bwd(dgates, gates, topk_idx, E: int) -> np.ndarray:
    """Gradient of the renormalised softmax gates w.r.t. the router scores:
    dL[t, e] = g_e (dg_e - sum_i g_i dg_i) for e in S_t, zero elsewhere."""
    dg = f64(dgates)
    g = f64(gates)
    idx = np.asarray(topk_idx).astype(np.int64)
    T, k = idx.shape
    inner = (g * dg).sum(axis=1, keepdims=True)
    vals = g * (dg - inner)
    dL = np.zeros((T, E))
    np.put_along_axis(dL, idx, vals, axis=1)
    return dL


def router_bwd(x, Wr, dlogits):
    """dx_r = dL Wr, dWr = dL^T x (router weight stored [E, d])."""
    dL = f64(dlogits)
    return dL @ f64(Wr), dL.T @ f64(x)


def unpermute_sum(dx_perm, slot_row, dx_r=None) -> np.ndarray:
    """dx[t] = dx_r[t] + sum_j dx_perm[slot_row[t, j]]."""
    D = f64(dx_perm)
    sr = np.asarray(slot_row)
    T, k = sr.shape
    dx = np.zeros((T, D.shape[1])) if dx_r is None else f64(dx_r).copy()
    for j in range(k):
        dx += D[sr[:, j]]
    return dx


# ----------------------------------------------------------------------------- composite
def shared_expert_fwd(x, W1s, W3s, W2s):
    """The always-on shared expert: the SwiGLU FFN applied to every token, i.e. the
    grouped FFN with one group spanning all T rows (bigchange.ai, "Olmo-core 3
    открывает стек обучения MoE…", section "Что инженер может попробовать на практике":
    top-four routing plus one shared expert).  W1s, W3s [1, fs, d], W2s [1, d, fs]."""
    X = f64(x)
    return expert_ffn_fwd(X, [0, X.shape[0]], W1s, W3s, W2s)


def layer_forward(x, W1, W3, W2, k: int, Wr=None, bias=None, select_logits=None,
                  topk_idx=None, gates=None, shared=None) -> dict:
    """Whole layer forward.

    Learned routing: pass Wr (and optionally bias).  The selection runs on
    ``select_logits`` when given (the scores whose fp32 comparison decides the
    integer routing), else on the fp64 scores.
    Given routing: pass topk_idx and gates; no router runs.
    shared: (W1s, W3s, W2s) of a shared expert, whose output is added to every token's.
    """
    E = f64(W1).shape[0]
    out = {}
    if topk_idx is None:
        L = router_logits(x, Wr, bias)
        out["logits"] = L
        sel = L if select_logits is None else f64(select_logits)
        idx, _ = topk_gates(sel, k)
        # the selection decides the integer routing; the gate values are the
        # oracle's own fp64 scores at the chosen experts
        g_sel = np.take_along_axis(L, idx.astype(np.int64), axis=1)
        w = np.exp(g_sel - g_sel[:, :1])
        out["gates"] = w / w.sum(axis=1, keepdims=True)
        out["topk_idx"] = idx
    else:
        out["topk_idx"] = np.asarray(topk_idx).astype(np.int32)
        out["gates"] = f64(gates)
    counts, offsets, slot_row, row_src = dispatch(out["topk_idx"], E)
    out.update(counts=counts, offsets=offsets, slot_row=slot_row, row_src=row_src)
    out["x_perm"] = permute(x, row_src)
    a, b, h, y_perm = expert_ffn_fwd(out["x_perm"], offsets, W1, W3, W2)
    out.update(a=a, b=b, h=h, y_perm=y_perm)
    out["y"] = combine(y_perm, out["gates"], slot_row)
    if shared is not None:
        a_s, b_s, h_s, y_s = shared_expert_fwd(x, *shared)
        out["shared"] = dict(a=a_s, b=b_s, h=h_s, y=y_s)
        out["y"] = y_s + out["y"]
    return out


def layer_backward(fw: dict, dy, x, W1, W3, W2, Wr=None, learned: bool = True, shared=None) -> dict:
    """Whole layer backward from the forward record ``fw`` (shared: the shared expert's
    weights when the forward had one)."""
    E = f64(W1).shape[0]
    g = {}
    dy_perm, dgates = combine_bwd(dy, fw["y_perm"], fw["gates"], fw["slot_row"])
    g["dy_perm"], g["dgates"] = dy_perm, dgates
    dx_perm, dW1, dW3, dW2, da, db = expert_ffn_bwd(dy_perm, fw["x_perm"], fw["a"], fw["b"],
                                                    fw["offsets"], W1, W3, W2)
    g.update(dx_perm=dx_perm, dW1=dW1, dW3=dW3, dW2=dW2, da=da, db=db)
    dx_r = None
    if learned:
        dL = route_bwd(dgates, fw["gates"], fw["topk_idx"], E)
        dx_r, dWr = router_bwd(x, Wr, dL)
        g.update(dlogits=dL, dWr=dWr, dx_r=dx_r)
    if shared is not None:
        T = f64(x).shape[0]
        sh = fw["shared"]
        dx_s, dW1s, dW3s, dW2s, _, _ = expert_ffn_bwd(dy, x, sh["a"], sh["b"], [0, T], *shared)
        g.update(dx_s=dx_s, dW1s=dW1s, dW3s=dW3s, dW2s=dW2s)
        dx_r = dx_s if dx_r is None else dx_r + dx_s
    g["dx"] = unpermute_sum(dx_perm, fw["slot_row"], dx_r)
    return g
