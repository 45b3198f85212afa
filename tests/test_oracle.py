"""Pins for the CPU oracle of the MoE layer (no GPU).

Each test checks the oracle against something other than itself: brute force
on tiny inputs, a different formulation (dense-masked experts), special cases
that reduce to library routines (softmax, a dense SwiGLU FFN through
torch.nn.functional.silu), invariants the routing must satisfy, and central
finite differences for every gradient.
"""
import itertools

import numpy as np
import pytest
import scipy.special
import torch

from oracle import moe_ref as ref


def _rand_case(seed, T, d, f, E, k, scale_w=0.3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    Wr = rng.standard_normal((E, d)) * scale_w
    W1 = rng.standard_normal((E, f, d)) * scale_w
    W3 = rng.standard_normal((E, f, d)) * scale_w
    W2 = rng.standard_normal((E, d, f)) * scale_w
    dy = rng.standard_normal((T, d))
    return x, Wr, W1, W3, W2, dy


# ------------------------------------------------------------------ top-k selection
def _rank_by_pairwise(L, k):
    """Brute force: expert e is chosen iff fewer than k experts beat it, where e'
    beats e when its score is larger, or equal with a lower index; its position
    in the output is the number of experts that beat it."""
    T, E = L.shape
    idx = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        for e in range(E):
            beaters = sum(1 for e2 in range(E)
                          if L[t, e2] > L[t, e] or (L[t, e2] == L[t, e] and e2 < e))
            if beaters < k:
                idx[t, beaters] = e
    return idx


@pytest.mark.parametrize("E,k", [(6, 1), (6, 3), (6, 6), (8, 2), (9, 4)])
def test_topk_matches_pairwise_bruteforce(E, k):
    rng = np.random.default_rng(E * 10 + k)
    # small integer scores force many exact ties
    L = rng.integers(-3, 4, size=(60, E)).astype(np.float64)
    idx, gates = ref.topk_gates(L, k)
    assert np.array_equal(idx, _rank_by_pairwise(L, k))
    # the chosen set maximises the score sum over all k-subsets
    for t in range(0, 60, 7):
        best = max(sum(L[t, list(c)]) for c in itertools.combinations(range(E), k))
        assert L[t, idx[t]].sum() == best


def test_topk_all_equal_and_signed_zero():
    L = np.zeros((3, 7))
    L[1] = 2.5
    L[2, :] = 0.0
    L[2, 3] = -0.0
    L[2, 0] = -0.0
    idx, gates = ref.topk_gates(L, 4)
    assert (idx == np.arange(4)).all()
    assert np.allclose(gates, 0.25, rtol=0, atol=1e-15)


def test_gates_closed_forms():
    rng = np.random.default_rng(3)
    L = rng.standard_normal((40, 8)) * 3
    # k = E: the gates are the full softmax, in selection order
    idx, g = ref.topk_gates(L, 8)
    sm = scipy.special.softmax(L, axis=1)
    assert np.allclose(g, np.take_along_axis(sm, idx.astype(np.int64), axis=1), rtol=1e-13, atol=0)
    # k = 1: a single gate of exactly 1 on the argmax
    idx1, g1 = ref.topk_gates(L, 1)
    assert (g1 == 1.0).all() and (idx1[:, 0] == L.argmax(axis=1)).all()
    # general k: softmax over all E renormalised over the chosen k
    idx4, g4 = ref.topk_gates(L, 4)
    p = np.take_along_axis(sm, idx4.astype(np.int64), axis=1)
    assert np.allclose(g4, p / p.sum(axis=1, keepdims=True), rtol=1e-13, atol=0)
    assert np.allclose(g4.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert (np.diff(g4, axis=1) <= 0).all()          # value-descending order


def test_router_bias_shifts_selection_and_gates():
    """A per-expert bias adds to every token's score: +12 on expert 2 puts it first for
    every token, -12 on expert 4 keeps it out, and the gates are the softmax of the
    biased scores of the chosen experts (scipy's softmax over a torch matmul)."""
    rng = np.random.default_rng(41)
    x = rng.standard_normal((50, 16))
    Wr = rng.standard_normal((6, 16)) * 0.05
    bias = np.zeros(6)
    bias[2], bias[4] = 12.0, -12.0
    L = ref.router_logits(x, Wr, bias)
    idx, g = ref.topk_gates(L, 3)
    assert (idx[:, 0] == 2).all() and not (idx == 4).any()
    raw = (torch.tensor(x) @ torch.tensor(Wr).T).numpy()
    chosen = np.take_along_axis(raw, idx.astype(np.int64), axis=1) + bias[idx]
    assert np.allclose(g, scipy.special.softmax(chosen, axis=1), rtol=1e-12, atol=0)
    assert (g[:, 0] > 0.99).all()
    fw = ref.layer_forward(x, rng.standard_normal((6, 8, 16)), rng.standard_normal((6, 8, 16)),
                           rng.standard_normal((6, 16, 8)), 3, Wr=Wr, bias=bias)
    assert (fw["counts"][2] == 50) and fw["counts"][4] == 0


# ------------------------------------------------------------------ dispatch
def _dispatch_loop(idx, E):
    T, k = idx.shape
    counts = [0] * E
    for t in range(T):
        for j in range(k):
            counts[idx[t, j]] += 1
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + counts[e])
    fill = list(offsets[:-1])
    slot_row = np.zeros((T, k), dtype=np.int64)
    for t in range(T):              # visiting slots in t*k + j order keeps the sort stable
        for j in range(k):
            e = idx[t, j]
            slot_row[t, j] = fill[e]
            fill[e] += 1
    return np.array(counts), np.array(offsets), slot_row


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (37, 5, 2), (64, 16, 4), (200, 128, 4)])
def test_dispatch_bruteforce_and_invariants(T, E, k):
    rng = np.random.default_rng(T + E + k)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, slot_row, row_src = ref.dispatch(idx, E)
    c2, o2, s2 = _dispatch_loop(idx, E)
    assert np.array_equal(counts, c2) and np.array_equal(offsets, o2) and np.array_equal(slot_row, s2)
    assert counts.sum() == T * k and offsets[0] == 0 and offsets[-1] == T * k
    assert (np.diff(offsets) >= 0).all() and (counts <= T).all()
    flat = slot_row.reshape(-1)
    assert np.array_equal(np.sort(flat), np.arange(T * k))          # bijection onto [0, T*k)
    assert (row_src[flat] == np.repeat(np.arange(T), k)).all()       # row_src inverts slot_row
    x = rng.standard_normal((T, 5))
    xp = ref.permute(x, row_src)
    for j in range(k):                                               # unpermute(permute(x)) == x
        assert np.array_equal(xp[slot_row[:, j]], x)
    for e in range(E):                                               # rows of one expert keep token order
        seg = row_src[offsets[e]:offsets[e + 1]]
        assert (np.diff(seg) > 0).all()


def test_validate_given_routing():
    idx = np.array([[0, 1], [2, 2], [3, 9], [-1, 0]], dtype=np.int32)
    flags = ref.validate_given_routing(idx, 8)
    assert flags.tolist() == [0, 2, 1, 1]


# ------------------------------------------------------------------ expert FFN forward
def test_single_expert_is_dense_swiglu():
    x, Wr, W1, W3, W2, _ = _rand_case(1, 30, 12, 20, 1, 1)
    fw = ref.layer_forward(x, W1, W3, W2, 1, Wr=Wr)
    xt = torch.tensor(x)
    h = torch.nn.functional.silu(xt @ torch.tensor(W1[0]).T) * (xt @ torch.tensor(W3[0]).T)
    y = (h @ torch.tensor(W2[0]).T).numpy()
    assert np.allclose(fw["gates"], 1.0)
    assert np.allclose(fw["y"], y, rtol=1e-12, atol=1e-12)


def test_dense_masked_formulation():
    x, Wr, W1, W3, W2, _ = _rand_case(2, 50, 16, 24, 7, 3)
    fw = ref.layer_forward(x, W1, W3, W2, 3, Wr=Wr)
    G = np.zeros((50, 7))
    np.put_along_axis(G, fw["topk_idx"].astype(np.int64), fw["gates"], axis=1)
    y = np.zeros((50, 16))
    for e in range(7):               # every expert on every token, masked by the gate matrix
        a = x @ W1[e].T
        b = x @ W3[e].T
        y += G[:, e:e + 1] * ((a / (1 + np.exp(-a)) * b) @ W2[e].T)
    assert np.allclose(fw["y"], y, rtol=1e-12, atol=1e-12)


def test_identical_experts_and_linearity():
    x, Wr, W1, W3, W2, dy = _rand_case(3, 40, 10, 14, 6, 2)
    W1[:] = W1[0]; W3[:] = W3[0]; W2[:] = W2[0]
    fw = ref.layer_forward(x, W1, W3, W2, 2, Wr=Wr)
    a = x @ W1[0].T
    ffn = (a * scipy.special.expit(a) * (x @ W3[0].T)) @ W2[0].T
    assert np.allclose(fw["y"], ffn, rtol=1e-12, atol=1e-12)   # gates sum to one
    bw = ref.layer_backward(fw, dy, x, W1, W3, W2, Wr=Wr)
    assert np.abs(bw["dlogits"]).max() < 1e-12 and np.abs(bw["dWr"]).max() < 1e-11
    fw2 = ref.layer_forward(x, W1, W3, 2.5 * W2, 2, Wr=Wr)
    assert np.allclose(fw2["y"], 2.5 * fw["y"], rtol=1e-12, atol=1e-12)


def test_empty_experts_get_zero_weight_grads():
    x, Wr, W1, W3, W2, dy = _rand_case(4, 20, 8, 12, 6, 2)
    idx = np.tile(np.array([[0, 3]], dtype=np.int32), (20, 1))
    gates = np.tile(np.array([[0.7, 0.3]]), (20, 1))
    fw = ref.layer_forward(x, W1, W3, W2, 2, topk_idx=idx, gates=gates)
    bw = ref.layer_backward(fw, dy, x, W1, W3, W2, learned=False)
    for e in (1, 2, 4, 5):
        assert not bw["dW1"][e].any() and not bw["dW3"][e].any() and not bw["dW2"][e].any()
    assert fw["counts"].tolist() == [20, 0, 0, 20, 0, 0]


# ------------------------------------------------------------------ backward via finite differences
def _loss(params, dy, k, learned=True, idx=None):
    x, Wr, W1, W3, W2, gates = params
    if learned:
        fw = ref.layer_forward(x, W1, W3, W2, k, Wr=Wr)
    else:
        fw = ref.layer_forward(x, W1, W3, W2, k, topk_idx=idx, gates=gates)
    return float((fw["y"] * dy).sum()), fw["topk_idx"]


def test_score_gradient_is_zero_outside_the_chosen_experts():
    """dlogits against central differences of the loss in every single score, with the
    selection held (the gates are a softmax over the k chosen scores): each token's
    gradient has exactly its k chosen experts' entries, zero elsewhere.  The un-permute
    that folds in the router's input gradient reads only those k entries per token."""
    T, d, f, E, k = 6, 8, 8, 5, 2
    x, Wr, W1, W3, W2, dy = _rand_case(21, T, d, f, E, k, scale_w=0.5)
    L = ref.router_logits(x, Wr)
    srt = np.sort(L, axis=1)[:, ::-1]
    assert (srt[:, k - 1] - srt[:, k]).min() > 1e-3          # the selection stays put under +-h
    fw = ref.layer_forward(x, W1, W3, W2, k, Wr=Wr)
    bw = ref.layer_backward(fw, dy, x, W1, W3, W2, Wr=Wr)

    def loss(Lp):
        idx, gates = ref.topk_gates(Lp, k)
        assert np.array_equal(idx, fw["topk_idx"])
        return float((ref.layer_forward(x, W1, W3, W2, k, topk_idx=idx, gates=gates)["y"] * dy).sum())

    h = 1e-6
    fd = np.zeros((T, E))
    for t in range(T):
        for e in range(E):
            Lp, Lm = L.copy(), L.copy()
            Lp[t, e] += h
            Lm[t, e] -= h
            fd[t, e] = (loss(Lp) - loss(Lm)) / (2 * h)
    chosen = np.zeros((T, E), dtype=bool)
    np.put_along_axis(chosen, fw["topk_idx"].astype(np.int64), True, axis=1)
    assert np.abs(fd[~chosen]).max() < 1e-8
    assert np.abs(bw["dlogits"][~chosen]).max() == 0.0
    assert np.allclose(bw["dlogits"][chosen], fd[chosen], rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("learned", [True, False])
def test_backward_finite_differences(learned):
    T, d, f, E, k = 24, 10, 12, 5, 2
    x, Wr, W1, W3, W2, dy = _rand_case(11, T, d, f, E, k, scale_w=0.5)
    rng = np.random.default_rng(12)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    gates = rng.dirichlet(np.ones(k), size=T)
    params = [x, Wr, W1, W3, W2, gates]
    if learned:
        fw = ref.layer_forward(x, W1, W3, W2, k, Wr=Wr)
        srt = np.sort(ref.router_logits(x, Wr), axis=1)[:, ::-1]
        assert (srt[:, k - 1] - srt[:, k]).min() > 1e-4      # selection stays put under +-h
        bw = ref.layer_backward(fw, dy, x, W1, W3, W2, Wr=Wr)
        grads = {0: bw["dx"], 1: bw["dWr"], 2: bw["dW1"], 3: bw["dW3"], 4: bw["dW2"]}
        assert np.allclose(bw["dlogits"].sum(axis=1), 0, atol=1e-12)
    else:
        fw = ref.layer_forward(x, W1, W3, W2, k, topk_idx=idx, gates=gates)
        bw = ref.layer_backward(fw, dy, x, W1, W3, W2, learned=False)
        grads = {0: bw["dx"], 2: bw["dW1"], 3: bw["dW3"], 4: bw["dW2"], 5: bw["dgates"]}
    h = 1e-5
    for pi, g in grads.items():
        for trial in range(2):
            D = rng.standard_normal(params[pi].shape)
            plus = [p.copy() for p in params]; plus[pi] = params[pi] + h * D
            minus = [p.copy() for p in params]; minus[pi] = params[pi] - h * D
            lp, ip = _loss(plus, dy, k, learned, idx)
            lm, im = _loss(minus, dy, k, learned, idx)
            assert np.array_equal(ip, fw["topk_idx"]) and np.array_equal(im, fw["topk_idx"])
            fd = (lp - lm) / (2 * h)
            an = float((g * D).sum())
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (pi, fd, an)


# ------------------------------------------------------------------ shared expert
def test_shared_expert_forward_per_token_bruteforce():
    """y = shared SwiGLU FFN of every token + the routed layer; the shared part checked
    token by token with matrix-vector products and torch's silu."""
    x, Wr, W1, W3, W2, _ = _rand_case(21, 17, 12, 20, 5, 2)
    rng = np.random.default_rng(22)
    fs = 16
    Ws = (rng.standard_normal((1, fs, 12)) * 0.3, rng.standard_normal((1, fs, 12)) * 0.3,
          rng.standard_normal((1, 12, fs)) * 0.3)
    fw = ref.layer_forward(x, W1, W3, W2, 2, Wr=Wr, shared=Ws)
    plain = ref.layer_forward(x, W1, W3, W2, 2, Wr=Wr)
    for t in range(17):
        xt = torch.tensor(x[t])
        ht = torch.nn.functional.silu(torch.tensor(Ws[0][0]) @ xt) * (torch.tensor(Ws[1][0]) @ xt)
        ys = (torch.tensor(Ws[2][0]) @ ht).numpy()
        assert np.allclose(fw["y"][t], plain["y"][t] + ys, rtol=1e-12, atol=1e-12)


def test_shared_expert_backward_finite_differences():
    T, d, f, E, k, fs = 16, 8, 10, 4, 2, 12
    x, Wr, W1, W3, W2, dy = _rand_case(23, T, d, f, E, k, scale_w=0.5)
    rng = np.random.default_rng(24)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    gates = rng.dirichlet(np.ones(k), size=T)
    Ws = [rng.standard_normal((1, fs, d)) * 0.5, rng.standard_normal((1, fs, d)) * 0.5,
          rng.standard_normal((1, d, fs)) * 0.5]
    params = [x, W1, W3, W2, *Ws]

    def loss(p):
        fw = ref.layer_forward(p[0], p[1], p[2], p[3], k, topk_idx=idx, gates=gates, shared=p[4:])
        return float((fw["y"] * dy).sum())

    fw = ref.layer_forward(x, W1, W3, W2, k, topk_idx=idx, gates=gates, shared=Ws)
    bw = ref.layer_backward(fw, dy, x, W1, W3, W2, learned=False, shared=Ws)
    grads = {0: bw["dx"], 1: bw["dW1"], 2: bw["dW3"], 3: bw["dW2"], 4: bw["dW1s"], 5: bw["dW3s"], 6: bw["dW2s"]}
    h = 1e-5
    for pi, g in grads.items():
        D = rng.standard_normal(params[pi].shape)
        plus = list(params); plus[pi] = params[pi] + h * D
        minus = list(params); minus[pi] = params[pi] - h * D
        fd = (loss(plus) - loss(minus)) / (2 * h)
        an = float((g * D).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (pi, fd, an)
