"""moe_route_noalloc (no workspace: a fixed array in the library's device memory) against
moe_route (caller's workspace), bit for bit, on two calls in a row with the second one
smaller, so whatever the first call left in the shared array must not reach the second."""
import numpy as np
import pytest
import torch

from gpu_common import host, say

pytestmark = pytest.mark.gpu


def _logits(T, E, seed):
    g = torch.Generator().manual_seed(seed)
    L = torch.randn(T, E, generator=g)
    n = min(T, 6)
    L[:n] = torch.randint(-2, 3, (n, E), generator=g).float()   # rows full of exact ties
    L[0, ::2] = -0.0
    return L.cuda()


def _outputs(T, E, k):
    i32 = torch.int32
    return dict(idx=torch.full((T, k), -7, dtype=i32, device="cuda"),
                gates=torch.full((T, k), -1.0, device="cuda"),
                counts=torch.full((E,), -7, dtype=i32, device="cuda"),
                offsets=torch.full((E + 1,), -7, dtype=i32, device="cuda"),
                slot=torch.full((T, k), -7, dtype=i32, device="cuda"))


def _route_both(T, E, k, seed):
    import mixture_experts_layer_logits_amd as m
    say(f"[gpu] route_noalloc vs route T={T} E={E} k={k}")
    s = m.make_shape(T, 64, 64, E, k)
    L = _logits(T, E, seed)
    a, b = _outputs(T, E, k), _outputs(T, E, k)
    ws = torch.empty(m.moe_workspace_size(s), dtype=torch.uint8, device="cuda")
    m.moe_route(s, L, a["idx"], a["gates"], a["counts"], a["offsets"], a["slot"], ws)
    m.moe_route_noalloc(s, L, b["idx"], b["gates"], b["counts"], b["offsets"], b["slot"])
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), (T, E, k, key)
    off = host(b["offsets"])
    assert off[0] == 0 and off[-1] == T * k
    assert np.array_equal(np.sort(host(b["slot"]).reshape(-1)), np.arange(T * k))


def test_route_noalloc_matches_route_on_two_calls():
    _route_both(65536, 128, 4, 11)   # 2 MiB of the 4 MiB array
    _route_both(1000, 96, 3, 12)     # smaller: the first call's histograms are still there


def test_route_noalloc_refuses_shapes_beyond_its_scratch():
    import mixture_experts_layer_logits_amd as m
    s = m.make_shape(200000, 64, 64, 128, 4)     # 6250 * 128 + 800000 int32 > 2^20
    T, E, k = 200000, 128, 4
    dummy = torch.empty(16, dtype=torch.int32, device="cuda")
    with pytest.raises(m.MoeError) as ei:
        m.moe_route_noalloc(s, dummy, dummy, dummy, dummy, dummy, dummy)
    assert ei.value.status == -7
