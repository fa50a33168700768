"""The allocation-free entry point moe_forward_noalloc against moe_forward.

It runs the same kernels on the library's fixed per-GPU scratch instead of a
caller workspace, so its outputs must equal moe_forward's bit for bit (which
is tighter than the oracle tolerance moe_forward is held to elsewhere). Two
calls in a row, the second on a smaller input, so the scratch holds the first
call's contents when the second starts; shapes on both FFN schedules, with
and without the permutation derived inside the gate/up pass, a split down
pass (dense layer at 64 rows), and the largest decode layer.
"""
import pytest
import torch

import workloads
from int8_weight_moe_amd import MoeError, moe_forward, moe_forward_noalloc
from int8_weight_moe_amd._lib import MOE_PATH_AUTO, MOE_PATH_STREAM, MOE_PATH_TILED
from oracle import moe as omoe
from tests.helpers import assert_close_to_oracle, experts_to_device, np64, quantize_experts_oracle

pytestmark = pytest.mark.gpu


def _layer(T, d, f, E, K, seed, bias=None):
    w = workloads.Workload("na", T=T, d=d, f=f, E=E, K=K, act="bf16", scale="bf16", weight_src="bf16", seed=seed)
    x = workloads.draw_activations(w)
    wr, _ = workloads.draw_router(w)
    src = workloads.draw_expert_weights(w, "cpu")
    W = quantize_experts_oracle(src, "bf16")
    b = None if bias is None else torch.tensor(bias, dtype=torch.float32).cuda()
    return x.cuda(), wr.cuda(), b, experts_to_device(W, torch.bfloat16), W


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16)) if a.dtype == torch.bfloat16 else torch.equal(a, b)


@pytest.mark.parametrize("T1,T2,d,f,E,K,path", [
    (200, 37, 256, 384, 16, 2, MOE_PATH_AUTO),       # tiled then stream (ids mode)
    (600, 130, 192, 320, 8, 2, MOE_PATH_TILED),      # tiled twice, ragged tiles
    (300, 100, 128, 1536, 16, 2, MOE_PATH_STREAM),   # stream with the permutation kernel, then ids mode
    (64, 9, 256, 512, 1, 1, MOE_PATH_STREAM),        # dense layer: down pass split over workgroups
])
def test_noalloc_equals_forward_two_calls(T1, T2, d, f, E, K, path):
    x, wr, b, ex, W = _layer(T1, d, f, E, K, seed=T1 + d, bias=[1.0] + [0.0] * (E - 1) if E > 1 else None)
    outs = []
    for T in (T1, T2):
        xs = x[:T].contiguous()
        y0, i0, g0 = moe_forward(xs, wr, b, ex, K, path=path)
        y1, i1, g1 = moe_forward_noalloc(xs, wr, b, ex, K, path=path)
        torch.cuda.synchronize()
        assert torch.equal(i0, i1) and torch.equal(g0, g1), f"routing differs at T={T}"
        assert _same(y0, y1), f"y differs from moe_forward at T={T}"
        outs.append((xs, y1, i1))
    # and the second, smaller call against the oracle
    xs, y1, i1 = outs[1]
    ref = omoe.moe_forward(np64(xs), np64(wr), None if b is None else np64(b), W, K, ids=i1.cpu().numpy())["y"]
    assert_close_to_oracle(np64(y1), ref, "noalloc y (second call)")


def test_noalloc_large_decode_layer_then_smaller():
    """The largest decode layer (Jamba-1.5-Large shape, T=64) fits the fixed scratch."""
    w = workloads.LARGE_DECODE
    from int8_weight_moe_amd import quantize_experts
    src = workloads.draw_expert_weights(w, "cuda")
    ex = quantize_experts(src["w_gate"], src["w_up"], src["w_down"], torch.bfloat16)
    del src
    wr = workloads.draw_router(w)[0].cuda()
    x = workloads.draw_activations(w).cuda()
    for T in (64, 24):
        xs = x[:T].contiguous()
        y0, i0, g0 = moe_forward(xs, wr, None, ex, 2)
        y1, i1, g1 = moe_forward_noalloc(xs, wr, None, ex, 2)
        torch.cuda.synchronize()
        assert torch.equal(i0, i1) and torch.equal(g0, g1) and _same(y0, y1), f"T={T}"
    del ex
    torch.cuda.empty_cache()


def test_noalloc_rejects_shapes_beyond_the_scratch():
    """40000 tokens need 41 MB of y_rows alone: rejected before anything is enqueued."""
    x, wr, b, ex, W = _layer(8, 128, 192, 4, 2, seed=5)
    big = torch.zeros((40000, 128), dtype=torch.bfloat16, device="cuda")
    y = torch.full((40000, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(MoeError, match="scratch"):
        moe_forward_noalloc(big, wr, None, ex, 2, y=y)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)          # nothing was written
