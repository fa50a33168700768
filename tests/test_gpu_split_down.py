"""The stream down pass with its reduction split over workgroups.

With 33-64 rows per expert on average and a split of the reduction, a down
pass given partial-sum planes (moe_forward, moe_mlp_forward and moe_expert_ffn
take them from their workspace, moe_expert_down from its optional one) lets
workgroups share each slice's activations through LDS, and a second kernel
adds the slices; without the planes the split stays inside one workgroup.
Both must give y_rows bit for bit, the fused calls must equal the staged ones,
and y must match the oracle. Shapes: MoE layers with one to three 64-row
passes per expert (ragged), and the dense MLP; int8, bf16 and fp8 weights.
"""
import numpy as np
import pytest
import torch

import workloads
from int8_weight_moe_amd import (moe_combine, moe_expert_down, moe_expert_ffn, moe_expert_gate_up, moe_forward,
                                 moe_mlp_forward, moe_permute, moe_route, pack_bf16_experts, quantize_experts_fp8)
from int8_weight_moe_amd._lib import MOE_PATH_AUTO, MOE_PATH_STREAM, MOE_W_INT8
from int8_weight_moe_amd.ops import make_shape, workspace_size
from oracle import fp8 as ofp8
from oracle import moe as omoe
from tests.helpers import assert_close_to_oracle, experts_to_device, np64, quantize_experts_oracle

pytestmark = pytest.mark.gpu


def _experts(fmt, w):
    src = workloads.draw_expert_weights(w, "cpu")
    if fmt == "int8":
        W = quantize_experts_oracle(src, w.scale)
        return experts_to_device(W, workloads.TORCH_DTYPE[w.scale]), W
    ws = [src[k].cuda() for k in ("w_gate", "w_up", "w_down")]
    if fmt == "bf16":
        W = {}
        for k in ("gate", "up", "down"):
            W["q_" + k] = np64(src["w_" + k])
            W["s_" + k] = np.ones(W["q_" + k].shape[:-1])
        return pack_bf16_experts(*ws), W
    W = {}
    for k in ("gate", "up", "down"):
        codes, sc = ofp8.quantize_rows_fp8(np64(src["w_" + k]), "bf16")
        W["q_" + k], W["s_" + k] = ofp8.e4m3_decode(codes), sc
    return quantize_experts_fp8(*ws, torch.bfloat16), W


def _base_workspace(T, d, f, E, K):
    """The workspace without partial-sum planes: ids, weights, offsets, slots, inverse map, h, y_rows."""
    r = lambda n: (n + 255) // 256 * 256
    S = T * K
    return r(S * 4) * 4 + r((E + 1) * 4) + r(S * f * 2) + r(S * d * 4)


@pytest.mark.parametrize("fmt,act", [("int8", "bf16"), ("bf16", "bf16"), ("fp8", "bf16"), ("int8", "f32")])
@pytest.mark.parametrize("T,d,f,E,K", [(300, 256, 512, 16, 2), (100, 512, 640, 4, 2), (150, 256, 1024, 2, 2),
                                       (64, 256, 24576, 1, 1), (400, 256, 1536, 16, 2)])
def test_fused_split_equals_staged_and_oracle(fmt, act, T, d, f, E, K):
    """The last two shapes take the one-wave-per-SIMD gate/up shape (48-channel
    items, two per workgroup, reductions cut in two) with int8 and fp8 weights:
    a dense layer with 256 workgroups, and 16 experts with 16 each."""
    w = workloads.Workload("split", T=T, d=d, f=f, E=E, K=K, act=act, scale=act, weight_src="f32" if act == "f32" else "bf16",
                           seed=21)
    x = workloads.draw_activations(w)
    wr, _ = workloads.draw_router(w)
    ex, W = _experts(fmt, w)
    shape = make_shape(T, d, f, E, K, workloads.TORCH_DTYPE[act], workloads.TORCH_DTYPE[act], MOE_PATH_STREAM, ex.fmt)
    assert workspace_size(shape) > _base_workspace(T, d, f, E, K), "the split down pass is not planned"
    xg, wrg = x.cuda(), wr.cuda()
    y, ids, gw = moe_forward(xg, wrg, None, ex, K, path=MOE_PATH_STREAM)
    ids2, gw2 = moe_route(xg, wrg, None, K)
    off, ss, s2r = moe_permute(ids2, E)
    rows = moe_expert_ffn(xg, off, ss, ex, K, path=MOE_PATH_STREAM)
    y2 = moe_combine(rows, s2r, gw2, x.dtype)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(gw, gw2)
    assert torch.equal(y, y2)
    # the down pass alone, with and without the planes
    h = moe_expert_gate_up(xg, off, ss, ex, K, path=MOE_PATH_STREAM)
    r_split = moe_expert_down(h, off, ex, T, K, act=x.dtype, path=MOE_PATH_STREAM)
    r_in = moe_expert_down(h, off, ex, T, K, act=x.dtype, path=MOE_PATH_STREAM, split_workspace=False)
    torch.cuda.synchronize()
    assert torch.equal(r_split, r_in) and torch.equal(r_split, rows)
    counts = np.diff(off.cpu().numpy())
    if (T, E) == (150, 2):
        assert counts.max() > 128    # an expert with three 64-row passes
    ref = omoe.moe_forward(np64(x), np64(wr), None, W, K, ids=ids.cpu().numpy())
    assert_close_to_oracle(np64(y), ref["y"], f"split down, {fmt} weights, T={T} E={E}")


@pytest.mark.parametrize("path", [MOE_PATH_STREAM, MOE_PATH_AUTO])
@pytest.mark.parametrize("T,act", [(40, "bf16"), (64, "bf16"), (48, "f32")])
def test_dense_mlp_split_equals_staged(path, T, act):
    """moe_mlp_forward with the down reduction split over workgroups writes y
    from the sum of the slices (the combine folded in): bitwise the staged
    calls' y, for bf16 and fp32 outputs."""
    w = workloads.Workload("dsplit", T=T, d=256, f=1024, E=1, K=1, act=act, scale=act,
                           weight_src="f32" if act == "f32" else "bf16", seed=8)
    x = workloads.draw_activations(w)
    ex, W = _experts("int8", w)
    adt = workloads.TORCH_DTYPE[act]
    assert workspace_size(make_shape(T, 256, 1024, 1, 1, adt, adt, path, MOE_W_INT8)) > \
        _base_workspace(T, 256, 1024, 1, 1)
    xg = x.cuda()
    y = moe_mlp_forward(xg, ex, path=path)
    ones = torch.ones((T, 1), dtype=torch.float32, device="cuda")
    off = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    ident = torch.arange(T, dtype=torch.int32, device="cuda")
    rows = moe_expert_ffn(xg, off, ident, ex, 1, path=MOE_PATH_STREAM)
    y2 = moe_combine(rows, ident, ones, adt)
    h = moe_expert_gate_up(xg, off, ident, ex, 1, path=MOE_PATH_STREAM)
    r_in = moe_expert_down(h, off, ex, T, 1, act=adt, path=MOE_PATH_STREAM, split_workspace=False)
    torch.cuda.synchronize()
    bits = torch.int16 if act == "bf16" else torch.int32
    assert torch.equal(y.view(bits), y2.view(bits))
    assert torch.equal(r_in, rows)
    ref = omoe.expert_swiglu(np64(x), W["q_gate"][0], W["s_gate"][0], W["q_up"][0], W["s_up"][0],
                             W["q_down"][0], W["s_down"][0])
    assert_close_to_oracle(np64(y), ref, f"dense MLP split down T={T}")
