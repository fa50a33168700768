"""Dense int8-weight MLP (moe_mlp_forward): the one-expert case of the layer.

ExpertsInt8 quantizes the MLP weights as well as the MoE weights (Jamba-1.5
paper, "Serving Considerations and Improvements"). The oracle for a dense MLP
is its expert FFN on every row; the textbook form (torch CPU fp64 silu on the
dequantized weights) is checked too. Small shapes cover both schedules and
ragged row counts; the Jamba-1.5-Large-shaped layer is checked on 256 sampled
rows in the launch configuration bench.py times.
"""
import numpy as np
import pytest
import torch

import workloads
from int8_weight_moe_amd import MoeError, moe_mlp_forward, quantize_experts
from int8_weight_moe_amd._lib import MOE_PATH_AUTO, MOE_PATH_STREAM, MOE_PATH_TILED
from oracle import moe as omoe
from oracle import quant as oquant
from tests.helpers import assert_close_to_oracle, experts_to_device, np64, quantize_experts_oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("path", [MOE_PATH_AUTO, MOE_PATH_STREAM, MOE_PATH_TILED])
@pytest.mark.parametrize("T,d,f,act", [(1, 256, 512, "bf16"), (70, 384, 640, "bf16"), (300, 256, 320, "f32"),
                                       (129, 128, 192, "bf16")])
def test_mlp_matches_oracle(path, T, d, f, act):
    w = workloads.Workload("mlp", T=T, d=d, f=f, E=1, K=1, act=act, scale=act,
                           weight_src="f32" if act == "f32" else "bf16", seed=21)
    x = workloads.draw_activations(w)
    src = workloads.draw_expert_weights(w, "cpu")
    W = quantize_experts_oracle(src, w.scale)
    ex = experts_to_device(W, workloads.TORCH_DTYPE[w.scale])
    y = moe_mlp_forward(x.cuda(), ex, path=path)
    torch.cuda.synchronize()
    x64 = np64(x)
    ref = omoe.expert_swiglu(x64, W["q_gate"][0], W["s_gate"][0], W["q_up"][0], W["s_up"][0],
                             W["q_down"][0], W["s_down"][0])
    assert_close_to_oracle(np64(y), ref, "dense MLP")
    deq = {k: torch.from_numpy(oquant.dequantize_rows(W["q_" + k][0], W["s_" + k][0])) for k in ("gate", "up", "down")}
    xt = torch.from_numpy(x64)
    text = (torch.nn.functional.silu(xt @ deq["gate"].T) * (xt @ deq["up"].T)) @ deq["down"].T
    assert_close_to_oracle(np64(y), text.numpy(), "dense MLP vs textbook SwiGLU")


def test_mlp_rejects_more_than_one_expert():
    w = workloads.Workload("mlp", T=4, d=64, f=64, E=2, K=1)
    x = workloads.draw_activations(w).cuda()
    src = workloads.draw_expert_weights(w, "cuda")
    ex = quantize_experts(src["w_gate"], src["w_up"], src["w_down"], torch.bfloat16)
    with pytest.raises((MoeError, ValueError)):
        moe_mlp_forward(x, ex)


@pytest.mark.parametrize("name", list(workloads.DENSE_WORKLOADS))
def test_large_mlp_sampled_rows(name):
    w = workloads.DENSE_WORKLOADS[name]
    dev = torch.device("cuda:0")
    src = workloads.draw_expert_weights(w, dev)
    ex = quantize_experts(src["w_gate"], src["w_up"], src["w_down"], torch.bfloat16)
    x_host = workloads.draw_activations(w)
    y = moe_mlp_forward(x_host.to(dev), ex)
    y2 = moe_mlp_forward(x_host.to(dev), ex)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    W = quantize_experts_oracle({k: v[0] for k, v in src.items()}, w.scale)
    rows = np.random.default_rng(0).choice(w.T, size=min(w.T, 256), replace=False)
    ref = omoe.expert_swiglu(np64(x_host)[rows], W["q_gate"], W["s_gate"], W["q_up"], W["s_up"],
                             W["q_down"], W["s_down"])
    assert_close_to_oracle(np64(y)[rows], ref, name)
