"""Weight-encoding comparator: the layer with bf16 expert weights (no quantization).

The Jamba-1.5 paper ("Serving Considerations and Improvements") says that
dequantizing the int8 weights inside the fused kernel is faster than running
with BF16 weights; the comparator is the same layer and kernels with the bf16
weights read as they are (MOE_W_BF16). Its oracle is the oracle's expert FFN
on the bf16 weights themselves with unit scales, in fp64; its tolerance is the
layer's. Small shapes cover both schedules, ragged row counts and the dense
(E = K = 1) case; mini-decode and mini-prefill are checked at full size on the
rows of sampled experts, in the launch configuration bench.py times.
"""
import sys

import numpy as np
import pytest
import torch

import workloads
from int8_weight_moe_amd import (moe_expert_ffn, moe_forward, moe_mlp_forward, moe_permute, moe_route,
                                 pack_bf16_experts)
from int8_weight_moe_amd._lib import MOE_PATH_AUTO, MOE_PATH_STREAM, MOE_PATH_TILED, MOE_W_BF16
from oracle import moe as omoe
from tests.helpers import assert_close_to_oracle, check_routing, np64, tiled_to_rowmajor

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[weights-test] {msg}", file=sys.stderr, flush=True)


def _unquantized(src: dict, experts=None) -> dict:
    """bf16 weights as the oracle's expert weights: codes = the weights (fp64), scales = 1."""
    W = {}
    for k in ("gate", "up", "down"):
        w = src["w_" + k] if experts is None else src["w_" + k][experts]
        W["q_" + k] = np64(w)
        W["s_" + k] = np.ones(W["q_" + k].shape[:-1])
    return W


def test_bf16_packing_is_the_byte_tiling():
    w = workloads.Workload("pack", T=1, d=128, f=192, E=2, K=1, act="bf16", scale="bf16", weight_src="bf16", seed=3)
    src = workloads.draw_expert_weights(w, "cpu")
    ex = pack_bf16_experts(*(src[k].cuda() for k in ("w_gate", "w_up", "w_down")))
    assert ex.fmt == MOE_W_BF16 and ex.s_gate is None
    for k in ("gate", "up", "down"):
        got = getattr(ex, "q_" + k).cpu().view(torch.int8).numpy()
        want = src["w_" + k].view(torch.int8).numpy()
        assert np.array_equal(tiled_to_rowmajor(got.reshape(want.shape)), want), k


@pytest.mark.parametrize("path", [MOE_PATH_AUTO, MOE_PATH_STREAM, MOE_PATH_TILED])
@pytest.mark.parametrize("T,d,f,E,K", [(64, 256, 512, 16, 2), (1, 128, 192, 4, 2), (300, 384, 640, 8, 2),
                                       (129, 256, 320, 4, 4), (40, 256, 256, 16, 2)])
def test_bf16_weights_match_oracle(path, T, d, f, E, K):
    w = workloads.Workload("bf16w", T=T, d=d, f=f, E=E, K=K, act="bf16", scale="bf16", weight_src="bf16", seed=11)
    x = workloads.draw_activations(w)
    wr, _ = workloads.draw_router(w)
    src = workloads.draw_expert_weights(w, "cpu")
    ex = pack_bf16_experts(*(src[k].cuda() for k in ("w_gate", "w_up", "w_down")))
    y, ids, gw = moe_forward(x.cuda(), wr.cuda(), None, ex, K, path=path)
    y2, _, _ = moe_forward(x.cuda(), wr.cuda(), None, ex, K, path=path)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    x64, wr64 = np64(x), np64(wr)
    logits = omoe.router_logits(x64, wr64)
    check_routing(ids.cpu().numpy(), gw.cpu().numpy(), logits, K)
    ref = omoe.moe_forward(x64, wr64, None, _unquantized(src), K, ids=ids.cpu().numpy())
    assert_close_to_oracle(np64(y), ref["y"], f"bf16 weights T={T} path={path}")


@pytest.mark.parametrize("path", [MOE_PATH_STREAM, MOE_PATH_TILED])
@pytest.mark.parametrize("T", [1, 64, 200])
def test_bf16_weights_dense_mlp(path, T):
    w = workloads.Workload("bf16mlp", T=T, d=256, f=384, E=1, K=1, act="bf16", scale="bf16", weight_src="bf16",
                           seed=5)
    x = workloads.draw_activations(w)
    src = workloads.draw_expert_weights(w, "cpu")
    ex = pack_bf16_experts(*(src[k].cuda() for k in ("w_gate", "w_up", "w_down")))
    y = moe_mlp_forward(x.cuda(), ex, path=path)
    torch.cuda.synchronize()
    W = _unquantized(src)
    ref = omoe.expert_swiglu(np64(x), W["q_gate"][0], W["s_gate"][0], W["q_up"][0], W["s_up"][0],
                             W["q_down"][0], W["s_down"][0])
    assert_close_to_oracle(np64(y), ref, f"bf16-weight MLP T={T}")


ROWS_PER_EXPERT = 256


@pytest.mark.parametrize("name,n_experts", [("mini-decode", 3), ("mini-prefill", 2)])
def test_bf16_weights_workload_sampled_rows(name, n_experts):
    w = workloads.WORKLOADS[name]
    dev = torch.device("cuda:0")
    _say(f"{name}: drawing bf16 weights")
    src = workloads.draw_expert_weights(w, dev)
    ex = pack_bf16_experts(src["w_gate"], src["w_up"], src["w_down"])
    wr, bias = workloads.draw_router(w)
    x_host = workloads.draw_activations(w)
    x = x_host.to(dev)
    wr_d = wr.to(dev)
    y, ids, gw = moe_forward(x, wr_d, None, ex, w.K)
    # staged calls in the same configuration: bitwise equal to the fused call
    ids_s, gw_s = moe_route(x, wr_d, None, w.K)
    off, ss, s2r = moe_permute(ids_s, w.E)
    rows = moe_expert_ffn(x, off, ss, ex, w.K)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids_s) and torch.equal(gw, gw_s)
    off_h, ss_h, rows_h = off.cpu().numpy(), ss.cpu().numpy(), rows.cpu().numpy()
    counts = np.diff(off_h)
    sample = [int(e) for e in np.argsort(-counts, kind="stable")[:n_experts]]
    _say(f"{name}: oracle evaluates experts {sample}")
    x64 = np64(x_host)
    for e in sample:
        r0, r1 = int(off_h[e]), int(min(off_h[e + 1], off_h[e] + ROWS_PER_EXPERT))
        if r1 <= r0:
            continue
        W = _unquantized({k: v[e] for k, v in src.items()})
        toks = ss_h[r0:r1] // w.K
        ref = omoe.expert_swiglu(x64[toks], W["q_gate"], W["s_gate"], W["q_up"], W["s_up"], W["q_down"],
                                 W["s_down"])
        assert_close_to_oracle(rows_h[r0:r1], ref, f"{name} bf16 weights, expert {e}")
    del src, ex
    torch.cuda.empty_cache()
