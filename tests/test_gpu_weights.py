"""Weight-encoding comparators: the layer with bf16 weights and with fp8 e4m3 weights.

The Jamba-1.5 paper ("Serving Considerations and Improvements") says that
dequantizing the int8 weights inside the fused kernel is faster than running
with BF16 weights and matches FP8. The comparators are the same layer and
kernels with
  * the bf16 weights read as they are (MOE_W_BF16); oracle: the oracle's
    expert FFN on the bf16 weights with unit scales;
  * OCP e4m3 codes with per-channel scales (MOE_W_FP8) from the library's
    fp8 quantizer, which must match the oracle's (oracle/fp8.py) bit for bit;
    oracle: the expert FFN on the decoded e4m3 values and scales.
Both in fp64 and to the layer's tolerance. Small shapes cover both schedules,
ragged row counts and the dense (E = K = 1) case; mini-decode and mini-prefill
are checked at full size on the rows of sampled experts, in the launch
configuration bench.py times.
"""
import sys

import numpy as np
import pytest
import torch

import workloads
from int8_weight_moe_amd import (moe_expert_ffn, moe_forward, moe_mlp_forward, moe_permute, moe_quantize_rows_fp8,
                                 moe_route, pack_bf16_experts, quantize_experts_fp8)
from int8_weight_moe_amd._lib import MOE_PATH_AUTO, MOE_PATH_STREAM, MOE_PATH_TILED, MOE_W_BF16, MOE_W_FP8
from oracle import fp8 as ofp8
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


def _fp8_oracle(src: dict, scale: str, experts=None) -> dict:
    """Oracle e4m3 quantization: codes decoded to their values, scales as stored."""
    W = {}
    for k in ("gate", "up", "down"):
        w = src["w_" + k] if experts is None else src["w_" + k][experts]
        codes, sc = ofp8.quantize_rows_fp8(np64(w), scale)
        W["q_" + k], W["s_" + k], W["c_" + k] = ofp8.e4m3_decode(codes), sc, codes
    return W


def _make(fmt, src, scale_dtype):
    ws = [src[k].cuda() for k in ("w_gate", "w_up", "w_down")]
    return pack_bf16_experts(*ws) if fmt == "bf16" else quantize_experts_fp8(*ws, scale_dtype)


def _oracle_weights(fmt, src, scale, experts=None):
    return _unquantized(src, experts) if fmt == "bf16" else _fp8_oracle(src, scale, experts)


# --------------------------------------------------------------------------- fp8 quantizer
@pytest.mark.parametrize("src_dt,scale", [("f32", "f32"), ("f32", "bf16"), ("bf16", "bf16"), ("bf16", "f32")])
def test_fp8_quantizer_is_bit_exact(src_dt, scale):
    rng = np.random.default_rng(31)
    w = (rng.standard_normal((96, 320)) * 0.02).astype(np.float32)
    w[3] = 0.0                                   # zero row
    w[5, 7] = -np.abs(w[5]).max() * 4            # negative absmax
    w[9, :64] *= 1e-5                            # subnormal codes
    # exact e4m3 midpoints times a power-of-two scale: ties to even
    vals = ofp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[1:] + vals[:-1]) / 2
    w[11, :] = 0.0
    w[11, 0] = 448.0 * 2.0 ** -10
    w[11, 1:1 + 100] = mids[::-1][:100] * 2.0 ** -10
    w[12] = -w[11]
    wt = torch.from_numpy(w)
    if src_dt == "bf16":
        wt = wt.to(torch.bfloat16)
    q, s = moe_quantize_rows_fp8(wt.cuda(), torch.float32 if scale == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    codes, sref = ofp8.quantize_rows_fp8(np64(wt), scale)
    assert np.array_equal(np64(s), sref)
    assert np.array_equal(q.cpu().numpy(), codes)


def test_bf16_packing_is_the_byte_tiling():
    w = workloads.Workload("pack", T=1, d=128, f=192, E=2, K=1, act="bf16", scale="bf16", weight_src="bf16", seed=3)
    src = workloads.draw_expert_weights(w, "cpu")
    ex = pack_bf16_experts(*(src[k].cuda() for k in ("w_gate", "w_up", "w_down")))
    assert ex.fmt == MOE_W_BF16 and ex.s_gate is None
    for k in ("gate", "up", "down"):
        got = getattr(ex, "q_" + k).cpu().view(torch.int8).numpy()
        want = src["w_" + k].view(torch.int8).numpy()
        assert np.array_equal(tiled_to_rowmajor(got.reshape(want.shape)), want), k


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("path", [MOE_PATH_AUTO, MOE_PATH_STREAM, MOE_PATH_TILED])
@pytest.mark.parametrize("T,d,f,E,K", [(64, 256, 512, 16, 2), (1, 128, 192, 4, 2), (300, 384, 640, 8, 2),
                                       (129, 256, 320, 4, 4), (40, 256, 256, 16, 2)])
def test_weight_formats_match_oracle(fmt, path, T, d, f, E, K):
    w = workloads.Workload("wfmt", T=T, d=d, f=f, E=E, K=K, act="bf16", scale="bf16", weight_src="bf16", seed=11)
    x = workloads.draw_activations(w)
    wr, _ = workloads.draw_router(w)
    src = workloads.draw_expert_weights(w, "cpu")
    ex = _make(fmt, src, torch.bfloat16)
    assert ex.fmt == (MOE_W_BF16 if fmt == "bf16" else MOE_W_FP8)
    y, ids, gw = moe_forward(x.cuda(), wr.cuda(), None, ex, K, path=path)
    y2, _, _ = moe_forward(x.cuda(), wr.cuda(), None, ex, K, path=path)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    x64, wr64 = np64(x), np64(wr)
    logits = omoe.router_logits(x64, wr64)
    check_routing(ids.cpu().numpy(), gw.cpu().numpy(), logits, K)
    ref = omoe.moe_forward(x64, wr64, None, _oracle_weights(fmt, src, "bf16"), K, ids=ids.cpu().numpy())
    assert_close_to_oracle(np64(y), ref["y"], f"{fmt} weights T={T} path={path}")


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("path", [MOE_PATH_STREAM, MOE_PATH_TILED])
@pytest.mark.parametrize("T", [1, 64, 200])
def test_weight_formats_dense_mlp(fmt, path, T):
    w = workloads.Workload("wmlp", T=T, d=256, f=384, E=1, K=1, act="bf16", scale="bf16", weight_src="bf16",
                           seed=5)
    x = workloads.draw_activations(w)
    src = workloads.draw_expert_weights(w, "cpu")
    ex = _make(fmt, src, torch.bfloat16)
    y = moe_mlp_forward(x.cuda(), ex, path=path)
    torch.cuda.synchronize()
    W = _oracle_weights(fmt, src, "bf16")
    ref = omoe.expert_swiglu(np64(x), W["q_gate"][0], W["s_gate"][0], W["q_up"][0], W["s_up"][0],
                             W["q_down"][0], W["s_down"][0])
    assert_close_to_oracle(np64(y), ref, f"{fmt}-weight MLP T={T}")


ROWS_PER_EXPERT = 256


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("name,n_experts", [("mini-decode", 3), ("mini-prefill", 2)])
def test_weight_formats_workload_sampled_rows(fmt, name, n_experts):
    w = workloads.WORKLOADS[name]
    dev = torch.device("cuda:0")
    _say(f"{name}: drawing weights ({fmt})")
    src = workloads.draw_expert_weights(w, dev)
    ex = pack_bf16_experts(src["w_gate"], src["w_up"], src["w_down"]) if fmt == "bf16" else \
        quantize_experts_fp8(src["w_gate"], src["w_up"], src["w_down"], workloads.TORCH_DTYPE[w.scale])
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
        W = _oracle_weights(fmt, {k: v[e] for k, v in src.items()}, w.scale)
        if fmt == "fp8":   # the library's codes and scales of this expert are the oracle's
            for k in ("gate", "up", "down"):
                got = tiled_to_rowmajor(getattr(ex, "q_" + k)[e].cpu().view(torch.int8).numpy()).view(np.uint8)
                assert np.array_equal(got, W["c_" + k]), f"fp8 codes differ (expert {e}, {k})"
                assert np.array_equal(np64(getattr(ex, "s_" + k)[e]), W["s_" + k])
        toks = ss_h[r0:r1] // w.K
        ref = omoe.expert_swiglu(x64[toks], W["q_gate"], W["s_gate"], W["q_up"], W["s_up"], W["q_down"],
                                 W["s_down"])
        assert_close_to_oracle(rows_h[r0:r1], ref, f"{name} {fmt} weights, expert {e}")
    del src, ex
    torch.cuda.empty_cache()
