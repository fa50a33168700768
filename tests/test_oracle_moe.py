"""Pins for the oracle MoE layer (oracle/moe.py).

Each test ties a part of the oracle to something other than its own formula:
  * gate: the closed form of a 2-way renormalised softmax (a logistic of the
    logit gap), a brute-force sort, the K = E case (plain softmax), K = 1;
  * permutation: a hand-written counting sort;
  * expert FFN: with E = 1, K = 1 the layer is the textbook dense SwiGLU MLP
    on the dequantized weights, evaluated with torch's CPU fp64 ops
    (torch.nn.functional.silu, matmul);
  * mixture: K = E equals the dense mixture over all experts;
  * whole layer: a scalar Python loop per token, and token-permutation
    equivariance.
"""
import math

import numpy as np
import pytest
import torch

from oracle import moe, quant


def _make_layer(rng, T, d, f, E, scale="bf16", bias=None):
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d)) * 0.3
    W = {}
    for name, shape in (("gate", (E, f, d)), ("up", (E, f, d)), ("down", (E, d, f))):
        q, s = quant.quantize_rows(rng.standard_normal(shape) * 0.1, scale)
        W["q_" + name], W["s_" + name] = q, s
    return x, wr, bias, W


# --------------------------------------------------------------------------- gate
def test_top2_weights_are_logistic_of_gap():
    rng = np.random.default_rng(10)
    l = rng.standard_normal((200, 16)) * 3
    ids, w = moe.topk_gate(l, 2)
    l1 = l[np.arange(200), ids[:, 0]]
    l2 = l[np.arange(200), ids[:, 1]]
    w1 = np.array([1.0 / (1.0 + math.exp(b - a)) for a, b in zip(l1, l2)])
    np.testing.assert_allclose(w[:, 0], w1, rtol=1e-13, atol=0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-15, atol=1e-15)
    assert np.all(l1 >= l2)


@pytest.mark.parametrize("K", [1, 2, 3, 5])
def test_topk_ids_match_bruteforce_sort(K):
    rng = np.random.default_rng(11)
    l = np.round(rng.standard_normal((300, 8)) * 2, 1)   # coarse values -> many exact ties
    ids, _ = moe.topk_gate(l, K)
    for t in range(l.shape[0]):
        want = sorted(range(8), key=lambda e: (-l[t, e], e))[:K]
        assert list(ids[t]) == want


def test_exact_ties_go_to_lower_index():
    l = np.array([[0.0, 1.0, 1.0, 1.0], [2.0, 2.0, -1.0, 2.0]])
    ids, w = moe.topk_gate(l, 2)
    assert ids.tolist() == [[1, 2], [0, 1]]
    np.testing.assert_allclose(w, 0.5)


def test_k_equals_e_gives_plain_softmax_and_k1_gives_one():
    rng = np.random.default_rng(12)
    l = rng.standard_normal((50, 6))
    ids, w = moe.topk_gate(l, 6)
    ex = np.exp(l)
    p = ex / ex.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(w, np.take_along_axis(p, ids.astype(np.int64), 1), rtol=1e-14)
    _, w1 = moe.topk_gate(l, 1)
    assert np.all(w1 == 1.0)


def test_near_tie_flags():
    l = np.array([
        [3.0, 2.0, 1.0, 0.0],          # clear
        [3.0, 3.0 - 5e-5, 1.0, 0.0],   # order of the two chosen is fragile
        [3.0, 2.0, 2.0 - 5e-5, 0.0],   # membership is fragile
        [3.0, 2.0, 1.0, 1.0 - 5e-5],   # tie outside the first K+1: not flagged
    ])
    assert moe.near_tie_flags(l, 2).tolist() == [False, True, True, False]


# --------------------------------------------------------------------------- permute
def test_permute_matches_counting_sort():
    rng = np.random.default_rng(13)
    for T, K, E in ((1, 1, 1), (7, 2, 16), (300, 2, 16), (64, 3, 5)):
        ids = rng.integers(0, E, size=(T, K))
        ids[: T // 3] = 0   # a hot expert
        off, ss, s2r = moe.permute(ids, E)
        flat = ids.reshape(-1).tolist()
        want_slots = [s for e in range(E) for s in range(len(flat)) if flat[s] == e]
        want_off = [0]
        for e in range(E):
            want_off.append(want_off[-1] + flat.count(e))
        assert off.tolist() == want_off
        assert ss.tolist() == want_slots
        for r, s in enumerate(want_slots):
            assert s2r[s] == r


def test_permute_rejects_bad_ids():
    with pytest.raises(ValueError):
        moe.permute(np.array([[0, 16]]), 16)


# --------------------------------------------------------------------------- experts
def test_single_expert_is_textbook_swiglu_mlp():
    rng = np.random.default_rng(14)
    x, wr, _, W = _make_layer(rng, T=9, d=32, f=48, E=1)
    out = moe.moe_forward(x, wr, None, W, K=1)
    deq = {k: torch.from_numpy(W["q_" + k].astype(np.float64)[0]) * torch.from_numpy(W["s_" + k][0])[:, None]
           for k in ("gate", "up", "down")}
    xt = torch.from_numpy(x)
    ref = (torch.nn.functional.silu(xt @ deq["gate"].T) * (xt @ deq["up"].T)) @ deq["down"].T
    assert np.all(out["ids"] == 0) and np.all(out["w"] == 1.0)
    np.testing.assert_allclose(out["y"], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_expert_hidden_is_textbook_gated_activation_on_any_channel_subset():
    """h = silu(x W_g^T) * (x W_u^T) on the dequantized weights (torch CPU fp64), and a
    subset of channels gives the same columns as the whole matrix."""
    rng = np.random.default_rng(15)
    x, _, _, W = _make_layer(rng, T=7, d=32, f=40, E=1)
    h = moe.expert_hidden(x, W["q_gate"][0], W["s_gate"][0], W["q_up"][0], W["s_up"][0])
    deq = {k: torch.from_numpy(W["q_" + k].astype(np.float64)[0]) * torch.from_numpy(W["s_" + k][0])[:, None]
           for k in ("gate", "up")}
    xt = torch.from_numpy(x)
    ref = torch.nn.functional.silu(xt @ deq["gate"].T) * (xt @ deq["up"].T)
    np.testing.assert_allclose(h, ref.numpy(), rtol=1e-12, atol=1e-12)
    ch = np.array([39, 0, 17, 17, 5])
    hs = moe.expert_hidden(x, W["q_gate"][0][ch], W["s_gate"][0][ch], W["q_up"][0][ch], W["s_up"][0][ch])
    np.testing.assert_allclose(hs, h[:, ch], rtol=1e-12, atol=1e-14)   # BLAS may sum in another order


def test_k_equals_e_is_dense_mixture():
    rng = np.random.default_rng(15)
    x, wr, _, W = _make_layer(rng, T=6, d=16, f=24, E=5)
    bias = rng.standard_normal(5)
    y = moe.moe_forward(x, wr, bias, W, K=5)["y"]
    np.testing.assert_allclose(y, moe.dense_mixture(x, wr, bias, W), rtol=1e-12, atol=1e-13)


def test_vectorised_layer_matches_scalar_loop():
    rng = np.random.default_rng(16)
    for K, scale in ((2, "bf16"), (3, "f32")):
        x, wr, _, W = _make_layer(rng, T=5, d=8, f=12, E=4, scale=scale)
        bias = np.array([0.5, 0.0, -0.25, 0.0])
        y = moe.moe_forward(x, wr, bias, W, K=K)["y"]
        np.testing.assert_allclose(y, moe.moe_forward_loop(x, wr, bias, W, K), rtol=1e-12, atol=1e-14)


def test_token_permutation_equivariance():
    rng = np.random.default_rng(17)
    x, wr, _, W = _make_layer(rng, T=40, d=32, f=40, E=16)
    y = moe.moe_forward(x, wr, None, W, K=2)
    perm = rng.permutation(40)
    yp = moe.moe_forward(x[perm], wr, None, W, K=2)
    assert np.array_equal(yp["ids"], y["ids"][perm])
    np.testing.assert_allclose(yp["y"], y["y"][perm], rtol=1e-12, atol=1e-14)


def test_forced_routing_recomputes_gate_weights():
    rng = np.random.default_rng(18)
    x, wr, _, W = _make_layer(rng, T=4, d=8, f=8, E=4)
    ids = np.array([[3, 0], [1, 2], [0, 1], [2, 3]], dtype=np.int32)
    out = moe.moe_forward(x, wr, None, W, K=2, ids=ids)
    l = moe.router_logits(x, wr)
    for t in range(4):
        a, b = l[t, ids[t, 0]], l[t, ids[t, 1]]
        assert abs(out["w"][t, 0] - 1.0 / (1.0 + math.exp(b - a))) < 1e-14
