"""Shared helpers of the parity tests: input construction and the tolerance.

Inputs come from workloads.py (draws only). Expected values come from the
oracle only. The tolerance is the one the layer is held to:
    |gpu - ref| <= 1e-2 * max|ref| + 1e-3   (elementwise, max over the compared set)
Routing ids must equal the oracle's except on near-tie tokens (a gap below
1e-4 between neighbouring sorted logits among the first K+1), where any
selection that is valid under the oracle's logits is accepted.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import moe as omoe
from oracle import quant as oquant

TIE_GAP = 1e-4
GATE_W_ATOL = 1e-5


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy() if t.is_floating_point() else t.detach().cpu().numpy()


def assert_close_to_oracle(gpu: np.ndarray, ref: np.ndarray, what: str = "output"):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    tol = 1e-2 * np.max(np.abs(ref)) + 1e-3
    err = np.max(np.abs(gpu - ref)) if gpu.size else 0.0
    assert err <= tol, f"{what}: max |gpu-ref| = {err:.3e} > tol {tol:.3e}"
    return err / tol if tol > 0 else 0.0


def quantize_experts_oracle(src: dict, scale: str) -> dict:
    """Oracle quantization of host weights dict(w_gate, w_up, w_down) -> q_*/s_* numpy."""
    W = {}
    for k in ("gate", "up", "down"):
        W["q_" + k], W["s_" + k] = oquant.quantize_rows(np64(src["w_" + k]), scale)
    return W


def experts_to_device(W: dict, scale_dtype: torch.dtype, device="cuda"):
    """Oracle codes and scales -> Int8Experts on the GPU (codes tiled by the library's moe_pack_rows)."""
    from int8_weight_moe_amd import pack_experts
    t = {}
    for k in ("gate", "up", "down"):
        t["q_" + k] = torch.from_numpy(W["q_" + k]).to(device)
        t["s_" + k] = torch.from_numpy(W["s_" + k]).to(scale_dtype).to(device)
    return pack_experts(t["q_gate"], t["q_up"], t["q_down"], t["s_gate"], t["s_up"], t["s_down"])


def tiled_to_rowmajor(p: np.ndarray) -> np.ndarray:
    """Inverse of the tiled int8 layout (include/moe_int8.h, moe_pack_rows): a pure index permutation.

    Tiled byte order per matrix [R, C]: block (rg, ks) of 16 rows x 64 columns at
    block index rg*(C/64)+ks, element (r, c) at 256*(c/16) + 16*r + c%16 inside it.
    """
    shape = p.shape
    C = shape[-1]
    R = p.size // C
    a = p.reshape(R // 16, C // 64, 4, 16, 16)          # [rg, ks, g, r, b]
    return a.transpose(0, 3, 1, 2, 4).reshape(shape)    # [rg, r, ks, g, b]


def rowmajor_to_tiled(q: np.ndarray) -> np.ndarray:
    shape = q.shape
    C = shape[-1]
    R = q.size // C
    a = q.reshape(R // 16, 16, C // 64, 4, 16)          # [rg, r, ks, g, b]
    return a.transpose(0, 2, 3, 1, 4).reshape(shape)    # [rg, ks, g, r, b]


def check_routing(ids_gpu: np.ndarray, w_gpu: np.ndarray, logits: np.ndarray, K: int):
    """Bit-exact ids except near ties; gate weights within GATE_W_ATOL of the oracle's.

    Returns the boolean mask of near-tie tokens.
    """
    ids_ref, w_ref = omoe.topk_gate(logits, K)
    flags = omoe.near_tie_flags(logits, K, TIE_GAP)
    ok = ~flags
    assert np.array_equal(ids_gpu[ok], ids_ref[ok]), "routing ids differ on a token that is not a near tie"
    np.testing.assert_allclose(w_gpu[ok], w_ref[ok], rtol=0, atol=GATE_W_ATOL)
    # near ties: the GPU's choice must be a valid top-K under the oracle's logits
    srt = np.sort(logits, axis=1)[:, ::-1]
    for t in np.nonzero(flags)[0]:
        chosen = logits[t, ids_gpu[t]]
        assert len(set(ids_gpu[t].tolist())) == K
        assert np.all(np.abs(chosen - srt[t, :K]) <= TIE_GAP), f"token {t}: invalid near-tie selection"
    assert np.all(np.abs(w_gpu.sum(axis=1) - 1.0) <= 1e-5)
    return flags


def oracle_for_routing(x64, wr64, bias64, W, ids, K):
    """Oracle output for the given routing (gate weights recomputed from the oracle's logits)."""
    return omoe.moe_forward(x64, wr64, bias64, W, K, ids=ids)["y"]
