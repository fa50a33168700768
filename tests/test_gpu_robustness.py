"""Large-magnitude activation rows through the layer, against the oracle.

Source: Jamba-1.5 paper, "Activation Loss": during pre-training some
activations grew to about 4e6 for certain tokens; the activation loss term
brought them down to a few thousand. The layer keeps activations in bf16 (no
fp16 range limit), so such rows must come out right on both FFN schedules.
Here a few token rows are scaled to those magnitudes (the bf16 values given to
the GPU are the values given to the oracle) and every token is checked on its
own: |y_t - ref_t| <= 1e-2 * max|ref_t| + 1e-3, so the small rows are held to
their own scale, not the big rows'.
"""
import numpy as np
import pytest
import torch

import workloads
from int8_weight_moe_amd import moe_forward
from int8_weight_moe_amd._lib import MOE_PATH_STREAM, MOE_PATH_TILED
from oracle import moe as omoe
from tests.helpers import GATE_W_ATOL, TIE_GAP, experts_to_device, np64, quantize_experts_oracle

pytestmark = pytest.mark.gpu


def _check_routing_scaled(ids_g, w_g, logits, K):
    """Routing check whose tie gap and weight tolerance scale with the row's
    logit magnitude: fp32 logits of a row of size ~s carry an absolute error of
    order 1e-7 * s * sqrt(d), far above the fixed gap of the unscaled rows."""
    ids_ref, w_ref = omoe.topk_gate(logits, K)
    mag = np.max(np.abs(logits), axis=1)
    gap = TIE_GAP + 1e-6 * mag
    srt = np.sort(logits, axis=1)[:, ::-1]
    for t in range(logits.shape[0]):
        chosen = logits[t, ids_g[t]]
        assert len(set(ids_g[t].tolist())) == K
        assert np.all(np.abs(chosen - srt[t, :K]) <= gap[t]), f"token {t}: not a top-{K} choice"
        if srt[t, K - 1] - srt[t, K] > gap[t] and np.all(np.diff(srt[t, :K]) < -gap[t]):
            assert np.array_equal(ids_g[t], ids_ref[t]), f"token {t}: ids differ without a near tie"
            atol = GATE_W_ATOL + 0.5 * gap[t]
            np.testing.assert_allclose(w_g[t], w_ref[t], rtol=0, atol=atol)
    assert np.all(np.abs(w_g.sum(axis=1) - 1.0) <= 1e-5)


@pytest.mark.parametrize("path", [MOE_PATH_STREAM, MOE_PATH_TILED])
@pytest.mark.parametrize("scale", [3.0e3, 4.0e6])
def test_large_magnitude_rows(path, scale):
    T, d, f, E, K = 300, 256, 512, 16, 2
    w = workloads.Workload("big", T=T, d=d, f=f, E=E, K=K, seed=17)
    x = workloads.draw_activations(w).float()
    rng = np.random.default_rng(23)
    big = rng.choice(T, size=24, replace=False)
    x[torch.from_numpy(big)] *= scale
    x = x.to(torch.bfloat16)
    wr, _ = workloads.draw_router(w)
    W = quantize_experts_oracle(workloads.draw_expert_weights(w, "cpu"), "bf16")
    ex = experts_to_device(W, torch.bfloat16)
    y, ids, gw = moe_forward(x.cuda(), wr.cuda(), None, ex, K, path=path)
    torch.cuda.synchronize()
    x64, wr64 = np64(x), np64(wr)
    assert np.max(np.abs(x64[big])) > 0.5 * scale
    logits = omoe.router_logits(x64, wr64, None)
    ids_g = ids.cpu().numpy()
    _check_routing_scaled(ids_g, gw.cpu().numpy(), logits, K)
    # silu(z) = z / (1 + exp(-z)): for z below about -709 exp overflows to inf
    # in fp64 and the quotient is -0, the correct limit
    with np.errstate(over="ignore"):
        ref = omoe.moe_forward(x64, wr64, None, W, K, ids=ids_g)["y"]
    yg = np64(y)
    assert np.all(np.isfinite(yg))
    tol = 1e-2 * np.max(np.abs(ref), axis=1) + 1e-3
    err = np.max(np.abs(yg - ref), axis=1)
    bad = np.nonzero(err > tol)[0]
    assert bad.size == 0, f"rows {bad[:8]}: err {err[bad[:8]]} > tol {tol[bad[:8]]}"
    # the big rows really are big at the output, the others are not
    assert np.median(np.max(np.abs(ref[big]), axis=1)) > 100 * np.median(np.max(np.abs(np.delete(ref, big, 0)), axis=1))
