"""ExpertsInt8 quantizer, oracle side (test infrastructure, see the package header).

Source: Jamba-1.5 paper, "Serving Considerations and Improvements": the MoE
and MLP weights are quantized to INT8 and stored that way, quantization takes
seconds at load time and needs no calibration, and the values are turned back
into BF16 before the contraction.

The paper does not give the granularity or the rounding. Reading taken here:
symmetric (no zero point), one scale per output channel (one row of the
(out, in) weight matrix), scale = max|w| / 127 rounded once, to nearest-even,
into the scale dtype, and codes q = round-half-even(w / stored scale) clamped
to [-127, 127]. An all-zero row stores scale 0 and codes 0.

All arithmetic is fp64 on exact copies of the fp32/bf16 source values.
"""
from __future__ import annotations

import numpy as np

BF16_MIN_EXP = -133   # 2**-133 is the smallest positive bf16 (subnormal) value


def round_to_bf16(v) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of each fp64 input, returned as fp64.

    bfloat16 carries 8 significant bits: write v = m * 2**e with 0.5 <= |m| < 1,
    then keep rint(m * 2**8) * 2**(e - 8). Values below the normal range are
    rounded on the fixed subnormal grid 2**-133. Non-finite or out-of-range
    inputs are rejected.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("round_to_bf16: non-finite input")
    m, e = np.frexp(v)
    step_exp = np.maximum(e - 8, BF16_MIN_EXP)
    out = np.ldexp(np.rint(np.ldexp(v, -step_exp)), step_exp)
    if np.any(np.abs(out) > 3.3895313892515355e38):  # largest finite bf16
        raise ValueError("round_to_bf16: value beyond the bf16 range")
    return out


def round_to_f32(v) -> np.ndarray:
    """Nearest fp32 value (ties to even; IEEE conversion), returned as fp64."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to(v, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16(v)
    if dtype == "f32":
        return round_to_f32(v)
    raise ValueError(f"unknown dtype {dtype!r}")


def quantize_rows(w, scale_dtype: str):
    """Per-row symmetric int8 quantization of w [..., rows, cols].

    Returns (q int8 [..., rows, cols], s fp64 [..., rows]) where every s is a
    value of `scale_dtype` and w ~= q * s[..., None].

    Exactness: w holds at most 24 significant bits and s at most 24, so their
    fp64 quotient can only land on a rounding midpoint when the exact quotient
    is that midpoint; one fp64 division followed by one rounding therefore
    gives the correctly rounded result of the exact rational, both for the
    scale (max|w| / 127) and for the codes (w / s).
    """
    w = np.asarray(w, dtype=np.float64)
    a = np.max(np.abs(w), axis=-1)
    s = round_to(a / 127.0, scale_dtype)
    safe = np.where(s > 0, s, 1.0)
    q = np.rint(w / safe[..., None])
    q = np.where((s > 0)[..., None], q, 0.0)
    q = np.clip(q, -127, 127).astype(np.int8)
    return q, s


def dequantize_rows(q, s) -> np.ndarray:
    """w_hat = q * s per row, in fp64 (exact: 8-bit times <=24-bit)."""
    return np.asarray(q, dtype=np.float64) * np.asarray(s, dtype=np.float64)[..., None]
