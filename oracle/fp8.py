"""FP8 (OCP e4m3) weight variant, oracle side (test infrastructure, see the package header).

Source: Jamba-1.5 paper, "Serving Considerations and Improvements": ExpertsInt8
is compared with FP8 weights, whose latency it matches; FP8 is the encoding
the paper's comparison uses on H100. The encoding here is OCP FP8 E4M3 ("fn"
variant, the one gfx950 converts natively): 1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits; exponent field 0 holds the subnormals m * 2**-9; the
largest finite value is 1.75 * 2**8 = 448; codes 0x7F and 0xFF are NaN; there
are no infinities.

The pages give no granularity for the FP8 weights. Reading taken here, the
same as the int8 scheme apart from the encoding: symmetric, one scale per
output channel (row), scale = max|w| / 448 rounded once, to nearest-even,
into the scale dtype; codes = the e4m3 value nearest to w / scale (ties to
the even mantissa), saturated to +-448; an all-zero row stores scale 0 and
codes 0.

All arithmetic is fp64 on exact copies of the fp32/bf16 source values.
"""
from __future__ import annotations

import numpy as np

from oracle import quant

E4M3_MAX = 448.0
E4M3_SUBNORMAL_EXP = -9      # subnormal quantum 2**-9 (exponent field 0)
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_BIAS = 7


def round_to_e4m3(v) -> np.ndarray:
    """Nearest e4m3 value of each fp64 input (ties to even), saturated to +-448; fp64 out.

    An e4m3 value carries 4 significant bits: with v = m * 2**e, 0.5 <= |m| < 1,
    the quantum of v's binade is 2**(e - 4), and never below the subnormal
    quantum 2**-9. Rounding v / quantum to the nearest integer (ties to even)
    and scaling back gives the nearest representable value; a carry into the
    next binade lands on its first value, which is representable too.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("round_to_e4m3: non-finite input")
    _, e = np.frexp(v)
    step = np.maximum(e - 4, E4M3_SUBNORMAL_EXP)
    out = np.ldexp(np.rint(np.ldexp(v, -step)), step)
    return np.clip(out, -E4M3_MAX, E4M3_MAX)


def e4m3_decode(codes) -> np.ndarray:
    """Value of each e4m3 code byte (fp64; NaN for 0x7F and 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    mf = c & 0x7
    sub = np.ldexp(mf.astype(np.float64), E4M3_SUBNORMAL_EXP)
    nor = np.ldexp(1.0 + mf / 8.0, ef - E4M3_BIAS)
    val = sign * np.where(ef == 0, sub, nor)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e4m3_encode(values) -> np.ndarray:
    """Code byte of each exact e4m3 value (the inverse of e4m3_decode on finite values)."""
    v = np.asarray(values, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > E4M3_MAX) or not np.all(np.isfinite(v)):
        raise ValueError("e4m3_encode: value outside the finite e4m3 range")
    m, e = np.frexp(a)                       # a = (2m) * 2**(e-1), 1 <= 2m < 2
    normal = a >= E4M3_MIN_NORMAL
    ef = np.where(normal, e - 1 + E4M3_BIAS, 0)
    mf = np.where(normal, (2.0 * m - 1.0) * 8.0, np.ldexp(a, -E4M3_SUBNORMAL_EXP))
    if not np.all(mf == np.round(mf)):
        raise ValueError("e4m3_encode: value is not an e4m3 value")
    code = (ef.astype(np.int64) << 3) | mf.astype(np.int64)
    code = np.where(np.signbit(v) & (a > 0), code | 0x80, code)
    return code.astype(np.uint8)


def quantize_rows_fp8(w, scale_dtype: str):
    """Per-row symmetric e4m3 quantization of w [..., rows, cols].

    Returns (codes uint8 [..., rows, cols], s fp64 [..., rows]) with
    w ~= e4m3_decode(codes) * s[..., None] and every s a value of `scale_dtype`.

    Exactness: w holds at most 24 significant bits and s at most 24, and the
    e4m3 rounding midpoints hold at most 5, so the fp64 quotient w / s can only
    land on a midpoint when the exact quotient is that midpoint; one fp64
    division followed by one rounding gives the correctly rounded result of
    the exact rational.
    """
    w = np.asarray(w, dtype=np.float64)
    a = np.max(np.abs(w), axis=-1)
    s = quant.round_to(a / E4M3_MAX, scale_dtype)
    safe = np.where(s > 0, s, 1.0)
    q = round_to_e4m3(w / safe[..., None])
    q = np.where((s > 0)[..., None], q, 0.0)
    return e4m3_encode(q), s


def dequantize_rows_fp8(codes, s) -> np.ndarray:
    """w_hat = e4m3 value * s per row, fp64 (exact: 4-bit times <=24-bit)."""
    return e4m3_decode(codes) * np.asarray(s, dtype=np.float64)[..., None]
