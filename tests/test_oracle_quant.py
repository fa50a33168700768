"""Pins for the oracle quantizer (oracle/quant.py).

The quantizer follows the ExpertsInt8 description (Jamba-1.5 paper, "Serving
Considerations and Improvements"); its exact form (symmetric, per output
channel, absmax/127, round-half-even) is the reading stated in the oracle.
These tests pin it to things other than its own formula:
  * bf16 rounding against torch's float32 -> bfloat16 conversion (a library
    routine) and against exact rational rounding;
  * the whole quantizer against exact rational arithmetic (fractions);
  * closed-form special cases and the round-trip bound |w - q s| <= s/2.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import quant


# --------------------------------------------------------------------------- exact reference helpers
def _frac_round_half_even(x: Fraction) -> int:
    n = x.numerator // x.denominator          # floor
    r = x - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def _frac_round_to_bits(v: Fraction, bits: int) -> Fraction:
    """Nearest number with `bits` significant bits (ties to even), exact."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    # v = sign * a * 2**e with 1 <= a < 2; spacing 2**(e - bits + 1)
    step = Fraction(2) ** (e - bits + 1)
    return sign * _frac_round_half_even(abs(v) / step) * step


def _frac_quantize_row(row, scale_bits):
    fr = [Fraction(float(v)) for v in row]
    a = max(abs(v) for v in fr)
    if a == 0:
        return [0] * len(fr), Fraction(0)
    s = _frac_round_to_bits(a / 127, scale_bits)
    q = [max(-127, min(127, _frac_round_half_even(v / s))) for v in fr]
    return q, s


# --------------------------------------------------------------------------- bf16 rounding
def test_round_to_bf16_matches_torch_conversion():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(0.02),
        rng.standard_normal(20000).astype(np.float32) * np.float32(1e-30),
        rng.standard_normal(20000).astype(np.float32) * np.float32(1e20),
    ])
    # exact midpoints between neighbouring bf16 values: low 16 bits = 0x8000
    bits = rng.integers(0x3000, 0x5000, size=4000, dtype=np.uint32) << 16 | 0x8000
    v = np.concatenate([v, bits.view(np.float32), -bits.view(np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = quant.round_to_bf16(v.astype(np.float64))
    assert np.array_equal(got, ref)


def test_round_to_bf16_matches_exact_rational_rounding():
    rng = np.random.default_rng(2)
    v = rng.standard_normal(500) * 10.0 ** rng.integers(-20, 20, size=500)
    got = quant.round_to_bf16(v)
    for a, g in zip(v, got):
        assert Fraction(float(g)) == _frac_round_to_bits(Fraction(float(a)), 8)


def test_round_to_bf16_subnormal_grid():
    tiny = 2.0 ** -133
    assert quant.round_to_bf16(np.array([tiny * 0.5]))[0] == 0.0          # tie -> even (0)
    assert quant.round_to_bf16(np.array([tiny * 1.5]))[0] == 2 * tiny     # tie -> even (2)
    assert quant.round_to_bf16(np.array([tiny * 0.51]))[0] == tiny


# --------------------------------------------------------------------------- quantizer
@pytest.mark.parametrize("src,scale,scale_bits", [("f32", "bf16", 8), ("bf16", "bf16", 8), ("f32", "f32", 24)])
def test_quantize_matches_exact_rationals(src, scale, scale_bits):
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((24, 40)) * 0.02).astype(np.float32)
    if src == "bf16":
        w = torch.from_numpy(w).to(torch.bfloat16).float().numpy()
    w[5] = 0.0                         # an all-zero row
    w[7, 3] = -np.abs(w[7]).max() * 2   # negative absmax
    q, s = quant.quantize_rows(w.astype(np.float64), scale)
    assert q.dtype == np.int8
    for r in range(w.shape[0]):
        qr, sr = _frac_quantize_row(w[r], scale_bits)
        assert Fraction(float(s[r])) == sr
        assert list(q[r].astype(int)) == qr


def test_quantize_round_trip_bound_and_range():
    rng = np.random.default_rng(4)
    w = rng.standard_normal((256, 512)).astype(np.float32) * np.float32(0.02)
    w = torch.from_numpy(w).to(torch.bfloat16).double().numpy()
    for scale in ("bf16", "f32"):
        q, s = quant.quantize_rows(w, scale)
        err = np.abs(w - q.astype(np.float64) * s[:, None])
        assert np.all(err <= s[:, None] / 2)
        assert q.min() >= -127 and q.max() <= 127
        # the absmax element always lands on +-127: |a/s| is within 2**-8 of 127
        assert np.all(np.abs(q).max(axis=1) == 127)


def test_quantize_power_of_two_grid_is_lossless():
    rng = np.random.default_rng(5)
    k = rng.integers(-127, 128, size=(8, 64))
    k[:, 0] = 127 * np.where(np.arange(8) % 2 == 0, 1, -1)
    w = k * 2.0 ** -7
    for scale in ("bf16", "f32"):
        q, s = quant.quantize_rows(w, scale)
        assert np.all(s == 2.0 ** -7)
        assert np.array_equal(q.astype(np.int64), k)
        assert np.array_equal(quant.dequantize_rows(q, s), w)


def test_quantize_zero_row():
    q, s = quant.quantize_rows(np.zeros((2, 16)), "bf16")
    assert np.all(s == 0) and np.all(q == 0)


def test_quantize_ties_go_to_even():
    # row absmax 127 * 2**-7 -> s = 2**-7; w = (n + 1/2) * s sits exactly on a tie
    w = np.array([[127 * 2.0 ** -7, 2.5 * 2.0 ** -7, 3.5 * 2.0 ** -7, -2.5 * 2.0 ** -7, -0.5 * 2.0 ** -7]])
    q, s = quant.quantize_rows(w, "bf16")
    assert s[0] == 2.0 ** -7
    assert list(q[0]) == [127, 2, 4, -2, 0]
