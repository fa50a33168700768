"""Pins for the oracle's FP8 (OCP e4m3) weight encoding (oracle/fp8.py).

The e4m3 format is pinned to torch's float8_e4m3fn type (a library routine:
the decoding of every code byte and the float32 -> e4m3 conversion), the
rounding to a brute-force nearest-value search over exact rationals, and the
quantizer (the reading stated in the oracle: per output channel, absmax/448,
ties to even, saturating) to exact rational arithmetic and closed forms.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import fp8
from tests.test_oracle_quant import _frac_round_to_bits

ALL_CODES = np.arange(256, dtype=np.uint8)


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _finite_table():
    """(value Fraction, code) of every finite non-negative e4m3 code, from torch's decoding."""
    vals = _torch_decode(ALL_CODES[:0x7F])
    return [(Fraction(float(v)), int(c)) for v, c in zip(vals, ALL_CODES[:0x7F])]


def _brute_round(x: Fraction, table) -> Fraction:
    """Nearest finite e4m3 value (ties to the even code), saturating beyond 448."""
    a = abs(x)
    best = min(table, key=lambda vc: (abs(a - vc[0]), vc[1] % 2))
    v = best[0]
    return -v if x < 0 else v


# --------------------------------------------------------------------------- the format
def test_decode_matches_torch_for_every_code():
    got = fp8.e4m3_decode(ALL_CODES)
    ref = _torch_decode(ALL_CODES)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])
    assert np.nanmax(got) == 448.0 and np.nanmin(got[got > 0]) == 2.0 ** -9
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def test_encode_inverts_decode():
    finite = ALL_CODES[(ALL_CODES & 0x7F) != 0x7F]
    finite = finite[finite != 0x80]                      # -0 encodes as the canonical +0
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_decode(finite)), finite)
    assert fp8.e4m3_encode(np.array([-0.0]))[0] == 0
    with pytest.raises(ValueError):
        fp8.e4m3_encode(np.array([449.0]))
    with pytest.raises(ValueError):
        fp8.e4m3_encode(np.array([1.0 + 2.0 ** -5]))     # not an e4m3 value


def test_round_matches_torch_conversion():
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.standard_normal(20000) * 100.0,
        rng.standard_normal(20000) * 2.0 ** -7,          # subnormal and lowest binades
        rng.uniform(-448, 448, 20000),
    ]).astype(np.float32)
    # exact midpoints between neighbouring finite values (both signs)
    vals = fp8.e4m3_decode(ALL_CODES[:0x7F])
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    v = np.concatenate([v[np.abs(v) <= 448], mids, -mids])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.round_to_e4m3(v.astype(np.float64))
    assert np.array_equal(got, ref)


def test_round_matches_brute_force_nearest():
    rng = np.random.default_rng(8)
    table = _finite_table()
    v = np.concatenate([rng.standard_normal(300) * 10.0 ** rng.integers(-3, 3, size=300),
                        [464.0, 480.0, 1000.0, -1000.0, 2.0 ** -10, 3 * 2.0 ** -11, -2.0 ** -10]])
    got = fp8.round_to_e4m3(v)
    for a, g in zip(v, got):
        assert Fraction(float(g)) == _brute_round(Fraction(float(a)), table), a


def test_round_saturates_and_ties_to_even():
    r = fp8.round_to_e4m3(np.array([448.0, 460.0, 464.0, 470.0, 1e6, -1e6, 2.0 ** -10, 3 * 2.0 ** -10,
                                     1.0625, 1.1875, -1.0625]))
    assert list(r) == [448.0, 448.0, 448.0, 448.0, 448.0, -448.0, 0.0, 2.0 ** -8, 1.0, 1.25, -1.0]


# --------------------------------------------------------------------------- the quantizer
def _frac_quantize_row_fp8(row, scale_bits, table):
    fr = [Fraction(float(v)) for v in row]
    a = max(abs(v) for v in fr)
    if a == 0:
        return [Fraction(0)] * len(fr), Fraction(0)
    s = _frac_round_to_bits(a / 448, scale_bits)
    return [_brute_round(v / s, table) for v in fr], s


@pytest.mark.parametrize("src,scale,scale_bits", [("f32", "bf16", 8), ("bf16", "bf16", 8), ("f32", "f32", 24)])
def test_quantize_fp8_matches_exact_rationals(src, scale, scale_bits):
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((12, 48)) * 0.02).astype(np.float32)
    if src == "bf16":
        w = torch.from_numpy(w).to(torch.bfloat16).float().numpy()
    w[4] = 0.0
    w[6, 2] = -np.abs(w[6]).max() * 3
    w[8, :8] *= 1e-4                       # tiny entries land in the subnormal codes
    codes, s = fp8.quantize_rows_fp8(w.astype(np.float64), scale)
    assert codes.dtype == np.uint8
    table = _finite_table()
    vals = fp8.e4m3_decode(codes)
    for r in range(w.shape[0]):
        qr, sr = _frac_quantize_row_fp8(w[r], scale_bits, table)
        assert Fraction(float(s[r])) == sr
        assert [Fraction(float(v)) for v in vals[r]] == qr


def test_quantize_fp8_absmax_lands_on_448_and_round_trip_bound():
    rng = np.random.default_rng(10)
    w = torch.from_numpy(rng.standard_normal((128, 256)).astype(np.float32) * np.float32(0.02)) \
        .to(torch.bfloat16).double().numpy()
    for scale in ("bf16", "f32"):
        codes, s = fp8.quantize_rows_fp8(w, scale)
        q = fp8.e4m3_decode(codes)
        assert np.all(np.abs(q).max(axis=1) == 448.0)
        # |w/s - q| is at most half the quantum of q's binade (4 significant bits)
        r = w / s[:, None]
        _, e = np.frexp(np.maximum(np.abs(q), np.abs(r)))
        half_quantum = np.ldexp(1.0, np.maximum(e - 4, -9) - 1)
        assert np.all(np.abs(r - q) <= half_quantum + 448.0 * 2.0 ** -8)   # + the scale rounding at the top


def test_quantize_fp8_zero_row_and_lossless_grid():
    codes, s = fp8.quantize_rows_fp8(np.zeros((2, 16)), "bf16")
    assert np.all(s == 0) and np.all(codes == 0)
    # rows that are e4m3 values times a power of two come back exactly
    rng = np.random.default_rng(11)
    finite = fp8.e4m3_decode(ALL_CODES[(ALL_CODES & 0x7F) != 0x7F])
    q = rng.choice(finite, size=(6, 32))
    q[:, 0] = 448.0
    w = q * 2.0 ** -12
    codes, s = fp8.quantize_rows_fp8(w, "bf16")
    assert np.all(s == 2.0 ** -12)
    assert np.array_equal(fp8.dequantize_rows_fp8(codes, s), w)
