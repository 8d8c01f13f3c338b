"""Pins for the oracle's FP8 format tables and its round-to-nearest-even encoder.

Independent references: the OCP 8-bit format constants (largest finite value,
smallest subnormal, code counts) and torch's CPU float8_e4m3fn / float8_e5m2
dtypes, whose casts round to nearest even.
"""
import math

import numpy as np
import pytest
import torch

import oracle

TORCH_DT = {oracle.E4M3: torch.float8_e4m3fn, oracle.E5M2: torch.float8_e5m2}


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_decode_table_matches_torch(fmt):
    tab = oracle.decode_table(fmt)
    ref = torch.arange(256, dtype=torch.uint8).view(TORCH_DT[fmt]).to(torch.float64).numpy()
    same = (tab == ref) | (np.isnan(tab) & np.isnan(ref))
    assert same.all(), np.nonzero(~same)
    # signed zero of code 0x80
    assert math.copysign(1.0, tab[0x80]) == -1.0


def test_format_constants():
    e4 = oracle.decode_table(oracle.E4M3)
    e5 = oracle.decode_table(oracle.E5M2)
    assert e4[0x7E] == 448.0 and e4[0x08] == 2.0 ** -6 and e4[0x01] == 2.0 ** -9
    assert e4[0x38] == 1.0 and np.isnan(e4[0x7F]) and np.isnan(e4[0xFF])
    assert np.isfinite(e4).sum() == 254
    assert e5[0x7B] == 57344.0 and e5[0x04] == 2.0 ** -14 and e5[0x01] == 2.0 ** -16
    assert e5[0x3C] == 1.0 and e5[0x7C] == math.inf and e5[0xFC] == -math.inf
    assert np.isfinite(e5).sum() == 248 and np.isnan(e5).sum() == 6
    # positive finite codes are ordered by magnitude
    assert (np.diff(e4[:0x7F]) > 0).all() and (np.diff(e5[:0x7C]) > 0).all()


def _torch_codes(vals32, fmt):
    t = torch.from_numpy(np.asarray(vals32, np.float32))
    return t.to(TORCH_DT[fmt]).view(torch.uint8).numpy()


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_encode_midpoints_against_torch(fmt):
    """Every rounding midpoint between neighbouring codes, and the fp32 values
    one ulp either side of it, with s = 1 (so the cast is the encoder)."""
    tab = oracle.decode_table(fmt)
    top = 0x7E if fmt == oracle.E4M3 else 0x7B
    pos = tab[: top + 1]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    vals = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                           pos.astype(np.float32)])
    vals = np.concatenate([vals, -vals])
    got = oracle.cast_f32(vals, 1.0, fmt)
    ref = _torch_codes(vals, fmt)
    assert (got == ref).all(), [(float(v), g, r) for v, g, r in zip(vals, got, ref) if g != r][:8]


def test_encode_printed_ties():
    # ties to even: 464 -> 448, 1.0625 -> 1.0, 1.1875 -> 1.25 (E4M3)
    assert oracle.encode_rne(oracle.E4M3, 464.0) == 0x7E
    assert oracle.encode_rne(oracle.E4M3, 1.0625) == 0x38
    assert oracle.encode_rne(oracle.E4M3, 1.1875) == 0x3A
    assert oracle.encode_rne(oracle.E4M3, -0.0) == 0x80
    assert oracle.encode_rne(oracle.E4M3, -1e-30) == 0x80
    assert oracle.encode_rne(oracle.E5M2, 2.0 ** -17) == 0x00  # tie with 0 -> even (0)
    assert oracle.encode_rne(oracle.E5M2, 3 * 2.0 ** -17) == 0x02  # tie 1 vs 2 -> 2


def test_double_to_bf16_against_torch_on_float32_values():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3e38)]
    got = oracle.double_to_bf16(f.astype(np.float64))
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (got == ref).all()


def test_double_to_bf16_exact_rounding_of_doubles():
    """Doubles that are not float32 values: compare with exact rational RNE."""
    from fractions import Fraction

    def rne_bf16(v):
        fr = Fraction(v)
        if fr == 0:
            return 0.0
        a = abs(fr)
        e = a.numerator.bit_length() - a.denominator.bit_length()
        if Fraction(2) ** e > a:
            e -= 1
        e = max(e, -126)
        q = Fraction(2) ** (e - 7)
        n = a / q
        fl = n.numerator // n.denominator
        rem = n - fl
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
            fl += 1
        r = fl * q
        return float(r) if fr > 0 else -float(r)

    rng = np.random.default_rng(3)
    vals = rng.standard_normal(3000) * np.exp2(rng.integers(-140, 60, 3000))
    # values just off bf16 midpoints (where double rounding via float32 would fail)
    base = rng.standard_normal(1000).astype(np.float32).astype(np.float64)
    mid = base * (1 + 2.0 ** -9) + base * 2.0 ** -40
    vals = np.concatenate([vals, mid, -mid])
    got = oracle.double_to_bf16(vals)
    gotf = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = np.array([rne_bf16(float(v)) for v in vals])
    assert (gotf == ref).all()
