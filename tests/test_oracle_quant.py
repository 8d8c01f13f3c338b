"""Pins for the oracle's dynamic tensorwise quantiser.

References: torch's CPU float32 division and float8 casts (round to nearest
even) on every finite bf16 pattern; invariants that follow from the
definition s = amax / fmax (bounded dequantised values, the amax element
maps to the largest code, idempotence, sign symmetry, power-of-two scaling,
per-element error bound of round-to-nearest).
"""

import numpy as np
import pytest
import torch

import oracle
from fp8_tensorwise_scaled_amd import synth

TORCH_DT = {oracle.E4M3: torch.float8_e4m3fn, oracle.E5M2: torch.float8_e5m2}
FMTS = [oracle.E4M3, oracle.E5M2]


def all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = synth.bf16_bits_to_f32(b)
    return b[np.isfinite(f)]


def torch_cast(xbits, s, fmt):
    x = torch.from_numpy(synth.bf16_bits_to_f32(xbits).copy())
    v = x / torch.tensor(s, dtype=torch.float32)
    fm = oracle.FMAX[fmt]
    v = v.clamp(-fm, fm)
    return v.to(TORCH_DT[fmt]).view(torch.uint8).numpy()


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("s", [2.0 ** -20, 1 / 448, 0.37, 1.0, 3.0, 2.0 ** 10, 7.006e-6, 0.0113])
def test_cast_exhaustive_bf16_against_torch(fmt, s):
    s = float(np.float32(s))
    x = all_finite_bf16().reshape(1, -1)
    got = oracle.cast(x, s, fmt)[0]
    ref = torch_cast(x[0], s, fmt)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(hex(x[0, i]), hex(got[i]), hex(ref[i])) for i in bad[:8]]


@pytest.mark.parametrize("fmt", FMTS)
def test_scale_formula_against_torch(fmt):
    amaxes = synth.bf16_bits_to_f32(all_finite_bf16())
    amaxes = np.unique(np.abs(amaxes))[1:]  # positive values
    fm = torch.tensor(oracle.FMAX[fmt], dtype=torch.float32)
    ref = (torch.from_numpy(amaxes) / fm).numpy()
    got = np.array([oracle.scale_from_amax(float(a), fmt) for a in amaxes[::37]], np.float32)
    assert (got == ref[::37]).all()
    assert oracle.scale_from_amax(0.0, fmt) == 1.0


@pytest.mark.parametrize("fmt", FMTS)
def test_quant_random_tensor_against_torch(fmt):
    x = synth.normal_bf16((96, 130), 1e-3, 99, outlier_frac=1e-2)
    q, s, a = oracle.quant(x, fmt)
    xf = synth.bf16_bits_to_f32(x)
    assert a == float(np.abs(xf).max())
    assert s == float(np.float32(np.float32(a) / np.float32(oracle.FMAX[fmt])))
    assert (q == torch_cast(x.reshape(-1), s, fmt).reshape(q.shape)).all()


@pytest.mark.parametrize("fmt", FMTS)
def test_zero_tensor(fmt):
    x = np.zeros((4, 8), np.uint16)
    x[1, 3] = 0x8000  # -0
    q, s, a = oracle.quant(x, fmt)
    assert s == 1.0 and a == 0.0
    assert q[1, 3] == 0x80 and (np.delete(q.reshape(-1), 11) == 0).all()


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(0, 8), (8, 0), (0, 0)])
def test_empty_tensor(fmt, shape):
    """An empty tensor has no elements to take a maximum over: amax = 0,
    hence s = 1 as for an all-zero tensor, and no codes."""
    q, s, a = oracle.quant(np.zeros(shape, np.uint16), fmt)
    assert q.shape == shape and s == 1.0 and a == 0.0


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("amax_bits", [0x0080, 0x0001, 0x0005, 0x00F0])  # 2^-126, 2^-133, ...
def test_tiny_amax(fmt, amax_bits):
    """Scales in the fp32 subnormal range: IEEE semantics, no flushing."""
    assert not torch.is_grad_enabled() or True
    x = all_finite_bf16()
    xf = synth.bf16_bits_to_f32(x)
    amax = synth.bf16_bits_to_f32(np.array([amax_bits], np.uint16))[0]
    x = x[np.abs(xf) <= amax]
    x = np.concatenate([x, np.array([amax_bits], np.uint16)]).reshape(1, -1)
    q, s, a = oracle.quant(x, fmt)
    assert a == float(amax)
    ref = torch_cast(x[0], s, fmt)
    assert (q[0] == ref).all()


def _dec(q, fmt):
    return oracle.decode_table(fmt)[q]


@pytest.mark.parametrize("fmt", FMTS)
def test_invariants_bound_and_amax_code(fmt):
    x = synth.normal_bf16((64, 257), 0.02, 5, outlier_frac=1e-2)
    q, s, a = oracle.quant(x, fmt)
    deq = np.abs(_dec(q, fmt)) * s
    assert (deq <= a * (1 + 2.0 ** -24)).all()                           # I1
    xf = synth.bf16_bits_to_f32(x)
    top = 0x7E if fmt == oracle.E4M3 else 0x7B
    i = np.argmax(np.abs(xf))
    assert q.reshape(-1)[i] == (top | (0x80 if xf.reshape(-1)[i] < 0 else 0))  # I2


@pytest.mark.parametrize("fmt", FMTS)
def test_invariant_idempotent(fmt):
    x = synth.normal_bf16((50, 211), 1.0, 11, outlier_frac=5e-3)
    q, s, a = oracle.quant(x, fmt)
    deq = _dec(q, fmt) * np.float64(s)
    x2 = oracle.double_to_bf16(deq)
    q2, s2, a2 = oracle.quant(x2, fmt)
    assert (q2 == q).all()                                                 # I3
    ulp = np.spacing(np.float32(s))
    assert abs(np.float32(s2) - np.float32(s)) <= ulp


@pytest.mark.parametrize("fmt", FMTS)
def test_invariant_error_bound(fmt):
    x = synth.normal_bf16((40, 300), 1.0, 12, outlier_frac=1e-2)
    q, s, a = oracle.quant(x, fmt)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    v = xf / s
    deq = _dec(q, fmt)
    mbits, emin = (3, -6) if fmt == oracle.E4M3 else (2, -14)
    e = np.maximum(np.floor(np.log2(np.maximum(np.abs(v), 1e-300))), emin)
    half_spacing = np.exp2(e - mbits) / 2
    # RN32(x/s) adds at most 2^-24 relative before the fp8 rounding
    assert (np.abs(deq - v) <= half_spacing + np.abs(v) * 2.0 ** -23).all()  # I4


@pytest.mark.parametrize("fmt", FMTS)
def test_invariant_sign_and_power_of_two(fmt):
    x = synth.normal_bf16((33, 65), 0.5, 13)
    q, s, a = oracle.quant(x, fmt)
    qn, sn, an = oracle.quant(x ^ np.uint16(0x8000), fmt)
    assert sn == s and (qn == (q ^ 0x80)).all()                           # I6 sign
    xs = oracle.double_to_bf16(synth.bf16_bits_to_f32(x).astype(np.float64) * 2.0 ** 5)
    q5, s5, a5 = oracle.quant(xs, fmt)
    assert s5 == s * 32 and (q5 == q).all()                                # I6 scaling
