"""Pins for the oracle's RMSNorm (the step before the MLP's input
quantisation): torch fp64 F.rms_norm, closed forms, and invariances that a
wrong axis, a missing eps or a dropped weight would break."""
import numpy as np
import pytest
import torch

import oracle
from fp8_tensorwise_scaled_amd import synth


def _bits(t):
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("with_gamma", [False, True])
def test_against_torch_fp64(with_gamma):
    x = synth.normal_bf16((64, 3072), 3.0, 81, outlier_frac=1e-3)
    g = synth.normal_bf16((3072,), 1.0, 82) if with_gamma else None
    xn, r = oracle.rmsnorm(x, g, 1e-6)
    xt = torch.from_numpy(oracle.bf16_bits_to_f64(x))
    gt = None if g is None else torch.from_numpy(oracle.bf16_bits_to_f64(g))
    ref = torch.nn.functional.rms_norm(xt, (3072,), gt, 1e-6)
    rref = 1.0 / torch.sqrt(xt.pow(2).mean(-1) + 1e-6)
    assert np.allclose(r, rref.numpy(), rtol=2 ** -22, atol=0)
    got = oracle.bf16_bits_to_f64(xn)
    exp = oracle.bf16_bits_to_f64(_bits(ref))
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(exp), 2.0 ** -126))) - 7)
    assert (np.abs(got - exp) <= ulp).all()
    assert (got == exp).mean() > 0.99


def test_closed_forms_and_invariances():
    # constant rows: X = sign * a / sqrt(a^2 + eps)
    x = np.zeros((3, 256), np.uint16)
    x[0] = 0x4040        # 3.0
    x[1] = 0xC040        # -3.0
    # x[2] all zero: r = 1/sqrt(eps), X = 0
    xn, r = oracle.rmsnorm(x, None, 1e-6)
    v = oracle.bf16_bits_to_f64(xn)
    assert (v[0] == 1.0).all() and (v[1] == -1.0).all() and (v[2] == 0.0).all()
    assert r[2] == np.float32(1.0 / np.sqrt(np.float32(1e-6)))
    # scale invariance of the input by 2^k (exact in every step), and a power-of-two weight scales X
    y = synth.normal_bf16((8, 512), 1.0, 83)
    y4 = _bits(torch.from_numpy(oracle.bf16_bits_to_f64(y)) * 4)
    a, ra = oracle.rmsnorm(y, None, 0.0)
    b, rb = oracle.rmsnorm(y4, None, 0.0)
    assert (a == b).all() and np.allclose(ra, 4 * rb, rtol=0)
    g2 = np.full(512, 0x4000, np.uint16)         # 2.0
    c, _ = oracle.rmsnorm(y, g2, 0.0)
    assert (oracle.bf16_bits_to_f64(c) == 2 * oracle.bf16_bits_to_f64(a)).all()
    # the mean is over the row: permuting columns permutes the output
    p = np.random.default_rng(1).permutation(512)
    d, _ = oracle.rmsnorm(np.ascontiguousarray(y[:, p]), None, 1e-6)
    e, _ = oracle.rmsnorm(y, None, 1e-6)
    assert (d == e[:, p]).all()
    # eps matters for small rows
    s = _bits(torch.from_numpy(oracle.bf16_bits_to_f64(y)) * 2.0 ** -12)
    assert not (oracle.rmsnorm(s, None, 1e-6)[0] == oracle.rmsnorm(s, None, 0.0)[0]).all()


def test_rmsnorm_quant_is_quant_of_rmsnorm():
    x = synth.normal_bf16((32, 768), 2.0, 84)
    q, s, a, xn, r = oracle.rmsnorm_quant(x, None, 1e-6, oracle.E4M3)
    q2, s2, a2 = oracle.quant(xn, oracle.E4M3)
    assert (q == q2).all() and s == s2 and a == a2
