"""Pins for the oracle's FP8 GEMMs (NT forward, NN grad-input, TN grad-weight).

References: exact rational arithmetic (Python Fractions) on tiny random
inputs, numpy's fp64 matmul with its own operand conventions, and closed
forms (identity, all-ones, one nonzero per row).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

E4, E5 = oracle.E4M3, oracle.E5M2


def finite_codes(fmt, rng, shape, lo_exp_codes=False):
    tab = oracle.decode_table(fmt)
    ok = np.nonzero(np.isfinite(tab))[0].astype(np.uint8)
    return rng.choice(ok, size=shape)


def bf16_of_fraction(fr):
    """Exact round-to-nearest-even of a rational to bf16, as a float."""
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
    r = float(fl * q)
    return r if fr > 0 else -r


def bits_to_f(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def exact_nt(a, fa, sa, b, fb, sb):
    ta = [Fraction(float(v)) if np.isfinite(v) else None for v in oracle.decode_table(fa)]
    tb = [Fraction(float(v)) if np.isfinite(v) else None for v in oracle.decode_table(fb)]
    p = Fraction(float(np.float32(np.float32(sa) * np.float32(sb))))
    M, K = a.shape
    N = b.shape[0]
    out = np.empty((M, N))
    for m in range(M):
        for n in range(N):
            acc = sum((ta[a[m, k]] * tb[b[n, k]] for k in range(K)), Fraction(0))
            out[m, n] = bf16_of_fraction(acc * p)
    return out


@pytest.mark.parametrize("fa,fb", [(E4, E4), (E5, E4), (E4, E5), (E5, E5)])
@pytest.mark.parametrize("shape", [(3, 5, 7), (8, 4, 64), (2, 3, 200)])
def test_gemm_nt_exact(fa, fb, shape):
    M, N, K = shape
    rng = np.random.default_rng(M * 100 + N * 10 + K + fa * 7 + fb * 3)
    a = finite_codes(fa, rng, (M, K))
    b = finite_codes(fb, rng, (N, K))
    sa, sb = 0.0137, 3.3e-5
    got = bits_to_f(oracle.gemm_nt(a, fa, sa, b, fb, sb))
    ref = exact_nt(a, fa, sa, b, fb, sb)
    assert (got == ref).all()


@pytest.mark.parametrize("fa,fb", [(E5, E4), (E4, E4)])
def test_gemm_nn_tn_exact(fa, fb):
    rng = np.random.default_rng(11)
    M, N, K = 6, 5, 9
    sa, sb = 1.7e-3, 0.021
    a = finite_codes(fa, rng, (M, N))
    b = finite_codes(fb, rng, (N, K))
    got = bits_to_f(oracle.gemm_nn(a, fa, sa, b, fb, sb))
    ref = exact_nt(a, fa, sa, np.ascontiguousarray(b.T), fb, sb)   # NN == NT with B^T
    assert (got == ref).all()
    a2 = finite_codes(fa, rng, (M, N))
    b2 = finite_codes(fb, rng, (M, K))
    got = bits_to_f(oracle.gemm_tn(a2, fa, sa, b2, fb, sb))
    ref = exact_nt(np.ascontiguousarray(a2.T), fa, sa, np.ascontiguousarray(b2.T), fb, sb)
    assert (got == ref).all()


def test_layouts_against_numpy_matmul():
    """numpy's matmul fixes the operand conventions independently."""
    rng = np.random.default_rng(5)
    M, N, K = 37, 29, 300
    ta, tb = oracle.decode_table(E5), oracle.decode_table(E4)
    p = float(np.float32(np.float32(0.5) * np.float32(0.25)))
    a = finite_codes(E5, rng, (M, N))
    a_codes_small = a
    b = finite_codes(E4, rng, (N, K))
    ref = oracle.double_to_bf16((ta[a_codes_small] @ tb[b]) * p)
    assert (oracle.gemm_nn(a, E5, 0.5, b, E4, 0.25) == ref).all()
    a = finite_codes(E5, rng, (K, M))
    b = finite_codes(E4, rng, (K, N))
    ref = oracle.double_to_bf16((ta[a].T @ tb[b]) * p)
    assert (oracle.gemm_tn(a, E5, 0.5, b, E4, 0.25) == ref).all()
    a = finite_codes(E4, rng, (M, K))
    b = finite_codes(E4, rng, (N, K))
    ref = oracle.double_to_bf16((tb[a] @ tb[b].T) * p)
    assert (oracle.gemm_nt(a, E4, 0.5, b, E4, 0.25) == ref).all()


def test_special_cases():
    rng = np.random.default_rng(9)
    K = 64
    one = 0x38
    # S1: B = identity (code for 1.0 on the diagonal): y = RN_bf16(p * dec(a))
    a = finite_codes(E4, rng, (K, K))
    eye = np.zeros((K, K), np.uint8)
    np.fill_diagonal(eye, one)
    s_a, s_b = 0.0375, 1.0
    y = bits_to_f(oracle.gemm_nt(a, E4, s_a, eye, E4, s_b))
    expect = torch.from_numpy((oracle.decode_table(E4)[a] * np.float32(s_a)).astype(np.float32))
    assert (y == expect.to(torch.bfloat16).to(torch.float64).numpy()).all()
    # S2: all ones: y = RN_bf16(p * K)
    ones = np.full((3, 1000), one, np.uint8)
    y = bits_to_f(oracle.gemm_nt(ones, E4, 1.0, ones, E4, 0.001))
    expect = float(torch.tensor(1000 * float(np.float32(0.001)), dtype=torch.float32).to(torch.bfloat16))
    assert (y == expect).all()
    # S3: one nonzero product per output: y equals the rounded single product
    a = np.zeros((4, 16), np.uint8)
    b = np.zeros((4, 16), np.uint8)
    for i in range(4):
        a[i, i] = 0x7E      # 448
        b[i, i] = 0x01      # 2^-9
    y = bits_to_f(oracle.gemm_nt(a, E4, 2.0, b, E4, 0.5))
    assert (np.diag(y) == 448 * 2.0 ** -9).all() and (y[~np.eye(4, dtype=bool)] == 0).all()


def test_empty_reduction_and_empty_outputs():
    """K = 0: every output is the empty sum, +0; M = 0 or N = 0: empty output."""
    for fn, a, b, shape in ((oracle.gemm_nt, np.zeros((5, 0), np.uint8), np.zeros((3, 0), np.uint8), (5, 3)),
                            (oracle.gemm_nn, np.zeros((5, 0), np.uint8), np.zeros((0, 3), np.uint8), (5, 3)),
                            (oracle.gemm_tn, np.zeros((0, 5), np.uint8), np.zeros((0, 3), np.uint8), (5, 3))):
        y = fn(a, E4, 0.5, b, E5, 3.0)
        assert y.shape == shape and (y == 0).all()
    assert oracle.gemm_nt(np.zeros((0, 16), np.uint8), E4, 1.0, np.ones((3, 16), np.uint8), E4, 1.0).shape == (0, 3)


def test_row_sampling_matches_full():
    rng = np.random.default_rng(2)
    a = finite_codes(E5, rng, (50, 70))
    b = finite_codes(E4, rng, (70, 33))
    rows = np.array([0, 7, 49, 13])
    full = oracle.gemm_nn(a, E5, 0.1, b, E4, 0.2)
    assert (oracle.gemm_nn(a, E5, 0.1, b, E4, 0.2, rows=rows) == full[rows]).all()
    b2 = finite_codes(E4, rng, (50, 33))
    full = oracle.gemm_tn(a, E5, 0.1, b2, E4, 0.2)
    assert (oracle.gemm_tn(a, E5, 0.1, b2, E4, 0.2, rows=rows[rows < 70]) == full[rows[rows < 70]]).all()
    b3 = finite_codes(E4, rng, (21, 70))
    full = oracle.gemm_nt(a, E5, 0.1, b3, E4, 0.2)
    assert (oracle.gemm_nt(a, E5, 0.1, b3, E4, 0.2, rows=rows) == full[rows]).all()
