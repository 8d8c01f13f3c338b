"""Pins for the oracle's Newton-Schulz orthogonalisation (Muon).

References that do not reuse the oracle's own formula: the singular value
decomposition (the iteration is the quintic p(s) = a s + b s^3 + c s^5
applied to every singular value of G / (||G|| + eps), singular vectors
unchanged), orthogonal invariance, torch's fp64 Frobenius norm, exact
power-of-two scale invariance of the normalisation, and the bf16 iteration
against the exact one within a budget that planted mistakes exceed."""
import numpy as np
import pytest
import torch

import oracle
from fp8_tensorwise_scaled_amd import synth

f64 = oracle.bf16_bits_to_f64


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("shape,seed", [((48, 80), 1), ((80, 48), 2), ((64, 64), 3), ((16, 200), 4)])
def test_exact_iteration_is_the_polynomial_on_singular_values(shape, seed):
    g = synth.normal_bf16(shape, 1.0, seed)
    gv = f64(g)
    u, s, vt = np.linalg.svd(gv, full_matrices=False)
    x0s = s / (np.sqrt(np.sum(gv * gv)) + oracle.NS_EPS)
    want = (u * oracle.ns_poly(x0s)) @ vt
    got = oracle.newton_schulz(g, exact=True)
    assert _rel(got, want) < 1e-12
    # the published coefficients bring every singular value of a Gaussian
    # matrix whose aspect ratio keeps its smallest singular value away from
    # zero (rows/cols <= 0.6) into [0.6, 1.2] after five steps
    sv = np.linalg.svd(got, compute_uv=False)
    assert sv.max() < 1.2, sv.max()
    if min(shape) / max(shape) <= 0.6:
        assert sv.min() > 0.6, sv.min()


def test_scalar_map():
    """p(s) = 3.4445 s - 4.7750 s^3 + 2.0315 s^5: fixed point 0, p(1) =
    0.701, and five steps from a small s multiply it by 3.4445^5 to first
    order."""
    assert oracle.ns_poly(0.0) == 0.0
    assert abs(oracle.ns_poly(1.0, steps=1) - (3.4445 - 4.7750 + 2.0315)) < 1e-15
    s = 1e-9
    assert abs(oracle.ns_poly(s) / (s * 3.4445 ** 5) - 1) < 1e-12


def test_orthogonal_invariance():
    """NS(Q G R) = Q NS(G) R for orthogonal Q, R.  Signed permutations keep
    a bf16 matrix a bf16 matrix exactly, so the oracle itself is run on the
    transformed input (exact iteration)."""
    g = synth.normal_bf16((40, 72), 1.0, 5)
    rng = np.random.default_rng(6)

    def signed_perm(n):
        m = np.zeros((n, n))
        m[np.arange(n), rng.permutation(n)] = rng.choice([-1.0, 1.0], n)
        return m

    q, r = signed_perm(40), signed_perm(72)
    gt = oracle.double_to_bf16(q @ f64(g) @ r)
    assert (f64(gt) == q @ f64(g) @ r).all()
    base = oracle.newton_schulz(g, exact=True)
    assert _rel(oracle.newton_schulz(gt, exact=True), q @ base @ r) < 1e-12


def test_normalise_against_torch_norm():
    g = synth.normal_bf16((96, 160), 3.0, 7, outlier_frac=1e-2)
    x0, n, den = oracle.ns_normalise(g)
    tn = float(torch.linalg.norm(torch.from_numpy(f64(g))))
    assert n == float(np.float32(tn))
    assert den == float(np.float32(np.float32(tn) + np.float32(oracle.NS_EPS)))
    # every element is the correctly rounded quotient, then one bf16 rounding
    xv = f64(x0)
    assert np.all(np.abs(xv - f64(g) / den) <= 2.0 ** -8 * np.abs(f64(g) / den) + 1e-30)
    assert abs(np.linalg.norm(xv) - 1.0) < 1e-3


def test_normalise_is_scale_invariant_for_powers_of_two():
    """Without eps, G and 2^k G give the same X0 bit for bit (every step of
    the normalisation commutes with an exact power-of-two scaling)."""
    g = synth.normal_bf16((32, 48), 1.0, 8)
    x0, _, _ = oracle.ns_normalise(g, eps=0.0)
    for k in (-3, 5):
        gk = oracle.double_to_bf16(f64(g) * 2.0 ** k)
        assert (oracle.ns_normalise(gk, eps=0.0)[0] == x0).all()


def test_orientation():
    """A tall matrix is iterated on its transpose: NS(G^T) = NS(G)^T."""
    g = synth.normal_bf16((72, 40), 1.0, 9)
    assert (oracle.newton_schulz(np.ascontiguousarray(g.T)) == oracle.newton_schulz(g).T).all()


# bf16 iteration against the exact one.  Each step rounds X, A and B to bf16
# (relative error up to 2^-9 per element); the small singular values are
# multiplied by up to 3.4445 per step, and with them the errors made in the
# early steps, so five steps end near 1.1-1.6% relative (measured on 48x80
# to 384x96 Gaussian matrices).  A 1.5% change of one coefficient already
# moves the result by 7-13%.
BUDGET = 0.03


@pytest.mark.parametrize("shape,seed", [((48, 80), 10), ((96, 384), 11), ((384, 96), 12)])
def test_bf16_iteration_within_budget(shape, seed):
    g = synth.normal_bf16(shape, 1.0, seed)
    e = oracle.newton_schulz(g, exact=True)
    o, tr = oracle.newton_schulz(g, trace=True)
    assert _rel(f64(o), e) < BUDGET
    assert len(tr) == oracle.NS_STEPS and tr[-1][2].shape == (min(shape), max(shape))


def test_budget_catches_planted_mistakes():
    g = synth.normal_bf16((96, 256), 1.0, 13)
    e = oracle.newton_schulz(g, exact=True)
    good = f64(oracle.newton_schulz(g))
    assert _rel(good, e) < BUDGET
    a, b, c = oracle.NS_COEFFS
    with np.errstate(over="ignore", invalid="ignore"):  # the swapped coefficients diverge
        bads = (oracle.newton_schulz(g, coeffs=(a, b, 2.0)),          # c off by 1.5%
                oracle.newton_schulz(g, steps=4),                      # a step short
                oracle.newton_schulz(g, coeffs=(a, c, b)))             # b and c swapped (diverges)
    for bad in bads:
        v = f64(bad)
        assert not np.isfinite(v).all() or _rel(v, e) > BUDGET


def test_bf16_product_closed_forms():
    """Small integers are exact in bf16 and their products and sums exact in
    fp64: the product is the integer matrix product, rounded once."""
    rng = np.random.default_rng(14)
    ai = rng.integers(-8, 9, (24, 40)).astype(np.float64)
    bi = rng.integers(-8, 9, (16, 40)).astype(np.float64)
    ci = rng.integers(-100, 101, (24, 16)).astype(np.float64)
    a, b, c = (oracle.double_to_bf16(v) for v in (ai, bi, ci))
    want = oracle.double_to_bf16(3.0 * (ai @ bi.T) - 2.0 * ci)
    assert (oracle.bf16_gemm_nt(a, b, 3.0, -2.0, c) == want).all()
    assert (oracle.bf16_gemm_nt(a, b) == oracle.double_to_bf16(ai @ bi.T)).all()
    # the iteration's first step is these products on X0
    g = synth.normal_bf16((32, 96), 1.0, 15)
    x0 = oracle.ns_normalise(g)[0]
    _, tr = oracle.newton_schulz(g, steps=1, trace=True)
    A, B, X1 = tr[0]
    a_, b_, c_ = oracle.NS_COEFFS
    assert (A == oracle.bf16_gemm_nt(x0, x0)).all()
    assert (B == oracle.bf16_gemm_nt(A, np.ascontiguousarray(A.T), c_, b_, A)).all()
    xt = np.ascontiguousarray(x0.T)
    assert (X1 == oracle.bf16_gemm_nt(B, xt, 1.0, a_, x0)).all()


def test_gram_products_are_exactly_symmetric():
    g = synth.normal_bf16((64, 200), 1.0, 16)
    _, tr = oracle.newton_schulz(g, steps=2, trace=True)
    for A, B, _ in tr:
        assert (A == A.T).all() and (B == B.T).all()
