"""Pins for the oracle's LM head fused with the softcapped cross-entropy.

References: torch fp64 autograd of the same loss written with torch's own
primitives (tanh, log_softmax / cross_entropy); closed forms (all-zero
logits, ignored rows, padded columns); exact fp64 accumulation of the
chunked grad-weight; the unquantised fp64 computation of the whole head
(within the FP8 error budget), with planted mistakes showing that budget
is tight enough to catch them."""
import numpy as np
import pytest
import torch

import oracle
from fp8_tensorwise_scaled_amd import synth

E4, E5 = oracle.E4M3, oracle.E5M2


def _logits(R, V, seed, scale=1.0):
    return synth.normal_bf16((R, V), scale, seed)


def _torch_ce(z_bits, targets, n_classes, c):
    z = torch.from_numpy(oracle.bf16_bits_to_f64(z_bits)[:, :n_classes]).requires_grad_(True)
    s = c * torch.tanh(z / c)
    t = torch.from_numpy(np.asarray(targets, dtype=np.int64))
    loss = torch.nn.functional.cross_entropy(s, t, ignore_index=-100, reduction="mean")
    loss.backward()
    return float(loss.detach()), z.grad.numpy()


@pytest.mark.parametrize("scale", [1.0, 8.0, 40.0])
def test_rows_against_torch_autograd(scale):
    R, V, n = 24, 300, 290
    z = _logits(R, V, 71, scale)
    rng = np.random.default_rng(5)
    t = rng.integers(0, n, R)
    t[[3, 11]] = -100
    n_valid = int((t >= 0).sum())
    loss_r, g, dz = oracle.softcap_ce_rows(z, t, n, 15.0, n_valid)
    ref_loss, ref_g = _torch_ce(z, t, n, 15.0)
    assert abs(loss_r.sum() / n_valid - ref_loss) <= 1e-12 * max(1.0, abs(ref_loss))
    assert np.allclose(g[:, :n], ref_g, rtol=1e-10, atol=1e-15)
    assert (g[:, n:] == 0).all() and (dz[:, n:] == 0).all()
    assert (dz == oracle.double_to_bf16(g)).all()


def test_saturated_rows_against_torch_autograd():
    """Logits far past the cap: the softcap written as c - 2c / (exp(2z/c) + 1)
    (the same function) gives torch's autograd a derivative without the
    cancellation of 1 - tanh^2; the oracle's gradient must follow it where
    tanh is 1 to fp64 precision."""
    R, V, n = 16, 256, 250
    z = _logits(R, V, 72, 250.0)
    zf = oracle.bf16_bits_to_f64(z)[:, :n]
    assert (np.abs(zf / 15.0) > 18.7).mean() > 0.2
    rng = np.random.default_rng(6)
    t = rng.integers(0, n, R)
    zt = torch.from_numpy(zf).requires_grad_(True)
    s = 15.0 - 30.0 / (torch.exp(2.0 * zt / 15.0) + 1.0)
    loss = torch.nn.functional.cross_entropy(s, torch.from_numpy(t), reduction="mean")
    loss.backward()
    loss_r, g, _ = oracle.softcap_ce_rows(z, t, n, 15.0, R)
    assert abs(loss_r.mean() - float(loss.detach())) <= 1e-12 * abs(float(loss.detach()))
    ref = zt.grad.numpy()
    assert (ref != 0).all() and (g[:, :n] != 0).all()
    assert np.allclose(g[:, :n], ref, rtol=1e-9, atol=0.0)


def test_closed_forms():
    R, V, n = 6, 64, 50
    z = np.zeros((R, V), np.uint16)
    t = np.array([0, 7, 49, -100, 3, 3])
    loss_r, g, _ = oracle.softcap_ce_rows(z, t, n, 15.0, 5)
    # zero logits: uniform softmax over n classes; tanh' = 1
    assert np.allclose(loss_r[[0, 1, 2, 4, 5]], np.log(n), rtol=0, atol=1e-15) and loss_r[3] == 0
    exp = np.full((R, n), 1.0 / n) / 5
    exp[np.arange(R), np.where(t >= 0, t, 0)] -= 1.0 / 5
    exp[3] = 0
    assert np.allclose(g[:, :n], exp, atol=1e-17)
    # a saturated row: the softcap bounds the logits to +-15
    z2 = np.full((1, V), 0x4780, np.uint16)  # bf16 65536
    loss2, g2, _ = oracle.softcap_ce_rows(z2, np.array([1]), n, 15.0, 1)
    assert abs(loss2[0] - np.log(n)) < 1e-12 and np.abs(g2).max() < 1e-12


def test_columns_match_rows():
    """The column form (given each row's log-sum-exp) reproduces the row form."""
    R, V, n = 20, 96, 90
    z = _logits(R, V, 72, 6.0)
    t = np.random.default_rng(2).integers(0, n, R)
    t[4] = -100
    t[9] = 93            # a padded class id: ignored
    nv = int(((t >= 0) & (t < n)).sum())
    _, g, dz = oracle.softcap_ce_rows(z, t, n, 15.0, nv)
    zz = oracle.bf16_bits_to_f64(z)[:, :n]
    s = 15.0 * np.tanh(zz / 15.0)
    lse = np.log(np.exp(s).sum(axis=1))
    cols = [0, 5, 89, 90, 95]
    gt, dzt = oracle.softcap_ce_columns(np.ascontiguousarray(z[:, cols].T), cols, lse, t, n, 15.0, nv)
    assert np.allclose(gt, g[:, cols].T, rtol=1e-12, atol=1e-18)
    assert (g[9] == 0).all() and (gt[:, 9] == 0).all() and (gt[3:] == 0).all()


def test_chunked_grad_weight_accumulation_is_exact():
    """Two chunks accumulated in fp64 equal one product over all rows, up to
    fp64 rounding; rounding the sum once equals the one-shot GEMM."""
    rng = np.random.default_rng(3)
    a = rng.integers(0, 0x7C, (64, 40)).astype(np.uint8)   # finite E5M2 codes
    b = rng.integers(0, 0x7E, (64, 24)).astype(np.uint8)
    acc = np.zeros((40, 24))
    oracle.gemm_tn_acc(a[:32], E5, 0.5, b[:32], E4, 0.25, acc)
    oracle.gemm_tn_acc(a[32:], E5, 0.5, b[32:], E4, 0.25, acc)
    full = np.zeros((40, 24))
    oracle.gemm_tn_acc(a, E5, 0.5, b, E4, 0.25, full)
    assert np.allclose(acc, full, rtol=1e-15, atol=0)
    assert (oracle.double_to_bf16(full) == oracle.gemm_tn(a, E5, 0.5, b, E4, 0.25)).all()


def _small_head(seed=9, M=96, K=128, V=320, n=300):
    x = synth.normal_bf16((M, K), 1.0, seed)
    w = synth.normal_bf16((V, K), 0.02, seed + 1)
    w[n:] = 0
    rng = np.random.default_rng(seed)
    t = rng.integers(0, n, M)
    t[::17] = -100
    return x, w, t, n


def _unquantised(x, w, t, n, c=15.0):
    """fp64 autograd of the unquantised head: loss, dX, dW."""
    X = torch.from_numpy(oracle.bf16_bits_to_f64(x)).requires_grad_(True)
    W = torch.from_numpy(oracle.bf16_bits_to_f64(w)).requires_grad_(True)
    s = c * torch.tanh((X @ W.T)[:, :n] / c)
    loss = torch.nn.functional.cross_entropy(s, torch.from_numpy(t), ignore_index=-100)
    loss.backward()
    return float(loss.detach()), X.grad.numpy(), W.grad.numpy()


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


# FP8 budget against the unquantised head: the dZ codes are E5M2, whose
# relative spacing is 2^-3..2^-2, i.e. an rms rounding error of about 4-7%
# per element; gradients summing many such terms with random signs keep
# about that relative rms.  Measured 2.6-5.3% (logits up to ~N(0, 27)).
BUDGET = 0.08


def test_fp8_head_within_budget_of_unquantised():
    x, w, t, n = _small_head()
    loss0, dx0, dw0 = _unquantised(x, w, t, n)
    for chunk in (None, 32):
        r = oracle.lm_head_ce(x, w, t, n, chunk=chunk)
        assert abs(r["loss"] - loss0) / loss0 < 2e-3, (r["loss"], loss0)
        assert _rel(oracle.bf16_bits_to_f64(r["dx"]), dx0) < BUDGET
        assert _rel(oracle.bf16_bits_to_f64(r["dw"]), dw0) < BUDGET
        assert (r["dw"][n:] == 0).all()
    # per-chunk scales: each chunk's dZ codes are its own tensor's quantisation
    r = oracle.lm_head_ce(x, w, t, n, chunk=32)
    for ch in r["chunks"]:
        q, s, _ = oracle.quant(ch["dz"], E5)
        assert (q == ch["dzq"]).all() and s == ch["sdz"]


def test_budget_catches_planted_mistakes():
    """Dropping the softcap derivative, or normalising by all rows instead of
    the non-ignored ones, moves the gradients outside the budget."""
    x, w, t, n = _small_head(seed=13, M=64, K=128, V=256, n=256)
    x = (synth.bf16_bits_to_f32(x) * 16).astype(np.float32)      # logits ~ N(0, 18)
    x = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    t[::2] = -100                                                 # half the rows ignored
    _, dx0, _ = _unquantised(x, w, t, n)
    good = oracle.lm_head_ce(x, w, t, n)
    assert _rel(oracle.bf16_bits_to_f64(good["dx"]), dx0) < BUDGET
    real = oracle.softcap_ce_rows
    try:
        def no_cap_derivative(z_bits, targets, n_classes, softcap, n_valid):
            loss, g, _ = real(z_bits, targets, n_classes, softcap, n_valid)
            tt = np.tanh(oracle.bf16_bits_to_f64(z_bits) / softcap)
            g = g / np.where(1 - tt * tt == 0, 1, 1 - tt * tt)
            return loss, g, oracle.double_to_bf16(g)

        def wrong_norm(z_bits, targets, n_classes, softcap, n_valid):
            return real(z_bits, targets, n_classes, softcap, len(targets))

        for planted in (no_cap_derivative, wrong_norm):
            oracle.softcap_ce_rows = planted
            bad = oracle.lm_head_ce(x, w, t, n)
            assert _rel(oracle.bf16_bits_to_f64(bad["dx"]), dx0) > BUDGET, planted.__name__
    finally:
        oracle.softcap_ce_rows = real
