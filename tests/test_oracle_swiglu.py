"""Pins for the oracle's gated (SwiGLU) MLP block: the gate and its
derivative against torch fp64 autograd of silu(G) * U, closed forms, the
fp64 two-term grad-input accumulation, and the quantised chain against the
unquantised fp64 block within the FP8 budget, with planted mistakes."""
import numpy as np
import torch

import oracle
from fp8_tensorwise_scaled_amd import synth

E4, E5 = oracle.E4M3, oracle.E5M2


def _f64(b):
    return oracle.bf16_bits_to_f64(b)


def test_gate_against_torch_autograd():
    g = synth.normal_bf16((64, 256), 3.0, 101)
    u = synth.normal_bf16((64, 256), 1.0, 102)
    da = synth.normal_bf16((64, 256), 1e-3, 103)
    G = torch.from_numpy(_f64(g)).requires_grad_(True)
    U = torch.from_numpy(_f64(u)).requires_grad_(True)
    A = torch.nn.functional.silu(G) * U
    A.backward(torch.from_numpy(_f64(da)))
    a = oracle.swiglu_gate(g, u)
    dg, du = oracle.swiglu_gate_bwd(g, u, da)
    for got, ref in ((a, A.detach().numpy()), (dg, G.grad.numpy()), (du, U.grad.numpy())):
        r = oracle.double_to_bf16(ref)
        v, rv = _f64(got), _f64(r)
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(rv), 2.0 ** -126))) - 7)
        assert (np.abs(v - rv) <= ulp).all() and (got == r).mean() > 0.999


def test_gate_closed_forms():
    g = np.array([[0x0000, 0x4120, 0xC120, 0x3F80]], np.uint16)      # 0, 10, -10, 1
    u = np.full((1, 4), 0x4000, np.uint16)                            # 2
    da = np.full((1, 4), 0x3F80, np.uint16)                           # 1
    a = _f64(oracle.swiglu_gate(g, u))[0]
    dg, du = (_f64(t)[0] for t in oracle.swiglu_gate_bwd(g, u, da))
    s1 = 1 / (1 + np.exp(-1.0))
    assert a[0] == 0 and abs(a[1] - 20.0) < 0.1 and abs(a[2]) < 1e-3
    assert dg[0] == 1.0            # silu'(0) = 1/2, times U = 2
    assert du[0] == 0.0 and abs(du[1] - 10.0) < 0.05
    assert abs(dg[3] - 2 * s1 * (1 + (1 - s1))) < 2 ** -6 and abs(du[3] - s1) < 2 ** -8


def test_two_term_grad_input_accumulation():
    rng = np.random.default_rng(4)
    a1, a2 = (rng.integers(0, 0x7C, (16, 48)).astype(np.uint8) for _ in range(2))
    b1, b2 = (rng.integers(0, 0x7E, (48, 24)).astype(np.uint8) for _ in range(2))
    acc = np.zeros((16, 24))
    oracle.gemm_nn_acc(a1, E5, 0.5, b1, E4, 0.25, acc)
    assert (oracle.double_to_bf16(acc) == oracle.gemm_nn(a1, E5, 0.5, b1, E4, 0.25)).all()
    oracle.gemm_nn_acc(a2, E5, 2.0, b2, E4, 0.125, acc)
    t = np.zeros((16, 24))
    oracle.gemm_nn_acc(np.concatenate([a1, a2], 1), E5, 0.5, np.concatenate([b1, b2 * 0], 0), E4, 0.25, t)
    t2 = np.zeros((16, 24))
    oracle.gemm_nn_acc(a2, E5, 2.0, b2, E4, 0.125, t2)
    assert np.allclose(acc, t + t2, rtol=1e-15, atol=0)
    rows = [3, 7]
    part = np.zeros((2, 24))
    oracle.gemm_nn_acc(a1, E5, 0.5, b1, E4, 0.25, part, rows=rows)
    full = np.zeros((16, 24))
    oracle.gemm_nn_acc(a1, E5, 0.5, b1, E4, 0.25, full)
    assert (part == full[rows]).all()


def _block(seed=41, M=128, d=96, h=264, sx=1.0, sw=0.1):
    x = synth.normal_bf16((M, d), sx, seed)
    wg = synth.normal_bf16((h, d), sw, seed + 1)
    wu = synth.normal_bf16((h, d), sw, seed + 2)
    wd = synth.normal_bf16((d, h), sw, seed + 3)
    dy = synth.normal_bf16((M, d), 1e-3, seed + 4)
    return x, wg, wu, wd, dy


def _unquantised(x, wg, wu, wd, dy):
    X, Wg, Wu, Wd = (torch.from_numpy(_f64(t)).requires_grad_(True) for t in (x, wg, wu, wd))
    Y = (torch.nn.functional.silu(X @ Wg.T) * (X @ Wu.T)) @ Wd.T
    Y.backward(torch.from_numpy(_f64(dy)))
    return Y.detach().numpy(), X.grad.numpy(), Wg.grad.numpy(), Wu.grad.numpy(), Wd.grad.numpy()


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


BUDGET = 0.12   # E4M3 operands (2^-4..2^-3 relative spacing) on every GEMM, E5M2 gradients


def test_chain_within_budget_and_catches_mistakes():
    x, wg, wu, wd, dy = _block()
    ref = _unquantised(x, wg, wu, wd, dy)
    f = oracle.swiglu_fwd(x, wg, wu, wd)
    b = oracle.swiglu_bwd(dy, f)
    got = (f["y"], b["dx"], b["dw_gate"], b["dw_up"], b["dw_down"])
    errs = [_rel(_f64(g), r) for g, r in zip(got, ref)]
    print("relative errors y, dx, dWg, dWu, dWd:", [f"{e:.3g}" for e in errs])
    assert max(errs) < BUDGET
    real = oracle.swiglu_gate_bwd
    try:
        def no_sigmoid_term(g_bits, u_bits, da_bits):          # silu'(g) taken as sigmoid(g)
            g, u, da = _f64(g_bits), _f64(u_bits), _f64(da_bits)
            s = 1 / (1 + np.exp(-g))
            return oracle.double_to_bf16(da * u * s), oracle.double_to_bf16(da * g * s)

        def swapped(g_bits, u_bits, da_bits):
            dg, du = real(g_bits, u_bits, da_bits)
            return du, dg

        for planted in (no_sigmoid_term, swapped):
            oracle.swiglu_gate_bwd = planted
            bb = oracle.swiglu_bwd(dy, f)
            e = max(_rel(_f64(bb["dx"]), ref[1]), _rel(_f64(bb["dw_gate"]), ref[2]), _rel(_f64(bb["dw_up"]), ref[3]))
            assert e > BUDGET, planted.__name__
    finally:
        oracle.swiglu_gate_bwd = real
