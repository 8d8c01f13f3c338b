"""Pins for the oracle's relu^2 steps and the wiring of the MLP block chain.

References: torch's float32 -> bf16 cast for the closed forms
relu(h)^2 and 2 relu(h) dA (both exact in fp32 before rounding); torch
float64 autograd of the unquantised block for the chain rule (a sanity bound
at the size of the FP8 error, not parity).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from fp8_tensorwise_scaled_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def to_bf16_bits(f32):
    return torch.from_numpy(np.ascontiguousarray(f32, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def test_relu2_closed_form():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    hf = synth.bf16_bits_to_f32(h)
    h = h[np.isfinite(hf)]
    hf = synth.bf16_bits_to_f32(h)
    r = np.maximum(hf, np.float32(0))
    with np.errstate(over="ignore"):  # squares past the fp32 range are inf, as in bf16
        assert (oracle.relu2(h) == to_bf16_bits(r * r)).all()


def test_relu2_bwd_closed_form():
    rng = np.random.default_rng(4)
    h = synth.normal_bf16((200000,), 3.0, 21)
    h[:3] = [0x0000, 0x8000, 0x0001]  # +0, -0, min subnormal
    da = synth.normal_bf16((200000,), 1e-3, 22)
    hf, daf = synth.bf16_bits_to_f32(h), synth.bf16_bits_to_f32(da)
    ref = to_bf16_bits(np.float32(2) * np.maximum(hf, np.float32(0)) * daf)
    got = oracle.relu2_bwd(h, da)
    assert (got == ref).all()
    # derivative is zero (with the sign of dA) for h <= 0
    neg = hf <= 0
    assert (synth.bf16_bits_to_f32(got)[neg] == 0).all()


@pytest.fixture(scope="module")
def small_block():
    w = synth.MLPWorkload(90, 256, 128, 512, sigma_up=128 ** -0.5, sigma_down=512 ** -0.5)
    x, wu, wd, dy = w.tensors()
    fwd = oracle.mlp_fwd(x, wu, wd)
    bwd = oracle.mlp_bwd(dy, fwd)
    return (x, wu, wd, dy), fwd, bwd


def test_chain_against_unquantised_autograd(small_block):
    (x, wu, wd, dy), fwd, bwd = small_block
    t = lambda b: torch.from_numpy(synth.bf16_bits_to_f32(b).astype(np.float64))
    X = t(x).requires_grad_()
    U = t(wu).requires_grad_()
    D = t(wd).requires_grad_()
    Y = torch.relu(X @ U.T).pow(2) @ D.T
    Y.backward(t(dy))
    f = lambda b: synth.bf16_bits_to_f32(b).astype(np.float64)

    def rel(got, ref):
        ref = ref.detach().numpy()
        return np.linalg.norm(f(got) - ref) / np.linalg.norm(ref)

    errs = dict(y=rel(fwd["y"], Y), dx=rel(bwd["dx"], X.grad), dw_up=rel(bwd["dw_up"], U.grad),
                dw_down=rel(bwd["dw_down"], D.grad))
    # FP8 (E4M3 forward, E5M2 backward) error budget: a few percent; wiring
    # mistakes (a transposed operand, the wrong saved tensor) give O(1).
    for k, v in errs.items():
        assert v < 0.12, errs
    print("relative errors vs unquantised fp64 chain:", errs)


def test_chain_uses_saved_forward_quantities(small_block):
    (x, wu, wd, dy), fwd, bwd = small_block
    # dH vanishes wherever the forward pre-activation is <= 0
    hf = synth.bf16_bits_to_f32(fwd["h"])
    dhf = synth.bf16_bits_to_f32(bwd["dh"])
    assert (dhf[hf <= 0] == 0).all()
    # amax(A) equals relu(max H)^2 rounded to bf16 (monotonicity)
    m = max(float(hf.max()), 0.0)
    assert fwd["amax_a"] == float(synth.bf16_bits_to_f32(to_bf16_bits(np.array([m * m], np.float32)))[0])


def test_chain_with_no_tokens():
    """M = 0: the forward is empty, the activation and gradient scales are 1
    (empty maxima), and both weight gradients are empty sums, i.e. zero."""
    x, wu, wd, dy = synth.MLPWorkload(41, 16, 32, 64).tensors()
    f = oracle.mlp_fwd(x[:0], wu, wd)
    b = oracle.mlp_bwd(dy[:0], f)
    assert f["y"].shape == (0, 32) and b["dx"].shape == (0, 32)
    assert f["sx"] == 1.0 and f["sa"] == 1.0 and b["sg"] == 1.0 and b["sh"] == 1.0
    assert f["su"] == oracle.quant(wu, oracle.E4M3)[1] and f["sd"] == oracle.quant(wd, oracle.E4M3)[1]
    assert b["dw_up"].shape == (64, 32) and (b["dw_up"] == 0).all()
    assert b["dw_down"].shape == (32, 64) and (b["dw_down"] == 0).all()


def test_pages_shapes_and_parameter_table():
    with open(os.path.join(HERE, "golden", "little_lm_config.json")) as fh:
        cfg = json.load(fh)
    m = cfg["model"]
    d, h = m["hidden_size"], m["intermediate_size"]
    assert h == 4 * d and m["hidden_act"] == "relu2" and not m["gated_mlp"]
    assert (synth.MLP_3P8B.d, synth.MLP_3P8B.h) == (d, h)
    kv = m["num_key_value_heads"] * m["head_dim"]
    q = m["num_attention_heads"] * m["head_dim"]
    per_layer = d * q + 2 * d * kv + q * d + 2 * d * h
    assert [p[1:] for p in synth.PROJ_SET.projections] == [(d, q), (d, kv), (d, kv), (q, d), (d, h), (h, d)]
    p = cfg["parameters_millions"]
    assert abs(m["num_hidden_layers"] * per_layer / 1e6 - p["decoder_layers"]) < 0.5
    vpad = -(-m["vocab_size"] // m["vocab_pad_to"]) * m["vocab_pad_to"]
    assert vpad == m["vocab_padded"] == synth.LM_HEAD_PADDED.N
    assert abs(vpad * d / 1e6 - p["lm_head"]) < 0.1
    assert abs(m["value_embedding_tables"] * vpad * kv / 1e6 - p["value_embeddings"]) < 0.1
    # The page's TFLOP/s counts 6 FLOPs per matmul parameter per token; the
    # MLP block's 12*M*d*h per fwd+bwd is that convention for its 2*d*h params.
    tp = cfg["throughput"]
    n_matmul = m["num_hidden_layers"] * per_layer + vpad * d
    implied = 6 * n_matmul * tp["tokens_per_s_node"] / tp["gpus"] / 1e12
    assert abs(implied / tp["tflops_per_gpu"] - 1) < 0.03
    assert synth.MLP_3P8B.flops == 6 * (2 * d * h) * synth.MLP_3P8B.M


def test_chain_bound_detects_planted_wiring_mistakes(small_block):
    """A planted mistake in the oracle chain (wrong operand for dW_up or a
    transposed weight for dX) must break the sanity bound used above."""
    (x, wu, wd, dy), fwd, bwd = small_block
    t = lambda b: torch.from_numpy(synth.bf16_bits_to_f32(b).astype(np.float64))
    X, U, D = (t(v).requires_grad_() for v in (x, wu, wd))
    (torch.relu(X @ U.T).pow(2) @ D.T).backward(t(dy))
    f = lambda b: synth.bf16_bits_to_f32(b).astype(np.float64)
    rel = lambda got, ref: np.linalg.norm(f(got) - ref.numpy()) / np.linalg.norm(ref.numpy())
    wrong_dw_up = oracle.gemm_tn(bwd["hq"], oracle.E5M2, bwd["sh"], fwd["xq"][::-1].copy(), oracle.E4M3, fwd["sx"])
    assert rel(wrong_dw_up, U.grad) > 0.5
    rolled_uq = np.roll(fwd["uq"], 1, axis=0)  # W_up rows off by one
    wrong_dx = oracle.gemm_nn(bwd["hq"], oracle.E5M2, bwd["sh"], rolled_uq, oracle.E4M3, fwd["su"])
    assert rel(wrong_dx, X.grad) > 0.5
