"""GPU parity of the relu^2 MLP block (relu2_mlp_fwd / relu2_mlp_bwd), in
both accumulation modes.

Every expected value is the oracle (tests/mlp_chain.py): each GEMM stage
against the oracle GEMM of the GPU's own FP8 operands (exact mode: the
strict bar), each cast bit-exact given its own bf16 input and equal to the
oracle chain's codes wherever that input agrees, the end-to-end outputs
against the oracle chain run from the same bf16 inputs (exact mode:
max-relative error <= 5e-3)."""
import numpy as np
import pytest
import torch

import oracle
from fp8_tensorwise_scaled_amd import synth
from tests.gpu_util import ACC_EXACT, ACC_FAST, ACCUMS, bits_f64, collect_block, to_dev_bf16, ulp_bf16
from tests.mlp_chain import compare_block, full_chain_scales, golden_scales, sampled_chain

pytestmark = pytest.mark.gpu
E4, E5 = oracle.E4M3, oracle.E5M2


def run_block(w, accum=ACC_FAST):
    from fp8_tensorwise_scaled_amd import api

    x, wu, wd, dy = w.tensors()
    M, d, h = w.M, w.d, w.h
    dev = torch.device("cuda:0")
    ws_f = api.relu2_mlp_fwd_workspace(M, d, h, dev)
    ws_b = api.relu2_mlp_bwd_workspace(M, d, h, dev)
    y, saved = api.relu2_mlp_fwd(to_dev_bf16(x), to_dev_bf16(wu), to_dev_bf16(wd), ws=ws_f, accum=accum)
    dx, dwu, dwd, bsc = api.relu2_mlp_bwd(to_dev_bf16(dy), saved, ws=ws_b, accum=accum)
    torch.cuda.synchronize()
    return collect_block((x, wu, wd, dy), y, saved, ws_f, ws_b, dx, dwu, dwd, bsc)


@pytest.fixture(scope="module", params=ACCUMS, ids=["fast", "exact"])
def small(request):
    return request.param, run_block(synth.MLP_SMALL, request.param)


def test_fwd_quantisation_bit_exact(small):
    _, g = small
    for name, src, q, si in (("X", g["x"], g["xq"], 0), ("W_up", g["wu"], g["uq"], 1), ("W_down", g["wd"], g["dq"], 2)):
        rq, rs, _ = oracle.quant(src, E4)
        assert np.float32(g["scales"][si]) == np.float32(rs), name
        assert (q == rq).all(), name


def test_small_block_every_stage(small):
    """M=2048, d=768, h=3072: every stage on every row and column against
    the oracle."""
    accum, g = small
    sc, _, _ = full_chain_scales(g["x"], g["wu"], g["wd"], g["dy"])
    rows, cols = np.arange(g["x"].shape[0]), np.arange(g["wu"].shape[0])
    o = sampled_chain(g["x"], g["wu"], g["wd"], g["dy"], sc, rows, cols)
    compare_block(g, o, sc, rows, cols, accum)


def test_end_to_end(small):
    """Oracle chain from the same bf16 inputs, whole outputs: relative
    Frobenius error <= 1e-2 in both modes; exact mode also max-relative
    error <= 5e-3 and >= 99% of the elements within one bf16 ulp (a one-ulp
    difference in H or dH moves an FP8 code of A or dH by a whole step
    wherever it flips a rounding, so single elements may differ by more)."""
    accum, g = small
    ref_f = oracle.mlp_fwd(g["x"], g["wu"], g["wd"])
    ref_b = oracle.mlp_bwd(g["dy"], ref_f)
    for name, got, ref in (("Y", g["y"], ref_f["y"]), ("dX", g["dx"], ref_b["dx"]),
                           ("dW_up", g["dw_up"], ref_b["dw_up"]), ("dW_down", g["dw_down"], ref_b["dw_down"])):
        gv, rv = bits_f64(got), bits_f64(ref)
        rel = np.abs(gv - rv).max() / np.abs(rv).max()
        fro = np.linalg.norm(gv - rv) / np.linalg.norm(rv)
        frac = float((np.abs(gv - rv) <= ulp_bf16(rv)).mean())
        print(f"end-to-end {name} ({'exact' if accum == ACC_EXACT else 'fast'}): max rel {rel:.3g}, "
              f"rel fro {fro:.3g}, within 1 ulp {frac:.5f}")
        assert fro <= 1e-2, (name, rel, fro, frac)
        if accum == ACC_EXACT:
            assert rel <= 5e-3 and frac >= 0.99, (name, rel, fro, frac)


@pytest.mark.parametrize("accum", ACCUMS, ids=["fast", "exact"])
def test_3p8b_block_sampled(accum):
    """M=8192, d=3072, h=12288: the block's tensor-wide scales against the
    stored oracle values, every stage on 32 sampled token rows and 32 sampled
    hidden columns against the oracle."""
    w = synth.MLP_3P8B
    g = run_block(w, accum)
    sc = golden_scales("mlp_3p8b", (g["x"], g["wu"], g["wd"], g["dy"]))
    rng = np.random.default_rng(11)
    rows = np.sort(rng.choice(w.M, 32, replace=False))
    cols = np.sort(rng.choice(w.h, 32, replace=False))
    o = sampled_chain(g["x"], g["wu"], g["wd"], g["dy"], sc, rows, cols)
    compare_block(g, o, sc, rows, cols, accum)


def test_no_tokens():
    """M = 0: empty Y and dX, activation and gradient scales 1, both weight
    gradients zero (empty sums), weight codes and scales as the oracle's."""
    from fp8_tensorwise_scaled_amd import api

    w = synth.MLPWorkload(41, 16, 64, 256)
    x, wu, wd, dy = w.tensors()
    ref_f = oracle.mlp_fwd(x[:0], wu, wd)
    ref_b = oracle.mlp_bwd(dy[:0], ref_f)
    dev = torch.device("cuda:0")
    y, saved = api.relu2_mlp_fwd(to_dev_bf16(x[:0]), to_dev_bf16(wu), to_dev_bf16(wd))
    dwu = torch.full((256, 64), 7, dtype=torch.int16, device=dev).view(torch.bfloat16)
    dwd = torch.full((64, 256), 7, dtype=torch.int16, device=dev).view(torch.bfloat16)
    dx, dwu, dwd, bsc = api.relu2_mlp_bwd(to_dev_bf16(dy[:0]), saved, dw_up=dwu, dw_down=dwd)
    torch.cuda.synchronize()
    sc = saved.scales.cpu().numpy()
    assert [float(v) for v in sc] == [ref_f["sx"], ref_f["su"], ref_f["sd"], ref_f["sa"]]
    assert [float(v) for v in bsc.cpu().numpy()] == [ref_b["sg"], ref_b["sh"]] == [1.0, 1.0]
    assert (saved.uq.cpu().numpy() == ref_f["uq"]).all() and (saved.dq.cpu().numpy() == ref_f["dq"]).all()
    from tests.gpu_util import bf16_bits
    assert (bf16_bits(dwu) == ref_b["dw_up"]).all() and (bf16_bits(dwd) == ref_b["dw_down"]).all()
    assert tuple(y.shape) == (0, 64) and tuple(dx.shape) == (0, 64)


def test_deterministic_and_reuse():
    """Two passes with the same buffers give identical bytes."""
    a = run_block(synth.MLPWorkload(21, 512, 256, 1024, sigma_up=1 / 16, sigma_down=1 / 32))
    b = run_block(synth.MLPWorkload(21, 512, 256, 1024, sigma_up=1 / 16, sigma_down=1 / 32))
    for k in ("y", "dx", "dw_up", "dw_down", "h", "aq", "hq"):
        assert (a[k] == b[k]).all(), k


@pytest.mark.parametrize("accum", ACCUMS, ids=["fast", "exact"])
def test_tiny_ragged_block(accum):
    """M=48, d=64, h=176: every GEMM is a single ragged tile; every stage on
    every row and column against the oracle."""
    w = synth.MLPWorkload(45, 48, 64, 176, sigma_up=1 / 8, sigma_down=1 / 13)
    g = run_block(w, accum)
    sc, _, _ = full_chain_scales(g["x"], g["wu"], g["wd"], g["dy"])
    rows, cols = np.arange(w.M), np.arange(w.h)
    o = sampled_chain(g["x"], g["wu"], g["wd"], g["dy"], sc, rows, cols)
    compare_block(g, o, sc, rows, cols, accum)


# (M, d, h, accum): the relu^2-backward GEMM dA [M, h] (K = d) on 256-row
# tiles whose interior tiles prefetch H in the main loop's last two
# iterations and whose ragged edge tiles load it after the loop:
# 4-wave 256x256 tiles with 3 reduction stages, the same with one stage
# (nothing prefetched before the last iteration), 8-wave 256x192 tiles
# (which also prefetch during the last iteration)
PREFETCH_CASES = [(2096, 384, 6208, ACC_FAST), (2096, 384, 6208, ACC_EXACT), (2096, 128, 6208, ACC_FAST),
                  (2096, 384, 4624, ACC_FAST)]


@pytest.mark.parametrize("M,d,h,accum", PREFETCH_CASES,
                         ids=["256x256-fast", "256x256-exact", "256x256-one-stage", "256x192-fast"])
def test_relu2_backward_prefetch_tiles(M, d, h, accum):
    """Every stage against the oracle on sampled rows and columns that cover
    interior and edge tiles of the relu^2-backward GEMM."""
    w = synth.MLPWorkload(M + d + h, M, d, h, sigma_up=d ** -0.5, sigma_down=h ** -0.5)
    g = run_block(w, accum)
    sc, _, _ = full_chain_scales(g["x"], g["wu"], g["wd"], g["dy"])
    rows = np.unique(np.concatenate([np.arange(0, M, 37), np.arange(M - 45, M), np.arange(250, 262)]))
    cols = np.unique(np.concatenate([np.arange(0, h, 29), np.arange(h - 60, h), np.arange(186, 198)]))
    o = sampled_chain(g["x"], g["wu"], g["wd"], g["dy"], sc, rows, cols)
    compare_block(g, o, sc, rows, cols, accum)
