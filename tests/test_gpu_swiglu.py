"""GPU parity of the gated (SwiGLU) MLP block (swiglu_mlp_fwd / swiglu_mlp_bwd),
in both accumulation modes.

Every expected value is the oracle (tests/swiglu_chain.py): each GEMM stage
against the oracle GEMM of the GPU's own FP8 operands (exact mode: the
strict bar), each cast bit-exact given its own input, the gate within the
bound of its fp32 evaluation, codes equal to the oracle chain's where their
input agrees, and the outputs against the oracle chain."""
import numpy as np
import pytest
import torch

import oracle
from fp8_tensorwise_scaled_amd import synth
from tests import swiglu_chain as sc_
from tests.gpu_util import ACC_EXACT, ACC_FAST, ACCUMS, bf16_bits, bits_f64, to_dev_bf16, ulp_bf16
from tests.mlp_chain import golden_scales

pytestmark = pytest.mark.gpu


def run_block(w, accum=ACC_FAST):
    from fp8_tensorwise_scaled_amd import api

    x, wg, wu, wd, dy = w.tensors()
    M, d, h = w.M, w.d, w.h
    dev = torch.device("cuda:0")
    ws_f = api.swiglu_mlp_workspace("fwd", M, d, h, dev)
    ws_b = api.swiglu_mlp_workspace("bwd", M, d, h, dev)
    y, saved = api.swiglu_mlp_fwd(to_dev_bf16(x), to_dev_bf16(wg), to_dev_bf16(wu), to_dev_bf16(wd), ws=ws_f,
                                  accum=accum)
    dx, dwg, dwu, dwd, bsc = api.swiglu_mlp_bwd(to_dev_bf16(dy), saved, ws=ws_b, accum=accum)
    torch.cuda.synchronize()
    return sc_.collect((x, wg, wu, wd, dy), y, saved, ws_f, ws_b, dx, dwg, dwu, dwd, bsc)


@pytest.fixture(scope="module", params=ACCUMS, ids=["fast", "exact"])
def small(request):
    return request.param, run_block(synth.SWIGLU_SMALL, request.param)


@pytest.fixture(scope="module")
def small_chain():
    x, wg, wu, wd, dy = synth.SWIGLU_SMALL.tensors()
    return sc_.full_chain_scales(x, wg, wu, wd, dy)


def test_small_block_every_stage(small, small_chain):
    """M=2048, d=768, h=2112: every stage on every token row and hidden
    column against the oracle."""
    accum, g = small
    sc, _, _ = small_chain
    rows, cols = np.arange(g["x"].shape[0]), np.arange(g["wg"].shape[0])
    o = sc_.sampled_chain(g["x"], g["wg"], g["wu"], g["wd"], g["dy"], sc, rows, cols)
    sc_.compare(g, o, sc, rows, cols, accum)


def test_end_to_end(small, small_chain):
    """Outputs against the full oracle chain: relative Frobenius <= 1e-2
    (a one-ulp difference in G, U or dA may move an FP8 code by a step);
    exact mode also max-relative error <= 5e-3."""
    accum, g = small
    _, f, b = small_chain
    for name, got, ref in (("Y", g["y"], f["y"]), ("dX", g["dx"], b["dx"]), ("dW_gate", g["dw_gate"], b["dw_gate"]),
                           ("dW_up", g["dw_up"], b["dw_up"]), ("dW_down", g["dw_down"], b["dw_down"])):
        gv, rv = bits_f64(got), bits_f64(ref)
        fro = np.linalg.norm(gv - rv) / np.linalg.norm(rv)
        rel = np.abs(gv - rv).max() / np.abs(rv).max()
        frac = float((np.abs(gv - rv) <= ulp_bf16(rv)).mean())
        print(f"end-to-end {name} ({'exact' if accum == ACC_EXACT else 'fast'}): max rel {rel:.3g}, "
              f"rel fro {fro:.3g}, within 1 ulp {frac:.5f}")
        assert fro <= 1e-2, (name, fro, frac)
        if accum == ACC_EXACT:
            assert rel <= 5e-3, (name, rel)


@pytest.mark.parametrize("accum", ACCUMS, ids=["fast", "exact"])
def test_3p8b_width_sampled(accum):
    """M=8192, d=3072, h=8448 (the gated block at the model width, ratio
    2.75): tensor-wide scales against the stored oracle values, every stage
    on 32 sampled token rows and 32 sampled hidden columns."""
    w = synth.SWIGLU_3P8B
    g = run_block(w, accum)
    sc = golden_scales("swiglu_3p8b", (g["x"], g["wg"], g["wu"], g["wd"], g["dy"]))
    rng = np.random.default_rng(12)
    rows = np.sort(rng.choice(w.M, 32, replace=False))
    cols = np.sort(rng.choice(w.h, 32, replace=False))
    o = sc_.sampled_chain(g["x"], g["wg"], g["wu"], g["wd"], g["dy"], sc, rows, cols)
    sc_.compare(g, o, sc, rows, cols, accum)


def test_no_tokens():
    """M = 0: empty Y and dX, activation and gradient scales 1, weight
    gradients zero, weight codes and scales as the oracle's."""
    from fp8_tensorwise_scaled_amd import api

    w = synth.SwigluWorkload(43, 16, 64, 176)
    x, wg, wu, wd, dy = w.tensors()
    f = oracle.swiglu_fwd(x[:0], wg, wu, wd)
    b = oracle.swiglu_bwd(dy[:0], f)
    dev = torch.device("cuda:0")
    y, saved = api.swiglu_mlp_fwd(to_dev_bf16(x[:0]), to_dev_bf16(wg), to_dev_bf16(wu), to_dev_bf16(wd))
    fill = lambda r, c: torch.full((r, c), 7, dtype=torch.int16, device=dev).view(torch.bfloat16)
    dx, dwg, dwu, dwd, bsc = api.swiglu_mlp_bwd(to_dev_bf16(dy[:0]), saved, dw_gate=fill(176, 64),
                                                dw_up=fill(176, 64), dw_down=fill(64, 176))
    torch.cuda.synchronize()
    assert [float(v) for v in saved.scales.cpu().numpy()] == [f["sx"], f["swg"], f["swu"], f["swd"], f["sa"]]
    assert [float(v) for v in bsc.cpu().numpy()] == [b["sg"], b["sdg"], b["sdu"]] == [1.0, 1.0, 1.0]
    for t, ref in ((saved.wgq, f["wgq"]), (saved.wuq, f["wuq"]), (saved.wdq, f["wdq"])):
        assert (t.cpu().numpy() == ref).all()
    for t, ref in ((dwg, b["dw_gate"]), (dwu, b["dw_up"]), (dwd, b["dw_down"])):
        assert (bf16_bits(t) == ref).all() and (ref == 0).all()
    assert tuple(y.shape) == (0, 64) and tuple(dx.shape) == (0, 64)


def test_deterministic_and_reuse():
    """Two passes give identical bytes (fixed summation order everywhere)."""
    w = synth.SwigluWorkload(22, 512, 256, 704, sigma_in=1 / 16, sigma_down=1 / 32)
    a, b = run_block(w), run_block(w)
    for k in ("y", "dx", "dw_gate", "dw_up", "dw_down", "g", "u", "a", "dg", "du", "dgq", "duq"):
        assert (a[k] == b[k]).all(), k


@pytest.mark.parametrize("accum", ACCUMS, ids=["fast", "exact"])
def test_whole_stage_width_block(accum):
    """M=256, d=192, h=384: h is a whole number of 128-deep stages, so dX is
    one launch over both products; every stage on every row and column
    against the oracle."""
    w = synth.SwigluWorkload(45, 256, 192, 384, sigma_in=1 / np.sqrt(192), sigma_down=1 / np.sqrt(384))
    g = run_block(w, accum)
    sc, _, b = sc_.full_chain_scales(g["x"], g["wg"], g["wu"], g["wd"], g["dy"])
    rows, cols = np.arange(w.M), np.arange(w.h)
    o = sc_.sampled_chain(g["x"], g["wg"], g["wu"], g["wd"], g["dy"], sc, rows, cols)
    sc_.compare(g, o, sc, rows, cols, accum)


@pytest.mark.parametrize("accum", ACCUMS, ids=["fast", "exact"])
def test_tiny_ragged_block(accum):
    """M=48, d=64, h=176: every GEMM is a single ragged tile; every stage on
    every row and column against the oracle."""
    w = synth.SwigluWorkload(44, 48, 64, 176, sigma_in=1 / 8, sigma_down=1 / 13)
    g = run_block(w, accum)
    sc, _, _ = sc_.full_chain_scales(g["x"], g["wg"], g["wu"], g["wd"], g["dy"])
    rows, cols = np.arange(w.M), np.arange(w.h)
    o = sc_.sampled_chain(g["x"], g["wg"], g["wu"], g["wd"], g["dy"], sc, rows, cols)
    sc_.compare(g, o, sc, rows, cols, accum)


@pytest.mark.parametrize("accum", ACCUMS, ids=["fast", "exact"])
@pytest.mark.parametrize("M,N,K,ld_pad", [(300, 200, 160, 0), (256, 384, 512, 24), (96, 1000, 3072, 0),
                                           (1, 8, 16, 0), (257, 136, 64, 8), (513, 264, 400, 0),
                                           (64, 200, 128, 1)])  # last: odd leading dimension, narrow stores
def test_gated_linear_fwd(M, N, K, ld_pad, accum):
    """fp8_gated_linear_fwd on its own: G and U within the GEMM bound of the
    oracle's products of the same codes; A within one bf16 ulp of the
    oracle's gate applied to the GPU's own G and U (fp32 against fp64
    evaluation), equal on at least 99.9%.  Ragged M and N (N = 200 leaves a
    partial second 128-column tile); with ld_pad the outputs are strided and
    the columns past N must stay untouched."""
    from fp8_tensorwise_scaled_amd import api
    from tests.gpu_util import check_gemm, to_dev_u8

    E4 = oracle.E4M3
    x = synth.normal_bf16((M, K), 1.0, 900 + M, outlier_frac=1e-3)
    wg = synth.normal_bf16((N, K), 0.02, 901 + N)
    wu = synth.normal_bf16((N, K), 0.02, 902 + N)
    xq, sx, _ = oracle.quant(x, E4)
    gq, sg, _ = oracle.quant(wg, E4)
    uq, su, _ = oracle.quant(wu, E4)
    dev = torch.device("cuda:0")
    s = lambda v: torch.tensor([v], dtype=torch.float32, device=dev)
    ld = N + ld_pad
    bufs = [torch.full((M, ld), 7, dtype=torch.int16, device=dev).view(torch.bfloat16) for _ in range(3)]
    g, u, a = api.fp8_gated_linear_fwd(to_dev_u8(xq), s(sx), to_dev_u8(gq), s(sg), to_dev_u8(uq), s(su),
                                       g=bufs[0][:, :N], u=bufs[1][:, :N], a=bufs[2][:, :N], accum=accum)
    torch.cuda.synchronize()
    gb, ub, ab = bf16_bits(g), bf16_bits(u), bf16_bits(a)
    check_gemm(gb, "nt", xq, E4, sx, gq, E4, sg, f"gated G {M}x{N}x{K}", accum=accum)
    check_gemm(ub, "nt", xq, E4, sx, uq, E4, su, f"gated U {M}x{N}x{K}", accum=accum)
    ref_a = oracle.swiglu_gate(gb, ub)
    err = np.abs(bits_f64(ab) - bits_f64(ref_a))
    assert (err <= ulp_bf16(bits_f64(ref_a))).all()
    eq = float((ab == ref_a).mean())
    print(f"[gated] {M}x{N}x{K}: A equal to the oracle gate on {eq:.6f}")
    assert eq >= 0.999
    if ld_pad:
        for t in bufs:
            assert (t.view(torch.int16)[:, N:] == 7).all()


def test_gated_linear_fwd_empty_reduction():
    """K = 0: G = U = 0 (empty sums) and A = silu(0) 0 = 0."""
    from fp8_tensorwise_scaled_amd import api

    dev = torch.device("cuda:0")
    s = torch.ones(1, dtype=torch.float32, device=dev)
    e = lambda r: torch.empty((r, 0), dtype=torch.uint8, device=dev)
    g, u, a = api.fp8_gated_linear_fwd(e(40), s, e(24), s, e(24), s,
                                       g=torch.full((40, 24), 7, dtype=torch.int16, device=dev).view(torch.bfloat16))
    torch.cuda.synchronize()
    for t in (g, u, a):
        assert (bf16_bits(t) == 0).all()


def test_grouped_grad_weights_equal_separate_launches(small):
    """The block's three grad-weights come out of one grouped launch; each is
    byte-identical to fp8_linear_wgrad on the same codes and scales (a tile's
    sums run over the same reduction in the same order whichever launch holds
    it), so grouping changes no value the oracle checks elsewhere."""
    from fp8_tensorwise_scaled_amd import api

    accum, g = small
    dev = torch.device("cuda:0")
    u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    f1 = lambda v: torch.tensor([float(v)], dtype=torch.float32, device=dev)
    sx, sa = g["scales"][0], g["scales"][4]
    for key, codes, s_codes, other, s_other in (("dw_down", g["gq"], g["bsc"][0], g["aq"], sa),
                                                ("dw_gate", g["dgq"], g["bsc"][1], g["xq"], sx),
                                                ("dw_up", g["duq"], g["bsc"][2], g["xq"], sx)):
        sep = api.fp8_linear_wgrad(u8(codes), f1(s_codes), u8(other), f1(s_other), api.E5M2, api.E4M3,
                                   accum=accum)
        torch.cuda.synchronize()
        got = bf16_bits(sep)
        print(f"{key}: grouped equal to separate on {float((got == g[key]).mean()):.6f}")
        assert got.shape == g[key].shape, key
        assert (got == g[key]).all(), key
