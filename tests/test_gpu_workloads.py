"""GPU parity of the two larger workloads, through the library's C ABI.

* Decoder projection set at M=32768 (hidden 3072, 24 query / 8 key-value
  heads of 128, relu^2 MLP at 12288): Q, K, V share one quantised input; O
  is its own linear; the MLP is the fused block.  Every quantisation is
  bit-exact on the whole tensor; every GEMM is checked on sampled rows
  against the oracle; the MLP block's stages are checked on sampled rows and
  columns against the oracle chain with its stored tensor-wide scales.
* LM head at M=16384, K=3072, vocabulary 50304 (padded to a multiple of 64)
  and 50257 (unpadded, bf16 row stride 50257; the grad-input GEMM reduces
  over exactly 50257 codes): parity of both against the oracle on sampled
  rows, and padding invariance - the padded problem is the unpadded one plus
  zero rows of W and zero columns of dLogits, so scales, codes and every
  output on the overlap are the same, and the padded rows of dW are zero."""
import numpy as np
import pytest
import torch

import oracle
from fp8_tensorwise_scaled_amd import synth
from tests.gpu_util import bf16_bits, check_gemm, collect_block, f32, to_dev_bf16, u8
from tests.mlp_chain import compare_block, golden_scales, sampled_chain

pytestmark = pytest.mark.gpu
E4, E5 = oracle.E4M3, oracle.E5M2


def _scale(t):
    return np.float32(f32(t)[0])


def _check_quant(host_x, fmt, qo, rows, cols, what):
    """QuantOut codes and scale bit-exact."""
    rq, rs, _ = oracle.quant(host_x, fmt)
    assert rq.shape == (rows, cols), what
    assert _scale(qo.scale) == np.float32(rs), what
    assert (u8(qo.q[:, :cols]) == rq).all(), what
    return rq, rs


# ----------------------------------------------------------- projection set
@pytest.fixture(scope="module")
def proj():
    from fp8_tensorwise_scaled_amd.workloads import ProjectionSetRunner

    w = synth.PROJ_SET
    host = {n: w.input(n) for n in w.INPUTS}
    host.update({n: w.grad(n) for n, _ in w.GRADS})
    for i, (name, _, _) in enumerate(w.projections):
        host["w_" + name] = w.weight(i)
    r = ProjectionSetRunner(w.M, torch.device("cuda:0"))
    r.step({k: to_dev_bf16(v) for k, v in host.items()})
    torch.cuda.synchronize()
    return w, host, r


@pytest.mark.parametrize("name", ["q", "k", "v", "o"])
def test_projection_linear(proj, name):
    w, host, r = proj
    lin = getattr(r, name)
    x = host["x_o"] if name == "o" else host["x_attn"]
    M = w.M
    xq, sx = _check_quant(x, E4, lin.xq, M, lin.n_in, f"X of {name}")
    wq, sw = _check_quant(host["w_" + name], E4, lin.wq, lin.n_out, lin.n_in, f"W_{name}")
    gq, sg = _check_quant(host["d" + name], E5, lin.gq, M, lin.n_out, f"dY of {name}")
    rng = np.random.default_rng(40 + ord(name))
    rows = np.sort(rng.choice(M, 16, replace=False))
    check_gemm(bf16_bits(lin.y)[rows], "nt", xq, E4, sx, wq, E4, sw, f"{name} fwd rows", rows=rows)
    check_gemm(bf16_bits(lin.dx)[rows], "nn", gq, E5, sg, wq, E4, sw, f"{name} dgrad rows", rows=rows)
    wr = np.sort(rng.choice(lin.n_out, 16, replace=False))
    check_gemm(bf16_bits(lin.dw)[wr], "tn", gq, E5, sg, xq, E4, sx, f"{name} wgrad rows", rows=wr)


def test_projection_mlp_block(proj):
    w, host, r = proj
    inputs = (host["x_mlp"], host["w_up"], host["w_down"], host["dy_mlp"])
    g = collect_block(inputs, r.y_mlp, r.saved, r.ws_f, r.ws_b, r.dx_mlp, r.dw_up, r.dw_down, r.bsc)
    sc = golden_scales("proj_set_mlp", inputs)
    rng = np.random.default_rng(12)
    rows = np.sort(rng.choice(w.M, 24, replace=False))
    cols = np.sort(rng.choice(12288, 24, replace=False))
    o = sampled_chain(*inputs, sc, rows, cols)
    compare_block(g, o, sc, rows, cols)


# ------------------------------------------------------------------ LM head
@pytest.fixture(scope="module")
def lm():
    from fp8_tensorwise_scaled_amd.workloads import LMHeadRunner

    w = synth.LM_HEAD_PADDED
    n = synth.LM_HEAD_UNPADDED.N
    x, wt, g = w.tensors()
    dev = torch.device("cuda:0")
    xd = to_dev_bf16(x)
    pad = LMHeadRunner(w.M, w.K, w.N, dev)
    pad.step(xd, to_dev_bf16(wt), to_dev_bf16(g))
    unp = LMHeadRunner(w.M, w.K, n, dev)
    unp.step(xd, to_dev_bf16(wt[:n]), to_dev_bf16(g[:, :n]))
    torch.cuda.synchronize()
    return dict(x=x, w=wt, g=g, n=n, pad=pad, unp=unp)


def _lm_parity(L, r, N, seed):
    M, K = r.M, r.K
    w, g = L["w"][:N], L["g"][:, :N]
    xq, sx = _check_quant(L["x"], E4, r.xq, M, K, "X")
    wq, sw = _check_quant(w, E4, r.wq, N, K, "W")
    gq, sg = _check_quant(g, E5, r.gq, M, N, "dLogits")
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(M, 12, replace=False))
    check_gemm(bf16_bits(r.y)[rows], "nt", xq, E4, sx, wq, E4, sw, f"LM head N={N} fwd rows", rows=rows)
    check_gemm(bf16_bits(r.dx)[rows], "nn", gq, E5, sg, wq, E4, sw, f"LM head N={N} dgrad rows", rows=rows)
    wr = np.sort(np.concatenate([rng.choice(L["n"], 12, replace=False), np.arange(L["n"], N)[:4]]))
    check_gemm(bf16_bits(r.dw)[wr], "tn", gq, E5, sg, xq, E4, sx, f"LM head N={N} wgrad rows", rows=wr)


def test_lm_head_padded(lm):
    _lm_parity(lm, lm["pad"], lm["pad"].N, 51)


def test_lm_head_unpadded(lm):
    _lm_parity(lm, lm["unp"], lm["n"], 52)


def test_lm_head_padding_invariance(lm):
    p, u, n = lm["pad"], lm["unp"], lm["n"]
    for what in ("xq", "wq", "gq"):
        assert _scale(getattr(p, what).scale) == _scale(getattr(u, what).scale), what
    assert (u8(p.wq.q[:n]) == u8(u.wq.q)).all()
    assert (u8(p.gq.q[:, :n]) == u8(u.gq.q[:, :n])).all()
    yp, yu = bf16_bits(p.y), bf16_bits(u.y)
    assert (yp[:, :n] == yu).all(), "logits differ on the overlap"
    assert (bf16_bits(p.dx) == bf16_bits(u.dx)).all(), "dX differs"
    dwp, dwu = bf16_bits(p.dw), bf16_bits(u.dw)
    assert (dwp[:n] == dwu).all(), "dW differs on the overlap"
    assert (dwp[n:] & 0x7FFF == 0).all(), "padded rows of dW are not zero"
    assert (yp[:, n:] & 0x7FFF == 0).all(), "padded logits are not zero"
