"""The quantiser's single-launch form against the oracle and against its
two-launch form, byte for byte.

A batch of dense, aligned, codes-only tensors of more than 2 * 65536
elements each is quantised in one pass over the data: one grid reads each
tensor once for its amax, every thread holding its first chunks in
registers across one grid-wide wait, and casts the held chunks without
reading them again.  The amax, the scale and the element-wise cast are the
ones of the two launches (amax pass, then cast), so every byte must match.
FP8MLP_QUANT_PATH=single makes a call fail rather than fall back, which
shows the single pass ran; =two forces the two launches."""
import numpy as np
import pytest
import torch

import oracle
from fp8_tensorwise_scaled_amd import api, synth
from fp8_tensorwise_scaled_amd._native import Fp8MlpError
from tests.gpu_util import f32, to_dev_bf16, u8

pytestmark = pytest.mark.gpu
FMTS = [oracle.E4M3, oracle.E5M2]


def with_path(monkeypatch, path, fn):
    monkeypatch.setenv("FP8MLP_QUANT_PATH", path)
    try:
        out = fn()
        torch.cuda.synchronize()
        return out
    finally:
        monkeypatch.delenv("FP8MLP_QUANT_PATH")


def quant(xd, fmt):
    q, _, s, a = api.fp8_amax_quant(xd, fmt)
    return q, s, a


# (256, 1024): two work units, the fewest; (777, 520) and (3, 65544): a
# thread's last chunk past the tensor in some units; (8192, 3072): the dY
# shape, every chunk held; (8192, 12288) and (8191, 12288): about half the
# chunks held, the rest read twice, a ragged last round of the grid-stride
# loop in the second
SHAPES = [(256, 1024), (777, 520), (3, 65544), (2048, 768), (8192, 3072), (8192, 12288), (8191, 12288)]
# too small for the single pass (fewer than three amax partials)
SMALL = [(1, 8), (5, 1000), (256, 512)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{r}x{c}" for r, c in SHAPES])
def test_single_launch_matches_oracle_and_two_launches(monkeypatch, fmt, shape):
    sigma = 1.0 if fmt == oracle.E4M3 else 1e-3
    x = synth.normal_bf16(shape, sigma, 7000 + shape[0] + fmt, outlier_frac=1e-3)
    rq, rs, ra = oracle.quant(x, fmt)
    xd = to_dev_bf16(x)
    q1, s1, a1 = with_path(monkeypatch, "single", lambda: quant(xd, fmt))
    q2, s2, a2 = with_path(monkeypatch, "two", lambda: quant(xd, fmt))
    assert np.float32(f32(s1)[0]) == np.float32(rs) and np.float32(f32(a1)[0]) == np.float32(ra)
    bad = np.argwhere(u8(q1) != rq)
    assert bad.size == 0, [(tuple(i), hex(x[tuple(i)]), u8(q1)[tuple(i)], rq[tuple(i)]) for i in bad[:5]]
    assert torch.equal(q1, q2) and torch.equal(s1, s2) and torch.equal(a1, a2)


@pytest.mark.parametrize("shape", SMALL, ids=[f"{r}x{c}" for r, c in SMALL])
def test_small_tensors_take_two_launches(monkeypatch, shape):
    x = synth.normal_bf16(shape, 1.0, 7300 + shape[0], outlier_frac=1e-3)
    xd = to_dev_bf16(x)
    with pytest.raises(Fp8MlpError):
        with_path(monkeypatch, "single", lambda: quant(xd, oracle.E4M3))
    q, s, _ = quant(xd, oracle.E4M3)
    torch.cuda.synchronize()
    rq, rs, _ = oracle.quant(x, oracle.E4M3)
    assert (u8(q) == rq).all() and np.float32(f32(s)[0]) == np.float32(rs)


@pytest.mark.parametrize("fmt", FMTS)
def test_single_launch_amax_at_the_last_element(monkeypatch, fmt):
    """amax set by one element, placed where the tensor ends, in the part
    that is read a second time: the barrier must publish that block's
    partial to every block."""
    x = synth.normal_bf16((8192, 12288), 0.02, 7100 + fmt)
    x[-1, -1] = 0x4480  # 1024.0
    rq, rs, ra = oracle.quant(x, fmt)
    q, s, a = with_path(monkeypatch, "single", lambda: quant(to_dev_bf16(x), fmt))
    assert np.float32(f32(a)[0]) == np.float32(ra) == np.float32(1024.0)
    assert np.float32(f32(s)[0]) == np.float32(rs)
    assert (u8(q) == rq).all()


def test_single_launch_refuses_strided_input(monkeypatch):
    """A strided tensor cannot take the single launch: with the override the
    call reports it instead of falling back; without it, the two launches
    run and match the oracle."""
    x = synth.normal_bf16((1024, 256), 1.0, 7200)
    buf = to_dev_bf16(np.zeros((1024, 320), np.uint16))
    buf[:, :256].copy_(to_dev_bf16(x))
    xd = buf[:, :256]
    with pytest.raises(Fp8MlpError):
        with_path(monkeypatch, "single", lambda: quant(xd, oracle.E4M3))
    q, s, _ = quant(xd, oracle.E4M3)
    torch.cuda.synchronize()
    rq, rs, _ = oracle.quant(x, oracle.E4M3)
    assert (u8(q) == rq).all() and np.float32(f32(s)[0]) == np.float32(rs)


@pytest.mark.parametrize("wl", ["mlp_small", "mlp_3p8b"])
def test_block_batches_single_vs_two(monkeypatch, wl):
    """The blocks' batched quantisations (X, W_up and W_down in one launch;
    dY in the backward) take the single launch; every saved code, scale and
    output is byte-identical to the two-launch run."""
    w = synth.MLP_SMALL if wl == "mlp_small" else synth.MLP_3P8B
    x, wu, wd, dy = (to_dev_bf16(t) for t in w.tensors())

    def step():
        y, saved = api.relu2_mlp_fwd(x, wu, wd)
        dx, dwu, dwd, bsc = api.relu2_mlp_bwd(dy, saved)
        return y, saved, dx, dwu, dwd, bsc

    r1 = with_path(monkeypatch, "single", step)
    r2 = with_path(monkeypatch, "two", step)
    for name in ("xq", "uq", "dq", "aq", "h", "scales"):
        assert torch.equal(getattr(r1[1], name), getattr(r2[1], name)), name
    for i, name in ((0, "y"), (2, "dx"), (3, "dw_up"), (4, "dw_down"), (5, "bwd_scales")):
        assert torch.equal(r1[i], r2[i]), name


@pytest.mark.parametrize("fmt", FMTS)
def test_wait_bound_reached_gives_nan(monkeypatch, fmt):
    """The single pass's wait is bounded.  With the bound set to zero polls
    (a host-side setting: no block waits, every kernel ends normally) no
    block can know the amax, and every output must show it: all codes NaN
    (0x7F) and the scale NaN.  The next call with the default bound is
    correct again."""
    x = synth.normal_bf16((2048, 768), 1.0, 7400 + fmt)
    xd = to_dev_bf16(x)
    monkeypatch.setenv("FP8MLP_QUANT_SPIN_LIMIT", "0")
    q, s, _ = with_path(monkeypatch, "single", lambda: quant(xd, fmt))
    monkeypatch.delenv("FP8MLP_QUANT_SPIN_LIMIT")
    assert (u8(q) == 0x7F).all()
    assert np.isnan(f32(s)[0])
    q, s, _ = with_path(monkeypatch, "single", lambda: quant(xd, fmt))
    rq, rs, _ = oracle.quant(x, fmt)
    assert (u8(q) == rq).all() and np.float32(f32(s)[0]) == np.float32(rs)
