"""GPU parity of fp8_amax_quant: codes, transposed codes and scales are
bit-identical to the oracle's."""
import numpy as np
import pytest
import torch

import oracle
from fp8_tensorwise_scaled_amd import synth
from tests.gpu_util import bf16_bits, f32, to_dev_bf16, u8

pytestmark = pytest.mark.gpu
FMTS = [oracle.E4M3, oracle.E5M2]


def run_quant(x_np, fmt, ld=None, qt=True, offset=0):
    """offset: elements between the allocation's start and x (2 bytes each,
    so an odd offset leaves x off a dword boundary)."""
    from fp8_tensorwise_scaled_amd import api

    rows, cols = x_np.shape
    if ld is None and offset == 0:
        xd = to_dev_bf16(x_np)
    else:
        ld = cols if ld is None else ld
        buf = np.zeros(offset + rows * ld, np.uint16)
        buf[offset:].reshape(rows, ld)[:, :cols] = x_np
        xd = to_dev_bf16(buf)[offset:].view(rows, ld)[:, :cols]
    q, qt_, s, a = api.fp8_amax_quant(xd, fmt, want_qt=qt)
    torch.cuda.synchronize()
    return u8(q), (u8(qt_) if qt else None), float(f32(s)[0]), float(f32(a)[0])


def check_against_oracle(x_np, fmt, **kw):
    """Scale, amax and codes against the oracle, with and without the
    transposed codes (the two are different cast paths) unless `qt` is
    given."""
    rq, rs, ra = oracle.quant(x_np, fmt)
    for want_qt in ((kw.pop("qt"),) if "qt" in kw else (True, False)):
        q, qt, s, a = run_quant(x_np, fmt, qt=want_qt, **kw)
        assert np.float32(s) == np.float32(rs) and np.float32(a) == np.float32(ra), (want_qt, s, rs, a, ra)
        bad = np.argwhere(q != rq)
        assert bad.size == 0, [(want_qt, tuple(i), hex(x_np[tuple(i)]), q[tuple(i)], rq[tuple(i)]) for i in bad[:5]]
        if qt is not None:
            assert (qt == rq.T).all()


@pytest.mark.parametrize("fmt", FMTS)
def test_exhaustive_bf16_patterns(fmt):
    """Every finite bf16 value, with amax set by the largest one present:
    the full tensor and a sweep of 48 amax cut-offs."""
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = b[np.isfinite(synth.bf16_bits_to_f32(b))]
    check_against_oracle(fin.reshape(-1, 256), fmt)   # 255 x 256: vector path
    mags = np.unique(fin & 0x7FFF)
    rng = np.random.default_rng(fmt)
    cuts = np.concatenate([mags[[1, 2, 100, 0x80, 0x300]], rng.choice(mags[1:], 43, replace=False)])
    for c in cuts:
        sel = fin[(fin & 0x7FFF) <= c]
        sel = np.concatenate([sel, [c]]).astype(np.uint16)
        n = sel.size
        cols = 128 if n >= 128 else n
        rows = -(-n // cols)
        pad = np.zeros(rows * cols, np.uint16)
        pad[:n] = sel
        check_against_oracle(pad.reshape(rows, cols), fmt)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(256, 512), (1024, 512), (300, 200), (1, 8), (129, 130), (7, 1000),
                                   (256, 384), (128, 260), (384, 1020)])  # last column tile 128, 4, 252 wide
def test_workload_like_shapes(fmt, shape):
    sigma = 1.0 if fmt == oracle.E4M3 else 1e-3
    x = synth.normal_bf16(shape, sigma, 1000 + shape[0] * 7 + shape[1], outlier_frac=1e-3)
    check_against_oracle(x, fmt)


def test_random_shapes():
    """Thirty seeded random cases: rows in [1, 700), cols in [1, 1100), a
    leading dimension equal to cols, padded, or odd, a base offset of 0 to 3
    elements, and a random format: every tile kind (whole, partial width,
    ragged rows, realigned rows, element path) against the oracle."""
    rng = np.random.default_rng(4242)
    for i in range(30):
        rows, cols = int(rng.integers(1, 700)), int(rng.integers(1, 1100))
        ld = [cols, cols + int(rng.integers(1, 40)), cols | 1][int(rng.integers(0, 3))]
        offset = int(rng.integers(0, 4))
        fmt = FMTS[int(rng.integers(0, 2))]
        x = synth.normal_bf16((rows, cols), 1.0 if fmt == oracle.E4M3 else 1e-3, 9000 + i, outlier_frac=1e-3)
        print(f"[quant random] {i}: {rows}x{cols} ld {ld} offset {offset} fmt {fmt}", flush=True)
        check_against_oracle(x, fmt, ld=ld, offset=offset)


@pytest.mark.parametrize("fmt", FMTS)
def test_strided_and_unaligned(fmt):
    x = synth.normal_bf16((200, 333), 1.0, 77)
    check_against_oracle(x, fmt, ld=341)     # odd leading dimension: element path
    x = synth.normal_bf16((256, 256), 1.0, 78)
    check_against_oracle(x, fmt, ld=264)     # aligned ld > cols: vector path
    q, qt, s, a = run_quant(x, fmt, qt=False)
    assert qt is None and (q == oracle.quant(x, fmt)[0]).all()


@pytest.mark.parametrize("fmt", FMTS)
def test_unaligned_rows_full_tiles(fmt):
    """Rows that are not 8-byte aligned go through the realigning buffer-load
    paths on whole tiles (and the element path on the ragged edge): with
    transposed codes or rows of codes off 8 bytes, 4 columns per lane;
    codes-only on 8-byte rows of codes, 16 bytes per lane shifted by the
    row's phase (an odd leading dimension alternates it row by row, base
    offsets 1-3 move it, 776 columns end in an 8-column tile)."""
    x = synth.normal_bf16((300, 776), 1.0, 82)
    for off in (1, 2, 3):
        check_against_oracle(x, fmt, ld=777, offset=off, qt=False)
    check_against_oracle(x, fmt, ld=780, offset=1, qt=False)  # even leading dimension, base off a dword
    x = synth.normal_bf16((300, 700), 1.0, 79)
    check_against_oracle(x, fmt, ld=701)             # odd leading dimension
    check_against_oracle(x, fmt, ld=702, offset=1)   # base off a dword boundary
    x = synth.normal_bf16((257, 1001), 1.0, 80)
    check_against_oracle(x, fmt)                     # dense, odd row length
    x = synth.normal_bf16((128, 512), 1.0, 81)
    check_against_oracle(x, fmt, ld=513, offset=3)   # whole tiles only, tensor ends mid-dword


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("bad", [0x7FC0, 0xFFC1, 0x7F80, 0xFF80], ids=["nan", "-nan", "inf", "-inf"])
def test_non_finite_input_gives_non_finite_scale(fmt, bad):
    """Outside the numeric contract, one guarantee: a NaN or an infinity
    anywhere in the tensor (here in the last row tile, past the first amax
    block) makes amax and the scale non-finite, NaN winning over infinity.
    The call completes; the codes are not checked."""
    x = synth.normal_bf16((300, 70000), 1.0, 61)
    x[297, 69011] = bad
    _, _, s, a = run_quant(x, fmt)
    want_nan = (bad & 0x7F) != 0
    assert not np.isfinite(s) and not np.isfinite(a), (s, a)
    assert np.isnan(a) == want_nan and np.isnan(s) == want_nan, (s, a)
    x[5, 3] = 0x7F80  # an infinity and a NaN together: NaN
    if want_nan:
        _, _, s, a = run_quant(x, fmt)
        assert np.isnan(s) and np.isnan(a)


def test_more_than_2_31_elements():
    """A [40000, 60000] tensor, 2.4e9 elements (4.8 GB): a seeded bf16 block
    T [125, 600] repeated (neither period divides the 128 x 256 cast tiles),
    and as the very last element, beyond element 2^31, -4 max|T|, which
    alone sets amax.  Scale, amax, codes and transposed codes against the
    oracle's quantisation of T's elements and that one."""
    from fp8_tensorwise_scaled_amd import api

    R, C, tr, tc = 40000, 60000, 125, 600
    assert R * C > 2 ** 31 and R % tr == 0 and C % tc == 0
    fmt = oracle.E5M2
    T = synth.normal_bf16((tr, tc), 1.0, 77)
    top = int((T & 0x7FFF).max())
    last = (top + 0x100) | 0x8000  # exponent + 2: exactly -4 max|T|
    vals = np.concatenate([T.ravel(), [last]]).astype(np.uint16).reshape(1, -1)
    rq, rs, ra = oracle.quant(vals, fmt)
    assert ra == 4 * float(synth.bf16_bits_to_f32(np.array([top], np.uint16))[0])

    dev = torch.device("cuda:0")
    x = to_dev_bf16(T).repeat(R // tr, C // tc)
    x.view(torch.int16)[-1, -1] = last - 65536
    q = torch.empty((R, C), dtype=torch.uint8, device=dev)
    qt = torch.empty((C, R), dtype=torch.uint8, device=dev)
    _, _, s, a = api.fp8_amax_quant(x, fmt, q=q, qt=qt)
    torch.cuda.synchronize()
    del x
    assert np.float32(f32(s)[0]) == np.float32(rs) and np.float32(f32(a)[0]) == np.float32(ra)
    code_last = int(rq[0, -1])
    assert int(q[-1, -1]) == code_last and int(qt[-1, -1]) == code_last
    tq = torch.from_numpy(np.ascontiguousarray(rq[0, :-1].reshape(tr, tc))).to(dev)
    q[-1, -1] = tq[-1, -1]  # the rest repeats T's codes
    qt[-1, -1] = tq[-1, -1]
    qv = q.view(R // tr, tr, C // tc, tc)
    for i in range(0, R // tr, 40):
        assert bool((qv[i:i + 40] == tq[None, :, None, :]).all()), ("q", i)
    tqt = tq.t().contiguous()
    qtv = qt.view(C // tc, tc, R // tr, tr)
    for i in range(0, C // tc, 20):
        assert bool((qtv[i:i + 20] == tqt[None, :, None, :]).all()), ("qt", i)
    del q, qt, qv, qtv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(0, 64), (64, 0), (0, 0)])
def test_empty_tensor(fmt, shape):
    """No elements: amax 0 and scale 1, as the oracle defines them."""
    from fp8_tensorwise_scaled_amd import api

    x = torch.empty(shape, dtype=torch.bfloat16, device="cuda:0")
    scale = torch.full((1,), 7.0, device="cuda:0")
    amax = torch.full((1,), 7.0, device="cuda:0")
    q, qt, s, a = api.fp8_amax_quant(x, fmt, want_qt=True, scale=scale, amax=amax)
    torch.cuda.synchronize()
    rq, rs, ra = oracle.quant(np.zeros(shape, np.uint16), fmt)
    assert float(f32(s)[0]) == rs == 1.0 and float(f32(a)[0]) == ra == 0.0
    assert tuple(q.shape) == shape and tuple(qt.shape) == shape[::-1]


@pytest.mark.parametrize("fmt", FMTS)
def test_zero_and_tiny(fmt):
    x = np.zeros((64, 64), np.uint16)
    x[3, 5] = 0x8000
    check_against_oracle(x, fmt)
    for amax_bits in (0x0001, 0x0080, 0x1000, 0x1380, 0x1400):  # 2^-133 .. 2^-87
        xx = synth.normal_bf16((64, 64), 1.0, int(amax_bits))
        xx = (xx & 0x8000) | np.minimum(xx & 0x7FFF, amax_bits).astype(np.uint16)
        xx[0, 0] = amax_bits
        check_against_oracle(xx, fmt)


@pytest.mark.parametrize("wl", ["linear", "mlp_small", "mlp_3p8b"])
def test_workload_tensors(wl):
    if wl == "linear":
        tensors = [(t, oracle.E4M3) for t in synth.LINEAR_SMALL.tensors()]
    else:
        w = synth.MLP_SMALL if wl == "mlp_small" else synth.MLP_3P8B
        x, wu, wd, dy = w.tensors()
        tensors = [(x, oracle.E4M3), (wu, oracle.E4M3), (wd, oracle.E4M3), (dy, oracle.E5M2)]
    for t, fmt in tensors:
        check_against_oracle(t, fmt)


def test_deterministic():
    from fp8_tensorwise_scaled_amd import api

    x = to_dev_bf16(synth.normal_bf16((1024, 1536), 1.0, 5, outlier_frac=1e-3))
    outs = [api.fp8_amax_quant(x, oracle.E5M2, want_qt=True) for _ in range(5)]
    torch.cuda.synchronize()
    for q, qt, s, a in outs[1:]:
        assert torch.equal(q, outs[0][0]) and torch.equal(qt, outs[0][1]) and torch.equal(s, outs[0][2])
