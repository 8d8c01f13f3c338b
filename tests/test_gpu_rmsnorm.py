"""GPU parity of fp8_rmsnorm_quant (RMSNorm fused with the tensorwise
quantisation of its output) against the oracle's rmsnorm_quant: the per-row
1/rms, the scale, the amax and every code are bit-identical."""
import numpy as np
import pytest
import torch

import oracle
from fp8_tensorwise_scaled_amd import synth
from tests.gpu_util import f32, to_dev_bf16, u8

pytestmark = pytest.mark.gpu
E4, E5 = oracle.E4M3, oracle.E5M2


def run(x, g, eps, fmt, ld=None, want_qt=True):
    """want_qt: also the transposed codes (a different cast path)."""
    from fp8_tensorwise_scaled_amd import api

    rows, cols = x.shape
    if ld is None:
        xd = to_dev_bf16(x)
    else:
        buf = np.zeros((rows, ld), np.uint16)
        buf[:, :cols] = x
        xd = to_dev_bf16(buf)[:, :cols]
    gd = None if g is None else to_dev_bf16(g)
    q, qt, s, a, r = api.fp8_rmsnorm_quant(xd, gd, eps, fmt, want_qt=want_qt)
    torch.cuda.synchronize()
    return u8(q), (u8(qt) if want_qt else None), float(f32(s)[0]), float(f32(a)[0]), f32(r)


@pytest.mark.parametrize("shape,ld,with_g,fmt", [
    ((8192, 3072), None, True, E4),     # the MLP input of the 3.8B-model block
    ((8192, 3072), None, False, E4),
    ((300, 700), 701, True, E4),        # ragged tiles, odd leading dimension
    ((256, 512), None, True, E5),
    ((17, 3072), None, True, E4),       # fewer rows than one statistics block
    ((33, 1000), None, True, E5),       # rows in registers, 125 16-byte chunks (not whole waves)
    ((40, 5120), None, True, E4),       # rows longer than the register path takes
    ((6, 4096), None, False, E4),       # the longest rows the register path takes; one block
    ((256, 392), None, True, E4),       # last column tile 136 wide: vector cast path with idle lanes
])
def test_bit_exact(shape, ld, with_g, fmt):
    x = synth.normal_bf16(shape, 2.5, 91, outlier_frac=1e-3)
    g = synth.normal_bf16((shape[1],), 1.0, 92) if with_g else None
    rq, rs, ra, _, rr = oracle.rmsnorm_quant(x, g, 1e-6, fmt)
    for want_qt in (True, False):
        q, qt, s, a, r = run(x, g, 1e-6, fmt, ld, want_qt)
        assert (r.view(np.uint32) == rr.view(np.uint32)).all(), "1/rms differs"
        assert np.float32(s) == np.float32(rs) and np.float32(a) == np.float32(ra), (s, rs, a, ra)
        assert (q == rq).all(), want_qt
        assert qt is None or (qt == rq.T).all()


def test_random_shapes():
    """Twenty seeded random cases: rows in [1, 600), cols in [1, 5000) (both
    statistics paths), a padded or odd leading dimension, with and without
    the weight, either format; r, the scale and every code bit-identical."""
    rng = np.random.default_rng(777)
    for i in range(20):
        rows, cols = int(rng.integers(1, 600)), int(rng.integers(1, 5000))
        ld = [None, cols + int(rng.integers(1, 24)), cols | 1][int(rng.integers(0, 3))]
        fmt = [E4, E5][int(rng.integers(0, 2))]
        x = synth.normal_bf16((rows, cols), float(rng.uniform(0.1, 4.0)), 9500 + i, outlier_frac=1e-3)
        g = synth.normal_bf16((cols,), 1.0, 9600 + i) if rng.integers(0, 2) else None
        want_qt = bool(i % 2)
        q, qt, s, a, r = run(x, g, 1e-6, fmt, ld, want_qt)
        rq, rs, ra, _, rr = oracle.rmsnorm_quant(x, g, 1e-6, fmt)
        what = (i, rows, cols, ld, fmt, g is not None, want_qt)
        assert (r.view(np.uint32) == rr.view(np.uint32)).all(), what
        assert np.float32(s) == np.float32(rs) and np.float32(a) == np.float32(ra), what
        assert (q == rq).all() and (qt is None or (qt == rq.T).all()), what


def test_zero_rows_and_empty():
    x = synth.normal_bf16((64, 256), 1.0, 93)
    x[5] = 0
    q, qt, s, a, r = run(x, None, 1e-6, E4)
    rq, rs, ra, _, rr = oracle.rmsnorm_quant(x, None, 1e-6, E4)
    assert (r.view(np.uint32) == rr.view(np.uint32)).all() and (q == rq).all() and s == rs
    q, qt, s, a, r = run(np.zeros((0, 256), np.uint16), None, 1e-6, E4)
    assert s == 1.0 and a == 0.0 and r.size == 0


def _run_path(monkeypatch, path, xd, gd, fmt, spin=None):
    from fp8_tensorwise_scaled_amd import api

    monkeypatch.setenv("FP8MLP_QUANT_PATH", path)
    if spin is not None:
        monkeypatch.setenv("FP8MLP_QUANT_SPIN_LIMIT", str(spin))
    try:
        q, _, s, a, r = api.fp8_rmsnorm_quant(xd, gd, 1e-6, fmt)
        torch.cuda.synchronize()
    finally:
        monkeypatch.delenv("FP8MLP_QUANT_PATH")
        if spin is not None:
            monkeypatch.delenv("FP8MLP_QUANT_SPIN_LIMIT")
    return u8(q), float(f32(s)[0]), float(f32(a)[0]), f32(r)


# rows of up to 3072 columns, at least three units of 16 rows: one pass, every
# block holding its 16 rows in registers across one grid-wide wait
SINGLE = [((8192, 3072), True, E4), ((8192, 3072), False, E5), ((48, 3072), True, E4), ((1000, 776), True, E4),
          ((33, 1000), False, E5), ((4096, 2048), True, E5)]


@pytest.mark.parametrize("shape,with_g,fmt", SINGLE, ids=[f"{s[0]}x{s[1]}-{'g' if w else 'nog'}-{f}" for s, w, f in SINGLE])
def test_single_pass_matches_oracle_and_two_launches(monkeypatch, shape, with_g, fmt):
    """r, scale, amax and codes of the single pass equal the oracle's and
    the two launches' bit for bit (1000 rows: a partial last unit; 776 and
    1000 columns: lanes past a row's last chunk)."""
    x = synth.normal_bf16(shape, 2.5, 93 + shape[0], outlier_frac=1e-3)
    x[shape[0] // 2] = 0  # a zero row
    g = synth.normal_bf16((shape[1],), 1.0, 94) if with_g else None
    xd, gd = to_dev_bf16(x), (None if g is None else to_dev_bf16(g))
    rq, rs, ra, _, rr = oracle.rmsnorm_quant(x, g, 1e-6, fmt)
    q1, s1, a1, r1 = _run_path(monkeypatch, "single", xd, gd, fmt)
    q2, s2, a2, r2 = _run_path(monkeypatch, "two", xd, gd, fmt)
    assert (r1.view(np.uint32) == rr.view(np.uint32)).all(), "1/rms differs"
    assert np.float32(s1) == np.float32(rs) and np.float32(a1) == np.float32(ra)
    assert (q1 == rq).all(), np.argwhere(q1 != rq)[:5]
    assert (q1 == q2).all() and s1 == s2 and a1 == a2 and (r1.view(np.uint32) == r2.view(np.uint32)).all()


def test_single_pass_refuses_long_rows(monkeypatch):
    """Rows longer than 3072 columns keep the two launches."""
    from fp8_tensorwise_scaled_amd._native import Fp8MlpError

    x = synth.normal_bf16((64, 4096), 1.0, 95)
    with pytest.raises(Fp8MlpError):
        _run_path(monkeypatch, "single", to_dev_bf16(x), None, E4)


def test_single_pass_wait_bound_gives_nan(monkeypatch):
    """With the wait's bound set to zero polls from the host (no block
    waits; every kernel ends normally) the codes are all NaN (0x7F) and the
    scale is NaN; r is still each row's own."""
    x = synth.normal_bf16((2048, 3072), 1.0, 96)
    rq, rs, _, _, rr = oracle.rmsnorm_quant(x, None, 1e-6, E4)
    q, s, _, r = _run_path(monkeypatch, "single", to_dev_bf16(x), None, E4, spin=0)
    assert (q == 0x7F).all() and np.isnan(s)
    assert (r.view(np.uint32) == rr.view(np.uint32)).all()
