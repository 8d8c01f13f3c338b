"""GPU parity of the three FP8 GEMMs of a linear layer.

fp8_linear_fwd (NT), fp8_linear_dgrad (NN) and fp8_linear_wgrad (TN) on
row-major codes, in both accumulation modes.  Inputs are FP8 codes and
scales produced by the oracle's quantiser, so both sides see identical
operands.  Exact mode: the strict bar (max|gpu - oracle| / max|oracle| <=
5e-3, >= 99.9% of the elements within one bf16 ulp) and its accumulation
bound.  Fast mode: the element-wise bound of the FP8 matrix core's truncating
group sums (tests/gpu_util.py, gemm_bound).

Operands live in buffers whose leading dimension is rounded up to 16 and
whose padding holds NaN codes (0x7F in both formats): a reduction that is not
a multiple of 16 must be masked, and padding past an MN-major operand's
extent may only reach outputs that are never stored."""
import numpy as np
import pytest
import torch

import oracle
from fp8_tensorwise_scaled_amd import synth
from tests.gpu_util import (ACC_EXACT, ACC_FAST, ACCUMS, bf16_bits, bits_f64, check_gemm, gemm_bound, gemm_stats,
                            to_dev_u8)

pytestmark = pytest.mark.gpu
E4, E5 = oracle.E4M3, oracle.E5M2
FORMATS = [(E4, E4), (E5, E4), (E4, E5), (E5, E5)]
LAYOUTS = ("nt", "nn", "tn")
NAN = 0x7F


def scal(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda:0")


def padded(a: np.ndarray, fill: int = NAN, ld: int | None = None) -> torch.Tensor:
    """Device copy of a [rows, cols] code matrix in a buffer with leading
    dimension ld (default: cols rounded up to 16), padding = fill."""
    rows, cols = a.shape
    ld = ld or max(16, -(-cols // 16) * 16)
    buf = torch.full((max(rows, 1), ld), fill, dtype=torch.uint8, device="cuda:0")
    view = buf[:rows, :cols]
    if a.size:
        view.copy_(to_dev_u8(a))
    return view


def storage(kind, M, N, R):
    """Stored shapes of A and B for an output [M, N] with reduction R."""
    return {"nt": ((M, R), (N, R)), "nn": ((M, R), (R, N)), "tn": ((R, M), (R, N))}[kind]


def run(kind, A, fa, sa, B, fb, sb, accum, out=None):
    from fp8_tensorwise_scaled_amd import api

    fn = {"nt": api.fp8_linear_fwd, "nn": api.fp8_linear_dgrad, "tn": api.fp8_linear_wgrad}[kind]
    return fn(A, scal(sa), B, scal(sb), fa, fb, out=out, accum=accum)


def operands(kind, M, N, R, fa, fb, seed, sig_a=1.0, sig_b=0.02, outliers=1e-3):
    sh_a, sh_b = storage(kind, M, N, R)
    a = synth.normal_bf16(sh_a, sig_a, seed, outlier_frac=outliers)
    b = synth.normal_bf16(sh_b, sig_b, seed + 1)
    qa, sa, _ = oracle.quant(a, fa)
    qb, sb, _ = oracle.quant(b, fb)
    return qa, sa, qb, sb


@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("kind", LAYOUTS)
@pytest.mark.parametrize("fa,fb", FORMATS)
@pytest.mark.parametrize("MNR", [(256, 1024, 512), (300, 200, 160), (64, 48, 16), (513, 257, 400),
                                 (256, 256, 1024), (1, 1, 16), (100, 60, 37), (257, 130, 1000), (40, 24, 1),
                                 (192, 200, 129)])
def test_layouts(accum, kind, fa, fb, MNR):
    """Every layout, format pair and accumulation mode on ragged tiles and
    reduction lengths that are not multiples of 16 (1, 37, 129, 1000)."""
    M, N, R = MNR
    qa, sa, qb, sb = operands(kind, M, N, R, fa, fb, 10 * M + N + R + fa + 2 * fb + 5 * LAYOUTS.index(kind))
    y = run(kind, padded(qa), fa, sa, padded(qb), fb, sb, accum)
    torch.cuda.synchronize()
    check_gemm(bf16_bits(y), kind, qa, fa, sa, qb, fb, sb, f"{kind} {MNR} fmt {fa}{fb}", accum=accum)


@pytest.mark.parametrize("accum", ACCUMS)
def test_random_shapes(accum):
    """Twenty-four seeded random shapes over the three layouts: M and N in
    [1, 700) (ragged tiles of both tile widths), any reduction length up to
    1100, random format pair."""
    rng = np.random.default_rng(2024 + accum)
    for i in range(24):
        kind = LAYOUTS[i % 3]
        M, N = (int(v) for v in rng.integers(1, 700, 2))
        R = int(rng.integers(1, 1100))
        fa, fb = (int(v) for v in rng.integers(0, 2, 2))
        qa, sa, qb, sb = operands(kind, M, N, R, fa, fb, 7000 + i)
        y = run(kind, padded(qa), fa, sa, padded(qb), fb, sb, accum)
        torch.cuda.synchronize()
        check_gemm(bf16_bits(y), kind, qa, fa, sa, qb, fb, sb, f"random {kind} {M}x{N}x{R} fmt {fa}{fb}",
                   accum=accum)


@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("kind", LAYOUTS)
def test_tile_threshold_shapes(accum, kind):
    """Output shapes on both sides of the switch between 256-row tiles and
    128x128 tiles (192 tiles of 256x192): 2816 x 3072 (176 tiles of 256x192,
    so 528 of 128x128), 3072 x 3072 (192 tiles of 256x192), and ragged
    neighbours of both; a reduction of 390 (not a multiple of 16).  Checked
    on sampled output rows, the first and last included."""
    rng = np.random.default_rng(31 + LAYOUTS.index(kind) + 10 * accum)
    for M, N in ((2816, 3072), (3072, 3072), (2811, 3000), (3059, 3112)):
        R = 390
        qa, sa, qb, sb = operands(kind, M, N, R, E5, E4, 8100 + M + N)
        y = run(kind, padded(qa), E5, sa, padded(qb), E4, sb, accum)
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 22, replace=False)]))
        got = bf16_bits(y)[rows]
        check_gemm(got, kind, qa, E5, sa, qb, E4, sb, f"threshold {kind} {M}x{N}x{R}", rows=rows, accum=accum)


@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("fa,fb", FORMATS)
def test_nt_wide_tiles_ragged(accum, fa, fb):
    """NT products that take 256x256 tiles (fast mode: 8 waves of 64x128;
    exact mode: 4 waves of 128x128): 2087 x 6199 is 9 x 25 = 225 such tiles,
    one wave over the CUs, ragged in M (39 rows) and N (55 columns), with a
    reduction of 390 (not a multiple of 16) and 2096 x 6208 x 3072 with whole
    16-byte chunks.  Checked on sampled output rows, the first and the last
    included."""
    rng = np.random.default_rng(77 + fa + 2 * fb + 10 * accum)
    for M, N, R in ((2087, 6199, 390), (2096, 6208, 3072)):
        qa, sa, qb, sb = operands("nt", M, N, R, fa, fb, 8300 + M + R)
        y = run("nt", padded(qa), fa, sa, padded(qb), fb, sb, accum)
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 22, replace=False)]))
        check_gemm(bf16_bits(y)[rows], "nt", qa, fa, sa, qb, fb, sb, f"wide tiles nt {M}x{N}x{R} fmt {fa}{fb}",
                   rows=rows, accum=accum)


@pytest.mark.parametrize("kind", LAYOUTS)
def test_exactly_representable_sums(kind):
    """Codes of magnitude in [1, 4) with unit scales: every product is a
    multiple of 2^-6 below 16, so each partial sum of 1024 of them is exact in
    fp32 and no product loses bits to the matrix core's group alignment.
    Both modes must then give RN_bf16 of the exact sum bit for bit: any wrong
    index, transposition or dropped product would show."""
    M, N, R = 272, 200, 1024
    rng = np.random.default_rng(77 + LAYOUTS.index(kind))
    sh_a, sh_b = storage(kind, M, N, R)

    def codes(fmt, shape):
        # E4M3: exponent fields 7..8 (1 <= |v| < 4), any mantissa; E5M2: 15..16
        e = rng.integers(7, 9, shape) if fmt == E4 else rng.integers(15, 17, shape)
        mbits = 3 if fmt == E4 else 2
        m = rng.integers(0, 1 << mbits, shape)
        return ((rng.integers(0, 2, shape) << 7) | (e << mbits) | m).astype(np.uint8)

    for fa, fb in FORMATS:
        a, b = codes(fa, sh_a), codes(fb, sh_b)
        ref = {"nt": oracle.gemm_nt, "nn": oracle.gemm_nn, "tn": oracle.gemm_tn}[kind](a, fa, 1.0, b, fb, 1.0)
        for accum in ACCUMS:
            y = run(kind, padded(a), fa, 1.0, padded(b), fb, 1.0, accum)
            torch.cuda.synchronize()
            got = bf16_bits(y)
            assert (got == ref).all(), (kind, fa, fb, accum, int((got != ref).sum()))


@pytest.mark.parametrize("accum", ACCUMS)
def test_linear_small_workload(accum):
    """Single linear forward: X [256x512] N(0,1), W [1024x512] N(0,0.02),
    both quantised on the GPU (codes and scales bit-exact)."""
    from fp8_tensorwise_scaled_amd import api
    from tests.gpu_util import to_dev_bf16

    x, w = synth.LINEAR_SMALL.tensors()
    xq, _, sx, _ = api.fp8_amax_quant(to_dev_bf16(x), E4)
    wq, _, sw, _ = api.fp8_amax_quant(to_dev_bf16(w), E4)
    y = api.fp8_linear_fwd(xq, sx, wq, sw, accum=accum)
    torch.cuda.synchronize()
    rx, rsx, _ = oracle.quant(x, E4)
    rw, rsw, _ = oracle.quant(w, E4)
    assert (xq.cpu().numpy() == rx).all() and (wq.cpu().numpy() == rw).all()
    assert float(sx.cpu()[0]) == np.float32(rsx) and float(sw.cpu()[0]) == np.float32(rsw)
    check_gemm(bf16_bits(y), "nt", rx, E4, rsx, rw, E4, rsw, "linear 256x1024x512", accum=accum)


@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("MNK", [(256, 1024, 512), (300, 200, 37), (1, 48, 16), (513, 257, 400)])
def test_linear_fwd_bf16(accum, MNK):
    """The linear forward from bf16 (both quantisations batched, then the
    GEMM): codes and scales bit-exact against the oracle's quantiser, Y at
    the GEMM bar on those codes, and every output byte-identical to the
    separate calls (fp8_amax_quant of X and of W, then fp8_linear_fwd)."""
    from fp8_tensorwise_scaled_amd import api
    from tests.gpu_util import to_dev_bf16

    M, N, K = MNK
    x = synth.normal_bf16((M, K), 1.0, 4100 + M, outlier_frac=1e-3)
    w = synth.normal_bf16((N, K), 0.02, 4200 + N)
    xd, wd = to_dev_bf16(x), to_dev_bf16(w)
    y, xq, wq, sc = api.fp8_linear_fwd_bf16(xd, wd, accum=accum)
    xq2, _, sx2, _ = api.fp8_amax_quant(xd, E4, q=padded(np.zeros((M, K), np.uint8)))
    wq2, _, sw2, _ = api.fp8_amax_quant(wd, E4, q=padded(np.zeros((N, K), np.uint8)))
    y2 = api.fp8_linear_fwd(xq2, sx2, wq2, sw2, accum=accum)
    torch.cuda.synchronize()
    rx, rsx, _ = oracle.quant(x, E4)
    rw, rsw, _ = oracle.quant(w, E4)
    scales = sc.cpu().numpy()
    assert (xq.cpu().numpy() == rx).all() and (wq.cpu().numpy() == rw).all()
    assert scales[0] == np.float32(rsx) and scales[1] == np.float32(rsw)
    check_gemm(bf16_bits(y), "nt", rx, E4, rsx, rw, E4, rsw, f"linear from bf16 {MNK}", accum=accum)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(xq, xq2) and torch.equal(wq, wq2)
    assert scales[0] == float(sx2.cpu()[0]) and scales[1] == float(sw2.cpu()[0])


def test_linear_fwd_bf16_empty():
    """No tokens: both scales written (X's is 1), no Y; no reduction: Y = 0."""
    from fp8_tensorwise_scaled_amd import api
    from tests.gpu_util import to_dev_bf16

    w = synth.normal_bf16((48, 64), 0.02, 4300)
    y, xq, wq, sc = api.fp8_linear_fwd_bf16(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda:0"),
                                            to_dev_bf16(w))
    torch.cuda.synchronize()
    assert y.shape == (0, 48)
    assert sc.cpu().numpy()[0] == 1.0 and sc.cpu().numpy()[1] == np.float32(oracle.quant(w, E4)[1])
    y, _, _, sc = api.fp8_linear_fwd_bf16(torch.empty((32, 0), dtype=torch.bfloat16, device="cuda:0"),
                                          torch.empty((48, 0), dtype=torch.bfloat16, device="cuda:0"))
    torch.cuda.synchronize()
    assert (y.float() == 0).all() and (sc.cpu().numpy() == 1.0).all()


@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("MNK", [(256, 512, 384), (208, 160, 96), (2048, 768, 3072)])
def test_dgrad_wgrad(accum, MNK):
    """dX = dY . W (NN) and dW = dY^T . X (TN) on the row-major codes of a
    linear layer: X [M,K] N(0,1), W [N,K] N(0,0.02), dY [M,N] N(0,1e-3) with
    0.1% x100 outliers (E5M2)."""
    from fp8_tensorwise_scaled_amd import api

    M, N, K = MNK
    g = synth.normal_bf16((M, N), 1e-3, M + N, outlier_frac=1e-3)
    w = synth.normal_bf16((N, K), 0.02, M + K)
    x = synth.normal_bf16((M, K), 1.0, N + K)
    gq, sg, _ = oracle.quant(g, E5)
    wq, sw, _ = oracle.quant(w, E4)
    xq, sx, _ = oracle.quant(x, E4)
    dx = api.fp8_linear_dgrad(to_dev_u8(gq), scal(sg), to_dev_u8(wq), scal(sw), accum=accum)
    dw = api.fp8_linear_wgrad(to_dev_u8(gq), scal(sg), to_dev_u8(xq), scal(sx), accum=accum)
    torch.cuda.synchronize()
    check_gemm(bf16_bits(dx), "nn", gq, E5, sg, wq, E4, sw, f"dgrad {MNK}", accum=accum)
    check_gemm(bf16_bits(dw), "tn", gq, E5, sg, xq, E4, sx, f"wgrad {MNK}", accum=accum)


@pytest.mark.parametrize("kind", LAYOUTS)
def test_strided_output_and_operands(kind):
    """Operands with leading dimensions well past their extents (NaN codes in
    between) and an output written into a wider buffer: columns past N stay
    untouched."""
    M, N, R = 200, 136, 192
    qa, sa, qb, sb = operands(kind, M, N, R, E4, E4, 99)
    r16 = lambda n: -(-n // 16) * 16
    A, B = padded(qa, ld=r16(qa.shape[1]) + 64), padded(qb, ld=r16(qb.shape[1]) + 48)
    C = torch.full((M, 200), 7, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
    run(kind, A, E4, sa, B, E4, sb, ACC_FAST, out=C[:, :N])
    torch.cuda.synchronize()
    Cb = bf16_bits(C)
    check_gemm(Cb[:, :N], kind, qa, E4, sa, qb, E4, sb, f"strided {kind}")
    assert (Cb[:, N:] == 7).all()   # columns past N untouched


def test_largest_operand_offsets():
    """Operand rows spaced as far apart as the library accepts.  K-major (NT):
    a 256-row tile spans (255 lda + K) < 2^31 bytes of 32-bit buffer offsets,
    lda = 8,421,488 with K = 4096.  MN-major (TN): every reduction row plus one
    stage of 128 rows read as zeros, (K + 128) ld + 256 < 2^31, ld = 5,368,704
    with K = 272.  16 bytes more is refused (tests/test_abi.py).  Ragged tiles
    in both directions; the bytes between rows are never read."""
    from fp8_tensorwise_scaled_amd import api

    dev = torch.device("cuda:0")
    M, N, K, LD = 300, 200, 4096, 8_421_488
    assert 255 * LD + K < 2 ** 31 <= 255 * (LD + 16) + K
    qa, sa, qb, sb = operands("nt", M, N, K, E4, E5, 4242)
    ra = torch.empty((M - 1) * LD + K, dtype=torch.uint8, device=dev)
    rb = torch.empty((N - 1) * LD + K, dtype=torch.uint8, device=dev)
    A, B = ra.as_strided((M, K), (LD, 1)), rb.as_strided((N, K), (LD, 1))
    A.copy_(to_dev_u8(qa))
    B.copy_(to_dev_u8(qb))
    y = api.fp8_linear_fwd(A, scal(sa), B, scal(sb), E4, E5)
    torch.cuda.synchronize()
    check_gemm(bf16_bits(y), "nt", qa, E4, sa, qb, E5, sb, "largest K-major offsets 300x200x4096")
    del ra, rb, A, B

    R, LDM = 272, 5_368_704
    assert (R + 128) * LDM + 256 < 2 ** 31 <= (R + 128) * (LDM + 16) + 256
    qa, sa, qb, sb = operands("tn", M, N, R, E5, E4, 4243)
    ra = torch.empty((R - 1) * LDM + M, dtype=torch.uint8, device=dev)
    rb = torch.empty((R - 1) * LDM + N, dtype=torch.uint8, device=dev)
    A, B = ra.as_strided((R, M), (LDM, 1)), rb.as_strided((R, N), (LDM, 1))
    A.copy_(to_dev_u8(qa))
    B.copy_(to_dev_u8(qb))
    y = api.fp8_linear_wgrad(A, scal(sa), B, scal(sb), E5, E4)
    torch.cuda.synchronize()
    check_gemm(bf16_bits(y), "tn", qa, E5, sa, qb, E4, sb, "largest MN-major offsets 300x200x272")
    del ra, rb, A, B
    torch.cuda.empty_cache()


def test_empty_sizes():
    """A reduction of length 0 writes the empty sum (+0) everywhere; M = 0 or
    N = 0 is a no-op.  Each of the three GEMMs, with the oracle's result."""
    from fp8_tensorwise_scaled_amd import api

    dev = torch.device("cuda:0")
    u8e = lambda r, c: torch.empty((r, c), dtype=torch.uint8, device=dev)
    s1, s2 = scal(0.5), scal(3.0)
    z = lambda r, c: np.zeros((r, c), np.uint8)
    for accum in ACCUMS:
        for name, call, ref in (
                ("fwd K=0", lambda out: api.fp8_linear_fwd(u8e(40, 0), s1, u8e(24, 0), s2, out=out, accum=accum),
                 oracle.gemm_nt(z(40, 0), E4, 0.5, z(24, 0), E4, 3.0)),
                ("dgrad N=0", lambda out: api.fp8_linear_dgrad(u8e(40, 0), s1, u8e(0, 24), s2, out=out, accum=accum),
                 oracle.gemm_nn(z(40, 0), E5, 0.5, z(0, 24), E4, 3.0)),
                ("wgrad M=0", lambda out: api.fp8_linear_wgrad(u8e(0, 40), s1, u8e(0, 24), s2, out=out, accum=accum),
                 oracle.gemm_tn(z(0, 40), E5, 0.5, z(0, 24), E4, 3.0))):
            out = torch.full((40, 24), 7, dtype=torch.int16, device=dev).view(torch.bfloat16)
            call(out)
            torch.cuda.synchronize()
            assert (bf16_bits(out) == ref).all() and (ref == 0).all(), (name, accum)
    # empty outputs: nothing to write, the call succeeds
    y = api.fp8_linear_fwd(u8e(0, 64), s1, u8e(24, 64), s2)
    y2 = api.fp8_linear_fwd(u8e(40, 64), s1, u8e(0, 64), s2)
    y3 = api.fp8_linear_wgrad(u8e(64, 0), s1, u8e(64, 24), s2)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (0, 24) and tuple(y2.shape) == (40, 0) and tuple(y3.shape) == (0, 24)


@pytest.mark.parametrize("kind", LAYOUTS)
def test_output_rows_not_16_byte_aligned(kind):
    """Odd leading dimension and a base 2 bytes off a dword: every row phase
    (0-14 bytes past a 16-byte boundary) occurs among the rows, so every
    store width the epilogue picks by alignment (2, 4, 8, 16 bytes) is used;
    the last column tile is 8 columns wide."""
    M, N, R = 264, 392, 256
    qa, sa, qb, sb = operands(kind, M, N, R, E4, E5, 98)
    ldc = 401
    flat = torch.full((1 + M * ldc,), 7, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
    C = flat[1:].view(M, ldc)
    run(kind, padded(qa), E4, sa, padded(qb), E5, sb, ACC_FAST, out=C[:, :N])
    torch.cuda.synchronize()
    Cb = bf16_bits(C)
    check_gemm(Cb[:, :N], kind, qa, E4, sa, qb, E5, sb, f"odd ldc {kind}")
    assert (Cb[:, N:] == 7).all() and int(bf16_bits(flat[:1])[0]) == 7   # nothing outside written


@pytest.mark.parametrize("accum", ACCUMS)
def test_wide_tiles_output_rows_not_16_byte_aligned(accum):
    """The unpadded-vocabulary case on 256x256 NT tiles: 2087 x 6199 outputs
    (ragged in both directions) into rows 6201 elements apart, 2 bytes past
    a dword.  Sampled rows against the oracle, the first and last included;
    no byte outside the output is written."""
    M, N, R = 2087, 6199, 272
    qa, sa, qb, sb = operands("nt", M, N, R, E4, E4, 8400 + accum)
    ldc = 6201
    flat = torch.full((1 + M * ldc,), 7, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
    C = flat[1:].view(M, ldc)
    run("nt", padded(qa), E4, sa, padded(qb), E4, sb, accum, out=C[:, :N])
    torch.cuda.synchronize()
    Cb = bf16_bits(C)
    rng = np.random.default_rng(91 + accum)
    rows = np.unique(np.concatenate([[0, 1, M - 2, M - 1], rng.choice(M, 20, replace=False)]))
    check_gemm(Cb[rows, :N], "nt", qa, E4, sa, qb, E4, sb, "wide tiles, odd ldc", rows=rows, accum=accum)
    assert (Cb[:, N:] == 7).all() and int(bf16_bits(flat[:1])[0]) == 7   # nothing outside written


@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("which", ["up_fwd", "down_dgrad", "up_wgrad"])
def test_full_size_sampled_rows(which, accum):
    """3.8B-model block shapes (M=8192, d=3072, h=12288) on the GPU in the
    layouts the block's GEMMs take, checked on 48 sampled output rows
    computed by the oracle."""
    from fp8_tensorwise_scaled_amd import api

    M, d, h = 8192, 3072, 12288
    rng = np.random.default_rng(3)
    if which == "up_fwd":
        qa, sa, qb, sb = operands("nt", M, h, d, E4, E4, 501)
        y = api.fp8_linear_fwd(to_dev_u8(qa), scal(sa), to_dev_u8(qb), scal(sb), accum=accum)
        rows = rng.choice(M, 48, replace=False)
        args = ("nt", qa, E4, sa, qb, E4, sb)
    elif which == "down_dgrad":   # dA [M, h] = dY [M, d] . W_down [d, h]
        g = synth.normal_bf16((M, d), 1e-3, 502, outlier_frac=1e-3)
        w = synth.normal_bf16((d, h), 0.02, 503)
        gq, sa, _ = oracle.quant(g, E5)
        wq, sb, _ = oracle.quant(w, E4)
        y = api.fp8_linear_dgrad(to_dev_u8(gq), scal(sa), to_dev_u8(wq), scal(sb), accum=accum)
        rows = rng.choice(M, 48, replace=False)
        args = ("nn", gq, E5, sa, wq, E4, sb)
    else:                         # dW_up [h, d] = dH [M, h]^T . X [M, d]
        g = synth.normal_bf16((M, h), 1e-3, 504, outlier_frac=1e-3)
        x = synth.normal_bf16((M, d), 1.0, 505)
        gq, sa, _ = oracle.quant(g, E5)
        xq, sb, _ = oracle.quant(x, E4)
        y = api.fp8_linear_wgrad(to_dev_u8(gq), scal(sa), to_dev_u8(xq), scal(sb), accum=accum)
        rows = rng.choice(h, 48, replace=False)
        args = ("tn", gq, E5, sa, xq, E4, sb)
    torch.cuda.synchronize()
    check_gemm(bf16_bits(y)[rows], *args, which, rows=rows, accum=accum)


@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("which", ["gate_fwd", "down_fwd", "gate_wgrad"])
def test_gated_width_sampled_rows(which, accum):
    """Shapes of the gated block at d=3072, h=8448 (33 tiles of 256, 44 of
    192 along h): G = Xq Wgq^T (N = 8448), Y = Aq Wdq^T (K = 8448) and
    dW_gate = dGq^T Xq (8448 output rows, K = 8192), on 48 sampled output
    rows computed by the oracle."""
    from fp8_tensorwise_scaled_amd import api

    M, d, h = 8192, 3072, 8448
    rng = np.random.default_rng(4)
    if which == "gate_fwd":
        qa, sa, qb, sb = operands("nt", M, h, d, E4, E4, 511)
        y = api.fp8_linear_fwd(to_dev_u8(qa), scal(sa), to_dev_u8(qb), scal(sb), accum=accum)
        rows = rng.choice(M, 48, replace=False)
        args = ("nt", qa, E4, sa, qb, E4, sb)
    elif which == "down_fwd":
        qa, sa, qb, sb = operands("nt", M, d, h, E4, E4, 512)
        y = api.fp8_linear_fwd(to_dev_u8(qa), scal(sa), to_dev_u8(qb), scal(sb), accum=accum)
        rows = rng.choice(M, 48, replace=False)
        args = ("nt", qa, E4, sa, qb, E4, sb)
    else:
        g = synth.normal_bf16((M, h), 1e-3, 513, outlier_frac=1e-3)
        x = synth.normal_bf16((M, d), 1.0, 514)
        gq, sa, _ = oracle.quant(g, E5)
        xq, sb, _ = oracle.quant(x, E4)
        y = api.fp8_linear_wgrad(to_dev_u8(gq), scal(sa), to_dev_u8(xq), scal(sb), accum=accum)
        rows = rng.choice(h, 48, replace=False)
        args = ("tn", gq, E5, sa, xq, E4, sb)
    torch.cuda.synchronize()
    check_gemm(bf16_bits(y)[rows], *args, which, rows=rows, accum=accum)


@pytest.mark.parametrize("kind", LAYOUTS)
def test_deterministic(kind):
    qa, sa, qb, sb = operands(kind, 1024, 1536, 2048, E5, E4, 7)
    A, B = to_dev_u8(qa), to_dev_u8(qb)
    for accum in ACCUMS:
        ys = [run(kind, A, E5, sa, B, E4, sb, accum) for _ in range(4)]
        torch.cuda.synchronize()
        for y in ys[1:]:
            assert torch.equal(y, ys[0])


def test_matrix_core_group_truncation():
    """The case that shows the two accumulation modes apart: one row holding
    256, -256 and sixty-two products of 2^-6 against ones.  The exact sum is
    62 * 2^-6 = 0.96875.  The FP8 matrix core truncates the 2^-6 products that
    share an 8-product group with the 256s, so the fast result differs from
    the exact one by more than a bf16 ulp, yet stays within
    7 * 2^-13 * sum|a b|; the exact mode returns 0.96875."""
    from fp8_tensorwise_scaled_amd import api

    one, c256, cm256, small = 0x38, 0x78, 0xF8, 0x08  # 1.0, 256, -256, 2^-6 (E4M3)
    assert [oracle.decode(E4, c) for c in (one, c256, cm256, small)] == [1.0, 256.0, -256.0, 2.0 ** -6]
    a = np.full((16, 64), small, np.uint8)
    a[:, 0], a[:, 1] = c256, cm256
    b = np.full((16, 64), one, np.uint8)
    ref = oracle.gemm_nt(a, E4, 1.0, b, E4, 1.0)
    assert (bits_f64(ref) == 0.96875).all()
    sabs = oracle.gemm_nt(a & 0x7F, E4, 1.0, b, E4, 1.0)
    fast = bits_f64(bf16_bits(api.fp8_linear_fwd(to_dev_u8(a), scal(1.0), to_dev_u8(b), scal(1.0))))
    exact = bits_f64(bf16_bits(api.fp8_linear_fwd(to_dev_u8(a), scal(1.0), to_dev_u8(b), scal(1.0),
                                                  accum=ACC_EXACT)))
    torch.cuda.synchronize()
    assert (np.abs(fast - 0.96875) > 2.0 ** -8).all()           # a real deviation from the exact sum
    assert (np.abs(fast - 0.96875) <= gemm_bound(ref, sabs, 64)).all()
    assert (exact == 0.96875).all()


@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("fa,fb", FORMATS)
def test_subnormal_codes(fa, fb, accum):
    """Subnormal FP8 operands (exponent field 0) reach the matrix cores as
    their values, not flushed to zero: an all-subnormal GEMM and one where
    half of the codes are subnormal, against the oracle.  With unit scales
    the all-subnormal products are 2^-18 .. 2^-12 (E4M3) and their sums stay
    normal in bf16."""
    rng = np.random.default_rng(31 + 2 * fa + fb)
    M, N, K = 96, 80, 256

    def subnormals(fmt, shape):
        mant = 0x07 if fmt == E4 else 0x03
        return (rng.integers(0, mant + 1, shape) | (rng.integers(0, 2, shape) << 7)).astype(np.uint8)

    def finite(fmt, shape):
        c = rng.integers(0, 256, shape).astype(np.uint8)
        nan = (c & 0x7F) == 0x7F if fmt == E4 else (c & 0x7C) == 0x7C
        return np.where(nan, c & 0x80, c).astype(np.uint8)

    sa_all, sb_all = subnormals(fa, (M, K)), subnormals(fb, (N, K))
    assert all(oracle.decode(fa, int(c)) == 0 or abs(oracle.decode(fa, int(c))) < 2.0 ** -6 for c in np.unique(sa_all))
    mask_a, mask_b = rng.integers(0, 2, (M, K)).astype(bool), rng.integers(0, 2, (N, K)).astype(bool)
    mixed_a = np.where(mask_a, subnormals(fa, (M, K)), finite(fa, (M, K))).astype(np.uint8)
    mixed_b = np.where(mask_b, subnormals(fb, (N, K)), finite(fb, (N, K))).astype(np.uint8)
    for what, a, b in (("all subnormal", sa_all, sb_all), ("half subnormal", mixed_a, mixed_b)):
        y = run("nt", to_dev_u8(a), fa, 1.0, to_dev_u8(b), fb, 1.0, accum)
        torch.cuda.synchronize()
        got = bf16_bits(y)
        check_gemm(got, "nt", a, fa, 1.0, b, fb, 1.0, f"{what} fmt {fa}{fb}", accum=accum)
        if what == "all subnormal":
            assert (bits_f64(got) != 0).mean() > 0.9  # not flushed


def test_fast_mode_statistics_reported():
    """The fast mode's one-ulp fraction and max-relative error on the 3.8B
    down-projection shape, printed beside the exact mode's for the same
    operands (the exact mode holds the strict bar; the fast mode holds its
    truncation bound, asserted in check_gemm)."""
    from fp8_tensorwise_scaled_amd import api

    M, N, K = 2048, 3072, 12288
    qa, sa, qb, sb = operands("nt", M, N, K, E4, E4, 515)
    rows = np.arange(0, M, 64)
    ref = oracle.gemm_nt(qa, E4, sa, qb, E4, sb, rows=rows)
    for accum in ACCUMS:
        y = api.fp8_linear_fwd(to_dev_u8(qa), scal(sa), to_dev_u8(qb), scal(sb), accum=accum)
        torch.cuda.synchronize()
        rel, within = gemm_stats(bf16_bits(y)[rows], ref)
        print(f"[stats] {'exact' if accum == ACC_EXACT else 'fast'} K={K}: max_rel={rel:.3g} within1={within:.6f}")
        check_gemm(bf16_bits(y)[rows], "nt", qa, E4, sa, qb, E4, sb, "stats", rows=rows, accum=accum)
