"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch


def dev():
    return torch.device("cuda:0")


def to_dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev())


def to_dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy()


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float32)


def bits_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    a = np.abs(v)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 7)


# Accuracy of the gfx950 FP8 matrix core (measured on the hardware): the 64
# products of one v_mfma_f32_32x32x64_f8f6f4 are summed in aligned groups of 8
# consecutive k; inside a group every product's magnitude is truncated to a
# multiple of 2^(e - 13), e the exponent of the group's largest product, and
# group sums are then combined without further loss.  So one dot product of
# length K differs from the exact sum by at most 7 * 2^-13 * sum_k |a_k b_k|,
# plus the fp32 accumulation over the K/64 instructions.
HW_GROUP_TRUNC = 7 * 2.0 ** -13


def gemm_bound(ref_bits: np.ndarray, sabs_bits: np.ndarray, K: int) -> np.ndarray:
    """Per-element tolerance for out = RN_bf16(RN32(acc * p)) against the
    oracle's RN_bf16(exact * p): if the pre-rounding values differ by D, the
    two bf16 roundings differ by at most D (1 + 2^-8) + 1.5 ulp(oracle).  D is
    bounded by the matrix-core truncation plus fp32 accumulation and scaling,
    (7 * 2^-13 + (K/64 + 2) * 2^-24) * p * sum|a b|; sabs_bits is the oracle
    GEMM on sign-cleared codes, i.e. RN_bf16(p * sum|a b|)."""
    r = bits_f64(ref_bits)
    sabs = bits_f64(sabs_bits) * (1 + 2.0 ** -7)
    return 1.5 * ulp_bf16(r) + (1 + 2.0 ** -8) * (HW_GROUP_TRUNC + (K / 64 + 2) * 2.0 ** -24) * sabs


def within_floors(K, heavy_tailed=False):
    """Aggregate floors (fraction within one and two bf16 ulps) that guard
    against a bound grown loose.  Measured: 99.68-99.97% / >= 99.87% for
    K <= 12288; the grad-weight GEMMs that reduce over 32768 tokens of a dY
    with 0.1% x100 outliers reach 99.49-99.59% / 99.71-99.76% (more outputs
    are small next to the sum of |products| their truncation error scales
    with); the LM head's 50304-long reduction, without outliers, 99.92%.
    heavy_tailed: a reduction whose operand is itself a product of such
    factors (the gated block's grad-weights) gets the long-reduction floors
    at any K."""
    return (0.995, 0.998) if (K is None or K <= 12288) and not heavy_tailed else (0.99, 0.995)


def gemm_close(got_bits: np.ndarray, ref_bits: np.ndarray, what: str = "", *, sabs_bits=None, K=None,
               bound=None, min_within1=None, min_within2=None):
    """GEMM output parity.

    Element-wise: |gpu - oracle| <= gemm_bound (or an explicit `bound`).
    Aggregate: the fraction of elements within one bf16 ulp of the oracle is
    at least min_within1, within two ulps at least min_within2 (defaults from
    within_floors(K)).  Also prints max|gpu - oracle| / max|oracle| and the
    one-ulp fraction."""
    f1, f2 = within_floors(K)
    min_within1 = f1 if min_within1 is None else min_within1
    min_within2 = f2 if min_within2 is None else min_within2
    g, r = bits_f64(got_bits), bits_f64(ref_bits)
    assert g.shape == r.shape, (g.shape, r.shape)
    err = np.abs(g - r)
    scale = np.abs(r).max()
    rel = err.max() / scale if scale > 0 else err.max()
    u = ulp_bf16(r)
    within = float((err <= u).mean())
    within2 = float((err <= 2 * u).mean())
    if bound is None:
        assert sabs_bits is not None and K is not None
        bound = gemm_bound(ref_bits, sabs_bits, K)
    over = err > bound
    print(f"[gemm_close] {what}: n={r.size} max_rel={rel:.3g} within1={within:.6f} within2={within2:.6f} "
          f"max_err/bound={float((err / bound).max()):.3g}")
    assert not over.any(), f"{what}: {int(over.sum())} elements beyond the bound, e.g. " + str(
        [(float(g.flat[i]), float(r.flat[i]), float(bound.flat[i])) for i in np.flatnonzero(over)[:4]])
    assert within >= min_within1 and within2 >= min_within2, (
        f"{what}: within 1 ulp {within:.6f}, within 2 ulps {within2:.6f}")
    return rel, within


def abs_codes(q: np.ndarray) -> np.ndarray:
    return q & np.uint8(0x7F)


def oracle_gemm(kind: str, a, fa, sa, b, fb, sb, rows=None):
    """Oracle GEMM of the given kind ('nt', 'nn', 'tn'), the same GEMM on the
    sign-cleared codes (sum of |products|, for the bound), and K."""
    import oracle

    fn = {"nt": oracle.gemm_nt, "nn": oracle.gemm_nn, "tn": oracle.gemm_tn}[kind]
    K = {"nt": a.shape[1], "nn": a.shape[1], "tn": a.shape[0]}[kind]
    ref = fn(a, fa, sa, b, fb, sb, rows=rows)
    sabs = fn(abs_codes(a), fa, sa, abs_codes(b), fb, sb, rows=rows)
    return ref, sabs, K


def check_gemm(got_bits, kind, a, fa, sa, b, fb, sb, what, rows=None, **floors):
    ref, sabs, K = oracle_gemm(kind, a, fa, sa, b, fb, sb, rows=rows)
    return gemm_close(got_bits, ref, what, sabs_bits=sabs, K=K, **floors)


def collect_block(inputs, y, saved, ws_f, ws_b, dx, dwu, dwd, bsc) -> dict:
    """Host copies of one relu^2 block pass: inputs, outputs, the saved
    forward quantities and the workspace intermediates (codes, dH)."""
    from fp8_tensorwise_scaled_amd import api

    x, wu, wd, dy = inputs
    M, d = x.shape
    h = wu.shape[0]
    of = api.workspace_layout("fwd", M, d, h)
    ob = api.workspace_layout("bwd", M, d, h)
    wf, wb = ws_f.cpu().numpy(), ws_b.cpu().numpy()
    sl = lambda buf, o, n: buf[o:o + n]
    return dict(
        x=x, wu=wu, wd=wd, dy=dy, y=bf16_bits(y), dx=bf16_bits(dx), dw_up=bf16_bits(dwu),
        dw_down=bf16_bits(dwd), h=bf16_bits(saved.h), scales=f32(saved.scales), bsc=f32(bsc),
        xq_t=u8(saved.xq_t), uq_t=u8(saved.uq_t), dq_t=u8(saved.dq_t), aq_t=u8(saved.aq_t),
        xq=sl(wf, of[0], M * d).reshape(M, d), uq=sl(wf, of[1], h * d).reshape(h, d),
        dq=sl(wf, of[2], d * h).reshape(d, h), aq=sl(wf, of[3], M * h).reshape(M, h),
        gq=sl(wb, ob[0], M * d).reshape(M, d), gq_t=sl(wb, ob[1], d * M).reshape(d, M),
        dh=sl(wb, ob[2], 2 * M * h).view(np.uint16).reshape(M, h), hq=sl(wb, ob[3], M * h).reshape(M, h),
        hq_t=sl(wb, ob[4], h * M).reshape(h, M))
