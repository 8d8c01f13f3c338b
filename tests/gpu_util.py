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


# GEMM accumulation modes of the library (FP8MLP_ACCUM_FAST / _EXACT).
ACC_FAST, ACC_EXACT = 0, 1
ACCUMS = (ACC_FAST, ACC_EXACT)

# The strict GEMM parity bar: max|gpu - oracle| / max|oracle| <= 5e-3 and at
# least 99.9% of the elements within one bf16 ulp of the oracle.
STRICT_MAX_REL = 5e-3
STRICT_WITHIN1 = 0.999

# Accuracy of the gfx950 FP8 matrix core (measured on the hardware): the 64
# products of one v_mfma_f32_32x32x64_f8f6f4 are summed in aligned groups of 8
# consecutive k; inside a group every product's magnitude is truncated to a
# multiple of 2^(e - 13), e the exponent of the group's largest product, and
# group sums are then combined without further loss.  So one dot product of
# length K differs from the exact sum by at most 7 * 2^-13 * sum_k |a_k b_k|,
# plus the fp32 accumulation over the K/64 instructions.  The exact mode's
# bf16 instructions multiply exactly (8-bit significands) and round once per
# 16 products into the fp32 accumulator.
HW_GROUP_TRUNC = 7 * 2.0 ** -13


def gemm_bound(ref_bits: np.ndarray, sabs_bits: np.ndarray, K: int, accum: int = ACC_FAST) -> np.ndarray:
    """Per-element tolerance for out = RN_bf16(RN32(acc * p)) against the
    oracle's RN_bf16(exact * p): if the pre-rounding values differ by D, the
    two bf16 roundings differ by at most D (1 + 2^-8) + 1.5 ulp(oracle).  D is
    bounded by the summation error plus the scaling: fast mode
    (7 * 2^-13 + (K/64 + 2) * 2^-24) * p * sum|a b|, exact mode
    (K/16 + 2) * 2^-24 * p * sum|a b|; sabs_bits is the oracle GEMM on
    sign-cleared codes, i.e. RN_bf16(p * sum|a b|)."""
    r = bits_f64(ref_bits)
    sabs = bits_f64(sabs_bits) * (1 + 2.0 ** -7)
    if accum == ACC_EXACT:
        term = (K / 16 + 2) * 2.0 ** -24
    else:
        term = HW_GROUP_TRUNC + (K / 64 + 2) * 2.0 ** -24
    return 1.5 * ulp_bf16(r) + (1 + 2.0 ** -8) * term * sabs


def gemm_stats(got_bits: np.ndarray, ref_bits: np.ndarray):
    """(max|gpu - oracle| / max|oracle|, fraction within one bf16 ulp)."""
    g, r = bits_f64(got_bits), bits_f64(ref_bits)
    err = np.abs(g - r)
    scale = np.abs(r).max() if r.size else 0.0
    rel = float(err.max() / scale) if scale > 0 else float(err.max() if err.size else 0.0)
    within = float((err <= ulp_bf16(r)).mean()) if r.size else 1.0
    return rel, within


def gemm_close(got_bits: np.ndarray, ref_bits: np.ndarray, what: str = "", *, sabs_bits=None, K=None,
               accum: int = ACC_FAST, bound=None):
    """GEMM output parity against the oracle on identical FP8 operands.

    Both modes: every element within gemm_bound (or an explicit `bound`).
    Exact mode: also the strict bar, max|gpu - oracle| / max|oracle| <= 5e-3
    and >= 99.9% of the elements within one bf16 ulp.  The fast mode's
    truncating group sums fall short of that bar by design (its element-wise
    bound is what the arithmetic guarantees); its max-relative error and
    one-ulp fraction are printed."""
    g, r = bits_f64(got_bits), bits_f64(ref_bits)
    assert g.shape == r.shape, (g.shape, r.shape)
    err = np.abs(g - r)
    rel, within = gemm_stats(got_bits, ref_bits)
    if bound is None:
        assert sabs_bits is not None and K is not None
        bound = gemm_bound(ref_bits, sabs_bits, K, accum)
    over = err > bound
    ratio = float((err / bound).max()) if err.size else 0.0
    print(f"[gemm_close] {what} ({'exact' if accum == ACC_EXACT else 'fast'}): n={r.size} max_rel={rel:.3g} "
          f"within1={within:.6f} max_err/bound={ratio:.3g}")
    assert not over.any(), f"{what}: {int(over.sum())} elements beyond the bound, e.g. " + str(
        [(float(g.flat[i]), float(r.flat[i]), float(bound.flat[i])) for i in np.flatnonzero(over)[:4]])
    if accum == ACC_EXACT:
        assert rel <= STRICT_MAX_REL, f"{what}: max|gpu - oracle| / max|oracle| = {rel:.3g} > {STRICT_MAX_REL}"
        assert within >= STRICT_WITHIN1, f"{what}: {within:.6f} of the elements within one ulp < {STRICT_WITHIN1}"
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


def check_gemm(got_bits, kind, a, fa, sa, b, fb, sb, what, rows=None, accum=ACC_FAST):
    ref, sabs, K = oracle_gemm(kind, a, fa, sa, b, fb, sb, rows=rows)
    return gemm_close(got_bits, ref, what, sabs_bits=sabs, K=K, accum=accum)


def collect_block(inputs, y, saved, ws_f, ws_b, dx, dwu, dwd, bsc) -> dict:
    """Host copies of one relu^2 block pass: inputs, outputs, the saved
    forward quantities (codes of X, W_up, W_down, A and H) and the backward
    workspace's intermediates (codes of dY, dH and its codes)."""
    from fp8_tensorwise_scaled_amd import api

    x, wu, wd, dy = inputs
    M, d = x.shape
    h = wu.shape[0]
    ob = api.workspace_layout("bwd", M, d, h)
    wb = ws_b.cpu().numpy()
    sl = lambda buf, o, n: buf[o:o + n]
    return dict(
        x=x, wu=wu, wd=wd, dy=dy, y=bf16_bits(y), dx=bf16_bits(dx), dw_up=bf16_bits(dwu),
        dw_down=bf16_bits(dwd), h=bf16_bits(saved.h), scales=f32(saved.scales), bsc=f32(bsc),
        xq=u8(saved.xq), uq=u8(saved.uq), dq=u8(saved.dq), aq=u8(saved.aq),
        gq=sl(wb, ob[0], M * d).reshape(M, d), dh=sl(wb, ob[1], 2 * M * h).view(np.uint16).reshape(M, h),
        hq=sl(wb, ob[2], M * h).reshape(M, h))
