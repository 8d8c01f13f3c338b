"""CPU oracle for FP8 tensorwise-scaled linears and the relu^2 MLP block.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product library
never calls it, and it imports nothing from the product package.

The arithmetic lives in ``fp8_oracle.c`` (plain C, fp64, OpenMP over output
rows); this module loads it with ctypes and composes the block from its
steps.  Every function takes and returns numpy arrays: bf16 tensors as
``uint16`` bit patterns, FP8 tensors as ``uint8`` codes.

Sources (the pages' statement of the method):
  * "Het trainen van een 3.8B LLM tot 0.384 CORE voor $998" (decomputer.nl),
    "Vroege experimenten" item 4 and the first bullet of "Doorvoer
    verhogen": all three GEMMs of every linear (one forward, two backward)
    in FP8 with dynamic tensorwise scaling, through a scaled matmul.
  * Same page, "Appendix: De configuratie": non-gated relu2 MLP with a 4x
    intermediate size, bf16 model dtype.
  * "little-lm" summary on manulx.blog (Japanese page), FP8 paragraph: the
    scaled matmul is torch._scaled_mm with dynamic per-tensor scales.
  * Same page, "Vroege experimenten" item 2 and the appendix: Muon for the
    matrix parameters; its Newton-Schulz orthogonalisation is taken as
    Muon's published quintic iteration (see ``newton_schulz``).
Readings where the pages are silent (formats, scale formula, rounding,
saturation, zero amax, operand layouts) are listed in the C file's header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

E4M3 = 0
E5M2 = 1
FMAX = {E4M3: 448.0, E5M2: 57344.0}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
               "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            i64, f32, c_int = ctypes.c_int64, ctypes.c_float, ctypes.c_int
            vp = ctypes.c_void_p
            lib.orc_decode.restype = ctypes.c_double
            lib.orc_decode.argtypes = [c_int, c_int]
            lib.orc_encode_rne.restype = c_int
            lib.orc_encode_rne.argtypes = [c_int, ctypes.c_double]
            lib.orc_double_to_bf16.restype = ctypes.c_uint16
            lib.orc_double_to_bf16.argtypes = [ctypes.c_double]
            lib.orc_double_to_bf16_array.restype = None
            lib.orc_double_to_bf16_array.argtypes = [vp, i64, vp]
            lib.orc_amax.restype = f32
            lib.orc_amax.argtypes = [vp, i64, i64, i64]
            lib.orc_scale_from_amax.restype = f32
            lib.orc_scale_from_amax.argtypes = [f32, c_int]
            lib.orc_cast.restype = None
            lib.orc_cast.argtypes = [vp, i64, i64, i64, f32, c_int, vp, i64]
            lib.orc_cast_f32.restype = None
            lib.orc_cast_f32.argtypes = [vp, i64, f32, c_int, vp]
            lib.orc_quant.restype = None
            lib.orc_quant.argtypes = [vp, i64, i64, i64, c_int, vp, i64, vp, vp]
            for name in ("orc_gemm_nt", "orc_gemm_nn", "orc_gemm_tn"):
                fn = getattr(lib, name)
                fn.restype = None
                fn.argtypes = [vp, i64, c_int, f32, vp, i64, c_int, f32, i64, i64, i64, vp, i64, vp, i64]
            lib.orc_gemm_tn_acc.restype = None
            lib.orc_gemm_tn_acc.argtypes = [vp, i64, c_int, f32, vp, i64, c_int, f32, i64, i64, i64, vp, i64]
            lib.orc_gemm_nn_acc.restype = None
            lib.orc_gemm_nn_acc.argtypes = [vp, i64, c_int, f32, vp, i64, c_int, f32, i64, i64, i64, vp, i64, vp, i64]
            lib.orc_rmsnorm.restype = None
            lib.orc_rmsnorm.argtypes = [vp, i64, i64, i64, vp, f32, vp, vp]
            lib.orc_relu2.restype = None
            lib.orc_relu2.argtypes = [vp, i64, vp]
            lib.orc_relu2_bwd.restype = None
            lib.orc_relu2_bwd.argtypes = [vp, vp, i64, vp]
            _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


# ------------------------------------------------------------------ formats
def decode(fmt: int, code: int) -> float:
    return _load().orc_decode(fmt, int(code))


def decode_table(fmt: int) -> np.ndarray:
    return np.array([decode(fmt, c) for c in range(256)], dtype=np.float64)


def encode_rne(fmt: int, value: float) -> int:
    return _load().orc_encode_rne(fmt, float(value))


def double_to_bf16(x) -> np.ndarray:
    """Round fp64 values to bf16 (one RNE step); returns bf16 bit patterns."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint16)
    _load().orc_double_to_bf16_array(_ptr(x), x.size, _ptr(out))
    return out


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------------ quantisation
def amax(x: np.ndarray) -> float:
    x = _c(x, np.uint16)
    r, c = x.shape
    return float(_load().orc_amax(_ptr(x), r, c, c))


def scale_from_amax(a: float, fmt: int) -> float:
    return float(np.float32(_load().orc_scale_from_amax(np.float32(a), fmt)))


def cast(x: np.ndarray, s: float, fmt: int) -> np.ndarray:
    """q = RNE_fp8(clamp(RN32(x / s), +-fmax)) for a given fp32 scale s."""
    x = _c(x, np.uint16)
    r, c = x.shape
    q = np.empty((r, c), dtype=np.uint8)
    _load().orc_cast(_ptr(x), r, c, c, np.float32(s), fmt, _ptr(q), c)
    return q


def cast_f32(x: np.ndarray, s: float, fmt: int) -> np.ndarray:
    x = _c(np.asarray(x, dtype=np.float32), np.float32)
    q = np.empty(x.shape, dtype=np.uint8)
    _load().orc_cast_f32(_ptr(x), x.size, np.float32(s), fmt, _ptr(q))
    return q


def quant(x: np.ndarray, fmt: int):
    """Dynamic tensorwise quantisation: returns (codes, scale, amax)."""
    x = _c(x, np.uint16)
    r, c = x.shape
    q = np.empty((r, c), dtype=np.uint8)
    s = np.zeros(1, dtype=np.float32)
    a = np.zeros(1, dtype=np.float32)
    _load().orc_quant(_ptr(x), r, c, c, fmt, _ptr(q), c, _ptr(s), _ptr(a))
    return q, float(s[0]), float(a[0])


# ------------------------------------------------------------------- GEMMs
def _gemm(name, a, fa, sa, b, fb, sb, M, N, K, out_rows, out_cols, rows):
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    idx = None
    n = 0
    if rows is not None:
        idx = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = idx.size
        out_rows = n
    y = np.empty((out_rows, out_cols), dtype=np.uint16)
    getattr(_load(), name)(_ptr(a), a.shape[1], fa, np.float32(sa), _ptr(b), b.shape[1], fb,
                           np.float32(sb), M, N, K, _ptr(y), out_cols,
                           None if idx is None else _ptr(idx), n)
    return y


def gemm_nt(a, fa, sa, b, fb, sb, rows=None):
    """y[m,n] = RN_bf16(RN32(sa*sb) * sum_k dec(a[m,k]) dec(b[n,k]))."""
    M, K = a.shape
    N, K2 = b.shape
    assert K == K2
    return _gemm("orc_gemm_nt", a, fa, sa, b, fb, sb, M, N, K, M, N, rows)


def gemm_nn(a, fa, sa, b, fb, sb, rows=None):
    """y[m,k] = RN_bf16(RN32(sa*sb) * sum_n dec(a[m,n]) dec(b[n,k]))."""
    M, N = a.shape
    N2, K = b.shape
    assert N == N2
    return _gemm("orc_gemm_nn", a, fa, sa, b, fb, sb, M, N, K, M, K, rows)


def gemm_tn(a, fa, sa, b, fb, sb, rows=None):
    """y[n,k] = RN_bf16(RN32(sa*sb) * sum_m dec(a[m,n]) dec(b[m,k]))."""
    M, N = a.shape
    M2, K = b.shape
    assert M == M2
    return _gemm("orc_gemm_tn", a, fa, sa, b, fb, sb, M, N, K, N, K, rows)


def gemm_tn_acc(a, fa, sa, b, fb, sb, acc: np.ndarray) -> None:
    """acc[n,k] += RN32(sa*sb) * sum_m dec(a[m,n]) dec(b[m,k]) in fp64, unrounded."""
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    M, N = a.shape
    M2, K = b.shape
    assert M == M2 and acc.shape == (N, K) and acc.dtype == np.float64 and acc.flags.c_contiguous
    _load().orc_gemm_tn_acc(_ptr(a), N, fa, np.float32(sa), _ptr(b), K, fb, np.float32(sb), M, N, K,
                            _ptr(acc), K)


def gemm_nn_acc(a, fa, sa, b, fb, sb, acc: np.ndarray, rows=None) -> None:
    """acc[i,k] += RN32(sa*sb) * sum_n dec(a[m,n]) dec(b[n,k]) (m = rows[i], or
    every row) in fp64, unrounded."""
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    M, N = a.shape
    N2, K = b.shape
    assert N == N2 and acc.dtype == np.float64 and acc.flags.c_contiguous and acc.shape[1] == K
    idx = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    assert acc.shape[0] == (M if idx is None else idx.size)
    _load().orc_gemm_nn_acc(_ptr(a), N, fa, np.float32(sa), _ptr(b), K, fb, np.float32(sb), M, N, K, _ptr(acc), K,
                            None if idx is None else _ptr(idx), 0 if idx is None else idx.size)


# --------------------------------------------------------------- RMSNorm
def rmsnorm(x: np.ndarray, gamma: np.ndarray | None, eps: float):
    """RMSNorm of bf16 rows (Llama-style, decomputer.nl appendix:
    rms_norm_eps 1.0e-6), each step in a stated precision:
      ms = RN32(RN64(sum_j x_j^2 / d))   (the sum in fp64)
      r  = RN32(1 / RN32(sqrt(RN32(ms + eps))))
      X_j = RN_bf16(RN32(RN32(x_j r) g_j))   (no g: RN_bf16(RN32(x_j r)))
    Returns (X as bf16 bits [rows, cols], r [rows] fp32)."""
    x = _c(x, np.uint16)
    r, c = x.shape
    out = np.empty((r, c), dtype=np.uint16)
    rstd = np.empty(r, dtype=np.float32)
    g = None if gamma is None else _c(np.asarray(gamma).reshape(-1), np.uint16)
    if g is not None:
        assert g.size == c
    _load().orc_rmsnorm(_ptr(x), r, c, c, None if g is None else _ptr(g), np.float32(eps), _ptr(out), _ptr(rstd))
    return out, rstd


def rmsnorm_quant(x: np.ndarray, gamma: np.ndarray | None, eps: float, fmt: int):
    """RMSNorm followed by the dynamic tensorwise quantisation of its output:
    returns (codes, scale, amax, X bits, rstd)."""
    xn, rstd = rmsnorm(x, gamma, eps)
    q, s, a = quant(xn, fmt)
    return q, s, a, xn, rstd


# --------------------------------------------------------------- relu^2
def relu2(h: np.ndarray) -> np.ndarray:
    h = _c(h, np.uint16)
    a = np.empty_like(h)
    _load().orc_relu2(_ptr(h), h.size, _ptr(a))
    return a


def relu2_bwd(h: np.ndarray, da: np.ndarray) -> np.ndarray:
    h = _c(h, np.uint16)
    da = _c(da, np.uint16)
    assert h.shape == da.shape
    dh = np.empty_like(h)
    _load().orc_relu2_bwd(_ptr(h), _ptr(da), h.size, _ptr(dh))
    return dh


# ------------------------------------------------------- FP8 linear layer
def linear_fwd(xq, fx, sx, wq, fw, sw, rows=None):
    """Forward GEMM of one FP8 linear: Y = X W^T (W stored [out, in])."""
    return gemm_nt(xq, fx, sx, wq, fw, sw, rows)


def linear_dgrad(dyq, fdy, sdy, wq, fw, sw, rows=None):
    """Grad-input GEMM: dX = dY W."""
    return gemm_nn(dyq, fdy, sdy, wq, fw, sw, rows)


def linear_wgrad(dyq, fdy, sdy, xq, fx, sx, rows=None):
    """Grad-weight GEMM: dW = dY^T X (overwrites; no accumulation)."""
    return gemm_tn(dyq, fdy, sdy, xq, fx, sx, rows)


# ------------------------------------------------------- relu^2 MLP block
def mlp_fwd(x, w_up, w_down):
    """Forward of Y = relu(X W_up^T)^2 W_down^T with FP8 on both GEMMs.

    X [M,d], W_up [h,d], W_down [d,h] as bf16 bits.  Returns every stage.
    """
    xq, sx, _ = quant(x, E4M3)
    uq, su, _ = quant(w_up, E4M3)
    dq, sd, _ = quant(w_down, E4M3)
    h = gemm_nt(xq, E4M3, sx, uq, E4M3, su)
    a = relu2(h)
    aq, sa, amax_a = quant(a, E4M3)
    y = gemm_nt(aq, E4M3, sa, dq, E4M3, sd)
    return dict(xq=xq, sx=sx, uq=uq, su=su, dq=dq, sd=sd, h=h, a=a, aq=aq, sa=sa,
                amax_a=amax_a, y=y)


def mlp_bwd(dy, saved):
    """Backward of the block given dY [M,d] (bf16 bits) and the forward stages."""
    gq, sg, _ = quant(dy, E5M2)
    dw_down = gemm_tn(gq, E5M2, sg, saved["aq"], E4M3, saved["sa"])
    da = gemm_nn(gq, E5M2, sg, saved["dq"], E4M3, saved["sd"])
    dh = relu2_bwd(saved["h"], da)
    hq, sh, amax_dh = quant(dh, E5M2)
    dw_up = gemm_tn(hq, E5M2, sh, saved["xq"], E4M3, saved["sx"])
    dx = gemm_nn(hq, E5M2, sh, saved["uq"], E4M3, saved["su"])
    return dict(gq=gq, sg=sg, dw_down=dw_down, da=da, dh=dh, hq=hq, sh=sh, amax_dh=amax_dh,
                dw_up=dw_up, dx=dx)


# ------------------------------------------- LM head + softcapped cross-entropy
def _sech2(x: np.ndarray) -> np.ndarray:
    """d tanh(x) / dx = 1 / cosh^2(x); 0 where cosh overflows (|x| > 710)."""
    with np.errstate(over="ignore"):
        return 1.0 / np.cosh(x) ** 2


def softcap_ce_rows(z_bits: np.ndarray, targets: np.ndarray, n_classes: int, softcap: float, n_valid: int):
    """Softcapped cross-entropy on bf16 logits Z [R, V] (bit patterns), in fp64.

    The model's logits are capped as S = c tanh(Z / c) (decomputer.nl,
    appendix: logit_softcap 15.0; loss LigerFusedLinearCrossEntropyLoss with
    softcap 15.0).  Over the first n_classes columns (the padded vocabulary
    rows of W are not classes):
      loss_r = logsumexp_j S_rj - S_r,t_r            (0 for ignored rows)
      G_rj   = (softmax_j(S_r) - [j = t_r]) (1 - tanh^2(Z_rj / c)) / n_valid
    with rows whose target is outside [0, n_classes) ignored (zero loss and
    gradient) and G = 0 in the padded columns.  The factor 1 - tanh^2 is
    evaluated as sech^2 = 1 / cosh^2, the same function: written as 1 - t*t
    it cancels to 0 in fp64 once |Z / c| > 18.7, where its value is still
    above 1e-16.  Returns (loss_r [R] fp64, G [R, V] fp64, dZ = RN_bf16(G)
    bits)."""
    R, V = z_bits.shape
    z = bf16_bits_to_f64(z_bits)[:, :n_classes]
    t = np.tanh(z / softcap)
    s = softcap * t
    m = s.max(axis=1, keepdims=True) if n_classes > 0 else np.zeros((R, 1))
    lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
    tg = np.asarray(targets, dtype=np.int64)
    valid = (tg >= 0) & (tg < n_classes)
    safe_t = np.where(valid, tg, 0)
    rows = np.arange(R)
    loss = np.where(valid, lse - s[rows, safe_t], 0.0)
    p = np.exp(s - lse[:, None])
    p[rows[valid], safe_t[valid]] -= 1.0
    g = np.zeros((R, V), dtype=np.float64)
    g[:, :n_classes] = p * _sech2(z / softcap) / max(n_valid, 1)
    g[~valid] = 0.0
    return loss, g, double_to_bf16(g)


def softcap_ce_columns(zt_bits: np.ndarray, cols, lse: np.ndarray, targets: np.ndarray, n_classes: int,
                       softcap: float, n_valid: int) -> np.ndarray:
    """Columns `cols` of the softcapped cross-entropy's logit gradient, given
    the logits of those columns for every row (zt_bits [ncols, R], bf16 bits,
    i.e. transposed) and every row's log-sum-exp (lse [R], fp64, over the
    classes).  Same formula as softcap_ce_rows; returns G^T [ncols, R] fp64
    and its bf16 bits."""
    cols = np.asarray(cols, dtype=np.int64)
    z = bf16_bits_to_f64(zt_bits)
    t = np.tanh(z / softcap)
    s = softcap * t
    p = np.exp(s - np.asarray(lse)[None, :])
    tg = np.asarray(targets, dtype=np.int64)
    valid = (tg >= 0) & (tg < n_classes)
    p -= (tg[None, :] == cols[:, None]).astype(np.float64)
    g = p * _sech2(z / softcap) / max(n_valid, 1)
    g[:, ~valid] = 0.0
    g[cols >= n_classes, :] = 0.0
    return g, double_to_bf16(g)


def lm_head_ce(x, w, targets, n_classes: int, softcap: float = 15.0, chunk: int | None = None):
    """FP8 LM head fused with the softcapped cross-entropy, chunked over rows.

    The head's GEMMs are FP8 linears with dynamic tensorwise scaling like
    every other linear (decomputer.nl, "Vroege experimenten" item 4).  The
    fusion (same page, "Doorvoer verhogen", fused linear cross-entropy
    bullet) processes `chunk` rows at a time so the full logits never exist:
      Xq, sx = Q(X, E4M3);  Wq, sw = Q(W, E4M3)        (whole tensors)
      per chunk k:  Z_k  = gemm(Xq_k, Wq)               (bf16 [C, V])
                    loss, dZ_k = softcap_ce_rows(Z_k)
                    dZq_k, s_k = Q(dZ_k, E5M2)           (the chunk's own scale)
                    dX_k = gemm(dZq_k, Wq)               (grad-input)
                    acc += RN32(s_k sx) dZq_k^T Xq_k     (fp64, unrounded)
      dW = RN_bf16(acc);  loss = sum of row losses / n_valid (0 if none).
    The dZ chunk is the operand of the chunk's two gradient GEMMs and never
    exists as a whole tensor, so its tensorwise scale is taken per chunk.
    Returns a dict with loss (fp64), dx, dw (bf16 bits), the scales and the
    per-chunk stages (z, g, dz, dzq, sdz, loss_rows)."""
    M, K = x.shape
    V = w.shape[0]
    C = M if chunk is None else int(chunk)
    tg = np.asarray(targets, dtype=np.int64)
    n_valid = int(((tg >= 0) & (tg < n_classes)).sum())
    xq, sx, _ = quant(x, E4M3)
    wq, sw, _ = quant(w, E4M3)
    acc = np.zeros((V, K), dtype=np.float64)
    dx = np.empty((M, K), dtype=np.uint16)
    loss_rows = np.zeros(M, dtype=np.float64)
    chunks = []
    for c0 in range(0, M, max(C, 1)):
        c1 = min(c0 + C, M)
        z = gemm_nt(xq[c0:c1], E4M3, sx, wq, E4M3, sw)
        lr, g, dz = softcap_ce_rows(z, tg[c0:c1], n_classes, softcap, n_valid)
        dzq, sdz, _ = quant(dz, E5M2)
        dx[c0:c1] = gemm_nn(dzq, E5M2, sdz, wq, E4M3, sw)
        gemm_tn_acc(dzq, E5M2, sdz, xq[c0:c1], E4M3, sx, acc)
        loss_rows[c0:c1] = lr
        chunks.append(dict(z=z, g=g, dz=dz, dzq=dzq, sdz=sdz))
    loss = float(loss_rows.sum() / n_valid) if n_valid > 0 else 0.0
    return dict(loss=loss, loss_rows=loss_rows, dx=dx, dw=double_to_bf16(acc), dw_acc=acc, xq=xq, sx=sx,
                wq=wq, sw=sw, n_valid=n_valid, chunks=chunks)


# ------------------------------------------------ gated (SwiGLU) MLP block
def silu(g: np.ndarray) -> np.ndarray:
    return g / (1.0 + np.exp(-g))


def swiglu_gate(g_bits: np.ndarray, u_bits: np.ndarray) -> np.ndarray:
    """A = RN_bf16(silu(G) U) from bf16 G and U (fp64 before the rounding)."""
    g, u = bf16_bits_to_f64(g_bits), bf16_bits_to_f64(u_bits)
    return double_to_bf16(silu(g) * u)


def swiglu_gate_bwd(g_bits, u_bits, da_bits):
    """dG = RN_bf16(dA U silu'(G)), dU = RN_bf16(dA silu(G)), with
    silu'(g) = sigmoid(g) (1 + g (1 - sigmoid(g)))."""
    g, u, da = bf16_bits_to_f64(g_bits), bf16_bits_to_f64(u_bits), bf16_bits_to_f64(da_bits)
    sg = 1.0 / (1.0 + np.exp(-g))
    return double_to_bf16(da * u * sg * (1.0 + g * (1.0 - sg))), double_to_bf16(da * g * sg)


def swiglu_fwd(x, w_gate, w_up, w_down):
    """Gated MLP Y = (silu(X Wg^T) * (X Wu^T)) Wd^T with FP8 GEMMs, the SwiGLU
    form the pages replaced by relu^2 (decomputer.nl, "Doorvoer verhogen",
    non-gated MLP bullet: three matmuls instead of two, intermediate ratio
    2.75).  X [M,d], Wg/Wu [h,d], Wd [d,h] bf16 bits; E4M3 for X, W and A."""
    xq, sx, _ = quant(x, E4M3)
    wgq, swg, _ = quant(w_gate, E4M3)
    wuq, swu, _ = quant(w_up, E4M3)
    wdq, swd, _ = quant(w_down, E4M3)
    g = gemm_nt(xq, E4M3, sx, wgq, E4M3, swg)
    u = gemm_nt(xq, E4M3, sx, wuq, E4M3, swu)
    a = swiglu_gate(g, u)
    aq, sa, amax_a = quant(a, E4M3)
    y = gemm_nt(aq, E4M3, sa, wdq, E4M3, swd)
    return dict(xq=xq, sx=sx, wgq=wgq, swg=swg, wuq=wuq, swu=swu, wdq=wdq, swd=swd, g=g, u=u, a=a, aq=aq, sa=sa,
                amax_a=amax_a, y=y)


def swiglu_bwd(dy, saved):
    """Backward of the gated block (gradients E5M2):
      Gq = Q(dY);  dWd = gemm(Gq^T, Aq);  dA = gemm(Gq, Wdq)
      dG, dU = swiglu_gate_bwd(G, U, dA);  dGq = Q(dG), dUq = Q(dU)
      dWg = gemm(dGq^T, Xq);  dWu = gemm(dUq^T, Xq)
      dX = RN_bf16(RN32(sdg swg) dGq.Wgq + RN32(sdu swu) dUq.Wuq)   (one rounding)"""
    gq, sg, _ = quant(dy, E5M2)
    dw_down = gemm_tn(gq, E5M2, sg, saved["aq"], E4M3, saved["sa"])
    da = gemm_nn(gq, E5M2, sg, saved["wdq"], E4M3, saved["swd"])
    dg, du = swiglu_gate_bwd(saved["g"], saved["u"], da)
    dgq, sdg, _ = quant(dg, E5M2)
    duq, sdu, _ = quant(du, E5M2)
    dw_gate = gemm_tn(dgq, E5M2, sdg, saved["xq"], E4M3, saved["sx"])
    dw_up = gemm_tn(duq, E5M2, sdu, saved["xq"], E4M3, saved["sx"])
    acc = np.zeros((dy.shape[0], saved["xq"].shape[1]))
    gemm_nn_acc(dgq, E5M2, sdg, saved["wgq"], E4M3, saved["swg"], acc)
    gemm_nn_acc(duq, E5M2, sdu, saved["wuq"], E4M3, saved["swu"], acc)
    return dict(gq=gq, sg=sg, dw_down=dw_down, da=da, dg=dg, du=du, dgq=dgq, sdg=sdg, duq=duq, sdu=sdu,
                dw_gate=dw_gate, dw_up=dw_up, dx=double_to_bf16(acc), dx_acc=acc)


# ------------------------------------------- Muon: Newton-Schulz iteration
# The pages train every matrix parameter with Muon (decomputer.nl, "Vroege
# experimenten" item 2: Muon for the matrix parameters, AdamW for the rest;
# its Newton-Schulz orthogonalisation costs about a quarter of a step;
# appendix: matrix optimizer Muon, lr 0.02, momentum 0.95).  The pages do
# not print the iteration; the plain reading is Muon's published quintic
# Newton-Schulz iteration (K. Jordan et al., "Muon: An optimizer for hidden
# layers in neural networks", 2024): normalise by the Frobenius norm, work
# on the wide orientation (rows <= cols), and repeat five times
#     A = X X^T,   B = b A + c A A,   X = a X + B X
# with (a, b, c) = (3.4445, -4.7750, 2.0315), which maps every singular
# value s of X to a s + b s^3 + c s^5 and so drives them towards 1 while
# keeping the singular vectors.  Precision: every tensor of the iteration is
# bf16 (the model dtype), formed with one rounding from the exact value;
# matrix products are fp64 BLAS products of the bf16 values (rounding error
# below 1e-12 of sum |products|, far under one bf16 ulp).
NS_COEFFS = (3.4445, -4.7750, 2.0315)
NS_EPS = 1e-7
NS_STEPS = 5


def bf16_gemm_nt(a_bits: np.ndarray, b_bits: np.ndarray, alpha: float = 1.0, beta: float = 0.0,
                 aux_bits: np.ndarray | None = None) -> np.ndarray:
    """One product of the iteration: RN_bf16(alpha A B^T + beta aux) from
    bf16 A [M,K], B [N,K] and aux [M,N], exact up to the fp64 product (one
    rounding at the end).  alpha and beta are taken as given (fp64)."""
    a = bf16_bits_to_f64(_c(a_bits, np.uint16))
    b = bf16_bits_to_f64(_c(b_bits, np.uint16))
    v = alpha * (a @ b.T)
    if aux_bits is not None:
        v = v + beta * bf16_bits_to_f64(_c(aux_bits, np.uint16))
    return double_to_bf16(v)


def _upper_mirrored(v: np.ndarray) -> np.ndarray:
    """X X^T and A A (A symmetric) are symmetric by definition; a BLAS
    product may still differ in the last fp64 bit between (i, j) and (j, i),
    so both take the value computed for the upper triangle."""
    return np.triu(v) + np.triu(v, 1).T


def ns_normalise(g_bits: np.ndarray, eps: float = NS_EPS):
    """X0 = RN_bf16(RN32(g / RN32(n + eps))), n = RN32(sqrt(sum g^2)) with the
    sum and the square root in fp64, the division in fp32 (IEEE).  Returns
    (X0 bits, n, the fp32 divisor)."""
    g = bf16_bits_to_f64(_c(g_bits, np.uint16))
    n = np.float32(np.sqrt(np.sum(g * g)))
    den = np.float32(n + np.float32(eps))
    x = g.astype(np.float32) / den
    return double_to_bf16(x.astype(np.float64)), float(n), float(den)


def ns_poly(s, steps: int = NS_STEPS, coeffs=NS_COEFFS):
    """The scalar map the iteration applies to every singular value."""
    a, b, c = coeffs
    s = np.asarray(s, dtype=np.float64)
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def newton_schulz(g_bits: np.ndarray, steps: int = NS_STEPS, coeffs=NS_COEFFS, eps: float = NS_EPS,
                  exact: bool = False, trace: bool = False):
    """Newton-Schulz orthogonalisation of a bf16 matrix G [rows, cols].

    exact=False: the iteration in the method's precision (bf16 tensors, each
    rounded once), returning bf16 bits of G's shape.  exact=True: the same
    steps in fp64 without any rounding (X0 = G / (||G|| + eps) in fp64),
    returning fp64 values.  trace=True also returns the list of per-step
    (A, B, X) in the wide orientation."""
    g_bits = _c(g_bits, np.uint16)
    a, b, c = coeffs
    if exact:
        g = bf16_bits_to_f64(g_bits)
        x = g / (np.sqrt(np.sum(g * g)) + eps)
        rnd = lambda v: v
    else:
        x = bf16_bits_to_f64(ns_normalise(g_bits, eps)[0])
        rnd = lambda v: bf16_bits_to_f64(double_to_bf16(v))
    tall = g_bits.shape[0] > g_bits.shape[1]
    if tall:
        x = np.ascontiguousarray(x.T)
    steps_out = []
    for _ in range(steps):
        A = rnd(_upper_mirrored(x @ x.T))
        B = rnd(b * A + c * _upper_mirrored(A @ A))
        x = rnd(a * x + B @ x)
        if trace:
            steps_out.append((A, B, x))
    if tall:
        x = np.ascontiguousarray(x.T)
    out = x if exact else double_to_bf16(x)
    if exact:
        return (out, steps_out) if trace else out
    conv = lambda v: double_to_bf16(v)
    return (out, [tuple(conv(t) for t in s) for s in steps_out]) if trace else out
