"""Python binding of the FP8 relu^2 MLP library (same names as the C ABI).

Marshalling only: torch tensors provide device memory and the current HIP
stream; every step of the computation runs in the library's kernels.  bf16
tensors are torch.bfloat16, FP8 codes torch.uint8, scales float32 device
scalars.  Outputs that are not given are allocated with torch.empty.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _native
from ._native import ACCUM_EXACT, ACCUM_FAST, E4M3, E5M2

FMAX = {E4M3: 448.0, E5M2: 57344.0}


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on the GPU (no CPU path)")


def _out(t, shape, dtype, device, name: str, dense: bool = False) -> torch.Tensor:
    """A caller-supplied output (checked: device, dtype, shape, and a layout
    the library can address) or a new empty one."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if t.device != torch.device(device) or t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a {dtype} tensor of shape {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")
    if dense and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not dense and t.dim() == 2 and t.numel() and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    return t


def _ws(t: torch.Tensor) -> torch.Tensor:
    if t.dtype != torch.uint8 or not t.is_contiguous() or not t.is_cuda:
        raise ValueError("workspace must be a contiguous uint8 GPU tensor")
    return t


def _ld(t: torch.Tensor) -> int:
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    if t.numel() == 0:  # empty: strides carry no layout
        return t.shape[1]
    if t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return t.stride(0)


def fp8_amax_quant(x: torch.Tensor, fmt: int = E4M3, *, q: torch.Tensor | None = None,
                   qt: torch.Tensor | None = None, want_q: bool = True, want_qt: bool = False,
                   scale: torch.Tensor | None = None, amax: torch.Tensor | None = None,
                   ws: torch.Tensor | None = None):
    """Dynamic tensorwise quantisation of a bf16 matrix.

    Returns (q, qt, scale, amax): codes [rows, cols] (or None), transposed
    codes [cols, rows] (or None), scale and amax as 1-element float32 tensors.
    """
    _check_dev(x)
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    rows, cols = x.shape
    dev = x.device
    if q is not None or want_q:
        q = _out(q, (rows, cols), torch.uint8, dev, "q")
    if qt is not None or want_qt:
        qt = _out(qt, (cols, rows), torch.uint8, dev, "qt")
    scale = _out(scale, (1,), torch.float32, dev, "scale", dense=True)
    amax = _out(amax, (1,), torch.float32, dev, "amax", dense=True)
    L = _native.lib()
    need = L.fp8_amax_quant_workspace_bytes(rows, cols)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev) if ws is None else _ws(ws)
    _native.call("fp8_amax_quant", _p(x), rows, cols, _ld(x), fmt, _p(q), 0 if q is None else _ld(q),
                 _p(qt), 0 if qt is None else _ld(qt), _p(scale), _p(amax), _p(ws), ws.numel(), _stream())
    return q, qt, scale, amax


def fp8_rmsnorm_quant(x: torch.Tensor, gamma: torch.Tensor | None = None, eps: float = 1e-6, fmt: int = E4M3, *,
                      q=None, qt=None, want_q: bool = True, want_qt: bool = False, scale=None, amax=None,
                      rstd=None, ws=None):
    """RMSNorm of the rows of x fused with the tensorwise quantisation of its
    output.  Returns (q, qt, scale, amax, rstd)."""
    _check_dev(x, gamma)
    if x.dtype != torch.bfloat16 or (gamma is not None and (gamma.dtype != torch.bfloat16 or not gamma.is_contiguous())):
        raise TypeError("x and gamma must be bfloat16 (gamma contiguous)")
    rows, cols = x.shape
    dev = x.device
    if gamma is not None and tuple(gamma.shape) not in ((cols,), (1, cols)):
        raise ValueError("gamma must hold one weight per column")
    if q is not None or want_q:
        q = _out(q, (rows, cols), torch.uint8, dev, "q")
    if qt is not None or want_qt:
        qt = _out(qt, (cols, rows), torch.uint8, dev, "qt")
    scale = _out(scale, (1,), torch.float32, dev, "scale", dense=True)
    amax = _out(amax, (1,), torch.float32, dev, "amax", dense=True)
    rstd = _out(rstd, (rows,), torch.float32, dev, "rstd", dense=True)
    if ws is None:
        ws = torch.empty(max(_native.lib().fp8_rmsnorm_quant_workspace_bytes(rows, cols), 16), dtype=torch.uint8,
                         device=dev)
    _ws(ws)
    _native.call("fp8_rmsnorm_quant", _p(x), _p(gamma), float(eps), rows, cols, _ld(x), fmt, _p(q),
                 0 if q is None else _ld(q), _p(qt), 0 if qt is None else _ld(qt), _p(scale), _p(amax), _p(rstd),
                 _p(ws), ws.numel(), _stream())
    return q, qt, scale, amax, rstd


def _gemm(name, a, fa, sa, b, fb, sb, M, N, K, out, out_shape, accum):
    _check_dev(a, b, sa, sb)
    out = _out(out, out_shape, torch.bfloat16, a.device, "out")
    _native.call(name, _p(a), _ld(a), fa, _p(sa), _p(b), _ld(b), fb, _p(sb), M, N, K, _p(out), _ld(out),
                 int(accum), _stream())
    return out


def fp8_linear_fwd(xq, sx, wq, sw, fx: int = E4M3, fw: int = E4M3, out=None, *, accum: int = ACCUM_FAST):
    """Y[M,N] = RN_bf16(RN32(sx*sw) * Xq[M,K] . Wq[N,K]^T)  (NT)."""
    M, K = xq.shape
    N = wq.shape[0]
    return _gemm("fp8_linear_fwd", xq, fx, sx, wq, fw, sw, M, N, K, out, (M, N), accum)


def _codes16(rows: int, cols: int, device) -> torch.Tensor:
    """[rows, cols] uint8 codes whose leading dimension is a multiple of 16
    (what the GEMMs read)."""
    ld = max(16, -(-cols // 16) * 16)
    return torch.empty((rows, ld), dtype=torch.uint8, device=device)[:, :cols]


def fp8_linear_fwd_bf16(x, w, *, xq=None, wq=None, scales=None, out=None, ws=None, accum: int = ACCUM_FAST):
    """One FP8 linear forward from bf16 X [M,K] and W [N,K]: both quantised
    to E4M3 with their own tensorwise scales (one amax launch and one cast
    launch for the two), then Y = RN_bf16(RN32(sx*sw) Xq . Wq^T).  Returns
    (y, xq, wq, scales) with scales = [sx, sw] (float32, on the device)."""
    _check_dev(x, w)
    if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise TypeError("x and w must be bfloat16")
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("x and w must have the same number of columns")
    dev = x.device
    xq = _codes16(M, K, dev) if xq is None else _out(xq, (M, K), torch.uint8, dev, "xq")
    wq = _codes16(N, K, dev) if wq is None else _out(wq, (N, K), torch.uint8, dev, "wq")
    scales = _out(scales, (2,), torch.float32, dev, "scales", dense=True)
    out = _out(out, (M, N), torch.bfloat16, dev, "out")
    if ws is None:
        ws = torch.empty(max(_native.lib().fp8_linear_fwd_bf16_workspace_bytes(M, N, K), 16), dtype=torch.uint8,
                         device=dev)
    _ws(ws)
    _native.call("fp8_linear_fwd_bf16", _p(x), _ld(x), _p(w), _ld(w), M, N, K, _p(xq), _ld(xq), _p(wq), _ld(wq),
                 _p(scales), _p(out), _ld(out), _p(ws), ws.numel(), int(accum), _stream())
    return out, xq, wq, scales


def fp8_linear_dgrad(dyq, sdy, wq, sw, fdy: int = E5M2, fw: int = E4M3, out=None, *, accum: int = ACCUM_FAST):
    """dX[M,K] = RN_bf16(RN32(sdy*sw) * dYq[M,N] . Wq[N,K])  (NN; the forward's weight codes)."""
    M, N = dyq.shape
    K = wq.shape[1]
    if wq.shape[0] != N:
        raise ValueError("shapes: dyq [M, N], wq [N, K]")
    return _gemm("fp8_linear_dgrad", dyq, fdy, sdy, wq, fw, sw, M, N, K, out, (M, K), accum)


def fp8_linear_wgrad(dyq, sdy, xq, sx, fdy: int = E5M2, fx: int = E4M3, out=None, *, accum: int = ACCUM_FAST):
    """dW[N,K] = RN_bf16(RN32(sdy*sx) * dYq[M,N]^T . Xq[M,K])  (TN; the forward's input codes)."""
    M, N = dyq.shape
    K = xq.shape[1]
    if xq.shape[0] != M:
        raise ValueError("shapes: dyq [M, N], xq [M, K]")
    return _gemm("fp8_linear_wgrad", dyq, fdy, sdy, xq, fx, sx, M, N, K, out, (N, K), accum)


def fp8_gated_linear_fwd(xq, sx, wgq, sg, wuq, su, *, g=None, u=None, a=None, accum: int = ACCUM_FAST):
    """The gated block's gate and up projections in one FP8 GEMM (E4M3 codes):
    G = RN_bf16(RN32(sx*sg) Xq Wgq^T), U = RN_bf16(RN32(sx*su) Xq Wuq^T),
    A = RN_bf16(silu(G) U).  Returns (g, u, a), each [M, N] bf16."""
    _check_dev(xq, sx, wgq, sg, wuq, su)
    M, K = xq.shape
    N = wgq.shape[0]
    if tuple(wuq.shape) != (N, K) or wgq.shape[1] != K:
        raise ValueError("shapes: xq [M, K], wgq and wuq [N, K]")
    if _ld(wuq) != _ld(wgq):
        raise ValueError("wgq and wuq must share a leading dimension")
    bf = torch.bfloat16
    g = _out(g, (M, N), bf, xq.device, "g")
    u = _out(u, (M, N), bf, xq.device, "u")
    a = _out(a, (M, N), bf, xq.device, "a")
    if not (_ld(g) == _ld(u) == _ld(a)):
        raise ValueError("g, u and a must share a leading dimension")
    _native.call("fp8_gated_linear_fwd", _p(xq), _ld(xq), _p(sx), _p(wgq), _p(sg), _p(wuq), _p(su), _ld(wgq),
                 M, N, K, _p(g), _p(u), _p(a), _ld(g), int(accum), _stream())
    return g, u, a


@dataclass
class Relu2MlpSaved:
    """Forward quantities the backward pass reads (device tensors): the
    row-major codes of X, W_up, W_down and A, H and the four scales."""
    xq: torch.Tensor
    uq: torch.Tensor
    dq: torch.Tensor
    aq: torch.Tensor
    h: torch.Tensor
    scales: torch.Tensor  # sx, su, sd, sa
    M: int
    d: int
    hid: int

    @staticmethod
    def empty(M: int, d: int, h: int, device) -> "Relu2MlpSaved":
        u8 = dict(dtype=torch.uint8, device=device)
        return Relu2MlpSaved(torch.empty((M, d), **u8), torch.empty((h, d), **u8), torch.empty((d, h), **u8),
                             torch.empty((M, h), **u8), torch.empty((M, h), dtype=torch.bfloat16, device=device),
                             torch.empty(4, dtype=torch.float32, device=device), M, d, h)

    def c_struct(self) -> _native.Relu2MlpSaved:
        M, d, h = self.M, self.d, self.hid
        for name, shape, dt in (("xq", (M, d), torch.uint8), ("uq", (h, d), torch.uint8),
                                ("dq", (d, h), torch.uint8), ("aq", (M, h), torch.uint8),
                                ("h", (M, h), torch.bfloat16), ("scales", (4,), torch.float32)):
            _out(getattr(self, name), shape, dt, self.scales.device, "saved." + name, dense=True)
        return _native.Relu2MlpSaved(self.xq.data_ptr(), self.uq.data_ptr(), self.dq.data_ptr(),
                                     self.aq.data_ptr(), self.h.data_ptr(), self.scales.data_ptr())


def relu2_mlp_fwd_workspace(M: int, d: int, h: int, device) -> torch.Tensor:
    n = _native.lib().relu2_mlp_fwd_workspace_bytes(M, d, h)
    if n == 0:
        raise ValueError(f"unsupported MLP shape M={M} d={d} h={h}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def relu2_mlp_bwd_workspace(M: int, d: int, h: int, device) -> torch.Tensor:
    n = _native.lib().relu2_mlp_bwd_workspace_bytes(M, d, h)
    if n == 0:
        raise ValueError(f"unsupported MLP shape M={M} d={d} h={h}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def workspace_layout(kind: str, M: int, d: int, h: int):
    n = 4 if kind == "fwd" else 6
    offs = (ctypes.c_size_t * n)()
    _native.call(f"relu2_mlp_{kind}_workspace_layout", M, d, h, offs, n)
    return list(offs)


def relu2_mlp_fwd(x, w_up, w_down, *, y=None, saved: Relu2MlpSaved | None = None, ws=None,
                  accum: int = ACCUM_FAST):
    """Y = relu(X W_up^T)^2 W_down^T with FP8 GEMMs.  Returns (y, saved)."""
    _check_dev(x, w_up, w_down)
    M, d = x.shape
    h = w_up.shape[0]
    if w_up.shape != (h, d) or w_down.shape != (d, h):
        raise ValueError("shapes: x [M,d], w_up [h,d], w_down [d,h]")
    for t in (x, w_up, w_down):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("x, w_up, w_down must be contiguous bfloat16")
    y = _out(y, (M, d), torch.bfloat16, x.device, "y", dense=True)
    if saved is None:
        saved = Relu2MlpSaved.empty(M, d, h, x.device)
    if (saved.M, saved.d, saved.hid) != (M, d, h):
        raise ValueError("saved was made for another shape")
    ws = relu2_mlp_fwd_workspace(M, d, h, x.device) if ws is None else _ws(ws)
    cs = saved.c_struct()
    _native.call("relu2_mlp_fwd", _p(x), _p(w_up), _p(w_down), M, d, h, _p(y), ctypes.byref(cs), _p(ws),
                 ws.numel(), int(accum), _stream())
    return y, saved


def relu2_mlp_bwd(dy, saved: Relu2MlpSaved, *, dx=None, dw_up=None, dw_down=None, bwd_scales=None, ws=None,
                  accum: int = ACCUM_FAST):
    """Backward of the block.  Returns (dx, dw_up, dw_down, bwd_scales[sg, sh])."""
    _check_dev(dy)
    M, d, h = saved.M, saved.d, saved.hid
    dev = dy.device
    if dy.shape != (M, d) or dy.dtype != torch.bfloat16 or not dy.is_contiguous():
        raise ValueError("dy must be a contiguous bfloat16 [M, d] tensor")
    bf = torch.bfloat16
    dx = _out(dx, (M, d), bf, dev, "dx", dense=True)
    dw_up = _out(dw_up, (h, d), bf, dev, "dw_up", dense=True)
    dw_down = _out(dw_down, (d, h), bf, dev, "dw_down", dense=True)
    bwd_scales = _out(bwd_scales, (2,), torch.float32, dev, "bwd_scales", dense=True)
    ws = relu2_mlp_bwd_workspace(M, d, h, dev) if ws is None else _ws(ws)
    cs = saved.c_struct()
    _native.call("relu2_mlp_bwd", _p(dy), ctypes.byref(cs), M, d, h, _p(dx), _p(dw_up), _p(dw_down),
                 _p(bwd_scales), _p(ws), ws.numel(), int(accum), _stream())
    return dx, dw_up, dw_down, bwd_scales


@dataclass
class SwigluMlpSaved:
    """Forward quantities the gated block's backward pass reads: the
    row-major codes of X, W_gate, W_up, W_down and A, G, U and five scales."""
    xq: torch.Tensor
    wgq: torch.Tensor
    wuq: torch.Tensor
    wdq: torch.Tensor
    aq: torch.Tensor
    g: torch.Tensor
    u: torch.Tensor
    scales: torch.Tensor  # sx, s_gate, s_up, s_down, sa
    M: int
    d: int
    hid: int

    @staticmethod
    def empty(M: int, d: int, h: int, device) -> "SwigluMlpSaved":
        u8 = dict(dtype=torch.uint8, device=device)
        bf = dict(dtype=torch.bfloat16, device=device)
        return SwigluMlpSaved(torch.empty((M, d), **u8), torch.empty((h, d), **u8), torch.empty((h, d), **u8),
                              torch.empty((d, h), **u8), torch.empty((M, h), **u8), torch.empty((M, h), **bf),
                              torch.empty((M, h), **bf), torch.empty(5, dtype=torch.float32, device=device),
                              M, d, h)

    def c_struct(self) -> _native.SwigluMlpSaved:
        M, d, h = self.M, self.d, self.hid
        u8, bf = torch.uint8, torch.bfloat16
        for name, shape, dt in (("xq", (M, d), u8), ("wgq", (h, d), u8), ("wuq", (h, d), u8),
                                ("wdq", (d, h), u8), ("aq", (M, h), u8), ("g", (M, h), bf), ("u", (M, h), bf),
                                ("scales", (5,), torch.float32)):
            _out(getattr(self, name), shape, dt, self.scales.device, "saved." + name, dense=True)
        return _native.SwigluMlpSaved(*(t.data_ptr() for t in (self.xq, self.wgq, self.wuq, self.wdq,
                                                               self.aq, self.g, self.u, self.scales)))


def swiglu_mlp_workspace(kind: str, M: int, d: int, h: int, device) -> torch.Tensor:
    n = getattr(_native.lib(), f"swiglu_mlp_{kind}_workspace_bytes")(M, d, h)
    if n == 0:
        raise ValueError(f"unsupported MLP shape M={M} d={d} h={h}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def swiglu_workspace_layout(kind: str, M: int, d: int, h: int):
    n = 6 if kind == "fwd" else 10
    offs = (ctypes.c_size_t * n)()
    _native.call(f"swiglu_mlp_{kind}_workspace_layout", M, d, h, offs, n)
    return list(offs)


def swiglu_mlp_fwd(x, w_gate, w_up, w_down, *, y=None, saved: SwigluMlpSaved | None = None, ws=None,
                   accum: int = ACCUM_FAST):
    """Y = (silu(X W_gate^T) * X W_up^T) W_down^T with FP8 GEMMs.  Returns (y, saved)."""
    _check_dev(x, w_gate, w_up, w_down)
    M, d = x.shape
    h = w_gate.shape[0]
    if w_gate.shape != (h, d) or w_up.shape != (h, d) or w_down.shape != (d, h):
        raise ValueError("shapes: x [M,d], w_gate [h,d], w_up [h,d], w_down [d,h]")
    for t in (x, w_gate, w_up, w_down):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("x, w_gate, w_up, w_down must be contiguous bfloat16")
    y = _out(y, (M, d), torch.bfloat16, x.device, "y", dense=True)
    if saved is None:
        saved = SwigluMlpSaved.empty(M, d, h, x.device)
    if (saved.M, saved.d, saved.hid) != (M, d, h):
        raise ValueError("saved was made for another shape")
    ws = swiglu_mlp_workspace("fwd", M, d, h, x.device) if ws is None else _ws(ws)
    cs = saved.c_struct()
    _native.call("swiglu_mlp_fwd", _p(x), _p(w_gate), _p(w_up), _p(w_down), M, d, h, _p(y), ctypes.byref(cs),
                 _p(ws), ws.numel(), int(accum), _stream())
    return y, saved


def swiglu_mlp_bwd(dy, saved: SwigluMlpSaved, *, dx=None, dw_gate=None, dw_up=None, dw_down=None,
                   bwd_scales=None, ws=None, accum: int = ACCUM_FAST):
    """Backward of the gated block.  Returns (dx, dw_gate, dw_up, dw_down,
    bwd_scales[s_dY, s_dG, s_dU])."""
    _check_dev(dy)
    M, d, h = saved.M, saved.d, saved.hid
    dev = dy.device
    if dy.shape != (M, d) or dy.dtype != torch.bfloat16 or not dy.is_contiguous():
        raise ValueError("dy must be a contiguous bfloat16 [M, d] tensor")
    bf = torch.bfloat16
    dx = _out(dx, (M, d), bf, dev, "dx", dense=True)
    dw_gate = _out(dw_gate, (h, d), bf, dev, "dw_gate", dense=True)
    dw_up = _out(dw_up, (h, d), bf, dev, "dw_up", dense=True)
    dw_down = _out(dw_down, (d, h), bf, dev, "dw_down", dense=True)
    bwd_scales = _out(bwd_scales, (3,), torch.float32, dev, "bwd_scales", dense=True)
    ws = swiglu_mlp_workspace("bwd", M, d, h, dev) if ws is None else _ws(ws)
    cs = saved.c_struct()
    _native.call("swiglu_mlp_bwd", _p(dy), ctypes.byref(cs), M, d, h, _p(dx), _p(dw_gate), _p(dw_up),
                 _p(dw_down), _p(bwd_scales), _p(ws), ws.numel(), int(accum), _stream())
    return dx, dw_gate, dw_up, dw_down, bwd_scales


def bf16_gemm_nt(a, b, alpha: float = 1.0, beta: float = 0.0, aux=None, *, out=None, out_t=None):
    """out = RN_bf16(alpha a b^T + beta aux) on the bf16 matrix cores
    (a [M,K], b [N,K], aux [M,N] or None); out_t, if given, receives out^T."""
    _check_dev(a, b)
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("shapes: a [M,K], b [N,K]")
    for t in (a, b) + ((aux,) if aux is not None else ()):
        if t.dtype != torch.bfloat16 or t.stride(-1) != 1:
            raise ValueError("a, b and aux must be bfloat16 with unit column stride")
    if aux is not None and tuple(aux.shape) != (M, N):
        raise ValueError("aux must be [M, N]")
    out = _out(out, (M, N), torch.bfloat16, a.device, "out")
    if out_t is not None:
        _out(out_t, (N, M), torch.bfloat16, a.device, "out_t")
    _native.call("bf16_gemm_nt", _p(a), _ld(a), _p(b), _ld(b), M, N, K, float(alpha), float(beta),
                 None if aux is None else _p(aux), 0 if aux is None else _ld(aux), _p(out), _ld(out),
                 None if out_t is None else _p(out_t), 0 if out_t is None else _ld(out_t), _stream())
    return out


def bf16_gemm_sym(a, alpha: float = 1.0, beta: float = 0.0, aux=None, *, out=None, ws=None):
    """Symmetric out = RN_bf16(alpha a a^T + beta aux) (aux symmetric or None),
    upper triangle multiplied and mirrored."""
    _check_dev(a)
    M, K = a.shape
    for t in (a,) + ((aux,) if aux is not None else ()):
        if t.dtype != torch.bfloat16 or t.stride(-1) != 1:
            raise ValueError("a and aux must be bfloat16 with unit column stride")
    if aux is not None and tuple(aux.shape) != (M, M):
        raise ValueError("aux must be [M, M]")
    out = _out(out, (M, M), torch.bfloat16, a.device, "out")
    if ws is None:
        n = _native.lib().bf16_gemm_sym_workspace_bytes(M, K)
        if n == 0:
            raise ValueError(f"unsupported symmetric product shape {M}x{K}")
        ws = torch.empty(n, dtype=torch.uint8, device=a.device)
    _ws(ws)
    _native.call("bf16_gemm_sym", _p(a), _ld(a), M, K, float(alpha), float(beta),
                 None if aux is None else _p(aux), 0 if aux is None else _ld(aux), _p(out), _ld(out), _p(ws),
                 ws.numel(), _stream())
    return out


def muon_ns_workspace(rows: int, cols: int, device) -> torch.Tensor:
    n = _native.lib().muon_ns_workspace_bytes(rows, cols)
    if n == 0:
        raise ValueError(f"unsupported Newton-Schulz shape {rows}x{cols}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def muon_newton_schulz(g, steps: int = 5, coeffs=None, eps: float = 1e-7, *, out=None, norm=None, ws=None):
    """Muon's Newton-Schulz orthogonalisation of a dense bf16 matrix.
    Returns (out [rows, cols] bf16, norm [2] fp32: ||G||_F and the divisor)."""
    _check_dev(g)
    if g.dtype != torch.bfloat16 or g.dim() != 2 or not g.is_contiguous():
        raise ValueError("g must be a contiguous 2-D bfloat16 tensor")
    rows, cols = g.shape
    dev = g.device
    out = _out(out, (rows, cols), torch.bfloat16, dev, "out", dense=True)
    norm = _out(norm, (2,), torch.float32, dev, "norm", dense=True)
    ws = muon_ns_workspace(rows, cols, dev) if ws is None else _ws(ws)
    c = None if coeffs is None else (ctypes.c_float * 3)(*coeffs)
    _native.call("muon_newton_schulz", _p(g), rows, cols, int(steps), c, float(eps), _p(out), _p(norm), _p(ws),
                 ws.numel(), _stream())
    return out, norm


def fp8_lm_head_ce_workspace(M: int, K: int, V: int, chunk: int, device) -> torch.Tensor:
    n = _native.lib().fp8_lm_head_ce_workspace_bytes(M, K, V, chunk)
    if n == 0:
        raise ValueError(f"unsupported LM-head shape M={M} K={K} V={V} chunk={chunk}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def lm_head_ce_layout(M: int, K: int, V: int, chunk: int):
    offs = (ctypes.c_size_t * 11)()
    _native.call("fp8_lm_head_ce_workspace_layout", M, K, V, chunk, offs, 11)
    return list(offs)


def fp8_lm_head_ce(x, w, targets, n_classes: int, softcap: float = 15.0, chunk: int = 2048, *, loss=None,
                   dx=None, dw=None, scales=None, ws=None, accum: int = ACCUM_FAST):
    """FP8 LM head fused with the softcapped cross-entropy, chunked over rows.

    x [M, K] bf16, w [V, K] bf16, targets [M] int32 (ids outside
    [0, n_classes) are ignored).  Returns (loss [1] fp32, dx [M, K] bf16,
    dw [V, K] bf16, scales [2 + ceil(M/chunk)] fp32: sx, sw, per-chunk dZ)."""
    _check_dev(x, w, targets)
    M, K = x.shape
    V = w.shape[0]
    if w.shape[1] != K or targets.shape != (M,) or targets.dtype != torch.int32:
        raise ValueError("shapes: x [M, K], w [V, K], targets [M] int32")
    for t in (x, w):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("x and w must be contiguous bfloat16")
    dev = x.device
    nchunks = (M + chunk - 1) // chunk if M > 0 else 0
    loss = _out(loss, (1,), torch.float32, dev, "loss", dense=True)
    dx = _out(dx, (M, K), torch.bfloat16, dev, "dx", dense=True)
    dw = _out(dw, (V, K), torch.bfloat16, dev, "dw", dense=True)
    scales = _out(scales, (2 + nchunks,), torch.float32, dev, "scales", dense=True)
    ws = fp8_lm_head_ce_workspace(M, K, V, chunk, dev) if ws is None else _ws(ws)
    if not targets.is_contiguous():
        raise ValueError("targets must be contiguous")
    _native.call("fp8_lm_head_ce", _p(x), _p(w), _p(targets), M, K, V, n_classes, float(softcap),
                 chunk, _p(loss), _p(dx), _p(dw), _p(scales), _p(ws), ws.numel(), int(accum), _stream())
    return loss, dx, dw, scales
