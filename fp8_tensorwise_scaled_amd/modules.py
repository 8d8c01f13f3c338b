"""PyTorch autograd modules over the C ABI: an FP8 linear layer and the
relu^2 MLP block, with dynamic tensorwise scaling on all three GEMMs of
every linear (decomputer.nl, "Doorvoer verhogen", first bullet).

Argument marshalling only: every quantisation and GEMM runs in
libfp8mlp.so through ``api``; there is no CPU path.  Inputs are bf16 with
any leading shape (flattened to rows); weights are bf16 [out, in].
"""
from __future__ import annotations

import math

import torch

from . import api


def _rows(x: torch.Tensor) -> torch.Tensor:
    return x.reshape(-1, x.shape[-1]).contiguous()


class _Fp8LinearFn(torch.autograd.Function):
    """y = x W^T with E4M3 x and W; backward with E5M2 dy:
    dx = dy W (NN) and dW = dy^T x (TN), both on the forward's row-major codes."""

    @staticmethod
    def forward(ctx, x, w):
        x2 = _rows(x)
        xq, _, sx, _ = api.fp8_amax_quant(x2, api.E4M3)
        wq, _, sw, _ = api.fp8_amax_quant(w.contiguous(), api.E4M3)
        y = api.fp8_linear_fwd(xq, sx, wq, sw)
        ctx.save_for_backward(xq, sx, wq, sw)
        ctx.x_shape = x.shape
        return y.reshape(*x.shape[:-1], w.shape[0])

    @staticmethod
    def backward(ctx, dy):
        xq, sx, wq, sw = ctx.saved_tensors
        need_dx, need_dw = ctx.needs_input_grad
        dy2 = _rows(dy.to(torch.bfloat16))
        gq, _, sg, _ = api.fp8_amax_quant(dy2, api.E5M2)
        dx = api.fp8_linear_dgrad(gq, sg, wq, sw).reshape(ctx.x_shape) if need_dx else None
        dw = api.fp8_linear_wgrad(gq, sg, xq, sx) if need_dw else None
        return dx, dw


class _Relu2MlpFn(torch.autograd.Function):
    """Y = relu(X W_up^T)^2 W_down^T through relu2_mlp_fwd / relu2_mlp_bwd."""

    @staticmethod
    def forward(ctx, x, w_up, w_down):
        x2 = _rows(x)
        y, saved = api.relu2_mlp_fwd(x2, w_up.contiguous(), w_down.contiguous())
        ctx.saved = saved
        ctx.x_shape = x.shape
        return y.reshape(x.shape)

    @staticmethod
    def backward(ctx, dy):
        if ctx.saved is None:
            raise RuntimeError("relu2_mlp: the saved FP8 codes are released by the first backward; "
                               "a second backward through the same forward is not supported")
        dx, dw_up, dw_down, _ = api.relu2_mlp_bwd(_rows(dy.to(torch.bfloat16)), ctx.saved)
        ctx.saved = None
        return dx.reshape(ctx.x_shape), dw_up, dw_down


def fp8_linear(x: torch.Tensor, weight: torch.Tensor) -> torch.Tensor:
    """Differentiable FP8 linear, y = x W^T (no bias)."""
    return _Fp8LinearFn.apply(x, weight)


def relu2_mlp(x: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor) -> torch.Tensor:
    """Differentiable non-gated relu^2 MLP block."""
    return _Relu2MlpFn.apply(x, w_up, w_down)


class FP8Linear(torch.nn.Module):
    """nn.Linear without bias whose three GEMMs run in FP8 with dynamic
    tensorwise scales.  in_features and out_features must be multiples of 16."""

    def __init__(self, in_features: int, out_features: int, device=None, std: float | None = None):
        super().__init__()
        std = 1.0 / math.sqrt(in_features) if std is None else std
        self.weight = torch.nn.Parameter(
            (std * torch.randn(out_features, in_features, device=device)).to(torch.bfloat16))

    def forward(self, x):
        return fp8_linear(x, self.weight)


class Relu2MLP(torch.nn.Module):
    """The non-gated relu^2 MLP block (hidden width h, usually 4 d), FP8 on
    all six GEMMs.  d, h and the token count must be multiples of 16."""

    def __init__(self, d: int, h: int, device=None, std_up: float | None = None, std_down: float | None = None):
        super().__init__()
        su = 1.0 / math.sqrt(d) if std_up is None else std_up
        sd = 1.0 / math.sqrt(h) if std_down is None else std_down
        self.w_up = torch.nn.Parameter((su * torch.randn(h, d, device=device)).to(torch.bfloat16))
        self.w_down = torch.nn.Parameter((sd * torch.randn(d, h, device=device)).to(torch.bfloat16))

    def forward(self, x):
        return relu2_mlp(x, self.w_up, self.w_down)
