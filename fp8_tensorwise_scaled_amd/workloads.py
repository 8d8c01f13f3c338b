"""Runners that sequence the library's C-ABI calls for the larger workloads.

Only buffer management and call order live here (torch provides the device
memory); every step runs in the library's kernels.

* `LinearSet`: one FP8 linear layer (forward, grad-input, grad-weight) with
  its own dynamic tensorwise scales - the unit the pages apply to every
  linear (decomputer.nl, "Doorvoer verhogen", first bullet).
* `ProjectionSetRunner`: the six projections of one decoder layer of the
  3.8B model (appendix configuration: hidden 3072, 24 query heads and 8
  key/value heads of 128, relu2 MLP at 12288): Q, K and V share one
  quantised input, O has its own, and the MLP runs as the fused block.
* `LMHeadRunner`: the LM head at the padded (50304, a multiple of 64) and
  the unpadded (50257) vocabulary (decomputer.nl, "Vroege experimenten"
  item 4; padded rows of W and columns of dLogits are zero).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import api
from .api import E4M3, E5M2


def _bf16(shape, device):
    return torch.empty(shape, dtype=torch.bfloat16, device=device)


def _u8(shape, device, zero=False):
    f = torch.zeros if zero else torch.empty
    return f(shape, dtype=torch.uint8, device=device)


def _f32(n, device):
    return torch.empty(n, dtype=torch.float32, device=device)


@dataclass
class QuantOut:
    """Row-major codes of a [rows, cols] tensor (q [rows, ld]) and its scale."""
    q: torch.Tensor
    scale: torch.Tensor
    amax: torch.Tensor
    ws: torch.Tensor

    @staticmethod
    def alloc(rows, cols, device, ld_multiple=1):
        """Codes with a leading dimension rounded up to ld_multiple (the
        columns past cols are never read: every GEMM masks its reduction)."""
        ld = -(-cols // ld_multiple) * ld_multiple
        ws = torch.empty(max(api._native.lib().fp8_amax_quant_workspace_bytes(rows, cols), 16),
                         dtype=torch.uint8, device=device)
        return QuantOut(_u8((rows, ld), device), _f32(1, device), _f32(1, device), ws)

    def run(self, x, fmt, cols):
        api.fp8_amax_quant(x, fmt, q=self.q[:, :cols], scale=self.scale, amax=self.amax, ws=self.ws)
        return self


class LinearSet:
    """Buffers and calls for one FP8 linear: Y = X W^T (NT), dX = dY W (NN),
    dW = dY^T X (TN), all three on the row-major codes of X, W and dY."""

    def __init__(self, M, n_in, n_out, device, x_quant: QuantOut | None = None, accum=api.ACCUM_FAST):
        self.M, self.n_in, self.n_out, self.accum = M, n_in, n_out, accum
        self.xq = x_quant or QuantOut.alloc(M, n_in, device)
        self.wq = QuantOut.alloc(n_out, n_in, device)
        self.gq = QuantOut.alloc(M, n_out, device)
        self.y = _bf16((M, n_out), device)
        self.dx = _bf16((M, n_in), device)
        self.dw = _bf16((n_out, n_in), device)

    def forward(self, x, w, quantize_x=True):
        if quantize_x:
            self.xq.run(x, E4M3, self.n_in)
        self.wq.run(w, E4M3, self.n_in)
        api.fp8_linear_fwd(self.xq.q[:, :self.n_in], self.xq.scale, self.wq.q[:, :self.n_in], self.wq.scale,
                           out=self.y, accum=self.accum)
        return self.y

    def backward(self, dy):
        self.gq.run(dy, E5M2, self.n_out)
        api.fp8_linear_dgrad(self.gq.q[:, :self.n_out], self.gq.scale, self.wq.q[:, :self.n_in], self.wq.scale,
                             out=self.dx, accum=self.accum)
        api.fp8_linear_wgrad(self.gq.q[:, :self.n_out], self.gq.scale, self.xq.q[:, :self.n_in], self.xq.scale,
                             out=self.dw, accum=self.accum)
        return self.dx, self.dw

    @property
    def flops(self):
        return 6 * self.M * self.n_in * self.n_out


class ProjectionSetRunner:
    """Q, K, V (shared input), O and the relu^2 MLP block of one decoder layer."""

    def __init__(self, M, device, d=3072, q_dim=3072, kv_dim=1024, h=12288, accum=api.ACCUM_FAST):
        self.M, self.d, self.h, self.accum = M, d, h, accum
        self.x_attn_q = QuantOut.alloc(M, d, device)
        self.q = LinearSet(M, d, q_dim, device, x_quant=self.x_attn_q, accum=accum)
        self.k = LinearSet(M, d, kv_dim, device, x_quant=self.x_attn_q, accum=accum)
        self.v = LinearSet(M, d, kv_dim, device, x_quant=self.x_attn_q, accum=accum)
        self.o = LinearSet(M, q_dim, d, device, accum=accum)
        self.saved = api.Relu2MlpSaved.empty(M, d, h, device)
        self.ws_f = api.relu2_mlp_fwd_workspace(M, d, h, device)
        self.ws_b = api.relu2_mlp_bwd_workspace(M, d, h, device)
        self.y_mlp = _bf16((M, d), device)
        self.dx_mlp = _bf16((M, d), device)
        self.dw_up = _bf16((h, d), device)
        self.dw_down = _bf16((d, h), device)
        self.bsc = _f32(2, device)

    def step(self, t):
        """t: dict of bf16 tensors x_attn, w_q, w_k, w_v, x_o, w_o, x_mlp, w_up, w_down,
        dq, dk, dv, do, dy_mlp.  One forward and backward of all six projections."""
        self.x_attn_q.run(t["x_attn"], E4M3, self.d)
        self.q.forward(None, t["w_q"], quantize_x=False)
        self.k.forward(None, t["w_k"], quantize_x=False)
        self.v.forward(None, t["w_v"], quantize_x=False)
        self.o.forward(t["x_o"], t["w_o"])
        api.relu2_mlp_fwd(t["x_mlp"], t["w_up"], t["w_down"], y=self.y_mlp, saved=self.saved, ws=self.ws_f,
                          accum=self.accum)
        self.q.backward(t["dq"])
        self.k.backward(t["dk"])
        self.v.backward(t["dv"])
        self.o.backward(t["do"])
        api.relu2_mlp_bwd(t["dy_mlp"], self.saved, dx=self.dx_mlp, dw_up=self.dw_up, dw_down=self.dw_down,
                          bwd_scales=self.bsc, ws=self.ws_b, accum=self.accum)

    @property
    def flops(self):
        return self.q.flops + self.k.flops + self.v.flops + self.o.flops + 12 * self.M * self.d * self.h


class LMHeadRunner:
    """LM head fwd+bwd for vocabulary N (padded or not).

    The unpadded vocabulary's codes of dLogits get a leading dimension
    rounded up to 128, so that every row starts on a 128-byte line as the
    padded vocabulary's rows do (the grad-input GEMM reads each row 128
    bytes per stage; rows on a 16-byte multiple only would straddle two
    lines per read); the grad-input GEMM reduces over exactly N of them,
    the kernel masking the tail."""

    def __init__(self, M, K, N, device, accum=api.ACCUM_FAST):
        self.M, self.K, self.N, self.accum = M, K, N, accum
        self.xq = QuantOut.alloc(M, K, device)
        self.wq = QuantOut.alloc(N, K, device)
        self.gq = QuantOut.alloc(M, N, device, ld_multiple=128)
        self.y = _bf16((M, N), device)
        self.dx = _bf16((M, K), device)
        self.dw = _bf16((N, K), device)

    def step(self, x, w, dlogits):
        K, N = self.K, self.N
        self.xq.run(x, E4M3, K)
        self.wq.run(w, E4M3, K)
        api.fp8_linear_fwd(self.xq.q, self.xq.scale, self.wq.q, self.wq.scale, out=self.y, accum=self.accum)
        self.gq.run(dlogits, E5M2, N)
        g = self.gq.q[:, :N]
        api.fp8_linear_dgrad(g, self.gq.scale, self.wq.q, self.wq.scale, out=self.dx, accum=self.accum)
        api.fp8_linear_wgrad(g, self.gq.scale, self.xq.q, self.xq.scale, out=self.dw, accum=self.accum)

    @property
    def flops(self):
        return 6 * self.M * self.K * self.N
