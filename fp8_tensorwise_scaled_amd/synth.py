"""Seeded synthetic inputs for the FP8 relu^2 MLP workloads.

This module only draws random numbers and rounds them to bf16; it holds none
of the method's arithmetic.  Both the HIP path (through tests and the
benchmark) and the CPU oracle consume the same bytes from here.

Recipe (one generator per tensor, seed = 1000 * workload_id + tensor_id):
  * numpy ``Generator(PCG64(seed))`` draws fp32 standard normals, multiplied
    by the standard deviation sigma (the second argument of N(0, sigma) is a
    standard deviation, as in the GPT-2 style init the decomputer.nl page
    mentions under "Wat niet werkte").
  * "outliers x100": exactly round(0.001 * n) distinct positions, drawn
    without replacement by a second generator (tensor id + 50), are scaled
    by 100 in fp32.
  * values are rounded to bf16 (round-to-nearest-even) by torch's CPU cast.
Shapes follow the little-lm appendix configuration on the decomputer.nl page
(hidden 3072, intermediate 12288, vocab 50257 padded to 50304, bf16).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


def _to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16(shape, sigma: float, seed: int, outlier_frac: float = 0.0,
                outlier_mult: float = 100.0) -> np.ndarray:
    """bf16 bit patterns of N(0, sigma) draws, optionally with outliers."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n = int(np.prod(shape))
    x = rng.standard_normal(n, dtype=np.float32) * np.float32(sigma)
    if outlier_frac > 0.0:
        k = int(round(outlier_frac * n))
        if k > 0:
            rng2 = np.random.Generator(np.random.PCG64(seed + 50))
            pos = rng2.choice(n, size=k, replace=False)
            x[pos] *= np.float32(outlier_mult)
    return _to_bf16_bits(x).reshape(shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class MLPWorkload:
    """relu^2 MLP block: X [M,d], W_up [h,d], W_down [d,h], dY [M,d]."""
    wid: int
    M: int
    d: int
    h: int
    sigma_x: float = 1.0
    sigma_up: float = 0.02
    sigma_down: float = 0.02
    sigma_dy: float = 1e-3
    dy_outliers: float = 1e-3
    name: str = ""

    def tensors(self):
        s = 1000 * self.wid
        x = normal_bf16((self.M, self.d), self.sigma_x, s + 1)
        w_up = normal_bf16((self.h, self.d), self.sigma_up, s + 2)
        w_down = normal_bf16((self.d, self.h), self.sigma_down, s + 3)
        dy = normal_bf16((self.M, self.d), self.sigma_dy, s + 4, self.dy_outliers)
        return x, w_up, w_down, dy

    @property
    def flops(self) -> int:
        """GEMM FLOPs of one fwd+bwd: six GEMMs of 2*M*d*h each."""
        return 12 * self.M * self.d * self.h


@dataclass
class SwigluWorkload:
    """Gated (SwiGLU) MLP block: X [M,d], W_gate [h,d], W_up [h,d],
    W_down [d,h], dY [M,d]."""
    wid: int
    M: int
    d: int
    h: int
    sigma_x: float = 1.0
    sigma_in: float = 0.02
    sigma_down: float = 0.02
    sigma_dy: float = 1e-3
    dy_outliers: float = 1e-3
    name: str = ""

    def tensors(self):
        s = 1000 * self.wid
        x = normal_bf16((self.M, self.d), self.sigma_x, s + 1)
        w_gate = normal_bf16((self.h, self.d), self.sigma_in, s + 2)
        w_up = normal_bf16((self.h, self.d), self.sigma_in, s + 3)
        w_down = normal_bf16((self.d, self.h), self.sigma_down, s + 4)
        dy = normal_bf16((self.M, self.d), self.sigma_dy, s + 5, self.dy_outliers)
        return x, w_gate, w_up, w_down, dy

    @property
    def flops(self) -> int:
        """GEMM FLOPs of one fwd+bwd: nine GEMMs of 2*M*d*h each."""
        return 18 * self.M * self.d * self.h


@dataclass
class LinearWorkload:
    """Single FP8 linear forward: X [M,K], W [N,K]."""
    wid: int
    M: int
    N: int
    K: int
    sigma_x: float = 1.0
    sigma_w: float = 0.02
    name: str = ""

    def tensors(self):
        s = 1000 * self.wid
        return (normal_bf16((self.M, self.K), self.sigma_x, s + 1),
                normal_bf16((self.N, self.K), self.sigma_w, s + 2))


@dataclass
class ProjectionSetWorkload:
    """All six projections of one decoder layer at M tokens (fwd+bwd)."""
    wid: int
    M: int
    projections: tuple = (("q", 3072, 3072), ("k", 3072, 1024), ("v", 3072, 1024),
                          ("o", 3072, 3072), ("up", 3072, 12288), ("down", 12288, 3072))
    name: str = ""
    sigma_in: float = 1.0
    sigma_grad: float = 1e-3
    grad_outliers: float = 1e-3

    def weight(self, i: int):
        """W_i [out, in] ~ N(0, 1/sqrt(in)); seeds 11..16 in projection order."""
        _, fin, fout = self.projections[i]
        return normal_bf16((fout, fin), 1.0 / math.sqrt(fin), 1000 * self.wid + 11 + i)

    INPUTS = ("x_attn", "x_o", "x_mlp")
    GRADS = (("dq", 3072), ("dk", 1024), ("dv", 1024), ("do", 3072), ("dy_mlp", 3072))

    def input(self, name: str):
        """Layer inputs [M, 3072] ~ N(0, 1): the attention input shared by Q,
        K and V (seed 21), the output-projection input (22) and the MLP input
        (23).  The down-projection input is the block's own relu^2 activation."""
        i = self.INPUTS.index(name)
        return normal_bf16((self.M, 3072), self.sigma_in, 1000 * self.wid + 21 + i)

    def grad(self, name: str):
        """Output gradients ~ N(0, 1e-3) with 0.1% x100 outliers: dQ, dK, dV,
        dO and the MLP block's dY (seeds 31..35)."""
        i = [g for g, _ in self.GRADS].index(name)
        return normal_bf16((self.M, self.GRADS[i][1]), self.sigma_grad, 1000 * self.wid + 31 + i,
                           self.grad_outliers)

    def mlp(self) -> "MLPWorkload":
        """The relu^2 block of the layer as an MLPWorkload-like view."""
        return _ProjMLP(self)

    def flops(self) -> int:
        return 6 * self.M * sum(fin * fout for _, fin, fout in self.projections)


class _ProjMLP:
    """X, W_up, W_down, dY of the projection set's MLP block, in the order
    MLPWorkload.tensors() returns them."""

    def __init__(self, p: ProjectionSetWorkload):
        self.p, self.M, self.d, self.h = p, p.M, 3072, 12288

    def tensors(self):
        return (self.p.input("x_mlp"), self.p.weight(4), self.p.weight(5), self.p.grad("dy_mlp"))

    @property
    def flops(self) -> int:
        return 12 * self.M * self.d * self.h


@dataclass
class LMHeadWorkload:
    """LM head linear fwd+bwd: X [M,K], W [N,K] (rows >= n_valid zero), dLogits [M,N]."""
    wid: int
    M: int
    K: int
    N: int
    n_valid: int = 50257
    name: str = ""

    def tensors(self):
        s = 1000 * self.wid
        x = normal_bf16((self.M, self.K), 1.0, s + 1)
        w = normal_bf16((self.n_valid, self.K), 0.02, s + 2)
        g = normal_bf16((self.M, self.n_valid), 1e-4, s + 4)
        if self.N > self.n_valid:
            w = np.concatenate([w, np.zeros((self.N - self.n_valid, self.K), np.uint16)], 0)
            g = np.concatenate([g, np.zeros((self.M, self.N - self.n_valid), np.uint16)], 1)
        return x, w, g

    @property
    def flops(self) -> int:
        return 6 * self.M * self.K * self.N


@dataclass
class LMHeadCEWorkload:
    """LM head fused with the softcapped cross-entropy: X [M,K] ~ N(0,1),
    W [V,K] ~ N(0, sigma_w) with rows >= n_classes zero, targets [M] int32
    uniform over the classes with a fraction set to -100 (ignored)."""
    wid: int
    M: int
    K: int
    V: int
    n_classes: int = 50257
    chunk: int = 4096
    softcap: float = 15.0
    sigma_w: float = 0.02
    ignored: float = 0.01
    name: str = ""

    def tensors(self):
        s = 1000 * self.wid
        x = normal_bf16((self.M, self.K), 1.0, s + 1)
        w = normal_bf16((self.n_classes, self.K), self.sigma_w, s + 2)
        if self.V > self.n_classes:
            w = np.concatenate([w, np.zeros((self.V - self.n_classes, self.K), np.uint16)], 0)
        rng = np.random.Generator(np.random.PCG64(s + 7))
        t = rng.integers(0, self.n_classes, self.M).astype(np.int32)
        k = int(round(self.ignored * self.M))
        if k > 0:
            t[np.random.Generator(np.random.PCG64(s + 57)).choice(self.M, size=k, replace=False)] = -100
        return x, w, t

    @property
    def flops(self) -> int:
        """GEMM FLOPs of the head: logits, grad-input, grad-weight."""
        return 6 * self.M * self.K * self.V


# The five workloads: a single linear, a small block, the 3.8B-model block,
# the full projection set and the LM head (padded / unpadded vocabulary).
LINEAR_SMALL = LinearWorkload(1, 256, 1024, 512, name="fp8 linear fwd 256x1024x512")
MLP_SMALL = MLPWorkload(2, 2048, 768, 3072, sigma_up=1 / math.sqrt(768),
                        sigma_down=1 / math.sqrt(3072), name="relu2 MLP M=2048 d=768 h=3072")
MLP_3P8B = MLPWorkload(3, 8192, 3072, 12288, name="relu2 MLP M=8192 d=3072 h=12288")
# intermediate ratio 2.75 (h = 2.75 d), the gated form's ratio on the pages
SWIGLU_SMALL = SwigluWorkload(7, 2048, 768, 2112, sigma_in=1 / math.sqrt(768), sigma_down=1 / math.sqrt(2112),
                              name="SwiGLU MLP M=2048 d=768 h=2112")
SWIGLU_3P8B = SwigluWorkload(8, 8192, 3072, 8448, name="SwiGLU MLP M=8192 d=3072 h=8448")
PROJ_SET = ProjectionSetWorkload(4, 32768, name="decoder projection set M=32768")
LM_HEAD_PADDED = LMHeadWorkload(5, 16384, 3072, 50304, name="LM head M=16384 K=3072 N=50304")
LM_HEAD_UNPADDED = LMHeadWorkload(5, 16384, 3072, 50257, name="LM head M=16384 K=3072 N=50257")
# chunks of 8192 rows: the logits buffer is half the [M, V] tensor (824 MB of
# 288 GB); 4096-row chunks measured 7% slower, 2048-row chunks 34% slower
LM_HEAD_CE = LMHeadCEWorkload(6, 16384, 3072, 50304, chunk=8192,
                              name="LM head + softcapped CE M=16384 K=3072 V=50304")
