// Gate arithmetic of the gated (SwiGLU) MLP block, used by the GEMM
// epilogues that apply the forward gate (merged gate/up projection) and its
// derivative (grad-input of the down projection), in fp32:
//   sigmoid(g) = 1 / (1 + e^-g)        (e^-g = +inf for very negative g gives 0)
//   A  = RN_bf16(silu(g) u),           silu(g) = g sigmoid(g)
//   dG = RN_bf16(dA u silu'(g)),       silu'(g) = sigmoid(g) (1 + g (1 - sigmoid(g)))
//   dU = RN_bf16(dA silu(g))
#pragma once
#include "device_common.h"

namespace fp8mlp {

__device__ __forceinline__ float sigmoid_f(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// bf16 bits of A = RN_bf16(silu(g) u)
__device__ __forceinline__ uint32_t swiglu_a_bits(float g, float u) { return f32_to_bf16_rne(g * sigmoid_f(g) * u); }

// bf16 bits of dG and dU from the bf16 values g, u and da
__device__ __forceinline__ void swiglu_bwd_bits(float g, float u, float da, uint32_t& dg, uint32_t& du) {
  const float s = sigmoid_f(g);
  dg = f32_to_bf16_rne(da * u * (s * (1.0f + g * (1.0f - s))));
  du = f32_to_bf16_rne(da * (g * s));
}

}  // namespace fp8mlp
