// Gate arithmetic of the gated (SwiGLU) MLP block, shared by the elementwise
// backward kernel and the GEMM epilogue that applies the forward gate, so
// that every path rounds the same fp32 expressions:
//   sigmoid(g) = 1 / (1 + e^-g)        (e^-g = +inf for very negative g gives 0)
//   A = RN_bf16(silu(g) u),            silu(g) = g sigmoid(g)
#pragma once
#include "device_common.h"

namespace fp8mlp {

__device__ __forceinline__ float sigmoid_f(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// bf16 bits of A = RN_bf16(silu(g) u)
__device__ __forceinline__ uint32_t swiglu_a_bits(float g, float u) { return f32_to_bf16_rne(g * sigmoid_f(g) * u); }

}  // namespace fp8mlp
