// Elementwise backward kernel of the gated (SwiGLU) MLP block on gfx950.
//
// The pages replaced this block by the non-gated relu^2 MLP (decomputer.nl,
// "Het trainen van een 3.8B LLM tot 0.384 CORE voor $998", "Doorvoer
// verhogen", non-gated MLP bullet: two matmuls instead of three, and the
// SwiGLU intermediate ratio of 2.75 replaced by 4x); the gated form runs here
// through the same FP8 linears so the two can be compared on MI355X.
//   forward:   A  = RN_bf16(silu(G) U),            silu(g) = g sigmoid(g)
//              (applied in the epilogue of the merged G/U GEMM, gemm.hip)
//   backward:  dG = RN_bf16(dA U silu'(G)),        silu'(g) = sigmoid(g) (1 + g (1 - sigmoid(g)))
//              dU = RN_bf16(dA silu(G))
// in fp32, with each output's per-block max |.| (bf16 magnitude bits) for the
// tensorwise scale of the next quantisation.  Memory-bound: 8 bf16 per lane
// per step, grid-stride over the dense [M, h] tensors.
#include "device_common.h"
#include "internal.h"
#include "swiglu_math.h"

namespace fp8mlp {

namespace {

constexpr int kGateThreads = 256;

__device__ __forceinline__ float lo16(uint32_t w) { return bf16_to_f32(w & 0xFFFFu); }
__device__ __forceinline__ float hi16(uint32_t w) { return bf16_to_f32(w >> 16); }

__global__ void __launch_bounds__(kGateThreads) swiglu_gate_bwd_kernel(const uint16_t* g, const uint16_t* u,
                                                                       const uint16_t* da, uint16_t* dg,
                                                                       uint16_t* du, int64_t n, uint32_t* pg,
                                                                       uint32_t* pu) {
  __shared__ uint32_t red[kGateThreads / 64];
  uint32_t mg = 0, mu = 0;
  const int64_t n8 = n / 8;
  for (int64_t i = (int64_t)blockIdx.x * kGateThreads + threadIdx.x; i < n8; i += (int64_t)gridDim.x * kGateThreads) {
    const v4u gv = reinterpret_cast<const v4u*>(g)[i];
    const v4u uv = reinterpret_cast<const v4u*>(u)[i];
    const v4u dv = reinterpret_cast<const v4u*>(da)[i];
    v4u og, ou;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t wg = 0, wu = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float gg = h ? hi16(gv[k]) : lo16(gv[k]);
        const float uu = h ? hi16(uv[k]) : lo16(uv[k]);
        const float dd = h ? hi16(dv[k]) : lo16(dv[k]);
        const float s = sigmoid_f(gg);
        const uint32_t bg = f32_to_bf16_rne(dd * uu * (s * (1.0f + gg * (1.0f - s))));
        const uint32_t bu = f32_to_bf16_rne(dd * (gg * s));
        wg |= bg << (16 * h);
        wu |= bu << (16 * h);
        mg = mg > (bg & 0x7FFFu) ? mg : (bg & 0x7FFFu);
        mu = mu > (bu & 0x7FFFu) ? mu : (bu & 0x7FFFu);
      }
      og[k] = wg;
      ou[k] = wu;
    }
    reinterpret_cast<v4u*>(dg)[i] = og;
    reinterpret_cast<v4u*>(du)[i] = ou;
  }
  mg = block_max_u32(mg, red);
  mu = block_max_u32(mu, red);
  if (threadIdx.x == 0) {
    pg[blockIdx.x] = mg;
    pu[blockIdx.x] = mu;
  }
}

}  // namespace

int swiglu_parts_for(int64_t n) {
  const int64_t b = (n / 8 + kGateThreads * 4 - 1) / (kGateThreads * 4);  // ~4 steps per thread
  return (int)(b < 1 ? 1 : (b > 1024 ? 1024 : b));
}

hipError_t launch_swiglu_gate_bwd(const uint16_t* g, const uint16_t* u, const uint16_t* da, uint16_t* dg,
                                  uint16_t* du, int64_t n, uint32_t* pg, uint32_t* pu, hipStream_t st) {
  hipLaunchKernelGGL(swiglu_gate_bwd_kernel, dim3(swiglu_parts_for(n)), dim3(kGateThreads), 0, st, g, u, da, dg,
                     du, n, pg, pu);
  return hipGetLastError();
}

}  // namespace fp8mlp
