// Device-side helpers shared by the gfx950 kernels of the FP8 relu^2 MLP.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8mlp {

constexpr int kE4M3 = 0;
constexpr int kE5M2 = 1;
constexpr float kFmaxE4M3 = 448.0f;
constexpr float kFmaxE5M2 = 57344.0f;

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef unsigned int v3u __attribute__((ext_vector_type(3)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round a finite fp32 value to bf16, nearest-even, on the bit pattern.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float fmt_max(int fmt) { return fmt == kE4M3 ? kFmaxE4M3 : kFmaxE5M2; }

// Clamp to +-fmax (keeps the sign of zero) and convert four values to packed
// FP8 codes with the hardware round-to-nearest-even conversion.
template <int FMT>
__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
  constexpr float fm = FMT == kE4M3 ? kFmaxE4M3 : kFmaxE5M2;
  a = __builtin_amdgcn_fmed3f(a, -fm, fm);
  b = __builtin_amdgcn_fmed3f(b, -fm, fm);
  c = __builtin_amdgcn_fmed3f(c, -fm, fm);
  d = __builtin_amdgcn_fmed3f(d, -fm, fm);
  int w;
  if constexpr (FMT == kE4M3) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  }
  return (uint32_t)w;
}

template <int FMT>
__device__ __forceinline__ uint32_t one_fp8(float a) {
  return pack4_fp8<FMT>(a, 0.f, 0.f, 0.f) & 0xFFu;
}

// Quotient x / s for the quantiser.  What must match RN32(x / s) exactly is
// the FP8 code it rounds to.  Fast form: a correctly rounded reciprocal
// r = RN(1/s) followed by two remainder corrections q <- q + (x - q s) r
// (Markstein's correction step, as presented in Muller et al., "Handbook of
// Floating-Point Arithmetic"), with the sign of x re-attached so that -0
// stays -0.  An exhaustive check over every bf16 amax and every bf16 x with
// |x| <= amax showed the fast form gives the same E4M3 and E5M2 codes as
// IEEE division whenever amax >= 2^-88 (the first differences appear below
// 2^-90); smaller tensors use the IEEE division.
struct Divider {
  float s, r;
  bool fast;
};

__device__ __forceinline__ Divider make_divider(float s, float amax) {
  Divider d;
  d.s = s;
  d.r = 1.0f / s;  // correctly rounded (IEEE division)
  d.fast = amax >= 0x1p-88f;
  return d;
}

__device__ __forceinline__ float div_rn(const Divider& d, float x) {
  if (d.fast) {
    float q0 = x * d.r;
    float e0 = __builtin_fmaf(-q0, d.s, x);
    float q1 = __builtin_fmaf(e0, d.r, q0);
    float e1 = __builtin_fmaf(-q1, d.s, x);
    return __builtin_copysignf(__builtin_fmaf(e1, d.r, q1), x);
  }
  return x / d.s;
}

// Wave (64 lanes) max of non-negative values given as uint bit patterns.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = __shfl_xor(v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

// Block-wide max; every thread gets the result.  `red` needs blockDim/64 slots.
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
  v = wave_max_u32(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  uint32_t m = 0;
  for (int i = 0; i < nw; ++i) m = m > red[i] ? m : red[i];
  return m;
}

// Raw buffer descriptor over [base, base + bytes): loads past the end return
// zeros (the range check of the buffer unit), offsets are 32-bit.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

}  // namespace fp8mlp
