// Dynamic tensorwise quantisation on gfx950: grid-wide amax, scale, cast.
//
// Dynamic tensorwise scaling (decomputer.nl, "Het trainen van een 3.8B LLM
// tot 0.384 CORE voor $998", "Vroege experimenten" item 4): one scale per
// tensor, recomputed from the tensor itself on every call.  Here
//   amax = max |x|,  s = RN32(amax / fmax) (1 if amax == 0),
//   q = RNE_fp8(clamp(RN32(x / s), +-fmax)).
//
// Two launches per batch of tensors, no atomics and no memsets:
//   1. amax_partials: every block writes the max of |x| over its slice, taken
//      as an integer max of the bf16 magnitude bits (monotone in the value,
//      order independent, hence bit-deterministic);
//   2. cast: every block first reduces the (<= 2048) partials of its tensor,
//      derives s itself, then streams 128x128 tiles: row-major codes go
//      straight to HBM, the transposed codes go through LDS so that both
//      outputs are written in full 128-byte rows.
#include "device_common.h"
#include "internal.h"

namespace fp8mlp {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 128;         // cast tile: 128 x 128 elements
constexpr int kLdsT = kTile + 16;  // transposed-tile row stride in LDS (bytes)

__device__ __forceinline__ const QuantJob& job_of(const QuantBatch& b, int& local_blk) {
  int j = 0;
#pragma unroll
  for (int i = 1; i < kMaxJobs; ++i)
    if (i < b.njobs && (int)blockIdx.x >= b.job[i].blk_begin) j = i;
  local_blk = blockIdx.x - b.job[j].blk_begin;
  return b.job[j];
}

__device__ __forceinline__ bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

__device__ __forceinline__ uint32_t absmax8(v4u v) {
  // two bf16 per dword: clear the sign bits, take the larger half
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t w = v[i] & 0x7FFF7FFFu;
    uint32_t lo = w & 0xFFFFu, hi = w >> 16;
    uint32_t t = lo > hi ? lo : hi;
    m = m > t ? m : t;
  }
  return m;
}

__global__ void __launch_bounds__(kThreads) amax_partials_kernel(QuantBatch b) {
  __shared__ uint32_t red[kThreads / 64];
  int lb;
  const QuantJob& jb = job_of(b, lb);
  const int64_t rows = jb.rows, cols = jb.cols, ldx = jb.ldx;
  const uint16_t* x = jb.x;
  const int nb = jb.nblocks;
  uint32_t m = 0;
  const bool vec = aligned16(x) && (ldx % 8 == 0) && (cols % 8 == 0);
  if (vec && ldx == cols) {
    // dense: one flat array of rows*cols/8 16-byte chunks
    const int64_t nch = rows * cols / 8;
    const v4u* xv = reinterpret_cast<const v4u*>(x);
    int64_t i = (int64_t)lb * kThreads + threadIdx.x;
    const int64_t step = (int64_t)nb * kThreads;
    for (; i + 3 * step < nch; i += 4 * step) {
      v4u v0 = __builtin_nontemporal_load(xv + i);
      v4u v1 = __builtin_nontemporal_load(xv + i + step);
      v4u v2 = __builtin_nontemporal_load(xv + i + 2 * step);
      v4u v3 = __builtin_nontemporal_load(xv + i + 3 * step);
      uint32_t t0 = absmax8(v0), t1 = absmax8(v1), t2 = absmax8(v2), t3 = absmax8(v3);
      t0 = t0 > t1 ? t0 : t1;
      t2 = t2 > t3 ? t2 : t3;
      t0 = t0 > t2 ? t0 : t2;
      m = m > t0 ? m : t0;
    }
    for (; i < nch; i += step) {
      uint32_t t = absmax8(xv[i]);
      m = m > t ? m : t;
    }
  } else if (vec) {
    const int64_t cpr = cols / 8;
    const int64_t nch = rows * cpr;
    for (int64_t i = (int64_t)lb * kThreads + threadIdx.x; i < nch; i += (int64_t)nb * kThreads) {
      int64_t r = i / cpr, c = (i - r * cpr) * 8;
      uint32_t t = absmax8(*reinterpret_cast<const v4u*>(x + r * ldx + c));
      m = m > t ? m : t;
    }
  } else {
    const int64_t n = rows * cols;
    for (int64_t i = (int64_t)lb * kThreads + threadIdx.x; i < n; i += (int64_t)nb * kThreads) {
      int64_t r = i / cols, c = i - r * cols;
      uint32_t t = x[r * ldx + c] & 0x7FFFu;
      m = m > t ? m : t;
    }
  }
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) jb.partials[lb] = m;
}

// Value the cast quantises, from the stored bf16 bits.
template <int MODE>
__device__ __forceinline__ float cast_value(uint32_t bits) {
  float f = bf16_to_f32(bits);
  if constexpr (MODE == kModeRelu2) {
    float r = __builtin_fmaxf(f, 0.0f);
    // r*r is exact in fp32 (8-bit significand); one rounding to bf16
    __bf16 a = (__bf16)(r * r);
    f = bf16_to_f32(__builtin_bit_cast(unsigned short, a));
  }
  return f;
}

template <int FMT, int MODE>
__device__ __forceinline__ uint32_t quant4(uint32_t w0, uint32_t w1, const Divider& d) {
  float a = div_rn(d, cast_value<MODE>(w0 & 0xFFFFu));
  float b = div_rn(d, cast_value<MODE>(w0 >> 16));
  float c = div_rn(d, cast_value<MODE>(w1 & 0xFFFFu));
  float e = div_rn(d, cast_value<MODE>(w1 >> 16));
  return pack4_fp8<FMT>(a, b, c, e);
}

template <int FMT, int MODE>
__device__ void cast_tiles(const QuantJob& jb, int lb, const Divider& d, uint8_t* lds) {
  const int64_t rows = jb.rows, cols = jb.cols, ldx = jb.ldx;
  const uint16_t* x = jb.x;
  uint8_t* q = jb.q;
  uint8_t* qt = jb.qt;
  const int64_t ntr = (rows + kTile - 1) / kTile, ntc = (cols + kTile - 1) / kTile;
  const int64_t ntiles = ntr * ntc;
  const bool vec_in = aligned16(x) && (ldx % 8 == 0);
  const bool vec_q = q == nullptr || (((reinterpret_cast<uintptr_t>(q) & 7u) == 0) && (jb.ldq % 8 == 0));
  const bool vec_qt = qt == nullptr || (aligned16(qt) && (jb.ldqt % 16 == 0));
  const int tid = threadIdx.x;
  for (int64_t t = lb; t < ntiles; t += jb.nblocks) {
    const int64_t r0 = (t / ntc) * kTile, c0 = (t % ntc) * kTile;
    const bool full = r0 + kTile <= rows && c0 + kTile <= cols && vec_in && vec_q && vec_qt;
    if (full) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int id = tid + kThreads * i;
        const int row = id >> 4, c16 = id & 15;
        const v4u v = __builtin_nontemporal_load(
            reinterpret_cast<const v4u*>(x + (r0 + row) * ldx + c0 + c16 * 8));
        const uint32_t lo = quant4<FMT, MODE>(v[0], v[1], d);
        const uint32_t hi = quant4<FMT, MODE>(v[2], v[3], d);
        if (q) {
          v2u o = {lo, hi};
          *reinterpret_cast<v2u*>(q + (r0 + row) * jb.ldq + c0 + c16 * 8) = o;
        }
        if (qt) {
          uint8_t* col = lds + (c16 * 8) * kLdsT + row;
#pragma unroll
          for (int e = 0; e < 4; ++e) col[e * kLdsT] = (uint8_t)(lo >> (8 * e));
#pragma unroll
          for (int e = 0; e < 4; ++e) col[(4 + e) * kLdsT] = (uint8_t)(hi >> (8 * e));
        }
      }
      if (qt) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int id = tid + kThreads * i;
          const int col = id >> 3, ch = id & 7;
          const v4u v = *reinterpret_cast<const v4u*>(lds + col * kLdsT + ch * 16);
          *reinterpret_cast<v4u*>(qt + (c0 + col) * jb.ldqt + r0 + ch * 16) = v;
        }
        __syncthreads();
      }
    } else {
      // ragged or unaligned tile: element by element
      for (int e = tid; e < kTile * kTile; e += kThreads) {
        const int row = e >> 7, col = e & (kTile - 1);
        if (r0 + row < rows && c0 + col < cols) {
          const uint32_t bits = x[(r0 + row) * ldx + c0 + col];
          const uint32_t code = pack4_fp8<FMT>(div_rn(d, cast_value<MODE>(bits)), 0.f, 0.f, 0.f) & 0xFFu;
          if (q) q[(r0 + row) * jb.ldq + c0 + col] = (uint8_t)code;
          if (qt) lds[col * kLdsT + row] = (uint8_t)code;
        }
      }
      if (qt) {
        __syncthreads();
        for (int e = tid; e < kTile * kTile; e += kThreads) {
          const int col = e >> 7, row = e & (kTile - 1);
          if (r0 + row < rows && c0 + col < cols)
            qt[(c0 + col) * jb.ldqt + r0 + row] = lds[col * kLdsT + row];
        }
        __syncthreads();
      }
    }
  }
}

__global__ void __launch_bounds__(kThreads) cast_kernel(QuantBatch b) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kTile * kLdsT];
  __shared__ uint32_t red[kThreads / 64];
  int lb;
  const QuantJob& jb = job_of(b, lb);
  // 1. amax from the partials (integer max of non-negative bit patterns)
  uint32_t m = 0;
  for (int i = threadIdx.x; i < jb.nparts; i += kThreads) {
    uint32_t v = jb.partials[i];
    m = m > v ? m : v;
  }
  m = block_max_u32(m, red);
  float amax;
  if (jb.mode == kModeRelu2) {
    // max over the tensor of RN_bf16(relu(h)^2) = RN_bf16(relu(max h)^2)
    // (x -> x^2 and rounding are monotone on x >= 0)
    const float mh = __uint_as_float(m);
    __bf16 a = (__bf16)(mh * mh);
    amax = bf16_to_f32(__builtin_bit_cast(unsigned short, a));
  } else {
    amax = bf16_to_f32(m);
  }
  const float fm = fmt_max(jb.fmt);
  const float s = amax == 0.0f ? 1.0f : amax / fm;  // IEEE division, correctly rounded
  if (lb == 0 && threadIdx.x == 0) {
    *jb.scale = s;
    if (jb.amax_out) *jb.amax_out = amax;
  }
  const Divider d = make_divider(s, amax);
  // 2. cast
  if (jb.fmt == kE4M3) {
    if (jb.mode == kModeRelu2) cast_tiles<kE4M3, kModeRelu2>(jb, lb, d, lds);
    else cast_tiles<kE4M3, kModePlain>(jb, lb, d, lds);
  } else {
    if (jb.mode == kModeRelu2) cast_tiles<kE5M2, kModeRelu2>(jb, lb, d, lds);
    else cast_tiles<kE5M2, kModePlain>(jb, lb, d, lds);
  }
}

int cast_blocks_for(int64_t rows, int64_t cols) {
  const int64_t tiles = ((rows + kTile - 1) / kTile) * ((cols + kTile - 1) / kTile);
  return (int)(tiles < 2048 ? tiles : 2048);
}

}  // namespace

int amax_parts_for(int64_t rows, int64_t cols) {
  // ~64K elements per block, at most 1024 blocks (4 per CU)
  const int64_t n = rows * cols;
  int64_t p = (n + 65535) / 65536;
  if (p < 1) p = 1;
  if (p > 1024) p = 1024;
  return (int)p;
}

hipError_t launch_amax_partials(QuantBatch& b, hipStream_t st) {
  int total = 0;
  for (int i = 0; i < b.njobs; ++i) {
    b.job[i].blk_begin = total;
    b.job[i].nblocks = b.job[i].nparts;
    total += b.job[i].nparts;
  }
  hipLaunchKernelGGL(amax_partials_kernel, dim3(total), dim3(kThreads), 0, st, b);
  return hipGetLastError();
}

hipError_t launch_cast(QuantBatch& b, hipStream_t st) {
  int total = 0;
  for (int i = 0; i < b.njobs; ++i) {
    b.job[i].blk_begin = total;
    b.job[i].nblocks = cast_blocks_for(b.job[i].rows, b.job[i].cols);
    total += b.job[i].nblocks;
  }
  hipLaunchKernelGGL(cast_kernel, dim3(total), dim3(kThreads), 0, st, b);
  return hipGetLastError();
}

}  // namespace fp8mlp
