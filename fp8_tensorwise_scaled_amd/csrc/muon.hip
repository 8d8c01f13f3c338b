// Newton-Schulz orthogonalisation of Muon on gfx950: the elementwise and
// data-movement kernels around the bf16 GEMMs (gemm.hip, kBF16 operands).
//
// The pages train every matrix parameter with Muon and put the cost of its
// Newton-Schulz orthogonalisation at about a quarter of a step
// (decomputer.nl, "Het trainen van een 3.8B LLM tot 0.384 CORE voor $998",
// "Vroege experimenten" item 2; appendix: matrix optimizer Muon).  The
// iteration is Muon's published quintic one:
//   X0 = RN_bf16(RN32(G / RN32(RN32(||G||_F) + eps)))   (wide orientation)
//   A  = RN_bf16(X X^T);  B = RN_bf16(b A + c A A);  X = RN_bf16(a X + B X)
// Here: the Frobenius norm (fp64 sum of squares, per-block partials reduced
// in a fixed order, so every block and every run sees the same value), the
// scaling with IEEE fp32 division, and a tiled bf16 transpose.
#include "device_common.h"
#include "internal.h"

namespace fp8mlp {

namespace {

constexpr int kNsThreads = 256;
constexpr int kNsMaxParts = 1024;

__device__ __forceinline__ double block_sum_f64(double v, double* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double s = 0.0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += red[i];  // fixed order
  __syncthreads();
  return s;
}

// partials[block] = sum over the block's slice of g^2 (fp64; a bf16 square
// is exact in fp64).  n is a multiple of 8.
__global__ void __launch_bounds__(kNsThreads) ns_sumsq_kernel(const uint16_t* g, int64_t n, double* partials) {
  __shared__ double red[kNsThreads / 64];
  double s = 0.0;
  const int64_t n8 = n / 8;
  for (int64_t i = (int64_t)blockIdx.x * kNsThreads + threadIdx.x; i < n8; i += (int64_t)gridDim.x * kNsThreads) {
    const v4u v = reinterpret_cast<const v4u*>(g)[i];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const double lo = bf16_to_f32(v[k] & 0xFFFFu), hi = bf16_to_f32(v[k] >> 16);
      s += lo * lo;
      s += hi * hi;
    }
  }
  s = block_sum_f64(s, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = s;
}

// x = RN_bf16(RN32(g / den)), den = RN32(RN32(sqrt(S)) + eps), S the sum of
// the partials.  Every block reduces the partials itself, in the same order.
__global__ void __launch_bounds__(kNsThreads) ns_scale_kernel(const uint16_t* g, int64_t n, const double* partials,
                                                             int nparts, float eps, uint16_t* x, float* norm_out) {
  __shared__ double red[kNsThreads / 64];
  double s = 0.0;
  for (int i = threadIdx.x; i < nparts; i += kNsThreads) s += partials[i];
  s = block_sum_f64(s, red);
  const float nrm = (float)__dsqrt_rn(s);
  const float den = nrm + eps;
  if (blockIdx.x == 0 && threadIdx.x == 0 && norm_out) {
    norm_out[0] = nrm;
    norm_out[1] = den;
  }
  const int64_t n8 = n / 8;
  for (int64_t i = (int64_t)blockIdx.x * kNsThreads + threadIdx.x; i < n8; i += (int64_t)gridDim.x * kNsThreads) {
    const v4u v = reinterpret_cast<const v4u*>(g)[i];
    v4u o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = f32_to_bf16_rne(__fdiv_rn(bf16_to_f32(v[k] & 0xFFFFu), den));
      const uint32_t hi = f32_to_bf16_rne(__fdiv_rn(bf16_to_f32(v[k] >> 16), den));
      o[k] = lo | (hi << 16);
    }
    reinterpret_cast<v4u*>(x)[i] = o;
  }
}

// dst [cols, rows] = src [rows, cols]^T, 64 x 64 tiles through LDS; rows and
// cols are multiples of 8 (whole 16-byte chunks).
constexpr int kTile = 64;
constexpr int kPitch = kTile + 2;  // elements; odd word pitch spreads a column over the banks
__global__ void __launch_bounds__(kNsThreads) transpose_bf16_kernel(const uint16_t* src, int64_t rows, int64_t cols,
                                                                   uint16_t* dst) {
  __shared__ uint16_t tile[kTile * kPitch];
  const int64_t r0 = (int64_t)blockIdx.y * kTile, c0 = (int64_t)blockIdx.x * kTile;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int id = threadIdx.x + kNsThreads * it;
    const int r = id >> 3, ch = id & 7;
    if (r0 + r < rows && c0 + ch * 8 < cols) {
      const v4u v = *reinterpret_cast<const v4u*>(src + (r0 + r) * cols + c0 + ch * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[r * kPitch + ch * 8 + e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
    }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int id = threadIdx.x + kNsThreads * it;
    const int c = id >> 3, ch = id & 7;
    if (c0 + c < cols && r0 + ch * 8 < rows) {
      v4u o;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = (uint32_t)tile[(ch * 8 + 2 * e) * kPitch + c] | ((uint32_t)tile[(ch * 8 + 2 * e + 1) * kPitch + c] << 16);
      *reinterpret_cast<v4u*>(dst + (c0 + c) * rows + r0 + ch * 8) = o;
    }
  }
}

// C = RN_bf16(fma(alpha, S, RN32(beta aux))) with S = ((p0 + p1) + ...) the
// fp32 partial sums of the upper-triangle split-K product, over the 64 x 64
// blocks (bi <= bj) of the symmetric M x M result: the block and its mirror
// are written from the same values, and a diagonal block takes its lower half
// from its upper half, so C is symmetric bit for bit.  M % 16 == 0.
constexpr int kSym = 64;
constexpr int kSymPitch = kSym + 2;
__global__ void __launch_bounds__(kNsThreads) sym_reduce_kernel(const float* parts, int nsplit, int64_t sstride,
                                                               int64_t M, float alpha, float beta,
                                                               const uint16_t* aux, int64_t ldaux, uint16_t* c,
                                                               int64_t ldc) {
  __shared__ uint16_t tile[kSym * kSymPitch];
  const int nb = (int)((M + kSym - 1) / kSym);
  int w = blockIdx.x, bi = 0;
  while (w >= nb - bi) { w -= nb - bi; ++bi; }
  const int bj = bi + w;
  const int64_t r0 = (int64_t)bi * kSym, c0 = (int64_t)bj * kSym;
  // 64 rows x 16 groups of 4 columns; each thread takes 4 groups
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int id = threadIdx.x + kNsThreads * it;
    const int r = id >> 4, q = id & 15;
    const int64_t gr = r0 + r, gc = c0 + q * 4;
    if (gr < M && gc < M) {
      const int64_t off = gr * M + gc;
      v4f sacc = *reinterpret_cast<const v4f*>(parts + off);
      for (int k = 1; k < nsplit; ++k) sacc += *reinterpret_cast<const v4f*>(parts + k * sstride + off);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = aux ? __builtin_fmaf(alpha, sacc[e], beta * bf16_to_f32(aux[gr * ldaux + gc + e]))
                            : alpha * sacc[e];
        tile[r * kSymPitch + q * 4 + e] = (uint16_t)f32_to_bf16_rne(v);
      }
    }
  }
  __syncthreads();
  if (bi == bj) {  // lower half of a diagonal block from its upper half
    uint16_t tmp[16];
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int id = threadIdx.x + kNsThreads * it, r = id >> 6, cc = id & 63;
      tmp[it] = r > cc ? tile[cc * kSymPitch + r] : tile[r * kSymPitch + cc];
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int id = threadIdx.x + kNsThreads * it, r = id >> 6, cc = id & 63;
      tile[r * kSymPitch + cc] = tmp[it];
    }
    __syncthreads();
  }
  // the block, rows of 8 columns (16 bytes)
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int id = threadIdx.x + kNsThreads * it, r = id >> 3, ch = id & 7;
    if (r0 + r < M && c0 + ch * 8 < M) {
      v4u o;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = (uint32_t)tile[r * kSymPitch + ch * 8 + 2 * e] | ((uint32_t)tile[r * kSymPitch + ch * 8 + 2 * e + 1] << 16);
      *reinterpret_cast<v4u*>(c + (r0 + r) * ldc + c0 + ch * 8) = o;
    }
  }
  if (bi == bj) return;
  // the mirror block: row cc of it is column cc of the tile
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int id = threadIdx.x + kNsThreads * it, cc = id >> 3, ch = id & 7;
    if (c0 + cc < M && r0 + ch * 8 < M) {
      v4u o;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = (uint32_t)tile[(ch * 8 + 2 * e) * kSymPitch + cc] |
               ((uint32_t)tile[(ch * 8 + 2 * e + 1) * kSymPitch + cc] << 16);
      *reinterpret_cast<v4u*>(c + (c0 + cc) * ldc + r0 + ch * 8) = o;
    }
  }
}

}  // namespace

hipError_t launch_sym_reduce(const float* parts, int nsplit, int64_t split_stride, int64_t M, float alpha,
                             float beta, const uint16_t* aux, int64_t ldaux, uint16_t* c, int64_t ldc,
                             hipStream_t st) {
  if (M == 0) return hipSuccess;
  const int64_t nb = (M + kSym - 1) / kSym;
  hipLaunchKernelGGL(sym_reduce_kernel, dim3((unsigned)(nb * (nb + 1) / 2)), dim3(kNsThreads), 0, st, parts, nsplit,
                     split_stride, M, alpha, beta, aux, ldaux, c, ldc);
  return hipGetLastError();
}

int ns_parts_for(int64_t n) {
  const int64_t b = (n / 8 + kNsThreads * 8 - 1) / (kNsThreads * 8);  // ~8 chunks per thread
  return (int)(b < 1 ? 1 : (b > kNsMaxParts ? kNsMaxParts : b));
}

hipError_t launch_ns_normalise(const uint16_t* g, int64_t n, float eps, double* partials, uint16_t* x,
                               float* norm_out, hipStream_t st) {
  const int np = ns_parts_for(n);
  hipLaunchKernelGGL(ns_sumsq_kernel, dim3(np), dim3(kNsThreads), 0, st, g, n, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nb = (n / 8 + kNsThreads * 4 - 1) / (kNsThreads * 4);
  const int grid = (int)(nb < 1 ? 1 : (nb > 4096 ? 4096 : nb));
  hipLaunchKernelGGL(ns_scale_kernel, dim3(grid), dim3(kNsThreads), 0, st, g, n, partials, np, eps, x, norm_out);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const uint16_t* src, int64_t rows, int64_t cols, uint16_t* dst, hipStream_t st) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const dim3 grid((unsigned)((cols + kTile - 1) / kTile), (unsigned)((rows + kTile - 1) / kTile));
  hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(kNsThreads), 0, st, src, rows, cols, dst);
  return hipGetLastError();
}

}  // namespace fp8mlp
