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
//      derives s itself, then streams 128x256 tiles: row-major codes go
//      straight to HBM, the transposed codes are built by byte permutes in
//      registers, so both outputs are written in full 128-byte lines.
#include "device_common.h"
#include "internal.h"

namespace fp8mlp {

namespace {

constexpr int kThreads = 256;      // amax kernel
constexpr int kCastThreads = 512;  // cast kernel: 8 waves
constexpr int kTR = 128;           // cast tile rows (8 waves x 16 rows)
constexpr int kTC = 256;           // cast tile columns (64 lanes x 4 columns)

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
  if (aligned16(x) && (ldx == cols || rows == 1)) {
    // dense: one flat array of rows*cols/8 16-byte chunks and a tail
    const int64_t n = rows * cols;
    const int64_t nch = n / 8;
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
    for (int64_t e = nch * 8 + (int64_t)lb * kThreads + threadIdx.x; e < n; e += step) {
      uint32_t t = x[e] & 0x7FFFu;
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

// RMSNorm output from the stored input bits, the row's r and the column's
// weight (has_g false: no weight): RN_bf16(RN32(RN32(x r) g)), as fp32.
__device__ __forceinline__ float norm_value(uint32_t bits, float r, float g, bool has_g) {
  float y = bf16_to_f32(bits) * r;
  if (has_g) y = y * g;
  const __bf16 b = (__bf16)y;  // v_cvt_pk_bf16_f32: round to nearest even
  return bf16_to_f32(__builtin_bit_cast(unsigned short, b));
}

template <int FMT>
__device__ __forceinline__ uint32_t quant4_norm(uint32_t w0, uint32_t w1, float r, const float g[4], bool has_g,
                                                const Divider& d) {
  float a = div_rn(d, norm_value(w0 & 0xFFFFu, r, g[0], has_g));
  float b = div_rn(d, norm_value(w0 >> 16, r, g[1], has_g));
  float c = div_rn(d, norm_value(w1 & 0xFFFFu, r, g[2], has_g));
  float e = div_rn(d, norm_value(w1 >> 16, r, g[3], has_g));
  return pack4_fp8<FMT>(a, b, c, e);
}

template <int FMT, int MODE>
__device__ __forceinline__ uint32_t quant4(uint32_t w0, uint32_t w1, const Divider& d) {
  float a = div_rn(d, cast_value<MODE>(w0 & 0xFFFFu));
  float b = div_rn(d, cast_value<MODE>(w0 >> 16));
  float c = div_rn(d, cast_value<MODE>(w1 & 0xFFFFu));
  float e = div_rn(d, cast_value<MODE>(w1 >> 16));
  return pack4_fp8<FMT>(a, b, c, e);
}

// 4x4 byte transpose: r[i] holds bytes (i,0..3); c[j] gets bytes (0..3,j).
__device__ __forceinline__ void transpose4x4(const uint32_t r[4], uint32_t c[4]) {
  // v_perm_b32(S0, S1, sel): selector byte values 0-3 pick bytes of S1, 4-7 bytes of S0
  const uint32_t t0 = __builtin_amdgcn_perm(r[1], r[0], 0x05010400u);  // r0b0 r1b0 r0b1 r1b1
  const uint32_t t1 = __builtin_amdgcn_perm(r[1], r[0], 0x07030602u);  // r0b2 r1b2 r0b3 r1b3
  const uint32_t t2 = __builtin_amdgcn_perm(r[3], r[2], 0x05010400u);  // r2b0 r3b0 r2b1 r3b1
  const uint32_t t3 = __builtin_amdgcn_perm(r[3], r[2], 0x07030602u);  // r2b2 r3b2 r2b3 r3b3
  c[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  c[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  c[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  c[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// Tiles of kTR x kTC elements: wave w takes rows [16w, 16w+16), lane l the
// 4 columns [4l, 4l+4).  Row-major codes leave as 4-byte stores (256
// contiguous bytes per row and wave instruction); transposed codes are
// assembled in registers, 16 rows of one column per 16-byte store, so each
// transposed row receives 128 contiguous bytes from the block.
// Transposed tile image in LDS: row c (tile column, 0..255) holds the 128
// codes of that column as eight 16-byte pieces k (tile rows 16k..16k+15).
// Piece k of row c sits at slot k ^ ((c >> 2) & 7) of physical row
// c ^ ((c >> 5) & 1): the 16 lanes of a 128-bit LDS access then hit 16
// distinct bank groups both when a wave parks column pieces (lanes 4 columns
// apart) and when it reads rows back (8 lanes per row).
constexpr int kTImage = kTC * kTR;  // bytes
__device__ __forceinline__ int timg_off(int c, int k) {
  return (c ^ ((c >> 5) & 1)) * kTR + ((k ^ ((c >> 2) & 7)) << 4);
}

template <int FMT, int MODE>
__device__ void cast_tiles(const QuantJob& jb, int lb, const Divider& d, uint8_t* tbuf) {
  const int64_t rows = jb.rows, cols = jb.cols, ldx = jb.ldx;
  const uint16_t* x = jb.x;
  uint8_t* q = jb.q;
  uint8_t* qt = jb.qt;
  const int64_t ntr = (rows + kTR - 1) / kTR, ntc = (cols + kTC - 1) / kTC;
  const int64_t ntiles = ntr * ntc;
  const bool vec_in = ((reinterpret_cast<uintptr_t>(x) & 7u) == 0) && (ldx % 4 == 0);
  // Rows that are not 8-byte aligned (odd leading dimension, unaligned base):
  // a lane's 8 bytes come from dword-aligned buffer loads (8 bytes, or 12
  // when they start mid-dword) realigned in registers.  The descriptor spans
  // the dwords that hold tensor bytes, so every dword loaded holds at least
  // one of them (and lies in the same page).
  const uintptr_t xa = reinterpret_cast<uintptr_t>(x);
  const uint32_t dlt = (uint32_t)(xa & 3u);
  const int64_t xbytes = ((rows - 1) * ldx + cols) * 2 + dlt;
  const bool buf_in = !vec_in && (xa & 1u) == 0 && xbytes < (int64_t{1} << 31);
  const __amdgpu_buffer_rsrc_t rx =
      make_rsrc(reinterpret_cast<const void*>(xa - dlt), buf_in ? (uint32_t)((xbytes + 3) & ~int64_t{3}) : 0u);
  const bool vec_q = q == nullptr || (((reinterpret_cast<uintptr_t>(q) & 3u) == 0) && (jb.ldq % 4 == 0));
  const bool vec_qt = qt == nullptr || (aligned16(qt) && (jb.ldqt % 16 == 0));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tile_parity = 0;  // LDS image buffer of the next transposed tile
  for (int64_t t = lb; t < ntiles; t += jb.nblocks) {
    const int64_t r0 = (t / ntc) * kTR, c0 = (t % ntc) * kTC;
    // A tile whose rows are all present takes the vector path when its width
    // is whole 4-column lane groups: lanes past the last column load nothing
    // and store nothing (the last column tile of a ragged width, e.g. 128 of
    // the 50304-column logits).
    const int64_t wv = cols - c0 < kTC ? cols - c0 : kTC;  // valid columns
    const bool full = r0 + kTR <= rows && wv % 4 == 0 && (vec_in || buf_in) && vec_q && vec_qt;
    if (full) {
      const int64_t rb = r0 + wave * 16, cb = c0 + lane * 4;
      const bool lane_ok = lane * 4 < wv;
      v2u in[16];
      if (!lane_ok) {
#pragma unroll
        for (int i = 0; i < 16; ++i) in[i] = v2u{0u, 0u};
      } else if (vec_in) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          in[i] = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(x + (rb + i) * ldx + cb));
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          // byte offset from the aligned base; its dword phase (0 or 2) is
          // the same for every lane of the wave (row-uniform)
          const uint32_t off = dlt + 2u * (uint32_t)((rb + i) * ldx + cb);
          if ((off & 3u) == 0) {
            in[i] = __builtin_amdgcn_raw_buffer_load_b64(rx, off, 0, 0);
          } else {
            const v3u w = __builtin_amdgcn_raw_buffer_load_b96(rx, off - 2u, 0, 0);
            in[i] = v2u{__builtin_amdgcn_alignbyte(w[1], w[0], 2), __builtin_amdgcn_alignbyte(w[2], w[1], 2)};
          }
        }
      }
      uint32_t code[16];  // codes of the 4 columns of each row
      if constexpr (MODE == kModeRmsNorm) {
        const bool has_g = jb.gamma != nullptr;
        float g[4] = {1.0f, 1.0f, 1.0f, 1.0f};
        if (has_g && lane_ok) {
#pragma unroll
          for (int e = 0; e < 4; ++e) g[e] = bf16_to_f32(jb.gamma[cb + e]);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) code[i] = quant4_norm<FMT>(in[i][0], in[i][1], jb.rstd[rb + i], g, has_g, d);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) code[i] = quant4<FMT, MODE>(in[i][0], in[i][1], d);
      }
      if (q && lane_ok) {
#pragma unroll
        for (int i = 0; i < 16; ++i) *reinterpret_cast<uint32_t*>(q + (rb + i) * jb.ldq + cb) = code[i];
      }
      if (qt) {
        // Transposed codes go through LDS so that the stores write whole
        // 128-byte rows of qt: the lane's 4x(16 rows) block is transposed
        // in registers, parked as four 16-byte pieces of the tile's
        // transposed image (256 rows of 128 bytes), and after one barrier
        // eight consecutive lanes store one 128-byte row.
        uint8_t* img = tbuf + (tile_parity & 1) * kTImage;
        uint32_t col[4][4];  // col[j][k]: column j, rows 4k..4k+3
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t c4[4];
          transpose4x4(code + 4 * k, c4);
#pragma unroll
          for (int j = 0; j < 4; ++j) col[j][k] = c4[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = lane * 4 + j;
          *reinterpret_cast<v4u*>(img + timg_off(c, wave)) = v4u{col[j][0], col[j][1], col[j][2], col[j][3]};
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kTC * (kTR / 16) / kCastThreads; ++i) {
          const int id = tid + kCastThreads * i;
          const int c = id >> 3, k = id & 7;
          const v4u o = *reinterpret_cast<const v4u*>(img + timg_off(c, k));
          if (c < wv) *reinterpret_cast<v4u*>(qt + (c0 + c) * jb.ldqt + r0 + 16 * k) = o;
        }
        ++tile_parity;
      }
    } else {
      // ragged or unaligned tile: element by element.  Each thread loads a
      // batch of elements before it converts and stores any of them, so the
      // batch's loads are in flight together (as far as the compiler knows
      // the stores could alias x, which would otherwise serialise every load
      // behind the previous store); the batch is small enough to leave the
      // kernel's register budget unchanged.
      constexpr int kElemBatch = MODE == kModeRmsNorm ? 2 : 4;
      static_assert((kTR * kTC) % (kCastThreads * kElemBatch) == 0, "whole element batches");
      const bool has_g = MODE == kModeRmsNorm && jb.gamma != nullptr;
      for (int e0 = tid; e0 < kTR * kTC; e0 += kCastThreads * kElemBatch) {
        uint32_t bits[kElemBatch];
        float rs[kElemBatch], gm[kElemBatch];
#pragma unroll
        for (int u = 0; u < kElemBatch; ++u) {
          const int e = e0 + u * kCastThreads;
          const int row = e / kTC, col = e % kTC;
          const bool ok = r0 + row < rows && c0 + col < cols;
          bits[u] = ok ? x[(r0 + row) * ldx + c0 + col] : 0u;
          if constexpr (MODE == kModeRmsNorm) {
            rs[u] = ok ? jb.rstd[r0 + row] : 0.0f;
            gm[u] = ok && has_g ? bf16_to_f32(jb.gamma[c0 + col]) : 1.0f;
          }
        }
#pragma unroll
        for (int u = 0; u < kElemBatch; ++u) {
          const int e = e0 + u * kCastThreads;
          const int row = e / kTC, col = e % kTC;
          if (r0 + row < rows && c0 + col < cols) {
            float v;
            if constexpr (MODE == kModeRmsNorm) {
              v = norm_value(bits[u], rs[u], gm[u], has_g);
            } else {
              v = cast_value<MODE>(bits[u]);
            }
            const uint32_t code = pack4_fp8<FMT>(div_rn(d, v), 0.f, 0.f, 0.f) & 0xFFu;
            if (q) q[(r0 + row) * jb.ldq + c0 + col] = (uint8_t)code;
            if (qt) qt[(c0 + col) * jb.ldqt + r0 + row] = (uint8_t)code;
          }
        }
      }
    }
  }
}

// RMSNorm statistics (RMSNorm of the decomputer.nl appendix, applied before
// the MLP's input quantisation): each wave takes two rows, kRmsRows rows per
// block; rows of up to 4096 columns are read once, both rows' loads in flight
// together, and kept in registers.
//   ms = RN32(RN64(sum x^2 / d))  (fp64 sum)   r = RN32(1 / RN32(sqrt(RN32(ms + eps))))
// rstd[row] = r; the block's partial is the max of |RN_bf16(RN32(RN32(x r) g))|,
// taken as RN_bf16 of the largest |RN32(RN32(x r) g)| (rounding to bf16 is
// monotone and odd), an integer max of the fp32 magnitude bits.
constexpr int kRmsRowsPerWave = 2;
constexpr int kRmsRows = 4 * kRmsRowsPerWave;  // four waves per block
constexpr int kRmsRegChunks = 8;  // rows of up to 64 x 8 x 8 = 4096 columns stay in registers

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// max |RN_bf16(RN32(RN32(x r) g))| over 8 columns; gv holds the 8 weights
// (bf16) when has_g.
__device__ __forceinline__ uint32_t norm_max8(v4u v, float r, v4u gv, bool has_g, uint32_t m) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float y = bf16_to_f32((v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) * r;
    if (has_g) y = y * bf16_to_f32((gv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
    const uint32_t mag = f32_to_bf16_rne(y) & 0x7FFFu;
    m = m > mag ? m : mag;
  }
  return m;
}

// Largest fp32 magnitude bits of RN32(RN32(x r) g) over 8 columns; gf holds
// the 8 weights as fp32 (all 1 without a weight: the product is then exact).
__device__ __forceinline__ uint32_t norm_maxbits8(v4u v, float r, const float gf[8], uint32_t m) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(v[i] << 16) * r * gf[2 * i];
    const float hi = __uint_as_float(v[i] & 0xFFFF0000u) * r * gf[2 * i + 1];
    const uint32_t a = __float_as_uint(lo) & 0x7FFFFFFFu, b = __float_as_uint(hi) & 0x7FFFFFFFu;
    m = max(m, max(a, b));
  }
  return m;
}

__device__ __forceinline__ double sumsq8(v4u v, double ss) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double lo = __uint_as_float(v[i] << 16), hi = __uint_as_float(v[i] & 0xFFFF0000u);
    ss = __builtin_fma(lo, lo, ss);  // lo * lo is exact in fp64
    ss = __builtin_fma(hi, hi, ss);
  }
  return ss;
}

__device__ __forceinline__ v4u load_g8(const uint16_t* g, int64_t col, bool g_vec) {
  if (!g) return v4u{0u, 0u, 0u, 0u};
  if (g_vec) return *reinterpret_cast<const v4u*>(g + col);
  v4u o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = (uint32_t)g[col + 2 * e] | ((uint32_t)g[col + 2 * e + 1] << 16);
  return o;
}

// IN_REGS (rows of at most 4096 columns, 16-byte aligned, as the host checks)
// is its own instance so that the register-resident path's registers do not
// lower the occupancy of the streaming path for longer rows.
template <bool IN_REGS>
__global__ void __launch_bounds__(256) rmsnorm_amax_kernel(QuantJob jb, float eps, float* rstd) {
  __shared__ uint32_t red[4];
  // the wave index is uniform across the wave: keep it (and the row descriptors) scalar
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t rows = jb.rows, cols = jb.cols, ldx = jb.ldx;
  const uint16_t* x = jb.x;
  const uint16_t* g = jb.gamma;
  const bool vec = aligned16(x) && (ldx % 8 == 0) && (cols % 8 == 0);
  const bool in_regs = IN_REGS;
  const bool g_vec = g != nullptr && aligned16(g);
  const int64_t nch = cols / 8;
  uint32_t m = 0;
  if (in_regs) {
    // this wave's rows base + wave + 4 i; the later ones may lie past the end
    // (a wave-uniform test); buffer loads past a row's end, or of a missing
    // row, return zeros
    const uint32_t row_bytes = (uint32_t)(2 * cols);
    int64_t row[kRmsRowsPerWave];
    bool has[kRmsRowsPerWave];
    v4u buf[kRmsRowsPerWave][kRmsRegChunks];
#pragma unroll
    for (int i = 0; i < kRmsRowsPerWave; ++i) {
      row[i] = (int64_t)blockIdx.x * kRmsRows + wave + 4 * i;
      has[i] = row[i] < rows;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(x + (has[i] ? row[i] : 0) * ldx, has[i] ? row_bytes : 0u);
#pragma unroll
      for (int k = 0; k < kRmsRegChunks; ++k)
        buf[i][k] = __builtin_amdgcn_raw_buffer_load_b128(rs, 16u * (uint32_t)(lane + 64 * k), 0, 0);
    }
    float r[kRmsRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRmsRowsPerWave; ++i) {
      double ss = 0.0;
#pragma unroll
      for (int k = 0; k < kRmsRegChunks; ++k) ss = sumsq8(buf[i][k], ss);
      ss = wave_sum_f64(ss);
      // correctly rounded square root and division
      r[i] = 1.0f / sqrtf((float)(ss / (double)cols) + eps);
      if (lane == 0 && has[i]) rstd[row[i]] = r[i];
    }
    uint32_t mb = 0;  // fp32 magnitude bits
#pragma unroll
    for (int k = 0; k < kRmsRegChunks; ++k) {
      const int64_t c = lane + 64 * k;
      if (c < nch) {
        float gf[8];
        const v4u gv = load_g8(g, 8 * c, g_vec);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          gf[2 * e] = g ? __uint_as_float(gv[e] << 16) : 1.0f;
          gf[2 * e + 1] = g ? __uint_as_float(gv[e] & 0xFFFF0000u) : 1.0f;
        }
#pragma unroll
        for (int i = 0; i < kRmsRowsPerWave; ++i)
          if (has[i]) mb = norm_maxbits8(buf[i][k], r[i], gf, mb);
      }
    }
    m = f32_to_bf16_rne(__uint_as_float(mb)) & 0x7FFFu;
  }
  for (int rr = wave; rr < kRmsRows && !in_regs; rr += 4) {
    const int64_t row = (int64_t)blockIdx.x * kRmsRows + rr;
    if (row >= rows) break;
    const uint16_t* xr = x + row * ldx;
    double ss = 0.0;
    if (vec) {
      for (int64_t c = lane; c < nch; c += 64) {
        const v4u v = *reinterpret_cast<const v4u*>(xr + 8 * c);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double f = bf16_to_f32((v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
          ss += f * f;
        }
      }
    } else {
      for (int64_t j = lane; j < cols; j += 64) {
        const double f = bf16_to_f32(xr[j]);
        ss += f * f;
      }
    }
    ss = wave_sum_f64(ss);
    const float ms = (float)(ss / (double)cols);
    const float r = 1.0f / sqrtf(ms + eps);  // correctly rounded square root and division
    if (lane == 0) rstd[row] = r;
    if (vec) {
      for (int64_t c = lane; c < nch; c += 64)
        m = norm_max8(*reinterpret_cast<const v4u*>(xr + 8 * c), r, load_g8(g, 8 * c, g_vec), g != nullptr, m);
    } else {
      for (int64_t j = lane; j < cols; j += 64) {
        float y = bf16_to_f32(xr[j]) * r;
        if (g) y = y * bf16_to_f32(g[j]);
        const uint32_t mag = f32_to_bf16_rne(y) & 0x7FFFu;
        m = m > mag ? m : mag;
      }
    }
  }
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) jb.partials[blockIdx.x] = m;
}

template <int FMT, int MODE>
__global__ void __launch_bounds__(kCastThreads) cast_kernel(QuantBatch b) {
  __shared__ uint32_t red[kCastThreads / 64];
  __shared__ __attribute__((aligned(16))) uint8_t tbuf[2 * kTImage];  // double-buffered transposed tile
  int lb;
  const QuantJob& jb = job_of(b, lb);
  // 1. amax from the partials (integer max of non-negative bit patterns)
  uint32_t m = 0;
  for (int i = threadIdx.x; i < jb.nparts; i += kCastThreads) {
    uint32_t v = jb.partials[i];
    m = m > v ? m : v;
  }
  m = block_max_u32(m, red);
  float amax;
  if constexpr (MODE == kModeRelu2) {
    // max over the tensor of RN_bf16(relu(h)^2) = RN_bf16(relu(max h)^2)
    // (x -> x^2 and rounding are monotone on x >= 0)
    const float mh = __uint_as_float(m);
    __bf16 a = (__bf16)(mh * mh);
    amax = bf16_to_f32(__builtin_bit_cast(unsigned short, a));
  } else {
    amax = bf16_to_f32(m);
  }
  constexpr float fm = FMT == kE4M3 ? kFmaxE4M3 : kFmaxE5M2;
  const float s = amax == 0.0f ? 1.0f : amax / fm;  // IEEE division, correctly rounded
  if (lb == 0 && threadIdx.x == 0) {
    *jb.scale = s;
    if (jb.amax_out) *jb.amax_out = amax;
  }
  const Divider d = make_divider(s, amax);
  // 2. cast
  cast_tiles<FMT, MODE>(jb, lb, d, tbuf);
}

int cast_blocks_for(int64_t rows, int64_t cols) {
  const int64_t tiles = ((rows + kTR - 1) / kTR) * ((cols + kTC - 1) / kTC);
  // at least one block: block 0 writes the scale even for an empty tensor
  return (int)(tiles < 1 ? 1 : (tiles < 2048 ? tiles : 2048));
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

int rmsnorm_parts_for(int64_t rows) {
  const int64_t p = (rows + kRmsRows - 1) / kRmsRows;
  return (int)(p < 1 ? 1 : p);
}

hipError_t launch_rmsnorm_amax(QuantJob& j, float eps, float* rstd, hipStream_t st) {
  j.blk_begin = 0;
  j.nblocks = rmsnorm_parts_for(j.rows);
  const bool in_regs = (reinterpret_cast<uintptr_t>(j.x) & 15u) == 0 && j.ldx % 8 == 0 && j.cols % 8 == 0 &&
                       j.cols <= 64 * 8 * kRmsRegChunks;
  if (in_regs)
    hipLaunchKernelGGL(rmsnorm_amax_kernel<true>, dim3(j.nblocks), dim3(256), 0, st, j, eps, rstd);
  else
    hipLaunchKernelGGL(rmsnorm_amax_kernel<false>, dim3(j.nblocks), dim3(256), 0, st, j, eps, rstd);
  return hipGetLastError();
}

hipError_t launch_cast(QuantBatch& b, hipStream_t st) {
  int total = 0;
  for (int i = 0; i < b.njobs; ++i) {
    // one launch handles jobs of a single format and mode
    if (b.job[i].fmt != b.job[0].fmt || b.job[i].mode != b.job[0].mode) return hipErrorInvalidValue;
    b.job[i].blk_begin = total;
    b.job[i].nblocks = cast_blocks_for(b.job[i].rows, b.job[i].cols);
    total += b.job[i].nblocks;
  }
  const int fmt = b.job[0].fmt, mode = b.job[0].mode;
  if (mode == kModeRmsNorm) {
    if (fmt == kE4M3)
      hipLaunchKernelGGL((cast_kernel<kE4M3, kModeRmsNorm>), dim3(total), dim3(kCastThreads), 0, st, b);
    else
      hipLaunchKernelGGL((cast_kernel<kE5M2, kModeRmsNorm>), dim3(total), dim3(kCastThreads), 0, st, b);
  } else if (fmt == kE4M3 && mode == kModePlain)
    hipLaunchKernelGGL((cast_kernel<kE4M3, kModePlain>), dim3(total), dim3(kCastThreads), 0, st, b);
  else if (fmt == kE4M3)
    hipLaunchKernelGGL((cast_kernel<kE4M3, kModeRelu2>), dim3(total), dim3(kCastThreads), 0, st, b);
  else if (mode == kModePlain)
    hipLaunchKernelGGL((cast_kernel<kE5M2, kModePlain>), dim3(total), dim3(kCastThreads), 0, st, b);
  else
    hipLaunchKernelGGL((cast_kernel<kE5M2, kModeRelu2>), dim3(total), dim3(kCastThreads), 0, st, b);
  return hipGetLastError();
}

}  // namespace fp8mlp
