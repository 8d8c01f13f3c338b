// FP8 GEMM on the gfx950 matrix cores:  C = RN_bf16(RN32(sa*sb) * A . B^T)
// with A [M,K] and B [N,K] both stored K-contiguous.  The same kernel also
// multiplies bf16 matrices (format kBF16): the data path moves bytes, so a
// bf16 row is a byte row twice as long, and each 32-byte fragment feeds two
// v_mfma_f32_32x32x16_bf16 instead of one FP8 instruction.  Both operands'
// fragments hold the same K positions at the same lane and register
// offsets, so every product pairs A[i][k] with B[j][k].
//
// All three GEMMs of an FP8 linear layer (decomputer.nl, "Doorvoer
// verhogen", first bullet: one forward and two backward GEMMs in FP8) map to
// this one kernel because the quantiser also writes transposed codes: the
// grad-input GEMM reduces over the output features (dY . W with W^T stored
// K-contiguous) and the grad-weight GEMM over the tokens (dY^T . X with both
// stored transposed).
//
// Design for CDNA4:
//  * v_mfma_f32_32x32x64_f8f6f4 (K = 64 per instruction, per-operand E4M3 or
//    E5M2 selected by the instruction), fp32 accumulation.
//  * 256x256 block tiles run 4 waves in a 2x2 grid, each wave a 128x128
//    tile (4x4 MFMA tiles, 256 accumulator registers: LDS traffic per MFMA
//    at its lowest).  256x192 tiles run 8 waves in a 4x2 grid of 64x96 wave
//    tiles, two waves per SIMD, so one wave's LDS and barrier waits overlap
//    the other's MFMAs.  With dense random FP8 operands the chip reaches its
//    power limit near 1.4-1.6 GHz, so both layouts trade MFMA utilisation
//    against the energy of the data they move.
//  * K is consumed 128 bytes per stage; stages are double-buffered in LDS,
//    loaded with 16-byte buffer loads into registers one stage ahead.  Rows
//    are 128 bytes; the 16-byte chunk c of row r is stored at c ^ ((r>>1)&7)
//    so that the ds_read_b128 fragment reads of sixteen consecutive rows hit
//    distinct banks.  Buffer-descriptor range checks return zeros for rows
//    past M/N and chunks past K, which handles ragged edges.
//  * The MFMA is issued with the B fragment first, so each lane holds four
//    consecutive output columns of one row: the epilogue packs them to bf16,
//    stages the tile in LDS and writes 16-byte row chunks to HBM.
//  * Workgroups are dispatched round-robin over the 8 XCDs; tile ids are
//    remapped so each XCD works on a contiguous run of tiles, grouped 4 tile
//    rows deep, so concurrently running tiles share operands in that XCD's L2.
//  * Epilogues (enum Epilogue in internal.h): plain bf16 store; the relu^2
//    block's relu^2-max and relu^2-backward fusions, whose tile maxima are
//    taken on fp32 values before the (monotone) bf16 rounding; fp32 store and
//    accumulate, and accumulate-then-round-to-bf16 for the last of several
//    summed products; the gated block's merged gate/up projection with the
//    gate applied; and, for bf16 operands, alpha/beta with an optional
//    transposed store and the upper-triangle split-K mode.
#include <type_traits>

#include "device_common.h"
#include "internal.h"
#include "swiglu_math.h"

namespace fp8mlp {

namespace {

constexpr int kBK = 128;  // bytes of K per stage
constexpr int kGroupM = 4;


// LDS placement of the 16-byte chunk c of tile row r: c ^ swz(r).  gfx950
// serves a 128-bit LDS access 16 lanes at a time across 64 four-byte banks,
// i.e. 256 bytes; 128-byte rows put rows r and r+1 in opposite bank halves,
// so the XOR key only has to differ between the 8 row pairs of any 16
// consecutive rows.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// WGM x WGN waves per block (64 * WGM * WGN threads), each owning a
// (BM/WGM) x (BN/WGN) sub-tile.
template <int FA, int FB, int BM, int BN, int WGM, int WGN, int EPI>
struct Gemm {
  static constexpr int THREADS = 64 * WGM * WGN;
  static constexpr int WM = BM / WGM, WN = BN / WGN;  // wave tile
  static constexpr int FM = WM / 32, FN = WN / 32;
  static_assert(FM * 32 == WM && FN * 32 == WN, "wave tile must be whole 32x32 MFMA tiles");
  static constexpr int A_BYTES = BM * kBK, B_BYTES = BN * kBK;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_LOADS = A_BYTES / (THREADS * 16);  // per thread per stage
  static constexpr int B_LOADS = B_BYTES / (THREADS * 16);
  static_assert(A_LOADS * THREADS * 16 == A_BYTES && B_LOADS * THREADS * 16 == B_BYTES, "whole loads");
  static constexpr int LOADS = A_LOADS + B_LOADS;
  static constexpr int CLD = BN * 2 + 16;  // epilogue C tile row stride (bytes)
  static constexpr int LDS = (2 * STAGE > BM * CLD) ? 2 * STAGE : BM * CLD;
};

template <int FA, int FB, int BM, int BN, int WGM, int WGN, int EPI>
__global__ void __launch_bounds__(64 * WGM * WGN, 1) gemm_nt_kernel(GemmArgs g, int tiles_m, int tiles_n) {
  using G = Gemm<FA, FB, BM, BN, WGM, WGN, EPI>;
  constexpr int kThreads = G::THREADS;
  __shared__ __attribute__((aligned(16))) uint8_t smem[G::LDS];
  __shared__ uint32_t red[kThreads / 64];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid % WGM, wn = wid / WGM;

  // ---- tile id: XCD-contiguous runs, grouped kGroupM tile-rows deep
  const int nt = gridDim.x;  // tiles, or work items of the upper-triangle mode
  const int bid = blockIdx.x;
  const int xcd = bid & 7, idx = bid >> 3, per = nt >> 3, rem = nt & 7;
  const int t = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  int tm, tn;
  int64_t kbeg = 0, kelems = g.K;
  float* cfp = g.cf;
  if (g.tri_tiles > 0) {
    // upper-triangle split-K work item: triangle tile t / ksplit in row-major
    // order over (tm <= tn), K slice t % ksplit
    const int ks = t % g.ksplit;
    int tri = t / g.ksplit;
    tm = 0;
    while (tri >= g.tri_tiles - tm) { tri -= g.tri_tiles - tm; ++tm; }
    tn = tm + tri;
    kbeg = ks * g.kchunk;
    kelems = min<int64_t>(g.kchunk, g.K - kbeg);
    cfp = g.cf + ks * g.split_stride;
  } else {
    const int in_group = kGroupM * tiles_n;
    const int first_m = (t / in_group) * kGroupM;
    const int gm = min(kGroupM, tiles_m - first_m);
    tm = first_m + (t % in_group) % gm;
    tn = (t % in_group) / gm;
  }
  // kEpiSwiGLU: a tile's BN B rows are BN/2 rows of the gate weights and the
  // same BN/2 rows of the up weights, so it covers BN/2 output columns
  constexpr bool kSwiGLU = EPI == kEpiSwiGLU;
  constexpr int BNO = kSwiGLU ? BN / 2 : BN;  // output columns per tile
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BNO;

  // operand bytes per element: K, lda and ldb below are in bytes
  constexpr int ES = FA == kBF16 ? 2 : 1;
  static_assert((FA == kBF16) == (FB == kBF16), "bf16 operands come in pairs");
  const int K = (int)kelems * ES;
  const int64_t lda = g.lda * ES, ldb = g.ldb * ES;
  const int rows_a = (int)min<int64_t>(BM, g.M - m0);
  const int rows_b = (int)min<int64_t>(BNO, g.N - n0);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.a + m0 * lda + kbeg * ES, (uint32_t)((rows_a - 1) * lda + K));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.b + n0 * ldb + kbeg * ES, (uint32_t)((rows_b - 1) * ldb + K));
  const __amdgpu_buffer_rsrc_t rb2 =
      kSwiGLU ? make_rsrc(g.b2 + n0 * ldb + kbeg * ES, (uint32_t)((rows_b - 1) * ldb + K)) : rb;

  // Per-thread 16-byte chunks loaded each stage: chunk id = tid + THREADS*j,
  // row = id / 8, logical column chunk = id % 8 (eight lanes cover one
  // 128-byte row, so a wave load is 8 full rows).  In LDS the chunk goes to
  // position logical ^ swz(row) of its row.  Loads j < A_LOADS are A rows,
  // the rest B rows.  Load j's row is row0 + j*(THREADS/8); THREADS/16 is a
  // multiple of 8, so swz() and the column are the same for every j and the
  // offsets are linear in j.
  constexpr int kRowStep = kThreads / 8;
  static_assert((kRowStep / 2) % 8 == 0, "swizzle must repeat every load step");
  const int row0 = tid >> 3, logical0 = tid & 7;
  const int colk0 = logical0 * 16;
  const uint32_t goff_a = (uint32_t)(row0 * lda) + colk0, goff_b = (uint32_t)(row0 * ldb) + colk0;
  const uint32_t gstep_a = (uint32_t)(kRowStep * lda), gstep_b = (uint32_t)(kRowStep * ldb);
  const uint32_t lds0 = row0 * kBK + ((logical0 ^ swz(row0)) << 4);

  v4u stg[G::LOADS];  // one stage in flight in registers
  // kEpiSwiGLU: B loads jj < B_LOADS/2 fill the gate half of the stage, the
  // rest the up half, from the same rows of the other operand
  static_assert(!kSwiGLU || (G::B_LOADS % 2 == 0 && (G::B_LOADS / 2) * kRowStep == BN / 2),
                "each B load must lie in one half");
  auto gload_one = [&](int j, int kt) {
    const int k0 = kt * kBK;
    const bool is_a = j < G::A_LOADS;
    const int jb = j - G::A_LOADS;
    const bool up = kSwiGLU && !is_a && jb >= G::B_LOADS / 2;
    const int jj = is_a ? j : (up ? jb - G::B_LOADS / 2 : jb);
    const uint32_t base = is_a ? goff_a + jj * gstep_a : goff_b + jj * gstep_b;
    const uint32_t off = (k0 + colk0 < K) ? base + k0 : 0x80000000u;  // out of range -> 0
    stg[j] = __builtin_amdgcn_raw_buffer_load_b128(is_a ? ra : (up ? rb2 : rb), off, 0, 0);
  };
  auto swrite_one = [&](int j, int buf) {
    const bool is_a = j < G::A_LOADS;
    const int jj = is_a ? j : j - G::A_LOADS;
    *reinterpret_cast<v4u*>(smem + buf * G::STAGE + (is_a ? 0 : G::A_BYTES) + lds0 + jj * kRowStep * kBK) =
        stg[j];
  };

  v16f acc[G::FM][G::FN];
#pragma unroll
  for (int i = 0; i < G::FM; ++i)
#pragma unroll
    for (int j = 0; j < G::FN; ++j) acc[i][j] = v16f{};

  // Fragments: lane reads row (lane & 31) of a 32-row block, the 32 bytes of
  // K starting at ks*64 + (lane >> 5)*32, as two 16-byte LDS reads.  Read r
  // of a fragment set (r < NR) is half r&1 of fragment r>>1 (A fragments
  // first, then B).
  constexpr int NM = G::FM * G::FN;        // MFMAs per 64-byte K substep
  constexpr int NR = 2 * (G::FM + G::FN);  // 16-byte LDS reads per substep
  const int frow = lane & 31, fhalf = lane >> 5;
  typedef v4i Frag[G::FM + G::FN][2];
  auto read_one = [&](int r, int buf, int ks, Frag& f) {
    const int fi = r >> 1, h = r & 1;
    const bool is_a = fi < G::FM;
    const int row = is_a ? wm * G::WM + fi * 32 + frow : wn * G::WN + (fi - G::FM) * 32 + frow;
    const int c = ks * 4 + fhalf * 2 + h;
    f[fi][h] = *reinterpret_cast<const v4i*>(smem + buf * G::STAGE + (is_a ? 0 : G::A_BYTES) + row * kBK +
                                             ((c ^ swz(row)) << 4));
  };
  auto mfma_one = [&](int t, const Frag& f) {
    const int i = t / G::FN, j = t % G::FN;
    const v4i* a = f[i];
    const v4i* b = f[G::FM + j];
    if constexpr (FA == kBF16) {
      // two K=16 bf16 instructions, one per 16-byte half of the fragment
      // (issuing the halves as two passes over the tiles measured slower)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, b[hh]),
                                                            __builtin_bit_cast(v8bf, a[hh]), acc[i][j], 0, 0, 0);
    } else {
      const v8i av = v8i{a[0][0], a[0][1], a[0][2], a[0][3], a[1][0], a[1][1], a[1][2], a[1][3]};
      const v8i bv = v8i{b[0][0], b[0][1], b[0][2], b[0][3], b[1][0], b[1][1], b[1][2], b[1][3]};
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv, av, acc[i][j], FB, FA, 0, 0, 0, 0);
    }
  };

  // Software pipeline over 128-byte K stages, two LDS buffers, one stage in
  // registers.  Iteration kt (stage kt in LDS buffer kt&1, its first-half
  // fragments F0 already in registers):
  //   A: MFMAs on F0; step t also issues read t of the second-half fragments
  //      F1, LDS write t of stage kt+1 (registers -> other buffer) and global
  //      load t of stage kt+2 into the register just written out;
  //   B: MFMAs on F1; the barrier that publishes stage kt+1 sits before the
  //      last kTail MFMAs, which hide the reads of stage kt+1's F0.
  // sched_barrier fences keep this order through instruction scheduling.
  constexpr int kTail = 4;
  constexpr int STEPS_A = NM > NR ? (NM > G::LOADS ? NM : G::LOADS) : (NR > G::LOADS ? NR : G::LOADS);
  const int nk = (K + kBK - 1) / kBK;
  Frag f0, f1;

#pragma unroll
  for (int j = 0; j < G::LOADS; ++j) gload_one(j, 0);
#pragma unroll
  for (int j = 0; j < G::LOADS; ++j) swrite_one(j, 0);
  if (nk > 1) {
#pragma unroll
    for (int j = 0; j < G::LOADS; ++j) gload_one(j, 1);
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < NR; ++r) read_one(r, 0, 0, f0);

  auto iteration = [&](int kt, auto has_next, auto has_next2) {
    constexpr bool HN = decltype(has_next)::value, HN2 = decltype(has_next2)::value;
    const int cur = kt & 1, nxt = cur ^ 1;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < STEPS_A; ++t) {
      if (t < NM) mfma_one(t, f0);
      if (t < NR) read_one(t, cur, 1, f1);
      if constexpr (HN) {
        if (t < G::LOADS) {
          swrite_one(t, nxt);
          if constexpr (HN2) gload_one(t, kt + 2);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = 0; t < NM - kTail; ++t) mfma_one(t, f1);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (HN) __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = NM - kTail; t < NM; ++t) {
      mfma_one(t, f1);
      if constexpr (HN) {
#pragma unroll
        for (int r = (t - (NM - kTail)) * NR / kTail; r < (t - (NM - kTail) + 1) * NR / kTail; ++r)
          read_one(r, nxt, 0, f0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using T = std::true_type;
  using F = std::false_type;
  int kt = 0;
  for (; kt + 2 < nk; ++kt) iteration(kt, T{}, T{});
  if (kt + 1 < nk) { iteration(kt, T{}, F{}); ++kt; }
  iteration(kt, F{}, F{});
  __syncthreads();

  // ---- alpha/beta epilogue (bf16 operands).  Each lane combines its four
  // consecutive columns of a row with the same elements of aux (when given),
  // so the sum is rounded once, and stages the bf16 result in LDS; the tile
  // then leaves as 16-byte row chunks and, with ct, as 16-byte chunks of
  // C^T rows (eight consecutive rows of one column).  In LDS the 16-byte
  // chunk c8 of tile row r sits at chunk c8 ^ ((r >> 3) & 7) of its row, so
  // that the column gathers of eight row groups hit distinct banks.  aux may
  // be the output itself: every aux element is read before the barrier that
  // precedes the stores, and each tile is one block's alone.
  if constexpr (EPI == kEpiAxpby) {
    const bool has_aux = g.aux != nullptr;
    const bool vaux = !has_aux || (((reinterpret_cast<uintptr_t>(g.aux) & 7u) == 0) && (g.ldaux % 4 == 0));
    auto lds_at = [&](int row, int col) {
      return row * G::CLD + (((col >> 3) ^ ((row >> 3) & 7)) << 4) + (col & 7) * 2;
    };
#pragma unroll
    for (int i = 0; i < G::FM; ++i) {
      const int row = wm * G::WM + i * 32 + frow;
      const int64_t gr = m0 + row;
#pragma unroll
      for (int j = 0; j < G::FN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = wn * G::WN + j * 32 + q * 8 + fhalf * 4;
          const int64_t gc = n0 + col;
          const v16f& a = acc[i][j];
          uint32_t o[4] = {0u, 0u, 0u, 0u};
          if (gr < g.M) {
            const uint16_t* src = g.aux + gr * g.ldaux + gc;
            if (!has_aux) {
#pragma unroll
              for (int e = 0; e < 4; ++e) o[e] = f32_to_bf16_rne(g.alpha * a[4 * q + e]);
            } else if (vaux && gc + 4 <= g.N) {
              const v2u x = *reinterpret_cast<const v2u*>(src);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const uint32_t xb = (x[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                o[e] = f32_to_bf16_rne(__builtin_fmaf(g.alpha, a[4 * q + e], g.beta * bf16_to_f32(xb)));
              }
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (gc + e < g.N)
                  o[e] = f32_to_bf16_rne(__builtin_fmaf(g.alpha, a[4 * q + e], g.beta * bf16_to_f32(src[e])));
            }
          }
          *reinterpret_cast<v2u*>(smem + lds_at(row, col)) = v2u{o[0] | (o[1] << 16), o[2] | (o[3] << 16)};
        }
      }
    }
    __syncthreads();
    // rows of C: 16-byte chunks
    constexpr int kCpr = BN / 8, kNch = BM * kCpr / kThreads;
    static_assert(kNch * kThreads == BM * kCpr, "whole row chunks");
    const bool vec_c = ((reinterpret_cast<uintptr_t>(g.c) & 15u) == 0) && (g.ldc % 8 == 0);
#pragma unroll
    for (int it = 0; it < kNch; ++it) {
      const int id = tid + kThreads * it;
      const int row = id / kCpr, c8 = id % kCpr;
      const int64_t gr = m0 + row, gc = n0 + c8 * 8;
      if (gr < g.M && gc < g.N) {
        const v4u v = *reinterpret_cast<const v4u*>(smem + lds_at(row, c8 * 8));
        uint16_t* dst = g.c + gr * g.ldc + gc;
        if (vec_c && gc + 8 <= g.N) {
          *reinterpret_cast<v4u*>(dst) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (gc + e < g.N) dst[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
    // rows of C^T: lanes take 8 consecutive columns x 8 consecutive row groups
    if (g.ct) {
      constexpr int kRg = BM / 8, kCo = BN / 8;  // row groups, column octets
      constexpr int kNt = BN * kRg / kThreads;
      static_assert(kNt * kThreads == BN * kRg && kRg % 8 == 0, "whole C^T chunks");
      const bool vec_t = ((reinterpret_cast<uintptr_t>(g.ct) & 15u) == 0) && (g.ldct % 8 == 0);
#pragma unroll
      for (int it = 0; it < kNt; ++it) {
        const int id = tid + kThreads * it;
        const int blk = id >> 6;
        const int col = (blk % kCo) * 8 + (id & 7);
        const int rg = (blk / kCo) * 8 + ((id >> 3) & 7);
        const int64_t gc = n0 + col, gr0 = m0 + rg * 8;
        if (gc < g.N && gr0 < g.M) {
          uint32_t h[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) h[e] = *reinterpret_cast<const uint16_t*>(smem + lds_at(rg * 8 + e, col));
          uint16_t* dst = g.ct + gc * g.ldct + gr0;
          if (vec_t && gr0 + 8 <= g.M) {
            *reinterpret_cast<v4u*>(dst) = v4u{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                               h[6] | (h[7] << 16)};
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (gr0 + e < g.M) dst[e] = (uint16_t)h[e];
          }
        }
      }
    }
    return;
  }

  // ---- fp32 epilogues: each lane writes its four consecutive columns of a
  // row straight from the accumulators (a 256-row fp32 tile would not fit in
  // LDS); the fp32 output is read-modify-written in place to accumulate.
  if constexpr (EPI == kEpiStoreF32 || EPI == kEpiAccF32 || EPI == kEpiAccF32Bf16) {
    float p;
    if constexpr (FA == kBF16) p = g.alpha;
    else p = (*g.sa) * (*g.sb);  // RN32(sa * sb)
    const bool vec = ((reinterpret_cast<uintptr_t>(cfp) & 15u) == 0) && (g.ldc % 4 == 0) &&
                     (EPI != kEpiAccF32Bf16 || (reinterpret_cast<uintptr_t>(g.c) & 7u) == 0);
#pragma unroll
    for (int i = 0; i < G::FM; ++i) {
      const int64_t gr = m0 + wm * G::WM + i * 32 + frow;
      if (gr >= g.M) continue;
#pragma unroll
      for (int j = 0; j < G::FN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t gc = n0 + wn * G::WN + j * 32 + q * 8 + fhalf * 4;
          const v16f& a = acc[i][j];
          v4f v = {a[4 * q + 0] * p, a[4 * q + 1] * p, a[4 * q + 2] * p, a[4 * q + 3] * p};
          float* dst = cfp + gr * g.ldc + gc;
          if constexpr (EPI == kEpiAccF32Bf16) {
            // the accumulated fp32 sum rounded once to bf16 (same ldc)
            uint16_t* out = g.c + gr * g.ldc + gc;
            if (vec && gc + 4 <= g.N) {
              v += *reinterpret_cast<const v4f*>(dst);
              *reinterpret_cast<v2u*>(out) = v2u{f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16),
                                                 f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16)};
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (gc + e < g.N) out[e] = (uint16_t)f32_to_bf16_rne(dst[e] + v[e]);
            }
          } else if (vec && gc + 4 <= g.N) {
            if constexpr (EPI == kEpiAccF32) v += *reinterpret_cast<const v4f*>(dst);
            *reinterpret_cast<v4f*>(dst) = v;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (gc + e < g.N) dst[e] = EPI == kEpiAccF32 ? dst[e] + v[e] : v[e];
          }
        }
      }
    }
    return;
  }

  // ---- epilogue
  // Each thread owns NCH 16-byte chunks of the output tile: chunk id
  // tid + THREADS*it is row id / CPR, 8-column group id % CPR.
  constexpr int CPR = BN / 8;  // 16-byte chunks per tile row
  constexpr int NCH = BM * CPR / kThreads;
  static_assert(NCH * kThreads == BM * CPR, "whole epilogue chunks");
  const bool vec_c = ((reinterpret_cast<uintptr_t>(g.c) & 15u) == 0) && (g.ldc % 8 == 0);
  const bool vec_aux = EPI != kEpiRelu2Bwd ||
                       (((reinterpret_cast<uintptr_t>(g.aux) & 15u) == 0) && (g.ldaux % 8 == 0));
  // The relu^2-backward epilogue needs H at its chunks.  With two waves per
  // SIMD (THREADS = 512) the loads are issued first, in flight while the tile
  // is staged in LDS; the 4-wave layout has no registers to spare next to its
  // 256 accumulators and issues them after staging.
  constexpr bool kEarlyH = EPI == kEpiRelu2Bwd && kThreads == 512;
  v4u hv[EPI == kEpiRelu2Bwd ? NCH : 1];
  auto load_h = [&]() {
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
      const int id = tid + kThreads * it;
      const int64_t gr = m0 + id / CPR, gc = n0 + (id % CPR) * 8;
      hv[it] = v4u{0u, 0u, 0u, 0u};
      if (gr < g.M && gc < g.N) {
        if (gc + 8 <= g.N && vec_c && vec_aux) {
          hv[it] = *reinterpret_cast<const v4u*>(g.aux + gr * g.ldaux + gc);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t lo = gc + 2 * e < g.N ? g.aux[gr * g.ldaux + gc + 2 * e] : 0u;
            const uint32_t hi = gc + 2 * e + 1 < g.N ? g.aux[gr * g.ldaux + gc + 2 * e + 1] : 0u;
            hv[it][e] = lo | (hi << 16);
          }
        }
      }
    }
  };
  if constexpr (kEarlyH) load_h();

  // scale, round to bf16 and stage the tile in LDS
  static_assert(!kSwiGLU || G::WN * 2 == BN, "kEpiSwiGLU: one wave column per half");
  float p;
  if constexpr (FA == kBF16) p = g.alpha;
  else if constexpr (kSwiGLU) p = (*g.sa) * (wn == 0 ? *g.sb : *g.sb2);  // gate or up half
  else p = (*g.sa) * (*g.sb);  // RN32(sa * sb)
  // relu^2-max epilogue: the tile's max of H = RN_bf16(x), x = RN32(acc p),
  // is RN_bf16 of the max of x (both roundings are monotone), so it is taken
  // here on the fp32 values.  Accumulators of rows past M or columns past N
  // are 0 (their operands load as zeros) and cannot raise a max that starts
  // at 0, so they need no mask.
  float hmax = 0.0f;
#pragma unroll
  for (int i = 0; i < G::FM; ++i) {
    const int row = wm * G::WM + i * 32 + frow;
#pragma unroll
    for (int j = 0; j < G::FN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = wn * G::WN + j * 32 + q * 8 + fhalf * 4;
        const v16f& a = acc[i][j];
        const float x0 = a[4 * q + 0] * p, x1 = a[4 * q + 1] * p, x2 = a[4 * q + 2] * p, x3 = a[4 * q + 3] * p;
        if constexpr (EPI == kEpiRelu2Max)
          hmax = __builtin_fmaxf(hmax, __builtin_fmaxf(__builtin_fmaxf(x0, x1), __builtin_fmaxf(x2, x3)));
        const __bf16 h0 = (__bf16)x0, h1 = (__bf16)x1;
        const __bf16 h2 = (__bf16)x2, h3 = (__bf16)x3;
        v2u w;
        w[0] = (uint32_t)__builtin_bit_cast(unsigned short, h0) |
               ((uint32_t)__builtin_bit_cast(unsigned short, h1) << 16);
        w[1] = (uint32_t)__builtin_bit_cast(unsigned short, h2) |
               ((uint32_t)__builtin_bit_cast(unsigned short, h3) << 16);
        *reinterpret_cast<v2u*>(smem + row * G::CLD + col * 2) = w;
      }
    }
  }
  __syncthreads();
  if constexpr (EPI == kEpiRelu2Bwd && !kEarlyH) load_h();

  if constexpr (kSwiGLU) {
    // Chunk pairs: row id / CPH, gate chunk id % CPH of the staged row and
    // the up chunk CPH chunks further along it.  G, U and A = RN_bf16(silu(G)
    // U) are written; the partial is the tile's max |A| (bf16 bits).
    constexpr int CPH = BN / 16;  // 16-byte chunks per half row
    constexpr int NP = BM * CPH / kThreads;
    static_assert(NP * kThreads == BM * CPH, "whole chunk pairs");
    const bool vec3 = vec_c && ((reinterpret_cast<uintptr_t>(g.c2) & 15u) == 0) &&
                      ((reinterpret_cast<uintptr_t>(g.c3) & 15u) == 0);
    uint32_t amx = 0;
#pragma unroll
    for (int it = 0; it < NP; ++it) {
      const int id = tid + kThreads * it;
      const int row = id / CPH, c8 = id % CPH;
      const int64_t gr = m0 + row, gc = n0 + c8 * 8;
      if (gr < g.M && gc < g.N) {
        const v4u gv = *reinterpret_cast<const v4u*>(smem + row * G::CLD + c8 * 16);
        const v4u uv = *reinterpret_cast<const v4u*>(smem + row * G::CLD + (c8 + CPH) * 16);
        v4u av;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t a0 = swiglu_a_bits(bf16_to_f32(gv[e] & 0xFFFFu), bf16_to_f32(uv[e] & 0xFFFFu));
          const uint32_t a1 = swiglu_a_bits(bf16_to_f32(gv[e] >> 16), bf16_to_f32(uv[e] >> 16));
          av[e] = a0 | (a1 << 16);
          if (gc + 2 * e < g.N) amx = amx > (a0 & 0x7FFFu) ? amx : (a0 & 0x7FFFu);
          if (gc + 2 * e + 1 < g.N) amx = amx > (a1 & 0x7FFFu) ? amx : (a1 & 0x7FFFu);
        }
        const int64_t o = gr * g.ldc + gc;
        if (gc + 8 <= g.N && vec3) {
          *reinterpret_cast<v4u*>(g.c + o) = gv;
          *reinterpret_cast<v4u*>(g.c2 + o) = uv;
          *reinterpret_cast<v4u*>(g.c3 + o) = av;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (gc + e < g.N) {
              const int sh = 16 * (e & 1);
              g.c[o + e] = (uint16_t)(gv[e >> 1] >> sh);
              g.c2[o + e] = (uint16_t)(uv[e >> 1] >> sh);
              g.c3[o + e] = (uint16_t)(av[e >> 1] >> sh);
            }
          }
        }
      }
    }
    amx = block_max_u32(amx, red);
    if (tid == 0 && g.partials) g.partials[t] = amx;
    return;
  }

  // epilogue max, as the partial's format wants it: relu^2-max the fp32 bit
  // pattern of a non-negative bf16 value, relu^2-backward the bf16 magnitude
  // bits.  The relu^2-backward max |dH| is likewise taken before rounding,
  // max |RN_bf16(y)| = RN_bf16(max |y|); chunk elements past N hold y = 0.
  uint32_t mx = 0;
  float dmax = 0.0f;
  if constexpr (EPI == kEpiRelu2Max) {
    const __bf16 hb = (__bf16)hmax;
    mx = ((uint32_t)__builtin_bit_cast(unsigned short, hb) << 16) & 0x7FFFFFFFu;  // -0 -> +0
  }
#pragma unroll
  for (int it = 0; it < NCH; ++it) {
    const int id = tid + kThreads * it;
    const int row = id / CPR, c8 = id % CPR;
    const int64_t gr = m0 + row, gc = n0 + c8 * 8;
    if (gr < g.M && gc < g.N) {
      v4u v = *reinterpret_cast<const v4u*>(smem + row * G::CLD + c8 * 16);
      const bool full = gc + 8 <= g.N && vec_c && vec_aux;
      if constexpr (EPI == kEpiRelu2Bwd) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t out = 0;
#pragma unroll
          for (int hlf = 0; hlf < 2; ++hlf) {
            const float h = bf16_to_f32((hv[it][e] >> (16 * hlf)) & 0xFFFFu);
            const float da = bf16_to_f32((v[e] >> (16 * hlf)) & 0xFFFFu);
            const float r = h > 0.0f ? h : 0.0f;
            const float y = (2.0f * r) * da;  // exact product
            dmax = __builtin_fmaxf(dmax, __builtin_fabsf(y));
            const __bf16 dh = (__bf16)y;  // one rounding
            out |= (uint32_t)__builtin_bit_cast(unsigned short, dh) << (16 * hlf);
          }
          v[e] = out;
        }
      }
      if (full) {
        *reinterpret_cast<v4u*>(g.c + gr * g.ldc + gc) = v;
      } else if (gc + 8 <= g.N) {
        // whole chunk, destination not 16-byte aligned (an odd or unaligned
        // leading dimension): the widest stores its alignment allows
        uint16_t* dst = g.c + gr * g.ldc + gc;
        const uintptr_t a = reinterpret_cast<uintptr_t>(dst);
        if ((a & 7u) == 0) {
          reinterpret_cast<v2u*>(dst)[0] = v2u{v[0], v[1]};
          reinterpret_cast<v2u*>(dst)[1] = v2u{v[2], v[3]};
        } else if ((a & 3u) == 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) reinterpret_cast<uint32_t*>(dst)[e] = v[e];
        } else {
          dst[0] = (uint16_t)v[0];
          uint32_t* mid = reinterpret_cast<uint32_t*>(dst + 1);
          mid[0] = __builtin_amdgcn_alignbyte(v[1], v[0], 2);
          mid[1] = __builtin_amdgcn_alignbyte(v[2], v[1], 2);
          mid[2] = __builtin_amdgcn_alignbyte(v[3], v[2], 2);
          dst[7] = (uint16_t)(v[3] >> 16);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (gc + e < g.N) g.c[gr * g.ldc + gc + e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
      }
    }
  }
  if constexpr (EPI == kEpiRelu2Bwd) {
    const __bf16 db = (__bf16)dmax;
    mx = (uint32_t)__builtin_bit_cast(unsigned short, db) & 0x7FFFu;
  }
  if constexpr (EPI != kEpiStore) {
    mx = block_max_u32(mx, red);
    if (tid == 0) g.partials[t] = mx;
  }
}

template <int FA, int FB, int BM, int BN, int WGM, int WGN, int EPI>
hipError_t launch_cfg(const GemmArgs& g, hipStream_t st) {
  constexpr int BNO = EPI == kEpiSwiGLU ? BN / 2 : BN;  // output columns per tile
  const int tiles_m = (int)((g.M + BM - 1) / BM), tiles_n = (int)((g.N + BNO - 1) / BNO);
  if (tiles_m == 0 || tiles_n == 0) return hipSuccess;  // empty output
  const int work = g.tri_tiles > 0 ? g.tri_tiles * (g.tri_tiles + 1) / 2 * g.ksplit : tiles_m * tiles_n;
  hipLaunchKernelGGL((gemm_nt_kernel<FA, FB, BM, BN, WGM, WGN, EPI>), dim3(work), dim3(64 * WGM * WGN), 0, st, g,
                     tiles_m, tiles_n);
  return hipGetLastError();
}

// Block tile width: 256x192 tiles when they fill the 256 CUs in whole waves
// better than 256x256 (e.g. an 8192x3072 output is 384 tiles of 256x256 =
// 1.5 waves, but 512 tiles of 256x192 = 2 waves).
int pick_bn(int64_t M, int64_t N) {
  auto eff = [&](int bn) {
    const int64_t t = ((M + 255) / 256) * ((N + bn - 1) / bn);
    const int64_t waves = (t + 255) / 256;
    return (double)(M * N) / (double)(waves * 256 * 256 * bn);
  };
  return eff(192) > eff(256) * 1.02 ? 192 : 256;
}

template <int FA, int FB, int BN, int WGM, int WGN>
hipError_t launch_bn(const GemmArgs& g, hipStream_t st) {
  if constexpr (FA == kBF16) {
    // bf16 products: the alpha/beta epilogue, or fp32 tiles of the
    // upper-triangle split-K mode
    if constexpr (BN == 192) {  // the 4-wave alpha/beta epilogue would spill
      if (g.epi == kEpiAxpby) return launch_cfg<FA, FB, 256, BN, WGM, WGN, kEpiAxpby>(g, st);
    }
    if (g.epi == kEpiStoreF32) return launch_cfg<FA, FB, 256, BN, WGM, WGN, kEpiStoreF32>(g, st);
    return hipErrorInvalidValue;
  } else {
  switch (g.epi) {
    case kEpiRelu2Max: return launch_cfg<FA, FB, 256, BN, WGM, WGN, kEpiRelu2Max>(g, st);
    case kEpiRelu2Bwd: return launch_cfg<FA, FB, 256, BN, WGM, WGN, kEpiRelu2Bwd>(g, st);
    case kEpiSwiGLU:
      // merged gate/up projection: E4M3 x E4M3 on 256x256 tiles (128 output columns)
      if constexpr (FA == kE4M3 && FB == kE4M3 && BN == 256) {
        return launch_cfg<FA, FB, 256, 256, 2, 2, kEpiSwiGLU>(g, st);
      } else {
        return hipErrorInvalidValue;
      }
    case kEpiStoreF32:
    case kEpiAccF32:
    case kEpiAccF32Bf16:
      // fp32 outputs are only produced for E5M2 x E4M3 (gradient x activation)
      if constexpr (FA == kE5M2 && FB == kE4M3) {
        if (g.epi == kEpiStoreF32) return launch_cfg<FA, FB, 256, BN, WGM, WGN, kEpiStoreF32>(g, st);
        if (g.epi == kEpiAccF32) return launch_cfg<FA, FB, 256, BN, WGM, WGN, kEpiAccF32>(g, st);
        return launch_cfg<FA, FB, 256, BN, WGM, WGN, kEpiAccF32Bf16>(g, st);
      } else {
        return hipErrorInvalidValue;
      }
    default: return launch_cfg<FA, FB, 256, BN, WGM, WGN, kEpiStore>(g, st);
  }
  }
}

template <int FA, int FB>
hipError_t launch_fmt(const GemmArgs& g, hipStream_t st) {
  // 256x192 tiles run 8 waves (4x2, 64x96 wave tiles, two waves per SIMD);
  // 256x256 tiles 4 waves (2x2, 128x128 wave tiles).  bf16 products always
  // take the 8-wave tiles: the 4-wave alpha/beta epilogue would spill.
  if constexpr (FA == kBF16) {
    // square 256x256 tiles for the upper-triangle mode (fp32 epilogue only)
    if (g.tri_tiles > 0) return launch_bn<FA, FB, 256, 2, 2>(g, st);
    return launch_bn<FA, FB, 192, 4, 2>(g, st);
  } else {
    if (g.epi == kEpiSwiGLU) return launch_bn<FA, FB, 256, 2, 2>(g, st);
    return pick_bn(g.M, g.N) == 192 ? launch_bn<FA, FB, 192, 4, 2>(g, st) : launch_bn<FA, FB, 256, 2, 2>(g, st);
  }
}

}  // namespace

int64_t gemm_num_tiles(int64_t M, int64_t N) {
  const int bn = pick_bn(M, N);
  return ((M + 255) / 256) * ((N + bn - 1) / bn);
}
int64_t gemm_max_tiles(int64_t M, int64_t N) { return ((M + 63) / 64) * ((N + 63) / 64); }
int64_t gemm_swiglu_tiles(int64_t M, int64_t N) { return ((M + 255) / 256) * ((N + 127) / 128); }

// Work split of the symmetric product: enough K slices that the triangle's
// tiles times the slices fill the 256 CUs about once, each slice at least
// 512 elements long and a whole number of 64-element stages.
int sym_ksplit(int64_t M, int64_t K) {
  const int64_t T = (M + 255) / 256, ntri = T * (T + 1) / 2;
  if (ntri == 0) return 1;  // empty product
  int64_t s = 256 / ntri;
  if (s > K / 512) s = K / 512;
  if (s > 8) s = 8;
  return (int)(s < 1 ? 1 : s);
}

static int64_t sym_kchunk(int64_t K, int s) { return ((K + s - 1) / s + 63) / 64 * 64; }

size_t sym_partials_bytes(int64_t M, int64_t K) { return (size_t)sym_ksplit(M, K) * (size_t)(M * M) * 4; }

hipError_t launch_sym_gemm(const uint16_t* a, int64_t lda, int64_t M, int64_t K, float alpha, float beta,
                           const uint16_t* aux, int64_t ldaux, uint16_t* c, int64_t ldc, float* partials,
                           hipStream_t st) {
  if (M == 0) return hipSuccess;
  const int s = sym_ksplit(M, K);
  const int64_t kc = sym_kchunk(K, s);
  const int nsplit = kc > 0 ? (int)((K + kc - 1) / kc) : 1;  // slices actually used
  GemmArgs g{};
  g.a = g.b = (const uint8_t*)a; g.lda = g.ldb = lda; g.fa = g.fb = kBF16;
  g.M = g.N = M; g.K = K; g.epi = kEpiStoreF32; g.alpha = 1.0f; g.cf = partials; g.ldc = M;
  g.tri_tiles = (int)((M + 255) / 256); g.ksplit = nsplit < 1 ? 1 : nsplit; g.kchunk = kc; g.split_stride = M * M;
  hipError_t e = launch_gemm(g, st);
  if (e != hipSuccess) return e;
  return launch_sym_reduce(partials, g.ksplit, M * M, M, alpha, beta, aux, ldaux, c, ldc, st);
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
  if (g.fa == kBF16 || g.fb == kBF16) {
    if (g.fa != g.fb) return hipErrorInvalidValue;
    return launch_fmt<kBF16, kBF16>(g, st);
  }
  if (g.fa == kE4M3 && g.fb == kE4M3) return launch_fmt<kE4M3, kE4M3>(g, st);
  if (g.fa == kE5M2 && g.fb == kE4M3) return launch_fmt<kE5M2, kE4M3>(g, st);
  if (g.fa == kE4M3 && g.fb == kE5M2) return launch_fmt<kE4M3, kE5M2>(g, st);
  return launch_fmt<kE5M2, kE5M2>(g, st);
}

}  // namespace fp8mlp
