// Templated GEMM kernel of the FP8 linear layers on the gfx950 matrix cores:
//   C = RN_bf16(RN32(sa*sb) * op(A) . op(B)),  fp32 accumulation,
// in the three layouts of a linear layer's GEMMs (decomputer.nl, "Doorvoer
// verhogen", first bullet: one forward and two backward GEMMs in FP8):
//   NT  C[m,n] = sum_k A[m,k] B[n,k]   forward      (both operands K-major)
//   NN  C[m,n] = sum_k A[m,k] B[k,n]   grad-input   (B MN-major)
//   TN  C[m,n] = sum_k A[k,m] B[k,n]   grad-weight  (both MN-major)
// "K-major": each stored row holds one output index and the reduction index
// runs along it; "MN-major": each stored row is one reduction index.  All
// operands are row-major FP8 codes as the quantiser writes them.  The same
// kernel also multiplies bf16 matrices (format kBF16, NT only): the data path
// moves bytes, so a bf16 row is a byte row twice as long, and each 32-byte
// fragment feeds two v_mfma_f32_32x32x16_bf16 instead of one FP8 instruction.
//
// Design for CDNA4:
//  * v_mfma_f32_32x32x64_f8f6f4 (K = 64 per instruction, per-operand E4M3 or
//    E5M2 selected by the instruction), fp32 accumulation.  Its hardware sum
//    is not exact: the 64 products are added in aligned groups of 8 whose
//    members are truncated to 13 bits below the group's largest product.
//    The exact mode (ACC == 1) decodes each fragment's codes to bf16 (every
//    E4M3 / E5M2 value is a bf16 value) and issues four K = 16 bf16
//    instructions instead, whose 8-bit-significand products are exact and
//    whose sums show no such truncation: the exact-product fp32 accumulation
//    of the numeric contract, at half the matrix-core rate.
//  * 256x256 block tiles run 4 waves in a 2x2 grid, each wave a 128x128
//    tile (4x4 MFMA tiles, 256 accumulator registers: LDS traffic per MFMA
//    at its lowest).  256x192 tiles run 8 waves in a 4x2 grid of 64x96 wave
//    tiles, two waves per SIMD, so one wave's LDS and barrier waits overlap
//    the other's MFMAs; so do the 256x256 tiles of NT FP8 products with a
//    plain or relu^2-max epilogue (64x128 wave tiles), the only ones whose
//    main loop fits the 256 registers of two waves per SIMD.  Small outputs, which 256-row tiles would spread
//    over too few CUs, take 128x128 tiles: 4 waves of 64x64, two blocks per
//    CU.
//  * K is consumed 128 codes per stage; stages are double-buffered in LDS,
//    loaded with 16-byte buffer loads into registers one stage ahead.
//    K-major tiles are 128-byte rows; the 16-byte chunk c of row r is stored
//    at c ^ ((r>>1)&7) so that the ds_read_b128 fragment reads of sixteen
//    consecutive rows hit distinct banks.  MN-major tiles are 128 rows of the
//    tile's width plus 32 bytes, so the rows' starts step through the 8
//    32-byte bank groups; fragments come from ds_read_b64_tr_b8, whose
//    16-lane groups return, to lane i, byte i&7 of the eight rows addressed
//    by lanes (i>>3) + 2b: pairs of lanes address one reduction row at
//    output offsets 0 and 8, and every lane receives 8 consecutive reduction
//    values of its own output index, the K-major fragment order.
//  * Buffer-descriptor range checks return zeros for rows past M/N and
//    chunks past K; a reduction length that is not a multiple of 16 has the
//    bytes past it cleared in the last stage (K-major operands) or ends at a
//    row past the descriptor's range (MN-major operands).
//  * The MFMA is issued with the B fragment first, so each lane holds four
//    consecutive output columns of one row: the epilogue packs them to bf16,
//    stages the tile in LDS and writes 16-byte row chunks to HBM.
//  * Workgroups are dispatched round-robin over the 8 XCDs; tile ids are
//    remapped so each XCD works on a contiguous run of tiles, grouped 1024
//    output rows deep, so concurrently running tiles share operands in that
//    XCD's L2.
//  * Epilogues (enum Epilogue in internal.h): plain bf16 store; the relu^2
//    block's relu^2-max and relu^2-backward fusions, whose tile maxima are
//    taken on fp32 values before the (monotone) bf16 rounding, the backward
//    one with H prefetched into the stage registers during the main loop's
//    last two iterations; fp32 store and accumulate, and
//    accumulate-then-round-to-bf16 for the last of several summed products;
//    two reduction segments with their own operands and scales, the first
//    segment's sum rescaled at the boundary, for a sum of two products (NN,
//    TN); up to three TN products with a shared reduction in one grouped
//    launch, so that their tiles fill the CUs together; the gated block's
//    merged gate/up projection with the gate applied, and its grad-input
//    with the gate's derivative applied (dG and dU leave the kernel, dA is
//    never stored); and, for bf16 operands, alpha/beta with an optional
//    transposed store and the upper-triangle split-K mode.
#pragma once
#include <type_traits>

#include "device_common.h"
#include "internal.h"
#include "swiglu_math.h"

namespace fp8mlp {
namespace gemm_detail {

constexpr int kBK = 128;  // reduction elements (FP8 codes, bytes) per stage
constexpr int kGroupM = 4;

// LDS placement of the 16-byte chunk c of K-major tile row r: c ^ swz(r).
// gfx950 serves a 128-bit LDS access 16 lanes at a time across 64 four-byte
// banks, i.e. 256 bytes; 128-byte rows put rows r and r+1 in opposite bank
// halves, so the XOR key only has to differ between the 8 row pairs of any
// 16 consecutive rows.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// ds_read_b64_tr_b8 on an LDS byte address.
__device__ __forceinline__ v2i lds_read_tr8(const uint8_t* p) {
  typedef __attribute__((address_space(3))) v2i lds_v2i;
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)((lds_u8*)p));
}

// Four FP8 codes (one dword) to four bf16 values (two dwords), exactly:
// every E4M3 and E5M2 value, subnormals included, is an fp32 value whose low
// 16 bits are zero, so its upper half is the bf16 encoding.
template <int F>
__device__ __forceinline__ v2u fp8x4_to_bf16x4(int w) {
  v2f lo, hi;
  if constexpr (F == kE4M3) {
    lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  } else {
    lo = __builtin_amdgcn_cvt_pk_f32_bf8(w, false);
    hi = __builtin_amdgcn_cvt_pk_f32_bf8(w, true);
  }
  return v2u{__builtin_amdgcn_perm(__float_as_uint(lo[1]), __float_as_uint(lo[0]), 0x07060302u),
             __builtin_amdgcn_perm(__float_as_uint(hi[1]), __float_as_uint(hi[0]), 0x07060302u)};
}

// Zero the bytes at positions >= nb (0 < nb < 16) of a 16-byte chunk.
__device__ __forceinline__ v4u keep_low_bytes(v4u x, int nb) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int v = nb - 4 * i;  // bytes of dword i to keep
    x[i] = v >= 4 ? x[i] : (v <= 0 ? 0u : (x[i] & ((1u << (8 * v)) - 1u)));
  }
  return x;
}

// WGM x WGN waves per block (64 * WGM * WGN threads), each owning a
// (BM/WGM) x (BN/WGN) sub-tile.  LAY: bit 0 = A MN-major, bit 1 = B MN-major.
template <int FA, int FB, int BM, int BN, int WGM, int WGN, int EPI, int LAY, int ACC>
struct Gemm {
  static constexpr bool AMN = (LAY & 1) != 0, BMN = (LAY & 2) != 0;
  static constexpr int THREADS = 64 * WGM * WGN;
  static constexpr int WM = BM / WGM, WN = BN / WGN;  // wave tile
  static constexpr int FM = WM / 32, FN = WN / 32;
  static_assert(FM * 32 == WM && FN * 32 == WN, "wave tile must be whole 32x32 MFMA tiles");
  // LDS row strides: a K-major tile is BM (BN) rows of kBK bytes, an
  // MN-major tile kBK rows of BM (BN) bytes plus 32 bytes
  static constexpr int A_LD = AMN ? BM + 32 : kBK, B_LD = BMN ? BN + 32 : kBK;
  static constexpr int A_BYTES = AMN ? kBK * A_LD : BM * kBK, B_BYTES = BMN ? kBK * B_LD : BN * kBK;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_LOADS = BM * kBK / (THREADS * 16);  // per thread per stage
  static constexpr int B_LOADS = BN * kBK / (THREADS * 16);
  static_assert(A_LOADS * THREADS * 16 == BM * kBK && B_LOADS * THREADS * 16 == BN * kBK, "whole loads");
  static constexpr int LOADS = A_LOADS + B_LOADS;
  static constexpr int CLD = BN * 2 + 16;  // epilogue C tile row stride (bytes)
  // LDS: two stages, or the staged C tile plus the epilogue's reduction
  // slots (RED, past the C tile), whichever is larger
  static constexpr int LDS = (2 * STAGE > BM * CLD + 64) ? 2 * STAGE : BM * CLD + 64;
  static constexpr int RED = LDS - 64;
  static_assert(LDS <= 160 * 1024 - 64, "LDS budget");
};

template <int FA, int FB, int BM, int BN, int WGM, int WGN, int EPI, int LAY, int ACC>
__global__ void __launch_bounds__(64 * WGM * WGN, BM == 128 ? 2 : 1) gemm_kernel(GemmArgs g, int tiles_m, int tiles_n) {
  using G = Gemm<FA, FB, BM, BN, WGM, WGN, EPI, LAY, ACC>;
  constexpr int kThreads = G::THREADS;
  constexpr bool AMN = G::AMN, BMN = G::BMN;
  __shared__ __attribute__((aligned(16))) uint8_t smem[G::LDS];
  uint32_t* red = reinterpret_cast<uint32_t*>(smem + G::RED);  // epilogue reductions only

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid % WGM, wn = wid / WGM;

  // ---- tile id: XCD-contiguous runs, grouped 1024 output rows deep
  const int nt = gridDim.x;  // tiles, or work items of the upper-triangle mode
  const int bid = blockIdx.x;
  const int xcd = bid & 7, idx = bid >> 3, per = nt >> 3, rem = nt & 7;
  const int t = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  // kEpiStoreGroup: this tile's problem replaces the operands, scales,
  // output and shape (selected with constant indices, so the arguments stay
  // in scalar registers), and its tile id and grid are the problem's own
  int tt = t, tms = tiles_m, tns = tiles_n;
  if constexpr (EPI == kEpiStoreGroup) {
    static_assert(LAY == 3 && FA != kBF16, "grouped products: TN FP8 only");
    const int p = (g.ngroup > 2 && t >= g.grp_first[2]) ? 2 : ((g.ngroup > 1 && t >= g.grp_first[1]) ? 1 : 0);
    auto take = [&](const GemmProblem& q) {
      g.a = q.a; g.b = q.b; g.sa = q.sa; g.sb = q.sb; g.c = q.c;
      g.lda = q.lda; g.ldb = q.ldb; g.ldc = q.ldc; g.M = q.M; g.N = q.N;
    };
    if (p == 2) take(g.grp[2]);
    else if (p == 1) take(g.grp[1]);
    else take(g.grp[0]);
    tt = t - (p == 2 ? g.grp_first[2] : (p == 1 ? g.grp_first[1] : 0));
    tms = (int)((g.M + BM - 1) / BM);
    tns = (int)((g.N + BN - 1) / BN);
  }
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
    constexpr int kGM = kGroupM * 256 / BM;  // tile rows per group: 1024 output rows
    const int in_group = kGM * tns;
    const int first_m = (tt / in_group) * kGM;
    const int gm = min(kGM, tms - first_m);
    tm = first_m + (tt % in_group) % gm;
    tn = (tt % in_group) / gm;
  }
  // kEpiSwiGLU: a tile's BN B rows are BN/2 rows of the gate weights and the
  // same BN/2 rows of the up weights, so it covers BN/2 output columns
  constexpr bool kSwiGLU = EPI == kEpiSwiGLU;
  static_assert(!kSwiGLU || LAY == 0, "the merged gate/up projection is an NT product");
  constexpr int BNO = kSwiGLU ? BN / 2 : BN;  // output columns per tile
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BNO;

  // operand bytes per element (K, lda and ldb below are in bytes)
  constexpr int ES = FA == kBF16 ? 2 : 1;
  static_assert((FA == kBF16) == (FB == kBF16), "bf16 operands come in pairs");
  static_assert(FA != kBF16 || (LAY == 0 && ACC == 0), "bf16 operands: NT products only");
  // kEpiStore2: two segments of K/2 (a multiple of kBK), each with its own
  // operands; descriptors span one segment
  constexpr bool kSeg2 = EPI == kEpiStore2;
  // (the last stage of each segment needs no byte patch: the caller keeps
  // both operands' descriptor ends dword-aligned)
  static_assert(!kSeg2 || ((LAY == 2 || LAY == 3) && FA != kBF16), "two-segment products: NN or TN FP8 only");
  if constexpr (kSeg2) kelems = g.K / 2;
  const int K = (int)kelems * ES;
  const int nseg1 = kSeg2 ? K / kBK : 0;  // stages of the first segment
  const int64_t lda = g.lda * ES, ldb = g.ldb * ES;
  const int rows_a = (int)min<int64_t>(BM, g.M - m0);
  const int rows_b = (int)min<int64_t>(BNO, g.N - n0);
  // Descriptors: K-major operands start at (row m0, k kbeg) and span their
  // rows of K bytes; MN-major ones start at (row kbeg, column m0) and span K
  // rows up to the tile's last column.
  auto rsrc_of = [&](const uint8_t* p, int64_t ld, int64_t mn0, int rows, bool mn_major) {
    if (mn_major)
      return make_rsrc(p + kbeg * ld + mn0, kelems > 0 ? (uint32_t)((kelems - 1) * ld + rows) : 0u);
    return make_rsrc(p + mn0 * ld + kbeg * ES, (uint32_t)((rows - 1) * ld + K));
  };
  const __amdgpu_buffer_rsrc_t ra = rsrc_of(g.a, lda, m0, rows_a, AMN);
  const __amdgpu_buffer_rsrc_t rb = rsrc_of(g.b, ldb, n0, rows_b, BMN);
  const __amdgpu_buffer_rsrc_t rb2 = kSwiGLU ? rsrc_of(g.b2, ldb, n0, rows_b, false) : rb;
  const __amdgpu_buffer_rsrc_t ra_2 = kSeg2 ? rsrc_of(g.a_2, lda, m0, rows_a, AMN) : ra;
  const __amdgpu_buffer_rsrc_t rb_2 = kSeg2 ? rsrc_of(g.b_2, ldb, n0, rows_b, BMN) : rb;

  // K-major loads.  Per-thread 16-byte chunks each stage: chunk id =
  // tid + THREADS*j, row = id / 8, logical column chunk = id % 8 (eight lanes
  // cover one 128-byte row, so a wave load is 8 full rows).  In LDS the chunk
  // goes to position logical ^ swz(row) of its row.  Load j's row is
  // row0 + j*(THREADS/8); THREADS/16 is a multiple of 8, so swz() and the
  // column are the same for every j and the offsets are linear in j.
  constexpr int kRowStep = kThreads / 8;
  static_assert((kRowStep / 2) % 8 == 0, "swizzle must repeat every load step");
  const int row0 = tid >> 3, logical0 = tid & 7;
  const int colk0 = logical0 * 16;
  const uint32_t goff_a = (uint32_t)(row0 * lda) + colk0, goff_b = (uint32_t)(row0 * ldb) + colk0;
  const uint32_t gstep_a = (uint32_t)(kRowStep * lda), gstep_b = (uint32_t)(kRowStep * ldb);
  const uint32_t lds0 = row0 * kBK + ((logical0 ^ swz(row0)) << 4);
  // The last stage of a reduction that is not a multiple of 16 holds one
  // chunk per row that ends past K: its bytes from K on are cleared.
  const int tail_keep = K - ((K - 1) / kBK) * kBK - colk0;  // bytes of this lane's last-stage chunk
  const bool tail_clip = (K & 15) != 0 && tail_keep > 0 && tail_keep < 16;

  // MN-major loads: a tile of width W (BM or BN) has W/16 chunks per
  // reduction row; chunk id = tid + THREADS*j is row id / (W/16), column
  // chunk id % (W/16).  Chunks whose first column is past the operand's
  // extent load as zeros (a chunk that straddles it reads bytes that only
  // reach outputs past the extent, which are never stored).
  auto mn_pos = [&](int jj, int width, int& krow, int& c) {
    const int cpr = width / 16;
    const int id = tid + kThreads * jj;
    krow = id / cpr;
    c = id % cpr;
  };
  const uint32_t kstep_a = (uint32_t)(kBK * lda), kstep_b = (uint32_t)(kBK * ldb);
  const int nk = (K + kBK - 1) / kBK * (kSeg2 ? 2 : 1);

  // The chunk that holds the last byte of an operand's descriptor range E
  // (the end of the last row it reads): when E is not a multiple of 4 the
  // buffer unit returns zero for the whole dword that straddles E, so that
  // dword's 1-3 valid bytes are fetched with byte loads when the last stage
  // is written.  end_j: which of this thread's loads holds it (-1: none);
  // end_off: its offset in the last stage; end_e: E.
  int end_ja = -1, end_jb = -1;
  uint32_t end_off_a = 0, end_off_b = 0, end_e_a = 0, end_e_b = 0;
  if (FA != kBF16 && nk > 0) {
    auto find_end = [&](bool mn_major, int width, int rows, int64_t ld, int nloads, int& end_j, uint32_t& end_off,
                        uint32_t& end_e) {
      if (mn_major) {
        end_e = (uint32_t)((kelems - 1) * ld + rows);
        if ((end_e & 3u) == 0) return;
        const int krow = (int)((kelems - 1) & (kBK - 1)), c = (rows - 1) >> 4;
        const int id = krow * (width / 16) + c;
        if (id >= tid && (id - tid) % kThreads == 0 && (id - tid) / kThreads < nloads) {
          end_j = (id - tid) / kThreads;
          end_off = (uint32_t)((kelems - 1) * ld) + c * 16;
        }
      } else {
        end_e = (uint32_t)((rows - 1) * ld + K);
        if ((end_e & 3u) == 0) return;
        const int r = rows - 1, l = ((K - 1) & (kBK - 1)) >> 4;
        if (l == logical0 && r >= row0 && (r - row0) % kRowStep == 0 && (r - row0) / kRowStep < nloads) {
          end_j = (r - row0) / kRowStep;
          end_off = (uint32_t)(r * ld) + (nk - 1) * kBK + l * 16;
        }
      }
    };
    find_end(AMN, BM, rows_a, lda, G::A_LOADS, end_ja, end_off_a, end_e_a);
    if (!kSwiGLU) find_end(BMN, BN, rows_b, ldb, G::B_LOADS, end_jb, end_off_b, end_e_b);
    if (end_jb >= 0) end_jb += G::A_LOADS;
  }
  auto patch_end = [&](v4u v, const __amdgpu_buffer_rsrc_t& rs, uint32_t off, uint32_t e) {
    const uint32_t p0 = e & ~3u;
    const int dw = (int)(p0 - off) >> 2;
    uint32_t w = 0;
    for (uint32_t p = p0; p < e; ++p)
      w |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, p, 0, 0) << (8 * (p - p0));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i == dw) v[i] = w;
    return v;
  };

  v4u stg[G::LOADS];  // one stage in flight in registers
  // kEpiSwiGLU: B loads jj < B_LOADS/2 fill the gate half of the stage, the
  // rest the up half, from the same rows of the other operand
  static_assert(!kSwiGLU || (G::B_LOADS % 2 == 0 && (G::B_LOADS / 2) * kRowStep == BN / 2),
                "each B load must lie in one half");
  auto gload_one = [&](int j, int ktg) {
    // stage ktg of the reduction; with two segments, stage kt of segment s
    const bool s2 = kSeg2 && ktg >= nseg1;
    const int kt = s2 ? ktg - nseg1 : ktg;
    const __amdgpu_buffer_rsrc_t& rsa = s2 ? ra_2 : ra;
    const __amdgpu_buffer_rsrc_t& rsb = s2 ? rb_2 : rb;
    const int k0 = kt * kBK;
    const bool is_a = j < G::A_LOADS;
    const int jb = j - G::A_LOADS;
    if ((is_a && AMN) || (!is_a && BMN)) {
      const int jj = is_a ? j : jb;
      int krow, c;
      mn_pos(jj, is_a ? BM : BN, krow, c);
      const bool inside = (is_a ? m0 : n0) + c * 16 < (is_a ? g.M : g.N);
      const uint32_t off = inside ? (uint32_t)(krow * (is_a ? lda : ldb)) + c * 16 + kt * (is_a ? kstep_a : kstep_b)
                                  : 0x80000000u;
      stg[j] = __builtin_amdgcn_raw_buffer_load_b128(is_a ? rsa : rsb, off, 0, 0);
    } else {
      const bool up = kSwiGLU && !is_a && jb >= G::B_LOADS / 2;
      const int jj = is_a ? j : (up ? jb - G::B_LOADS / 2 : jb);
      const uint32_t base = is_a ? goff_a + jj * gstep_a : goff_b + jj * gstep_b;
      const uint32_t off = (k0 + colk0 < K) ? base + k0 : 0x80000000u;  // out of range -> 0
      stg[j] = __builtin_amdgcn_raw_buffer_load_b128(is_a ? rsa : (up ? rb2 : rsb), off, 0, 0);
    }
  };
  // last: the stage written is the last one of the reduction
  auto swrite_one = [&](int j, int buf, bool last) {
    const bool is_a = j < G::A_LOADS;
    const int jj = is_a ? j : j - G::A_LOADS;
    uint8_t* base = smem + buf * G::STAGE + (is_a ? 0 : G::A_BYTES);
    if (last && (j == end_ja || j == end_jb))
      stg[j] = is_a ? patch_end(stg[j], ra, end_off_a, end_e_a) : patch_end(stg[j], rb, end_off_b, end_e_b);
    if ((is_a && AMN) || (!is_a && BMN)) {
      int krow, c;
      mn_pos(jj, is_a ? BM : BN, krow, c);
      *reinterpret_cast<v4u*>(base + krow * (is_a ? G::A_LD : G::B_LD) + c * 16) = stg[j];
    } else {
      v4u v = stg[j];
      if (last && tail_clip) v = keep_low_bytes(v, tail_keep);
      *reinterpret_cast<v4u*>(base + lds0 + jj * kRowStep * kBK) = v;
    }
  };

  v16f acc[G::FM][G::FN];
#pragma unroll
  for (int i = 0; i < G::FM; ++i)
#pragma unroll
    for (int j = 0; j < G::FN; ++j) acc[i][j] = v16f{};

  // Epilogue chunks: each thread owns NCH 16-byte chunks of the output tile,
  // chunk id tid + THREADS*it being row id / CPR, 8-column group id % CPR.
  constexpr int CPR = BN / 8;  // 16-byte chunks per tile row
  constexpr int NCH = BM * CPR / kThreads;
  static_assert(NCH * kThreads == BM * CPR, "whole epilogue chunks");
  const bool vec_c = ((reinterpret_cast<uintptr_t>(g.c) & 15u) == 0) && (g.ldc % 8 == 0);
  constexpr bool kSgBwd = EPI == kEpiSwiGLUBwd;
  const bool vec_aux = (EPI != kEpiRelu2Bwd && !kSgBwd) ||
                       (((reinterpret_cast<uintptr_t>(g.aux) & 15u) == 0) && (g.ldaux % 8 == 0) &&
                        (!kSgBwd || (((reinterpret_cast<uintptr_t>(g.aux2) & 15u) == 0) &&
                                     ((reinterpret_cast<uintptr_t>(g.c2) & 15u) == 0))));
  // chunk `it` of a bf16 [M, N] input with leading dimension ldaux; zeros
  // past N and for rows past M
  auto load_chunk = [&](const uint16_t* src, int it) {
    const int id = tid + kThreads * it;
    const int64_t gr = m0 + id / CPR, gc = n0 + (id % CPR) * 8;
    v4u v = v4u{0u, 0u, 0u, 0u};
    if (gr < g.M && gc < g.N) {
      if (gc + 8 <= g.N && vec_c && vec_aux) {
        v = *reinterpret_cast<const v4u*>(src + gr * g.ldaux + gc);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = gc + 2 * e < g.N ? src[gr * g.ldaux + gc + 2 * e] : 0u;
          const uint32_t hi = gc + 2 * e + 1 < g.N ? src[gr * g.ldaux + gc + 2 * e + 1] : 0u;
          v[e] = lo | (hi << 16);
        }
      }
    }
    return v;
  };
  // The relu^2-backward epilogue reads H at its chunks.  H is prefetched in
  // the last two iterations of the main loop, where every CU would otherwise
  // wait for it at once after the loop.  Chunk t < kPf1 is loaded as soon as
  // the stage register it reuses has been written to LDS (the second-to-last
  // iteration issues no global loads); with two waves per SIMD the next kPf2
  // chunks are loaded during the last iteration.  Only for tiles whose every
  // chunk takes the vector path; the other chunks are loaded after the loop.
  // (The gated backward's G and U, prefetched the same way, measured slower
  // than loading them chunk by chunk in the epilogue.)
  constexpr bool kPfH = EPI == kEpiRelu2Bwd;
  v4u hv[kPfH ? NCH : 1];
  constexpr int kPf1 = NCH < G::LOADS ? NCH : G::LOADS;
  constexpr int kPf2Max = kThreads == 512 ? 5 : 0;  // register budget of the last iteration
  constexpr int kPf2 = NCH - kPf1 < kPf2Max ? NCH - kPf1 : kPf2Max;
  const bool pf_h = kPfH && m0 + BM <= g.M && n0 + BN <= g.N && vec_c && vec_aux;
  auto h_vec = [&](int it) {
    const int id = tid + kThreads * it;
    return *reinterpret_cast<const v4u*>(g.aux + (m0 + id / CPR) * g.ldaux + n0 + (id % CPR) * 8);
  };

  // Fragments: lane reads output index (lane & 31) of a 32-wide block, the
  // 32 reduction values starting at ks*64 + (lane >> 5)*32, in two 16-byte
  // halves: one ds_read_b128 each from a K-major tile, two transposing
  // ds_read_b64_tr_b8 each from an MN-major one.  Read r of a fragment set
  // (r < NR) is half r&1 of fragment r>>1 (A fragments first, then B).
  constexpr int NM = G::FM * G::FN;        // MFMAs per 64-element K substep
  constexpr int NR = 2 * (G::FM + G::FN);  // 16-byte fragment halves per substep
  const int frow = lane & 31, fhalf = lane >> 5;
  // MN-major fragment reads: lanes 2i and 2i+1 of a 16-lane group address
  // reduction row i of the group's 8 at output offsets 0 and 8 of its 16
  const int tr_k = fhalf * 32 + ((lane & 15) >> 1);
  const int tr_mn = ((lane >> 4) & 1) * 16 + (lane & 1) * 8;
  typedef v4i Frag[G::FM + G::FN][2];
  auto read_one = [&](int r, int buf, int ks, Frag& f) {
    const int fi = r >> 1, h = r & 1;
    const bool is_a = fi < G::FM;
    const uint8_t* base = smem + buf * G::STAGE + (is_a ? 0 : G::A_BYTES);
    const int fb = is_a ? wm * G::WM + fi * 32 : wn * G::WN + (fi - G::FM) * 32;
    if ((is_a && AMN) || (!is_a && BMN)) {
      const int ld = is_a ? G::A_LD : G::B_LD;
      const uint8_t* p = base + (ks * 64 + 16 * h + tr_k) * ld + fb + tr_mn;
      const v2i lo = lds_read_tr8(p), hi = lds_read_tr8(p + 8 * ld);
      f[fi][h] = v4i{lo[0], lo[1], hi[0], hi[1]};
    } else {
      const int row = fb + frow;
      const int c = ks * 4 + fhalf * 2 + h;
      f[fi][h] = *reinterpret_cast<const v4i*>(base + row * kBK + ((c ^ swz(row)) << 4));
    }
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
    } else if constexpr (ACC == 1) {
      // exact products: instruction q takes codes 8q..8q+7 of both fragments,
      // decoded to bf16, so every k is multiplied once with its partner
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v2u a0 = fp8x4_to_bf16x4<FA>(a[q >> 1][2 * (q & 1)]);
        const v2u a1 = fp8x4_to_bf16x4<FA>(a[q >> 1][2 * (q & 1) + 1]);
        const v2u b0 = fp8x4_to_bf16x4<FB>(b[q >> 1][2 * (q & 1)]);
        const v2u b1 = fp8x4_to_bf16x4<FB>(b[q >> 1][2 * (q & 1) + 1]);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(v8bf, v4u{b0[0], b0[1], b1[0], b1[1]}),
            __builtin_bit_cast(v8bf, v4u{a0[0], a0[1], a1[0], a1[1]}), acc[i][j], 0, 0, 0);
      }
    } else {
      const v8i av = v8i{a[0][0], a[0][1], a[0][2], a[0][3], a[1][0], a[1][1], a[1][2], a[1][3]};
      const v8i bv = v8i{b[0][0], b[0][1], b[0][2], b[0][3], b[1][0], b[1][1], b[1][2], b[1][3]};
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv, av, acc[i][j], FB, FA, 0, 0, 0, 0);
    }
  };

  // Software pipeline over 128-element K stages, two LDS buffers, one stage
  // in registers.  Iteration kt (stage kt in LDS buffer kt&1, its first-half
  // fragments F0 already in registers):
  //   A: MFMAs on F0; step t also issues read t of the second-half fragments
  //      F1, LDS write t of stage kt+1 (registers -> other buffer) and global
  //      load t of stage kt+2 into the register just written out;
  //   B: MFMAs on F1; the barrier that publishes stage kt+1 sits before the
  //      last kTail MFMAs, which hide the reads of stage kt+1's F0.
  // sched_barrier fences keep this order through instruction scheduling.
  constexpr int kTail = 4;
  constexpr int STEPS_A = NM > NR ? (NM > G::LOADS ? NM : G::LOADS) : (NR > G::LOADS ? NR : G::LOADS);
  static_assert(kPf2 <= STEPS_A, "the last iteration issues one H prefetch per step");
  Frag f0, f1;

#pragma unroll
  for (int j = 0; j < G::LOADS; ++j) gload_one(j, 0);
#pragma unroll
  for (int j = 0; j < G::LOADS; ++j) swrite_one(j, 0, nk == 1);
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
          swrite_one(t, nxt, !HN2);  // stage kt+1 is the last one when kt+2 does not exist
          if constexpr (HN2) gload_one(t, kt + 2);
          if constexpr (kPfH && !HN2) {
            if (t < kPf1 && pf_h) hv[t] = h_vec(t);
          }
        }
      }
      if constexpr (kPfH && !HN && kPf2 > 0) {
        if (t < kPf2 && pf_h) hv[kPf1 + t] = h_vec(kPf1 + t);
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
  // kEpiStore2: at the first stage of the second segment the accumulators
  // hold the first segment's sum; scaled by RN32(p1 / p2) they continue as
  // if its products carried the second segment's scale
  auto boundary = [&](int kt) {
    if constexpr (kSeg2) {
      if (kt == nseg1) {
        const float p1 = (*g.sa) * (*g.sb), p2 = (*g.sa_2) * (*g.sb_2);
        const float r = p1 / p2;
#pragma unroll
        for (int i = 0; i < G::FM; ++i)
#pragma unroll
          for (int j = 0; j < G::FN; ++j) acc[i][j] *= r;
      }
    }
  };
  int kt = 0;
  for (; kt + 2 < nk; ++kt) { boundary(kt); iteration(kt, T{}, T{}); }
  if (kt + 1 < nk) { boundary(kt); iteration(kt, T{}, F{}); ++kt; }
  boundary(kt);
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
  // H chunks the main loop did not prefetch are loaded here: with two waves
  // per SIMD (THREADS = 512) before the tile is staged in LDS, so that they
  // are in flight while it is; the 4-wave layout has no registers to spare
  // next to its 256 accumulators and loads them after staging.
  constexpr bool kEarlyH = kPfH && kThreads == 512;
  auto load_h = [&]() {
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
      const bool pre = pf_h && (it < kPf1 ? nk >= 2 : it < kPf1 + kPf2);
      if (!pre) hv[it] = load_chunk(g.aux, it);
    }
  };
  if constexpr (kEarlyH) load_h();

  // scale, round to bf16 and stage the tile in LDS
  static_assert(!kSwiGLU || G::WN * 2 == BN, "kEpiSwiGLU: one wave column per half");
  float p;
  if constexpr (FA == kBF16) p = g.alpha;
  else if constexpr (kSwiGLU) p = (*g.sa) * (wn == 0 ? *g.sb : *g.sb2);  // gate or up half
  else if constexpr (kSeg2) p = (*g.sa_2) * (*g.sb_2);  // the second segment's scale
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
  if constexpr (kPfH && !kEarlyH) load_h();

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

  // One 16-byte chunk of bf16 outputs at (gr, gc) of an [M, N] output with
  // leading dimension ldc: one vector store when the chunk is whole and
  // aligned, the widest stores its alignment allows when it is whole but not
  // 16-byte aligned (an odd or unaligned leading dimension), else elements.
  auto store_chunk = [&](uint16_t* base, int64_t gr, int64_t gc, const v4u& v, bool full) {
    uint16_t* dst = base + gr * g.ldc + gc;
    if (full) {
      *reinterpret_cast<v4u*>(dst) = v;
    } else if (gc + 8 <= g.N) {
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
        if (gc + e < g.N) dst[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
    }
  };

  // epilogue max, as the partial's format wants it: relu^2-max the fp32 bit
  // pattern of a non-negative bf16 value, relu^2-backward and the gated
  // backward the bf16 magnitude bits.  The relu^2-backward max |dH| is taken
  // before rounding, max |RN_bf16(y)| = RN_bf16(max |y|); chunk elements past
  // N hold y = 0.  The gated backward's inputs past N load as zeros, so its
  // outputs there are +-0 and their magnitude bits 0.
  uint32_t mx = 0, mx2 = 0;
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
      if constexpr (kSgBwd) {
        // dA (staged bf16) with G and U at the same chunk
        const v4u gv = load_chunk(g.aux, it), uv = load_chunk(g.aux2, it);
        v4u dgv, duv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t wg = 0, wu = 0;
#pragma unroll
          for (int hlf = 0; hlf < 2; ++hlf) {
            const int sh = 16 * hlf;
            uint32_t bg, bu;
            swiglu_bwd_bits(bf16_to_f32((gv[e] >> sh) & 0xFFFFu), bf16_to_f32((uv[e] >> sh) & 0xFFFFu),
                            bf16_to_f32((v[e] >> sh) & 0xFFFFu), bg, bu);
            mx = mx > (bg & 0x7FFFu) ? mx : (bg & 0x7FFFu);
            mx2 = mx2 > (bu & 0x7FFFu) ? mx2 : (bu & 0x7FFFu);
            wg |= bg << sh;
            wu |= bu << sh;
          }
          dgv[e] = wg;
          duv[e] = wu;
        }
        store_chunk(g.c, gr, gc, dgv, full);
        store_chunk(g.c2, gr, gc, duv, full);
      } else {
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
        store_chunk(g.c, gr, gc, v, full);
      }
    }
  }
  if constexpr (EPI == kEpiRelu2Bwd) {
    const __bf16 db = (__bf16)dmax;
    mx = (uint32_t)__builtin_bit_cast(unsigned short, db) & 0x7FFFu;
  }
  if constexpr (EPI == kEpiRelu2Max || EPI == kEpiRelu2Bwd || kSgBwd) {
    mx = block_max_u32(mx, red);
    if (tid == 0) g.partials[t] = mx;
  }
  if constexpr (kSgBwd) {
    mx2 = block_max_u32(mx2, red);
    if (tid == 0) g.partials2[t] = mx2;
  }
}

template <int FA, int FB, int BM, int BN, int WGM, int WGN, int EPI, int LAY, int ACC>
hipError_t launch_cfg(const GemmArgs& g, hipStream_t st) {
  constexpr int BNO = EPI == kEpiSwiGLU ? BN / 2 : BN;  // output columns per tile
  const int tiles_m = (int)((g.M + BM - 1) / BM), tiles_n = (int)((g.N + BNO - 1) / BNO);
  if (tiles_m == 0 || tiles_n == 0) return hipSuccess;  // empty output
  const int work = g.tri_tiles > 0 ? g.tri_tiles * (g.tri_tiles + 1) / 2 * g.ksplit : tiles_m * tiles_n;
  hipLaunchKernelGGL((gemm_kernel<FA, FB, BM, BN, WGM, WGN, EPI, LAY, ACC>), dim3(work), dim3(64 * WGM * WGN), 0,
                     st, g, tiles_m, tiles_n);
  return hipGetLastError();
}

// A grouped launch: the problems' tiles one after another, grp_first set
// here; every problem reduces over the same K.
template <int FA, int FB, int BM, int BN, int WGM, int WGN, int LAY, int ACC>
hipError_t launch_group(const GemmArgs& g0, hipStream_t st) {
  GemmArgs g = g0;
  int total = 0;
  for (int p = 0; p < g.ngroup; ++p) {
    g.grp_first[p] = total;
    total += (int)(((g.grp[p].M + BM - 1) / BM) * ((g.grp[p].N + BN - 1) / BN));
  }
  g.grp_first[g.ngroup] = total;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<FA, FB, BM, BN, WGM, WGN, kEpiStoreGroup, LAY, ACC>), dim3(total),
                     dim3(64 * WGM * WGN), 0, st, g, 0, 0);
  return hipGetLastError();
}

// Block tile width: 256x192 tiles when they fill the 256 CUs in whole waves
// better than 256x256 (e.g. an 8192x3072 output is 384 tiles of 256x256 =
// 1.5 waves, but 512 tiles of 256x192 = 2 waves).
inline int pick_bn(int64_t M, int64_t N) {
  auto eff = [&](int bn) {
    const int64_t t = ((M + 255) / 256) * ((N + bn - 1) / bn);
    const int64_t waves = (t + 255) / 256;
    return (double)(M * N) / (double)(waves * 256 * 256 * bn);
  };
  return eff(192) > eff(256) * 1.02 ? 192 : 256;
}

// Block tile of an FP8 product with an M x N output: 128 for 128x128 tiles,
// else the width of a 256-row tile (pick_bn).  128x128 tiles (a third more
// LDS reads per MFMA, two blocks per CU) are taken when 256-row tiles would
// leave a quarter of the 256 CUs or more without a tile, e.g. a 1024 x 3072
// grad-weight (64 tiles of 256x192, 192 of 128x128).
inline int pick_tile(int64_t M, int64_t N) {
  const int bn = pick_bn(M, N);
  const int64_t t = ((M + 255) / 256) * ((N + bn - 1) / bn);
  return t < 192 ? 128 : bn;
}

// FP8 products of one layout and accumulation mode.  Epilogues beyond the
// plain store exist for the format pairs and layouts that use them: the
// relu^2 block's forward (E4M3 x E4M3, NT) and backward (E5M2 x E4M3, NT or
// NN), the gated block's projection (E4M3 x E4M3, NT) and backward (E5M2 x
// E4M3, NN), and the summed gradient products (E5M2 x E4M3): fp32 store and
// accumulate epilogues, and two-segment sums (NN, TN).
template <int LAY, int ACC, int FA, int FB, int BM, int BN, int WGM, int WGN>
hipError_t launch_bn(const GemmArgs& g, hipStream_t st) {
  switch (g.epi) {
    case kEpiStore: return launch_cfg<FA, FB, BM, BN, WGM, WGN, kEpiStore, LAY, ACC>(g, st);
    case kEpiRelu2Max:
      if constexpr (LAY == 0 && FA == kE4M3 && FB == kE4M3)
        return launch_cfg<FA, FB, BM, BN, WGM, WGN, kEpiRelu2Max, LAY, ACC>(g, st);
      break;
    case kEpiRelu2Bwd:
      if constexpr (LAY != 3 && FA == kE5M2 && FB == kE4M3)
        return launch_cfg<FA, FB, BM, BN, WGM, WGN, kEpiRelu2Bwd, LAY, ACC>(g, st);
      break;
    case kEpiSwiGLU:
      if constexpr (LAY == 0 && FA == kE4M3 && FB == kE4M3 && BM == 256 && BN == 256)
        return launch_cfg<FA, FB, 256, 256, 2, 2, kEpiSwiGLU, LAY, ACC>(g, st);
      break;
    case kEpiStore2:  // not on 4-wave 256x256 tiles, whose registers hold no second descriptor set
      if constexpr ((LAY == 2 || LAY == 3) && FA == kE5M2 && FB == kE4M3 && !(BM == 256 && BN == 256))
        return launch_cfg<FA, FB, BM, BN, WGM, WGN, kEpiStore2, LAY, ACC>(g, st);
      break;
    case kEpiSwiGLUBwd:
      if constexpr (LAY == 2 && FA == kE5M2 && FB == kE4M3)
        return launch_cfg<FA, FB, BM, BN, WGM, WGN, kEpiSwiGLUBwd, LAY, ACC>(g, st);
      break;
    case kEpiStoreGroup:
      if constexpr (LAY == 3 && FA == kE5M2 && FB == kE4M3 && BM == 256)
        return launch_group<FA, FB, BM, BN, WGM, WGN, LAY, ACC>(g, st);
      break;
    case kEpiStoreF32:
    case kEpiAccF32:
    case kEpiAccF32Bf16:
      if constexpr (FA == kE5M2 && FB == kE4M3) {
        if (g.epi == kEpiStoreF32) return launch_cfg<FA, FB, BM, BN, WGM, WGN, kEpiStoreF32, LAY, ACC>(g, st);
        if (g.epi == kEpiAccF32) return launch_cfg<FA, FB, BM, BN, WGM, WGN, kEpiAccF32, LAY, ACC>(g, st);
        return launch_cfg<FA, FB, BM, BN, WGM, WGN, kEpiAccF32Bf16, LAY, ACC>(g, st);
      }
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <int LAY, int ACC, int FA, int FB>
hipError_t launch_fmt(const GemmArgs& g, hipStream_t st) {
  // 256x192 tiles run 8 waves (4x2, 64x96 wave tiles, two waves per SIMD);
  // 256x256 tiles 4 waves (2x2, 128x128 wave tiles), except the NT FP8
  // plain-store and relu^2-max products, which run 8 waves (4x2, 64x128 wave
  // tiles: their main loop fits 256 registers with both operands K-major;
  // with an MN-major operand, exact products or the other epilogues it
  // spills); 128x128 tiles 4 waves (2x2, 64x64 wave tiles), two blocks per CU
  if (g.epi == kEpiSwiGLU) return launch_bn<LAY, ACC, FA, FB, 256, 256, 2, 2>(g, st);
  if (g.epi == kEpiStoreGroup) {
    // the tile width that fills whole waves best over all the problems' tiles
    auto eff = [&](int bn) {
      int64_t t = 0, work = 0;
      for (int p = 0; p < g.ngroup; ++p) {
        t += ((g.grp[p].M + 255) / 256) * ((g.grp[p].N + bn - 1) / bn);
        work += g.grp[p].M * g.grp[p].N;
      }
      const int64_t waves = (t + 255) / 256;
      return waves > 0 ? (double)work / (double)(waves * 256 * 256 * bn) : 1.0;
    };
    if (eff(192) > eff(256) * 1.02) return launch_bn<LAY, ACC, FA, FB, 256, 192, 4, 2>(g, st);
    return launch_bn<LAY, ACC, FA, FB, 256, 256, 2, 2>(g, st);
  }
  switch (pick_tile(g.M, g.N)) {
    case 128: return launch_bn<LAY, ACC, FA, FB, 128, 128, 2, 2>(g, st);
    case 192: return launch_bn<LAY, ACC, FA, FB, 256, 192, 4, 2>(g, st);
    default:
      if (g.epi == kEpiStore2) return launch_bn<LAY, ACC, FA, FB, 256, 192, 4, 2>(g, st);
      if constexpr (LAY == 0 && ACC == 0 && FA != kBF16) {
        if (g.epi == kEpiStore) return launch_cfg<FA, FB, 256, 256, 4, 2, kEpiStore, LAY, ACC>(g, st);
        if constexpr (FA == kE4M3 && FB == kE4M3) {
          if (g.epi == kEpiRelu2Max) return launch_cfg<FA, FB, 256, 256, 4, 2, kEpiRelu2Max, LAY, ACC>(g, st);
        }
      }
      return launch_bn<LAY, ACC, FA, FB, 256, 256, 2, 2>(g, st);
  }
}

template <int LAY, int ACC>
hipError_t launch_layout(const GemmArgs& g, hipStream_t st) {
  if (g.fa == kE4M3 && g.fb == kE4M3) return launch_fmt<LAY, ACC, kE4M3, kE4M3>(g, st);
  if (g.fa == kE5M2 && g.fb == kE4M3) return launch_fmt<LAY, ACC, kE5M2, kE4M3>(g, st);
  if (g.fa == kE4M3 && g.fb == kE5M2) return launch_fmt<LAY, ACC, kE4M3, kE5M2>(g, st);
  if (g.fa == kE5M2 && g.fb == kE5M2) return launch_fmt<LAY, ACC, kE5M2, kE5M2>(g, st);
  return hipErrorInvalidValue;
}

}  // namespace gemm_detail
}  // namespace fp8mlp
