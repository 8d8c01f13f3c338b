// Host-side interfaces between the C-ABI layer and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8mlp {

// How the cast kernel obtains the values it quantises and its amax.
enum CastMode : int {
  kModePlain = 0,  // values = x (bf16); partials = per-block max of |x| as bf16 bits
  kModeRelu2 = 1,  // values = RN_bf16(relu(x)^2) with x = H; partials = per-tile
                   // max of max(H, 0) as fp32 bits (written by the up-GEMM epilogue)
  kModeRmsNorm = 2,  // values = RN_bf16(RN32(RN32(x r_row) g_col)): RMSNorm with the
                     // per-row r written by rmsnorm_amax; partials as plain
};

struct QuantJob {
  const uint16_t* x;
  int64_t rows, cols, ldx;
  uint8_t* q;   // [rows, cols] codes or nullptr
  int64_t ldq;
  uint8_t* qt;  // [cols, rows] codes or nullptr
  int64_t ldqt;
  float* scale;     // out
  float* amax_out;  // out or nullptr
  uint32_t* partials;
  int nparts;
  int fmt;
  int mode;
  int blk_begin;  // first block of this job inside a batched launch
  int nblocks;    // blocks given to this job
  const float* rstd;      // kModeRmsNorm: per-row 1/rms (written by rmsnorm_amax)
  const uint16_t* gamma;  // kModeRmsNorm: per-column weight (bf16) or nullptr
};

constexpr int kMaxJobs = 4;
struct QuantBatch {
  QuantJob job[kMaxJobs];
  int njobs;
};

// Number of amax partials used for a tensor of `n` elements.
int amax_parts_for(int64_t rows, int64_t cols);

// amax partial kernel for every job of the batch (mode plain only).
hipError_t launch_amax_partials(QuantBatch& b, hipStream_t st);
// amax and cast of every job of the batch (mode plain): one pass over the
// data (a one-block clear, then one grid that holds part of the tensors in
// registers across a grid-wide wait) when every job is dense, 16-byte
// aligned and codes-only and the batch gives at least 256 work units, else
// launch_amax_partials then launch_cast.  Uses
// at most each job's nparts partials.
hipError_t launch_amax_cast(QuantBatch& b, hipStream_t st);
// RMSNorm statistics, amax and cast of one job (mode kModeRmsNorm): one pass
// (a one-block clear, then a grid that holds 16 rows per block in registers
// across a grid-wide wait) for dense rows of at most 3072 columns with codes
// only and at least 256 units of 16 rows, else launch_rmsnorm_amax then
// launch_cast.  Uses at most the job's
// nparts partials.
hipError_t launch_rmsnorm_quant(QuantBatch& b, float eps, float* rstd, hipStream_t st);
// RMSNorm statistics and amax partials of one job (mode kModeRmsNorm): writes
// rstd[row] and one partial per block of rows (rmsnorm_parts_for of them).
int rmsnorm_parts_for(int64_t rows);
hipError_t launch_rmsnorm_amax(QuantJob& j, float eps, float* rstd, hipStream_t st);
// cast kernel for every job of the batch.
hipError_t launch_cast(QuantBatch& b, hipStream_t st);

// GEMM operand format beside E4M3 (0) and E5M2 (1): bf16, for both operands.
constexpr int kBF16 = 2;

// GEMM epilogues.
enum Epilogue : int {
  kEpiStore = 0,      // C = RN_bf16(p * acc)
  kEpiRelu2Max = 1,   // C = H = RN_bf16(p * acc); partial[tile] = max over tile of max(H, 0)
  kEpiRelu2Bwd = 2,   // dA = RN_bf16(p * acc); C = dH = RN_bf16(2 relu(aux) dA);
                      // partial[tile] = max |dH| (bf16 bits)
  kEpiStoreF32 = 3,   // Cf = RN32(p * acc)              (fp32 output, cf)
  kEpiAccF32 = 4,     // Cf = RN32(Cf + RN32(p * acc))   (fp32 accumulation, cf)
  kEpiAxpby = 5,      // C = RN_bf16(fma(alpha, acc, RN32(beta * aux))), aux optional,
                      // optionally also C^T into ct   (bf16 operands only)
  kEpiAccF32Bf16 = 7, // C = RN_bf16(RN32(Cf + RN32(p * acc)))  (reads cf, writes bf16 c;
                      // the last of several fp32-accumulated products, ldc for both)
  kEpiSwiGLU = 6,     // merged gate/up projection of the gated MLP: a tile covers
                      // BN/2 output columns n; its first half multiplies B rows
                      // of b (gate), its second half the same rows of b2 (up).
                      // G = RN_bf16(RN32(sa sb) acc) -> c, U = RN_bf16(RN32(sa sb2)
                      // acc) -> c2, A = RN_bf16(silu(G) U) -> c3 (all ldc);
                      // partial[tile] = max |A| (bf16 bits) when partials is set
  kEpiStore2 = 9,     // two reduction segments (a, b then a_2, b_2, each K/2 long):
                      // C = RN_bf16(p2 (acc_2 + RN32(p1 / p2) acc_1)),
                      // p1 = RN32(sa sb), p2 = RN32(sa_2 sb_2)  (NN or TN; K/2 a
                      // multiple of 128 and dword-aligned operand ends)
  kEpiStoreGroup = 10,  // plain bf16 store of up to three TN products in one launch
                        // (grp[0..ngroup), each with its own operands, scales, output
                        // and shape; the reduction length K shared): the launch's tile
                        // t belongs to the problem p with grp_first[p] <= t < grp_first[p+1]
  kEpiSwiGLUBwd = 8,  // gated MLP backward: dA = RN_bf16(p * acc) (not stored), with G
                      // (aux) and U (aux2): dG = RN_bf16(dA U silu'(G)) -> c,
                      // dU = RN_bf16(dA silu(G)) -> c2 (ldc); partial[tile] =
                      // max |dG|, partials2[tile] = max |dU| (bf16 bits)
};

// GEMM operand layouts: bit 0 set = A is MN-major ([K, M], the output index
// contiguous), bit 1 set = B is MN-major ([K, N]); otherwise K-major.
enum GemmLayout : int {
  kLayNT = 0,  // A [M, K], B [N, K]: forward
  kLayNN = 2,  // A [M, K], B [K, N]: grad-input
  kLayTN = 3,  // A [K, M], B [K, N]: grad-weight
};

// Accumulation of FP8 products (the FP8MLP_ACCUM_* values of the C ABI).
enum GemmAccum : int {
  kAccFast = 0,   // FP8 matrix cores (group-truncated sums)
  kAccExact = 1,  // codes decoded to bf16, exact products on the bf16 matrix cores
};

// One problem of a grouped launch (kEpiStoreGroup).
struct GemmProblem {
  const uint8_t* a;
  const uint8_t* b;
  const float* sa;
  const float* sb;
  uint16_t* c;
  int64_t lda, ldb, ldc, M, N;
};

struct GemmArgs {
  const uint8_t* a;  // [M, K] (K-major) or [K, M] (MN-major) codes, or bf16 values [M, K]
  const uint8_t* b;  // [N, K] (K-major) or [K, N] (MN-major) codes, or bf16 values [N, K]
  int64_t lda, ldb;
  int layout;  // GemmLayout (bf16 operands: NT only)
  int accum;   // GemmAccum (FP8 operands)
  int fa, fb;
  const float* sa;
  const float* sb;
  int64_t M, N, K;
  uint16_t* c;  // [M, N] bf16
  int64_t ldc;
  int epi;
  const uint16_t* aux;  // H for kEpiRelu2Bwd, G for kEpiSwiGLUBwd ([M, N], ldaux)
  const uint16_t* aux2;  // U for kEpiSwiGLUBwd ([M, N], ldaux)
  int64_t ldaux;
  uint32_t* partials;   // one per tile for the max epilogues
  uint32_t* partials2;  // kEpiSwiGLUBwd: the second output's, one per tile
  float* cf;           // [M, N] fp32 (ldc) for the fp32 epilogues
  // bf16 operands (fa == fb == kBF16): a, b hold bf16 values, lda, ldb and K
  // count elements, and the output scale is alpha instead of sa * sb.
  float alpha, beta;
  uint16_t* ct;  // kEpiAxpby: optional transposed copy of C ([N, M], ldct)
  int64_t ldct;
  // kEpiSwiGLU: the up projection's codes [N, K] (ldb) and scale, and the U
  // and A outputs ([M, N], ldc); kEpiSwiGLUBwd: the dU output in c2
  const uint8_t* b2;
  const float* sb2;
  uint16_t* c2;
  uint16_t* c3;
  // kEpiStore2: the second segment's operands (same leading dimensions) and
  // scales
  const uint8_t* a_2;
  const uint8_t* b_2;
  const float* sa_2;
  const float* sb_2;
  // Upper-triangle split-K mode (M == N, A and B the same matrix's rows):
  // tri_tiles > 0 is the number of 256-wide tile rows; work item w covers
  // triangle tile w / ksplit (tile row <= tile column) and the K range
  // [(w % ksplit) * kchunk, +kchunk); its fp32 result goes to
  // cf + (w % ksplit) * split_stride with the kEpiStoreF32 epilogue.
  int tri_tiles, ksplit;
  int64_t kchunk, split_stride;
  // kEpiStoreGroup: the problems and their first tiles (set by the launcher)
  int ngroup;
  int grp_first[4];
  GemmProblem grp[3];
};

// Number of output tiles the GEMM will use (size of `partials`).
int64_t gemm_num_tiles(int64_t M, int64_t N);
// FP8 products of one layout and accumulation mode (one translation unit each).
hipError_t launch_gemm_nt_fast(const GemmArgs& g, hipStream_t st);
hipError_t launch_gemm_nt_exact(const GemmArgs& g, hipStream_t st);
hipError_t launch_gemm_nn_fast(const GemmArgs& g, hipStream_t st);
hipError_t launch_gemm_nn_exact(const GemmArgs& g, hipStream_t st);
hipError_t launch_gemm_tn_fast(const GemmArgs& g, hipStream_t st);
hipError_t launch_gemm_tn_exact(const GemmArgs& g, hipStream_t st);
int64_t gemm_swiglu_tiles(int64_t M, int64_t N);  // kEpiSwiGLU with N output columns
int64_t gemm_max_tiles(int64_t M, int64_t N);  // upper bound over tile configurations
hipError_t launch_gemm(const GemmArgs& g, hipStream_t st);

// LM head fused with the softcapped cross-entropy (lm_head_ce.hip).
// n_valid = number of targets in [0, n_classes).
hipError_t launch_count_valid(const int32_t* targets, int64_t M, int64_t n_classes, int32_t* n_valid,
                              hipStream_t st);
// Rows [0, rows) of a chunk: logits Z (bf16, [rows, V], ld ldz) become dZ in
// place; loss_rows[r] and partials[r] (max |dZ| as bf16 bits) are written.
hipError_t launch_softcap_ce(uint16_t* z, int64_t rows, int64_t V, int64_t ldz, int64_t n_classes,
                             float softcap, const int32_t* targets, const int32_t* n_valid,
                             float* loss_rows, uint32_t* partials, hipStream_t st);
int64_t lm_ce_max_vocab();  // largest vocabulary the row kernel takes
// loss = sum(loss_rows) / n_valid (0 if none).
hipError_t launch_lm_ce_loss(const float* loss_rows, int64_t M, const int32_t* n_valid, float* loss,
                             hipStream_t st);

// dst = RN_bf16(src) over n elements (n % 8 == 0); src == nullptr writes zeros.
hipError_t launch_f32_to_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t st);

// Newton-Schulz orthogonalisation helpers (muon.hip).
int ns_parts_for(int64_t n);
// x = RN_bf16(g / RN32(RN32(||g||_F) + eps)) over n elements (n % 8 == 0);
// partials: ns_parts_for(n) doubles; norm_out (may be NULL): n and the divisor.
hipError_t launch_ns_normalise(const uint16_t* g, int64_t n, float eps, double* partials, uint16_t* x,
                               float* norm_out, hipStream_t st);
// dst [cols, rows] = src [rows, cols]^T, both dense; rows, cols % 8 == 0.
hipError_t launch_transpose_bf16(const uint16_t* src, int64_t rows, int64_t cols, uint16_t* dst, hipStream_t st);

// Symmetric product C = RN_bf16(fma(alpha, A A^T, RN32(beta aux))) (aux
// symmetric or NULL) through the upper-triangle split-K GEMM and a reduction
// that writes both halves from the upper one (gemm.hip + muon.hip).
int sym_ksplit(int64_t M, int64_t K);
size_t sym_partials_bytes(int64_t M, int64_t K);
hipError_t launch_sym_gemm(const uint16_t* a, int64_t lda, int64_t M, int64_t K, float alpha, float beta,
                           const uint16_t* aux, int64_t ldaux, uint16_t* c, int64_t ldc, float* partials,
                           hipStream_t st);
hipError_t launch_sym_reduce(const float* parts, int nsplit, int64_t split_stride, int64_t M, float alpha,
                             float beta, const uint16_t* aux, int64_t ldaux, uint16_t* c, int64_t ldc,
                             hipStream_t st);

}  // namespace fp8mlp
