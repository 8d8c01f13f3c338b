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
// cast kernel for every job of the batch.
hipError_t launch_cast(QuantBatch& b, hipStream_t st);

// GEMM epilogues.
enum Epilogue : int {
  kEpiStore = 0,      // C = RN_bf16(p * acc)
  kEpiRelu2Max = 1,   // C = H = RN_bf16(p * acc); partial[tile] = max over tile of max(H, 0)
  kEpiRelu2Bwd = 2,   // dA = RN_bf16(p * acc); C = dH = RN_bf16(2 relu(aux) dA);
                      // partial[tile] = max |dH| (bf16 bits)
};

struct GemmArgs {
  const uint8_t* a;  // [M, K] codes, K contiguous
  const uint8_t* b;  // [N, K] codes, K contiguous
  int64_t lda, ldb;
  int fa, fb;
  const float* sa;
  const float* sb;
  int64_t M, N, K;
  uint16_t* c;  // [M, N] bf16
  int64_t ldc;
  int epi;
  const uint16_t* aux;  // H for kEpiRelu2Bwd ([M, N], ldaux)
  int64_t ldaux;
  uint32_t* partials;  // one per tile for the max epilogues
};

// Number of output tiles the GEMM will use (size of `partials`).
int64_t gemm_num_tiles(int64_t M, int64_t N);
int64_t gemm_max_tiles(int64_t M, int64_t N);  // upper bound over tile configurations
hipError_t launch_gemm(const GemmArgs& g, hipStream_t st);

}  // namespace fp8mlp
