// GEMM dispatch: the bf16 products (NT, Newton-Schulz), the FP8 products of
// the three layouts (each instantiated in its own translation unit from
// gemm_kernel.h) and the tile arithmetic the callers size workspaces with.
#include "gemm_kernel.h"

namespace fp8mlp {

namespace {

using gemm_detail::launch_cfg;

// bf16 products: the alpha/beta epilogue on 8-wave 256x192 tiles (the 4-wave
// alpha/beta epilogue would spill), or fp32 256x256 tiles of the
// upper-triangle split-K mode
hipError_t launch_bf16(const GemmArgs& g, hipStream_t st) {
  if (g.tri_tiles > 0) {
    if (g.epi != kEpiStoreF32) return hipErrorInvalidValue;
    return launch_cfg<kBF16, kBF16, 256, 256, 2, 2, kEpiStoreF32, kLayNT, kAccFast>(g, st);
  }
  if (g.epi == kEpiAxpby) return launch_cfg<kBF16, kBF16, 256, 192, 4, 2, kEpiAxpby, kLayNT, kAccFast>(g, st);
  if (g.epi == kEpiStoreF32) return launch_cfg<kBF16, kBF16, 256, 192, 4, 2, kEpiStoreF32, kLayNT, kAccFast>(g, st);
  return hipErrorInvalidValue;
}

}  // namespace

int64_t gemm_num_tiles(int64_t M, int64_t N) {
  const int tile = gemm_detail::pick_tile(M, N);
  const int bm = tile == 128 ? 128 : 256, bn = tile;
  return ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
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

// Two-segment sums: each segment a whole number of 128-deep stages, and the
// descriptor ranges of both operands ending on dword boundaries (the kernel
// patches the bytes of a straddling dword only at the last stage of the
// whole reduction).  MN-major operands end at their last row's M (N)
// extent, K-major ones at their rows' K/2.
bool seg2_ok(const GemmArgs& g) {
  if (g.K % 256 != 0 || g.lda % 4 != 0 || g.ldb % 4 != 0) return false;
  const bool amn = g.layout == kLayTN, bmn = g.layout == kLayNN || g.layout == kLayTN;
  return (!amn || g.M % 4 == 0) && (!bmn || g.N % 4 == 0) && g.a_2 && g.b_2 && g.sa_2 && g.sb_2;
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
  if (g.epi == kEpiStore2 && (!seg2_ok(g) || (g.layout != kLayNN && g.layout != kLayTN))) return hipErrorInvalidValue;
  if (g.epi == kEpiStoreGroup) {  // one to three TN problems over the same K, E5M2 x E4M3
    if (g.layout != kLayTN || g.ngroup < 1 || g.ngroup > 3 || g.fa != kE5M2 || g.fb != kE4M3) return hipErrorInvalidValue;
    for (int p = 0; p < g.ngroup; ++p) {
      const GemmProblem& q = g.grp[p];
      if (q.M < 0 || q.N < 0 || !q.sa || !q.sb || (q.M > 0 && q.N > 0 && (!q.c || q.ldc < q.N))) return hipErrorInvalidValue;
    }
  }
  if (g.fa == kBF16 || g.fb == kBF16) {
    if (g.fa != g.fb || g.layout != kLayNT) return hipErrorInvalidValue;
    return launch_bf16(g, st);
  }
  const bool exact = g.accum == kAccExact;
  switch (g.layout) {
    case kLayNT: return exact ? launch_gemm_nt_exact(g, st) : launch_gemm_nt_fast(g, st);
    case kLayNN: return exact ? launch_gemm_nn_exact(g, st) : launch_gemm_nn_fast(g, st);
    case kLayTN: return exact ? launch_gemm_tn_exact(g, st) : launch_gemm_tn_fast(g, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fp8mlp
