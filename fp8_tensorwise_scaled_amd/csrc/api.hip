// C ABI of the FP8 tensorwise-scaled linear layer and relu^2 MLP block
// (declarations and the numeric contract: include/fp8mlp.h).
//
// Every entry point validates its arguments on the host before enqueuing
// anything, never allocates, never synchronises, and launches only on the
// caller's stream.
#include <mutex>

#include "../../include/fp8mlp.h"
#include "internal.h"

using namespace fp8mlp;

namespace {

// Scratch memory of fp8_amax_quant_noalloc: the per-block amax partials
// (amax_parts_for() never exceeds 1024) in a file-scope device array, one
// copy per GPU, held until the process ends.  Host code uses the array only
// through the device address hipGetSymbolAddress returns for each GPU.
constexpr int kNoAllocScratchWords = 1024;
static __device__ __align__(256) uint32_t scratch[kNoAllocScratchWords];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
uint32_t* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device with
// that device current.
int scratch_of_current_device(uint32_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FP8MLP_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return FP8MLP_ENOTSUP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FP8MLP_EHIP;
    g_scratch_ptr[dev] = static_cast<uint32_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return FP8MLP_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool a2(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 1u) == 0; }
bool fmt_ok(int f) { return f == FP8MLP_E4M3 || f == FP8MLP_E5M2; }

int hip_status(hipError_t e) { return e == hipSuccess ? FP8MLP_OK : FP8MLP_EHIP; }

bool accum_ok(int a) { return a == FP8MLP_ACCUM_FAST || a == FP8MLP_ACCUM_EXACT; }

// GEMM operand tiles are addressed with 32-bit buffer offsets: a K-major
// operand from the first of a tile's 256 rows to the end of its last row, an
// MN-major one over every reduction row (plus one stage of 128 rows read
// past the end as zeros).
constexpr int64_t kTileRows = 256;
bool tile_range_ok(int64_t ld, int64_t K) { return (kTileRows - 1) * ld + K < (int64_t(1) << 31); }
bool mn_range_ok(int64_t ld, int64_t K) { return (K + 128) * ld + kTileRows < (int64_t(1) << 31); }

// FP8 GEMM C[M,N] = op(A) op(B) in `layout` (kLayNT / kLayNN / kLayTN): a
// K-major operand has rows of K codes (ld >= K), an MN-major one K rows of
// M (N) codes (ld >= M (N)).
int check_gemm(int layout, const uint8_t* a, int64_t lda, int fa, const float* sa, const uint8_t* b,
               int64_t ldb, int fb, const float* sb, int64_t M, int64_t N, int64_t K, const uint16_t* c,
               int64_t ldc, int accum) {
  if (!sa || !sb) return FP8MLP_EINVAL;
  if (M < 0 || N < 0 || K < 0) return FP8MLP_EINVAL;
  if (!fmt_ok(fa) || !fmt_ok(fb) || !accum_ok(accum)) return FP8MLP_EINVAL;
  if (M == 0 || N == 0) return FP8MLP_OK;  // empty output: nothing read or written
  if (!c || ldc < N) return FP8MLP_EINVAL;
  if (!a2(c)) return FP8MLP_EALIGN;
  if (K == 0) return FP8MLP_OK;  // empty sums: C = 0, the operands are not read
  const bool amn = (layout & 1) != 0, bmn = (layout & 2) != 0;
  if (!a || !b || lda < (amn ? M : K) || ldb < (bmn ? N : K)) return FP8MLP_EINVAL;
  if (!a16(a) || !a16(b) || lda % 16 || ldb % 16) return FP8MLP_EALIGN;
  if (!(amn ? mn_range_ok(lda, K) : tile_range_ok(lda, K)) || !(bmn ? mn_range_ok(ldb, K) : tile_range_ok(ldb, K)))
    return FP8MLP_ENOTSUP;
  if (M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return FP8MLP_ENOTSUP;
  return FP8MLP_OK;
}

int run_gemm(int layout, const uint8_t* a, int64_t lda, int fa, const float* sa, const uint8_t* b, int64_t ldb,
             int fb, const float* sb, int64_t M, int64_t N, int64_t K, uint16_t* c, int64_t ldc, int accum,
             void* stream) {
  int st = check_gemm(layout, a, lda, fa, sa, b, ldb, fb, sb, M, N, K, c, ldc, accum);
  if (st) return st;
  if (M == 0 || N == 0) return FP8MLP_OK;  // empty output; K == 0 writes zeros
  GemmArgs g{};
  g.a = a; g.b = b; g.lda = lda; g.ldb = ldb; g.fa = fa; g.fb = fb; g.sa = sa; g.sb = sb;
  g.layout = layout; g.accum = accum;
  if (K == 0) { g.lda = g.ldb = 0; g.layout = kLayNT; }  // operand descriptors cover no bytes
  g.M = M; g.N = N; g.K = K; g.c = c; g.ldc = ldc; g.epi = kEpiStore;
  return hip_status(launch_gemm(g, (hipStream_t)stream));
}

// ---- MLP workspace layouts (offsets in bytes from ws).  The forward's codes
// and H live in the caller's saved set; the workspaces hold what one pass
// needs for itself.
enum FwdSlot { F_PX, F_PU, F_PD, F_PH, F_COUNT };
enum BwdSlot { B_GQ, B_DH, B_HQ, B_PG, B_PDH, B_SC, B_COUNT };

size_t layout_fwd(int64_t M, int64_t d, int64_t h, size_t* off) {
  const size_t sz[F_COUNT] = {(size_t)amax_parts_for(M, d) * 4, (size_t)amax_parts_for(h, d) * 4,
                              (size_t)amax_parts_for(d, h) * 4, (size_t)gemm_max_tiles(M, h) * 4};
  size_t o = 0;
  for (int i = 0; i < F_COUNT; ++i) { off[i] = o; o = align_up(o + sz[i]); }
  return o;
}

size_t layout_bwd(int64_t M, int64_t d, int64_t h, size_t* off) {
  const size_t sz[B_COUNT] = {(size_t)(M * d), (size_t)(M * h) * 2, (size_t)(M * h),
                              (size_t)amax_parts_for(M, d) * 4, (size_t)gemm_max_tiles(M, h) * 4, 8};
  size_t o = 0;
  for (int i = 0; i < B_COUNT; ++i) { off[i] = o; o = align_up(o + sz[i]); }
  return o;
}

int check_mlp_dims(int64_t M, int64_t d, int64_t h) {
  if (M < 0 || d <= 0 || h <= 0) return FP8MLP_EINVAL;
  if (M % 16 || d % 16 || h % 16) return FP8MLP_ENOTSUP;
  if (!tile_range_ok(M, M) || !tile_range_ok(h, h) || !tile_range_ok(d, d)) return FP8MLP_ENOTSUP;
  if (M > INT32_MAX / 2 || d > INT32_MAX / 2 || h > INT32_MAX / 2) return FP8MLP_ENOTSUP;
  return FP8MLP_OK;
}

QuantJob make_job(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, uint8_t* q,
                  int64_t ldq, uint8_t* qt, int64_t ldqt, float* scale, float* amax,
                  uint32_t* partials, int nparts, int mode) {
  QuantJob j{};
  j.x = x; j.rows = rows; j.cols = cols; j.ldx = ldx; j.q = q; j.ldq = ldq; j.qt = qt;
  j.ldqt = ldqt; j.scale = scale; j.amax_out = amax; j.partials = partials; j.nparts = nparts;
  j.fmt = fmt; j.mode = mode;
  return j;
}

// ---- gated (SwiGLU) MLP workspaces (the forward's codes, G and U live in
// the caller's saved set)
enum SgFwdSlot { SF_A, SF_PX, SF_PWG, SF_PWU, SF_PWD, SF_PA, SF_COUNT };
enum SgBwdSlot { SB_GQ, SB_DG, SB_DU, SB_DGQ, SB_DUQ, SB_DXF, SB_PG, SB_PDG, SB_PDU, SB_SC, SB_COUNT };

size_t layout_sg_fwd(int64_t M, int64_t d, int64_t h, size_t* off) {
  const size_t sz[SF_COUNT] = {
      (size_t)(M * h) * 2, (size_t)amax_parts_for(M, d) * 4, (size_t)amax_parts_for(h, d) * 4,
      (size_t)amax_parts_for(h, d) * 4, (size_t)amax_parts_for(d, h) * 4, (size_t)gemm_swiglu_tiles(M, h) * 4};
  size_t o = 0;
  for (int i = 0; i < SF_COUNT; ++i) { off[i] = o; o = align_up(o + sz[i]); }
  return o;
}

size_t layout_sg_bwd(int64_t M, int64_t d, int64_t h, size_t* off) {
  const size_t mh = (size_t)(M * h);
  const size_t sz[SB_COUNT] = {
      (size_t)(M * d), mh * 2, mh * 2, mh, mh, (size_t)(M * d) * 4, (size_t)amax_parts_for(M, d) * 4,
      (size_t)gemm_num_tiles(M, h) * 4, (size_t)gemm_num_tiles(M, h) * 4, 16};
  size_t o = 0;
  for (int i = 0; i < SB_COUNT; ++i) { off[i] = o; o = align_up(o + sz[i]); }
  return o;
}

GemmArgs gemm_args(const uint8_t* a, int64_t lda, int fa, const float* sa, const uint8_t* b, int64_t ldb, int fb,
                   const float* sb, int64_t M, int64_t N, int64_t K, int epi) {
  GemmArgs g{};
  g.a = a; g.lda = lda; g.fa = fa; g.sa = sa; g.b = b; g.ldb = ldb; g.fb = fb; g.sb = sb;
  g.M = M; g.N = N; g.K = K; g.epi = epi;
  return g;
}

// ---- LM head + softcapped cross-entropy workspace
enum LmSlot { L_XQ, L_WQ, L_Z, L_DZQ, L_DWF, L_LOSS, L_PX, L_PW, L_PZ, L_NV, L_SC, L_COUNT };

int64_t pad16(int64_t v) { return (v + 15) / 16 * 16; }

size_t layout_lm_ce(int64_t M, int64_t K, int64_t V, int64_t C, size_t* off) {
  const int64_t Vp = pad16(V), nchunks = M > 0 ? (M + C - 1) / C : 0;
  const size_t sz[L_COUNT] = {
      (size_t)(M * K), (size_t)(V * K), (size_t)(C * Vp) * 2, (size_t)(C * Vp), (size_t)(V * K) * 4,
      (size_t)M * 4, (size_t)amax_parts_for(M, K) * 4, (size_t)amax_parts_for(V, K) * 4, (size_t)C * 4, 16,
      (size_t)(2 + nchunks) * 4};
  size_t o = 0;
  for (int i = 0; i < L_COUNT; ++i) { off[i] = o; o = align_up(o + sz[i]); }
  return o;
}

int check_lm_ce_dims(int64_t M, int64_t K, int64_t V, int64_t n_classes, int64_t C) {
  if (M < 0 || K <= 0 || V <= 0 || C <= 0 || n_classes <= 0 || n_classes > V) return FP8MLP_EINVAL;
  if (M % 16 || K % 16 || C % 16) return FP8MLP_ENOTSUP;
  if (V > lm_ce_max_vocab()) return FP8MLP_ENOTSUP;
  if (!tile_range_ok(K, K) || !tile_range_ok(M, M) || !tile_range_ok(pad16(V), pad16(V)) ||
      !tile_range_ok(C, C))
    return FP8MLP_ENOTSUP;
  return FP8MLP_OK;
}

// Argument checks shared by fp8_amax_quant and fp8_amax_quant_noalloc.
int check_amax_quant(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, const uint8_t* q,
                     int64_t ldq, const uint8_t* qt, int64_t ldqt, const float* scale) {
  if (!scale) return FP8MLP_EINVAL;
  if (rows < 0 || cols < 0 || ldx < cols || !fmt_ok(fmt)) return FP8MLP_EINVAL;
  if (rows > 0 && cols > 0) {  // an empty tensor only gets its scale (1) and amax (0)
    if (!x || (!q && !qt)) return FP8MLP_EINVAL;
    if ((q && ldq < cols) || (qt && ldqt < rows)) return FP8MLP_EINVAL;
    if ((q && (const void*)q == (const void*)x) || (qt && (const void*)qt == (const void*)x))
      return FP8MLP_EINVAL;
    if (!a2(x)) return FP8MLP_EALIGN;
  }
  return FP8MLP_OK;
}

// The amax pass and the cast of one tensor, with `partials` holding
// amax_parts_for(rows, cols) u32.
int run_amax_quant(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, uint8_t* q, int64_t ldq,
                   uint8_t* qt, int64_t ldqt, float* scale, float* amax, uint32_t* partials, void* stream,
                   bool two_launches = false) {
  QuantBatch b{};
  b.njobs = 1;
  b.job[0] = make_job(x, rows, cols, ldx, fmt, q, ldq, qt, ldqt, scale, amax, partials, amax_parts_for(rows, cols),
                      kModePlain);
  hipStream_t st = (hipStream_t)stream;
  if (!two_launches) return hip_status(launch_amax_cast(b, st));
  if (launch_amax_partials(b, st) != hipSuccess) return FP8MLP_EHIP;
  return hip_status(launch_cast(b, st));
}

}  // namespace

extern "C" {

int fp8mlp_abi_version(void) { return FP8MLP_ABI_VERSION; }

const char* fp8mlp_status_string(int status) {
  switch (status) {
    case FP8MLP_OK: return "ok";
    case FP8MLP_EINVAL: return "invalid argument (null pointer, negative size, ld < cols or unknown format)";
    case FP8MLP_EALIGN: return "misaligned pointer or leading dimension";
    case FP8MLP_EWORKSPACE: return "workspace missing or too small";
    case FP8MLP_EHIP: return "HIP launch failed";
    case FP8MLP_ENOTSUP: return "shape not supported (operand offsets beyond 2 GiB, or a size limit)";
    default: return "unknown status";
  }
}

size_t fp8_amax_quant_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return 0;
  return align_up((size_t)amax_parts_for(rows, cols) * 4);
}

int fp8_amax_quant(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, uint8_t* q,
                   int64_t ldq, uint8_t* qt, int64_t ldqt, float* scale, float* amax, void* ws,
                   size_t ws_bytes, void* stream) {
  int st = check_amax_quant(x, rows, cols, ldx, fmt, q, ldq, qt, ldqt, scale);
  if (st) return st;
  if (!ws || ws_bytes < fp8_amax_quant_workspace_bytes(rows, cols)) return FP8MLP_EWORKSPACE;
  if (!a16(ws)) return FP8MLP_EALIGN;
  return run_amax_quant(x, rows, cols, ldx, fmt, q, ldq, qt, ldqt, scale, amax, (uint32_t*)ws, stream);
}

int fp8_amax_quant_noalloc(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, uint8_t* q,
                           int64_t ldq, uint8_t* qt, int64_t ldqt, float* scale, float* amax, void* stream) {
  int st = check_amax_quant(x, rows, cols, ldx, fmt, q, ldq, qt, ldqt, scale);
  if (st) return st;
  if ((size_t)amax_parts_for(rows, cols) * 4 > sizeof(scratch)) return FP8MLP_ENOTSUP;
  uint32_t* parts = nullptr;
  st = scratch_of_current_device(&parts);
  if (st) return st;
  // every partial the cast reads is written by this call's amax pass first:
  // nothing in the scratch has to start at zero
  return run_amax_quant(x, rows, cols, ldx, fmt, q, ldq, qt, ldqt, scale, amax, parts, stream, true);
}

size_t fp8_rmsnorm_quant_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return 0;
  return align_up((size_t)rmsnorm_parts_for(rows) * 4);
}

int fp8_rmsnorm_quant(const uint16_t* x, const uint16_t* gamma, float eps, int64_t rows, int64_t cols,
                      int64_t ldx, int fmt, uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt, float* scale,
                      float* amax, float* rstd, void* ws, size_t ws_bytes, void* stream) {
  if (!scale) return FP8MLP_EINVAL;
  if (rows < 0 || cols < 0 || ldx < cols || !fmt_ok(fmt)) return FP8MLP_EINVAL;
  if (!(eps >= 0.0f) || !(eps < 1e30f)) return FP8MLP_EINVAL;
  if (rows > 0 && cols > 0) {
    if (!x || !rstd || (!q && !qt)) return FP8MLP_EINVAL;
    if ((q && ldq < cols) || (qt && ldqt < rows)) return FP8MLP_EINVAL;
    if ((q && (const void*)q == (const void*)x) || (qt && (const void*)qt == (const void*)x))
      return FP8MLP_EINVAL;
    if (!a2(x) || !a2(gamma) || ((uintptr_t)rstd & 3u)) return FP8MLP_EALIGN;
  }
  if (!ws || ws_bytes < fp8_rmsnorm_quant_workspace_bytes(rows, cols)) return FP8MLP_EWORKSPACE;
  if (!a16(ws)) return FP8MLP_EALIGN;
  QuantBatch b{};
  b.njobs = 1;
  b.job[0] = make_job(x, rows, cols, ldx, fmt, q, ldq, qt, ldqt, scale, amax, (uint32_t*)ws,
                      rmsnorm_parts_for(rows), kModeRmsNorm);
  b.job[0].rstd = rstd;
  b.job[0].gamma = gamma;
  hipStream_t st = (hipStream_t)stream;
  if (rows > 0 && cols > 0) return hip_status(launch_rmsnorm_quant(b, eps, rstd, st));
  {
    // no elements: amax 0, scale 1 (the partial the cast reads is written by
    // the plain amax pass over nothing)
    b.job[0].mode = kModePlain;
    b.job[0].nparts = amax_parts_for(rows, cols);
    if (launch_amax_partials(b, st) != hipSuccess) return FP8MLP_EHIP;
  }
  return hip_status(launch_cast(b, st));
}

int fp8_linear_fwd(const uint8_t* xq, int64_t ldx, int fx, const float* sx, const uint8_t* wq,
                   int64_t ldw, int fw, const float* sw, int64_t M, int64_t N, int64_t K, uint16_t* y,
                   int64_t ldy, int accum, void* stream) {
  // Y[M,N] = sum_k X[m,k] W[n,k]: NT
  return run_gemm(kLayNT, xq, ldx, fx, sx, wq, ldw, fw, sw, M, N, K, y, ldy, accum, stream);
}

size_t fp8_linear_fwd_bf16_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return 0;
  return align_up((size_t)amax_parts_for(M, K) * 4) + align_up((size_t)amax_parts_for(N, K) * 4);
}

int fp8_linear_fwd_bf16(const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw, int64_t M, int64_t N,
                        int64_t K, uint8_t* xq, int64_t ldxq, uint8_t* wq, int64_t ldwq, float* scales,
                        uint16_t* y, int64_t ldy, void* ws, size_t ws_bytes, int accum, void* stream) {
  if (!scales) return FP8MLP_EINVAL;
  if ((uintptr_t)scales & 3u) return FP8MLP_EALIGN;
  int st = check_amax_quant(x, M, K, ldx, FP8MLP_E4M3, xq, ldxq, nullptr, 0, &scales[0]);
  if (!st) st = check_amax_quant(w, N, K, ldw, FP8MLP_E4M3, wq, ldwq, nullptr, 0, &scales[1]);
  if (!st) st = check_gemm(kLayNT, xq, ldxq, FP8MLP_E4M3, &scales[0], wq, ldwq, FP8MLP_E4M3, &scales[1], M, N, K, y,
                           ldy, accum);
  if (st) return st;
  if (M > 0 && N > 0 && K > 0 && (const void*)xq == (const void*)wq) return FP8MLP_EINVAL;
  if (!ws || ws_bytes < fp8_linear_fwd_bf16_workspace_bytes(M, N, K)) return FP8MLP_EWORKSPACE;
  if (!a16(ws)) return FP8MLP_EALIGN;
  // 1. amax of X and W in one launch, 2. both casts in one launch, 3. Y = Xq . Wq^T (NT)
  uint32_t* px = (uint32_t*)ws;
  uint32_t* pw = (uint32_t*)((uint8_t*)ws + align_up((size_t)amax_parts_for(M, K) * 4));
  QuantBatch b{};
  b.njobs = 2;
  b.job[0] = make_job(x, M, K, ldx, FP8MLP_E4M3, xq, ldxq, nullptr, 0, &scales[0], nullptr, px, amax_parts_for(M, K),
                      kModePlain);
  b.job[1] = make_job(w, N, K, ldw, FP8MLP_E4M3, wq, ldwq, nullptr, 0, &scales[1], nullptr, pw, amax_parts_for(N, K),
                      kModePlain);
  hipStream_t s = (hipStream_t)stream;
  if (launch_amax_cast(b, s) != hipSuccess) return FP8MLP_EHIP;
  return run_gemm(kLayNT, xq, ldxq, FP8MLP_E4M3, &scales[0], wq, ldwq, FP8MLP_E4M3, &scales[1], M, N, K, y, ldy,
                  accum, stream);
}

int fp8_linear_dgrad(const uint8_t* dyq, int64_t lddy, int fdy, const float* sdy, const uint8_t* wq,
                     int64_t ldw, int fw, const float* sw, int64_t M, int64_t N, int64_t K,
                     uint16_t* dx, int64_t lddx, int accum, void* stream) {
  // dX[M,K] = sum_n dY[m,n] W[n,k]: NN with reduction length N
  return run_gemm(kLayNN, dyq, lddy, fdy, sdy, wq, ldw, fw, sw, M, K, N, dx, lddx, accum, stream);
}

int fp8_linear_wgrad(const uint8_t* dyq, int64_t lddy, int fdy, const float* sdy, const uint8_t* xq,
                     int64_t ldx, int fx, const float* sx, int64_t M, int64_t N, int64_t K,
                     uint16_t* dw, int64_t lddw, int accum, void* stream) {
  // dW[N,K] = sum_m dY[m,n] X[m,k]: TN with reduction length M
  return run_gemm(kLayTN, dyq, lddy, fdy, sdy, xq, ldx, fx, sx, N, K, M, dw, lddw, accum, stream);
}

int fp8_gated_linear_fwd(const uint8_t* xq, int64_t ldx, const float* sx, const uint8_t* wgq, const float* sg,
                         const uint8_t* wuq, const float* su, int64_t ldw, int64_t M, int64_t N, int64_t K,
                         uint16_t* g, uint16_t* u, uint16_t* a, int64_t ldo, int accum, void* stream) {
  int st = check_gemm(kLayNT, xq, ldx, FP8MLP_E4M3, sx, wgq, ldw, FP8MLP_E4M3, sg, M, N, K, g, ldo, accum);
  if (st) return st;
  if (!su) return FP8MLP_EINVAL;
  if (M == 0 || N == 0) return FP8MLP_OK;
  if (K % 16) return FP8MLP_ENOTSUP;  // the merged projection takes whole 16-byte chunks of both weights
  if (!u || !a) return FP8MLP_EINVAL;
  if (!a2(u) || !a2(a)) return FP8MLP_EALIGN;
  if (K > 0 && !wuq) return FP8MLP_EINVAL;
  if (K > 0 && !a16(wuq)) return FP8MLP_EALIGN;
  GemmArgs gs = gemm_args(xq, ldx, FP8MLP_E4M3, sx, wgq, ldw, FP8MLP_E4M3, sg, M, N, K, kEpiSwiGLU);
  gs.b2 = wuq; gs.sb2 = su; gs.c = g; gs.c2 = u; gs.c3 = a; gs.ldc = ldo; gs.accum = accum;
  if (K == 0) gs.lda = gs.ldb = 0;  // operand descriptors cover no bytes: G = U = A = 0
  return hip_status(launch_gemm(gs, (hipStream_t)stream));
}

size_t relu2_mlp_fwd_workspace_bytes(int64_t M, int64_t d, int64_t h) {
  if (check_mlp_dims(M, d, h)) return 0;
  size_t off[F_COUNT];
  return layout_fwd(M, d, h, off);
}

size_t relu2_mlp_bwd_workspace_bytes(int64_t M, int64_t d, int64_t h) {
  if (check_mlp_dims(M, d, h)) return 0;
  size_t off[B_COUNT];
  return layout_bwd(M, d, h, off);
}

int relu2_mlp_fwd_workspace_layout(int64_t M, int64_t d, int64_t h, size_t* offsets, int n) {
  if (check_mlp_dims(M, d, h) || !offsets || n < F_COUNT) return FP8MLP_EINVAL;
  layout_fwd(M, d, h, offsets);
  return FP8MLP_OK;
}

int relu2_mlp_bwd_workspace_layout(int64_t M, int64_t d, int64_t h, size_t* offsets, int n) {
  if (check_mlp_dims(M, d, h) || !offsets || n < B_COUNT) return FP8MLP_EINVAL;
  layout_bwd(M, d, h, offsets);
  return FP8MLP_OK;
}

int relu2_mlp_fwd(const uint16_t* x, const uint16_t* w_up, const uint16_t* w_down, int64_t M,
                  int64_t d, int64_t h, uint16_t* y, const relu2_mlp_saved* saved, void* ws,
                  size_t ws_bytes, int accum, void* stream) {
  if (!w_up || !w_down || !saved || !saved->uq || !saved->dq || !saved->scales) return FP8MLP_EINVAL;
  if (!accum_ok(accum)) return FP8MLP_EINVAL;
  int st = check_mlp_dims(M, d, h);
  if (st) return st;
  // buffers with M rows may be NULL when M == 0 (no tokens)
  if (M > 0 && (!x || !y || !saved->xq || !saved->aq || !saved->h)) return FP8MLP_EINVAL;
  const void* ptrs[] = {x, w_up, w_down, y, saved->xq, saved->uq, saved->dq, saved->aq, saved->h};
  for (const void* p : ptrs)
    if (!a16(p)) return FP8MLP_EALIGN;
  if (((uintptr_t)saved->scales & 3u) != 0) return FP8MLP_EALIGN;
  size_t off[F_COUNT];
  const size_t need = layout_fwd(M, d, h, off);
  if (!ws || ws_bytes < need) return FP8MLP_EWORKSPACE;
  if (!a16(ws)) return FP8MLP_EALIGN;

  uint8_t* w8 = (uint8_t*)ws;
  uint32_t* px = (uint32_t*)(w8 + off[F_PX]);
  uint32_t* pu = (uint32_t*)(w8 + off[F_PU]);
  uint32_t* pd = (uint32_t*)(w8 + off[F_PD]);
  uint32_t* ph = (uint32_t*)(w8 + off[F_PH]);
  float* sc = saved->scales;
  hipStream_t s = (hipStream_t)stream;

  // 1-2. quantise X, W_up, W_down (E4M3) in one amax launch and one cast launch
  QuantBatch b{};
  b.njobs = 3;
  b.job[0] = make_job(x, M, d, d, FP8MLP_E4M3, saved->xq, d, nullptr, 0, &sc[0], nullptr, px,
                      amax_parts_for(M, d), kModePlain);
  b.job[1] = make_job(w_up, h, d, d, FP8MLP_E4M3, saved->uq, d, nullptr, 0, &sc[1], nullptr, pu,
                      amax_parts_for(h, d), kModePlain);
  b.job[2] = make_job(w_down, d, h, h, FP8MLP_E4M3, saved->dq, h, nullptr, 0, &sc[2], nullptr, pd,
                      amax_parts_for(d, h), kModePlain);
  if (launch_amax_cast(b, s) != hipSuccess) return FP8MLP_EHIP;

  // 3. H = Xq . Uq^T (NT) with the relu^2 max epilogue
  GemmArgs g = gemm_args(saved->xq, d, FP8MLP_E4M3, &sc[0], saved->uq, d, FP8MLP_E4M3, &sc[1], M, h, d,
                         kEpiRelu2Max);
  g.c = saved->h; g.ldc = h; g.partials = ph; g.accum = accum;
  if (launch_gemm(g, s) != hipSuccess) return FP8MLP_EHIP;

  // 4. Aq = quant(RN_bf16(relu(H)^2)), amax from the epilogue's partials
  QuantBatch ba{};
  ba.njobs = 1;
  ba.job[0] = make_job(saved->h, M, h, h, FP8MLP_E4M3, saved->aq, h, nullptr, 0, &sc[3], nullptr, ph,
                       (int)gemm_num_tiles(M, h), kModeRelu2);
  if (launch_cast(ba, s) != hipSuccess) return FP8MLP_EHIP;

  // 5. Y = Aq . Dq^T (NT)
  GemmArgs g2 = gemm_args(saved->aq, h, FP8MLP_E4M3, &sc[3], saved->dq, h, FP8MLP_E4M3, &sc[2], M, d, h, kEpiStore);
  g2.c = y; g2.ldc = d; g2.accum = accum;
  return hip_status(launch_gemm(g2, s));
}

int relu2_mlp_bwd(const uint16_t* dy, const relu2_mlp_saved* saved, int64_t M, int64_t d, int64_t h,
                  uint16_t* dx, uint16_t* dw_up, uint16_t* dw_down, float* bwd_scales, void* ws,
                  size_t ws_bytes, int accum, void* stream) {
  if (!saved || !dw_up || !dw_down || !saved->uq || !saved->dq || !saved->scales) return FP8MLP_EINVAL;
  if (!accum_ok(accum)) return FP8MLP_EINVAL;
  int st = check_mlp_dims(M, d, h);
  if (st) return st;
  if (M > 0 && (!dy || !dx || !saved->xq || !saved->aq || !saved->h)) return FP8MLP_EINVAL;
  const void* ptrs[] = {dy, dx, dw_up, dw_down, saved->xq, saved->uq, saved->dq, saved->aq, saved->h};
  for (const void* p : ptrs)
    if (!a16(p)) return FP8MLP_EALIGN;
  if (((uintptr_t)saved->scales & 3u) != 0 || ((uintptr_t)bwd_scales & 3u) != 0) return FP8MLP_EALIGN;
  size_t off[B_COUNT];
  const size_t need = layout_bwd(M, d, h, off);
  if (!ws || ws_bytes < need) return FP8MLP_EWORKSPACE;
  if (!a16(ws)) return FP8MLP_EALIGN;

  uint8_t* w8 = (uint8_t*)ws;
  uint8_t *gq = w8 + off[B_GQ], *hq = w8 + off[B_HQ];
  uint16_t* dh = (uint16_t*)(w8 + off[B_DH]);
  uint32_t* pg = (uint32_t*)(w8 + off[B_PG]);
  uint32_t* pdh = (uint32_t*)(w8 + off[B_PDH]);
  float* bsc = bwd_scales ? bwd_scales : (float*)(w8 + off[B_SC]);
  const float* sc = saved->scales;
  hipStream_t s = (hipStream_t)stream;

  // 1. Gq = quant(dY) (E5M2)
  QuantBatch b{};
  b.njobs = 1;
  b.job[0] = make_job(dy, M, d, d, FP8MLP_E5M2, gq, d, nullptr, 0, &bsc[0], nullptr, pg, amax_parts_for(M, d),
                      kModePlain);
  if (launch_amax_cast(b, s) != hipSuccess) return FP8MLP_EHIP;

  // 2. dW_down[d,h] = Gq^T . Aq (TN, reduction over the M tokens)
  GemmArgs g = gemm_args(gq, d, FP8MLP_E5M2, &bsc[0], saved->aq, h, FP8MLP_E4M3, &sc[3], d, h, M, kEpiStore);
  g.layout = kLayTN; g.c = dw_down; g.ldc = h; g.accum = accum;
  if (launch_gemm(g, s) != hipSuccess) return FP8MLP_EHIP;

  // 3. dA = Gq . Dq (NN, reduction over d), fused dH = RN_bf16(2 relu(H) dA) and max |dH|
  GemmArgs g2 = gemm_args(gq, d, FP8MLP_E5M2, &bsc[0], saved->dq, h, FP8MLP_E4M3, &sc[2], M, h, d, kEpiRelu2Bwd);
  g2.layout = kLayNN; g2.c = dh; g2.ldc = h; g2.aux = saved->h; g2.ldaux = h; g2.partials = pdh; g2.accum = accum;
  if (launch_gemm(g2, s) != hipSuccess) return FP8MLP_EHIP;

  // 4. Hq = quant(dH) (E5M2), amax from the epilogue's partials
  QuantBatch bh{};
  bh.njobs = 1;
  bh.job[0] = make_job(dh, M, h, h, FP8MLP_E5M2, hq, h, nullptr, 0, &bsc[1], nullptr, pdh, (int)gemm_num_tiles(M, h),
                       kModePlain);
  if (launch_cast(bh, s) != hipSuccess) return FP8MLP_EHIP;

  // 5. dW_up[h,d] = Hq^T . Xq (TN, reduction over the M tokens)
  GemmArgs g3 = gemm_args(hq, h, FP8MLP_E5M2, &bsc[1], saved->xq, d, FP8MLP_E4M3, &sc[0], h, d, M, kEpiStore);
  g3.layout = kLayTN; g3.c = dw_up; g3.ldc = d; g3.accum = accum;
  if (launch_gemm(g3, s) != hipSuccess) return FP8MLP_EHIP;

  // 6. dX[M,d] = Hq . Uq (NN, reduction over h)
  GemmArgs g4 = gemm_args(hq, h, FP8MLP_E5M2, &bsc[1], saved->uq, d, FP8MLP_E4M3, &sc[1], M, d, h, kEpiStore);
  g4.layout = kLayNN; g4.c = dx; g4.ldc = d; g4.accum = accum;
  return hip_status(launch_gemm(g4, s));
}

size_t fp8_lm_head_ce_workspace_bytes(int64_t M, int64_t K, int64_t V, int64_t chunk) {
  if (check_lm_ce_dims(M, K, V, 1, chunk)) return 0;
  size_t off[L_COUNT];
  return layout_lm_ce(M, K, V, chunk, off);
}

int fp8_lm_head_ce_workspace_layout(int64_t M, int64_t K, int64_t V, int64_t chunk, size_t* offsets, int n) {
  if (check_lm_ce_dims(M, K, V, 1, chunk) || !offsets || n < L_COUNT) return FP8MLP_EINVAL;
  layout_lm_ce(M, K, V, chunk, offsets);
  return FP8MLP_OK;
}

int fp8_lm_head_ce(const uint16_t* x, const uint16_t* w, const int32_t* targets, int64_t M, int64_t K,
                   int64_t V, int64_t n_classes, float softcap, int64_t chunk, float* loss, uint16_t* dx,
                   uint16_t* dw, float* scales, void* ws, size_t ws_bytes, int accum, void* stream) {
  if (!w || !dw || !loss || !accum_ok(accum)) return FP8MLP_EINVAL;
  int st = check_lm_ce_dims(M, K, V, n_classes, chunk);
  if (st) return st;
  if (!(softcap > 0.0f) || !(softcap < 1e30f)) return FP8MLP_EINVAL;
  if (M > 0 && (!x || !targets || !dx)) return FP8MLP_EINVAL;
  const void* ptrs[] = {x, w, dx, dw};
  for (const void* p : ptrs)
    if (!a16(p)) return FP8MLP_EALIGN;
  if (((uintptr_t)loss & 3u) || ((uintptr_t)scales & 3u) || ((uintptr_t)targets & 3u)) return FP8MLP_EALIGN;
  size_t off[L_COUNT];
  const size_t need = layout_lm_ce(M, K, V, chunk, off);
  if (!ws || ws_bytes < need) return FP8MLP_EWORKSPACE;
  if (!a16(ws)) return FP8MLP_EALIGN;

  const int64_t Vp = pad16(V), C = chunk;
  uint8_t* w8 = (uint8_t*)ws;
  uint8_t *xq = w8 + off[L_XQ], *wq = w8 + off[L_WQ];
  uint16_t* zb = (uint16_t*)(w8 + off[L_Z]);
  uint8_t* dzq = w8 + off[L_DZQ];
  float* dwf = (float*)(w8 + off[L_DWF]);
  float* loss_rows = (float*)(w8 + off[L_LOSS]);
  uint32_t* px = (uint32_t*)(w8 + off[L_PX]);
  uint32_t* pw = (uint32_t*)(w8 + off[L_PW]);
  uint32_t* pz = (uint32_t*)(w8 + off[L_PZ]);
  int32_t* nv = (int32_t*)(w8 + off[L_NV]);
  float* sc = scales ? scales : (float*)(w8 + off[L_SC]);
  hipStream_t s = (hipStream_t)stream;

  // 1. targets that count, then X and W quantised tensorwise (E4M3) in one
  //    amax and one cast launch
  if (launch_count_valid(targets, M, n_classes, nv, s) != hipSuccess) return FP8MLP_EHIP;
  QuantBatch b{};
  b.njobs = 2;
  b.job[0] = make_job(x, M, K, K, FP8MLP_E4M3, xq, K, nullptr, 0, &sc[0], nullptr, px, amax_parts_for(M, K),
                      kModePlain);
  b.job[1] = make_job(w, V, K, K, FP8MLP_E4M3, wq, K, nullptr, 0, &sc[1], nullptr, pw, amax_parts_for(V, K),
                      kModePlain);
  if (launch_amax_cast(b, s) != hipSuccess) return FP8MLP_EHIP;

  // 2. chunks of C rows: logits, loss and dZ, dZ codes, grad-input, grad-weight.
  //    Two equal chunks (a multiple of 128 rows, V a multiple of 4, so that
  //    both reduction segments end on whole stages and dwords) keep the first
  //    chunk's dZ codes in the fp32 slot, which they then do not need, and
  //    take dW as one two-segment product after the loop:
  //    dW = RN_bf16(p_2 (S_2 + RN32(p_1 / p_2) S_1)), p_k = RN32(s_k sx).
  const bool seg2 = M == 2 * C && C % 128 == 0 && V % 4 == 0 && C * Vp <= V * K * 4;
  int64_t k = 0;
  for (int64_t c0 = 0; c0 < M; c0 += C, ++k) {
    uint8_t* dzk = (seg2 && k == 0) ? reinterpret_cast<uint8_t*>(dwf) : dzq;  // this chunk's dZ codes
    const int64_t rows = M - c0 < C ? M - c0 : C;
    // Z = Xq_k . Wq^T (NT; bf16, leading dimension Vp)
    GemmArgs g = gemm_args(xq + c0 * K, K, FP8MLP_E4M3, &sc[0], wq, K, FP8MLP_E4M3, &sc[1], rows, V, K, kEpiStore);
    g.c = zb; g.ldc = Vp; g.accum = accum;
    if (launch_gemm(g, s) != hipSuccess) return FP8MLP_EHIP;
    if (launch_softcap_ce(zb, rows, V, Vp, n_classes, softcap, targets + c0, nv, loss_rows + c0, pz, s) !=
        hipSuccess)
      return FP8MLP_EHIP;
    QuantBatch bz{};  // dZ codes with this chunk's own scale (row partials)
    bz.njobs = 1;
    bz.job[0] = make_job(zb, rows, V, Vp, FP8MLP_E5M2, dzk, Vp, nullptr, 0, &sc[2 + k], nullptr, pz, (int)rows,
                         kModePlain);
    if (launch_cast(bz, s) != hipSuccess) return FP8MLP_EHIP;
    // dX_k = dZq_k . Wq (NN, reduction over the V classes' rows of the vocabulary)
    GemmArgs gd = gemm_args(dzk, Vp, FP8MLP_E5M2, &sc[2 + k], wq, K, FP8MLP_E4M3, &sc[1], rows, K, V, kEpiStore);
    gd.layout = kLayNN; gd.c = dx + c0 * K; gd.ldc = K; gd.accum = accum;
    if (launch_gemm(gd, s) != hipSuccess) return FP8MLP_EHIP;
    if (seg2) continue;
    // dW (+)= RN32(s_k sx) dZq_k^T . Xq_k (TN, reduction over the chunk's rows)
    GemmArgs gw = gemm_args(dzq, Vp, FP8MLP_E5M2, &sc[2 + k], xq + c0 * K, K, FP8MLP_E4M3, &sc[0], V, K, rows,
                            kEpiStore);
    gw.layout = kLayTN; gw.cf = dwf; gw.ldc = K; gw.accum = accum;
    // fp32 accumulation over the chunks; the last chunk adds its product and
    // rounds the sum once to bf16 into dw (a single chunk rounds directly)
    const bool last = c0 + C >= M;
    gw.epi = !last ? (k == 0 ? kEpiStoreF32 : kEpiAccF32) : (k == 0 ? kEpiStore : kEpiAccF32Bf16);
    if (last) gw.c = dw;
    if (launch_gemm(gw, s) != hipSuccess) return FP8MLP_EHIP;
  }

  if (seg2) {
    GemmArgs gw = gemm_args(reinterpret_cast<const uint8_t*>(dwf), Vp, FP8MLP_E5M2, &sc[2], xq, K, FP8MLP_E4M3,
                            &sc[0], V, K, M, kEpiStore2);
    gw.layout = kLayTN; gw.a_2 = dzq; gw.b_2 = xq + C * K; gw.sa_2 = &sc[3]; gw.sb_2 = &sc[0];
    gw.c = dw; gw.ldc = K; gw.accum = accum;
    if (launch_gemm(gw, s) != hipSuccess) return FP8MLP_EHIP;
  }

  // 3. dW is zero without tokens; the mean loss
  if (M == 0 && launch_f32_to_bf16(nullptr, dw, V * K, s) != hipSuccess) return FP8MLP_EHIP;
  return hip_status(launch_lm_ce_loss(loss_rows, M, nv, loss, s));
}

size_t swiglu_mlp_fwd_workspace_bytes(int64_t M, int64_t d, int64_t h) {
  if (check_mlp_dims(M, d, h)) return 0;
  size_t off[SF_COUNT];
  return layout_sg_fwd(M, d, h, off);
}

size_t swiglu_mlp_bwd_workspace_bytes(int64_t M, int64_t d, int64_t h) {
  if (check_mlp_dims(M, d, h)) return 0;
  size_t off[SB_COUNT];
  return layout_sg_bwd(M, d, h, off);
}

int swiglu_mlp_fwd_workspace_layout(int64_t M, int64_t d, int64_t h, size_t* offsets, int n) {
  if (check_mlp_dims(M, d, h) || !offsets || n < SF_COUNT) return FP8MLP_EINVAL;
  layout_sg_fwd(M, d, h, offsets);
  return FP8MLP_OK;
}

int swiglu_mlp_bwd_workspace_layout(int64_t M, int64_t d, int64_t h, size_t* offsets, int n) {
  if (check_mlp_dims(M, d, h) || !offsets || n < SB_COUNT) return FP8MLP_EINVAL;
  layout_sg_bwd(M, d, h, offsets);
  return FP8MLP_OK;
}

int swiglu_mlp_fwd(const uint16_t* x, const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                   int64_t M, int64_t d, int64_t h, uint16_t* y, const swiglu_mlp_saved* sv, void* ws,
                   size_t ws_bytes, int accum, void* stream) {
  if (!w_gate || !w_up || !w_down || !sv || !sv->wgq || !sv->wuq || !sv->wdq || !sv->scales) return FP8MLP_EINVAL;
  if (!accum_ok(accum)) return FP8MLP_EINVAL;
  int st = check_mlp_dims(M, d, h);
  if (st) return st;
  if (M > 0 && (!x || !y || !sv->xq || !sv->aq || !sv->g || !sv->u)) return FP8MLP_EINVAL;
  const void* ptrs[] = {x, w_gate, w_up, w_down, y, sv->xq, sv->wgq, sv->wuq, sv->wdq, sv->aq, sv->g, sv->u};
  for (const void* p : ptrs)
    if (!a16(p)) return FP8MLP_EALIGN;
  if ((uintptr_t)sv->scales & 3u) return FP8MLP_EALIGN;
  size_t off[SF_COUNT];
  if (!ws || ws_bytes < layout_sg_fwd(M, d, h, off)) return FP8MLP_EWORKSPACE;
  if (!a16(ws)) return FP8MLP_EALIGN;
  uint8_t* w8 = (uint8_t*)ws;
  uint16_t* a = (uint16_t*)(w8 + off[SF_A]);
  uint32_t* pa = (uint32_t*)(w8 + off[SF_PA]);
  float* sc = sv->scales;
  hipStream_t s = (hipStream_t)stream;

  // 1. X, W_gate, W_up, W_down (E4M3), one amax and one cast launch
  QuantBatch b{};
  b.njobs = 4;
  b.job[0] = make_job(x, M, d, d, FP8MLP_E4M3, sv->xq, d, nullptr, 0, &sc[0], nullptr, (uint32_t*)(w8 + off[SF_PX]),
                      amax_parts_for(M, d), kModePlain);
  b.job[1] = make_job(w_gate, h, d, d, FP8MLP_E4M3, sv->wgq, d, nullptr, 0, &sc[1], nullptr,
                      (uint32_t*)(w8 + off[SF_PWG]), amax_parts_for(h, d), kModePlain);
  b.job[2] = make_job(w_up, h, d, d, FP8MLP_E4M3, sv->wuq, d, nullptr, 0, &sc[2], nullptr,
                      (uint32_t*)(w8 + off[SF_PWU]), amax_parts_for(h, d), kModePlain);
  b.job[3] = make_job(w_down, d, h, h, FP8MLP_E4M3, sv->wdq, h, nullptr, 0, &sc[3], nullptr,
                      (uint32_t*)(w8 + off[SF_PWD]), amax_parts_for(d, h), kModePlain);
  if (launch_amax_cast(b, s) != hipSuccess) return FP8MLP_EHIP;

  // 2. G, U and A = silu(G) U in one NT GEMM over the gate and up codes, with
  //    the per-tile max |A| partials
  GemmArgs gs = gemm_args(sv->xq, d, FP8MLP_E4M3, &sc[0], sv->wgq, d, FP8MLP_E4M3, &sc[1], M, h, d, kEpiSwiGLU);
  gs.b2 = sv->wuq; gs.sb2 = &sc[2];
  gs.c = sv->g; gs.c2 = sv->u; gs.c3 = a; gs.ldc = h; gs.partials = pa; gs.accum = accum;
  if (launch_gemm(gs, s) != hipSuccess) return FP8MLP_EHIP;

  // 3. Aq, 4. Y = Aq . Wdq^T (NT)
  QuantBatch ba{};
  ba.njobs = 1;
  ba.job[0] = make_job(a, M, h, h, FP8MLP_E4M3, sv->aq, h, nullptr, 0, &sc[4], nullptr, pa,
                       (int)gemm_swiglu_tiles(M, h), kModePlain);
  if (launch_cast(ba, s) != hipSuccess) return FP8MLP_EHIP;
  GemmArgs gy = gemm_args(sv->aq, h, FP8MLP_E4M3, &sc[4], sv->wdq, h, FP8MLP_E4M3, &sc[3], M, d, h, kEpiStore);
  gy.c = y; gy.ldc = d; gy.accum = accum;
  return hip_status(launch_gemm(gy, s));
}

int swiglu_mlp_bwd(const uint16_t* dy, const swiglu_mlp_saved* sv, int64_t M, int64_t d, int64_t h, uint16_t* dx,
                   uint16_t* dw_gate, uint16_t* dw_up, uint16_t* dw_down, float* bwd_scales, void* ws,
                   size_t ws_bytes, int accum, void* stream) {
  if (!sv || !dw_gate || !dw_up || !dw_down || !sv->wgq || !sv->wuq || !sv->wdq || !sv->scales) return FP8MLP_EINVAL;
  if (!accum_ok(accum)) return FP8MLP_EINVAL;
  int st = check_mlp_dims(M, d, h);
  if (st) return st;
  if (M > 0 && (!dy || !dx || !sv->xq || !sv->aq || !sv->g || !sv->u)) return FP8MLP_EINVAL;
  const void* ptrs[] = {dy, dx, dw_gate, dw_up, dw_down, sv->xq, sv->wgq, sv->wuq, sv->wdq, sv->aq, sv->g, sv->u};
  for (const void* p : ptrs)
    if (!a16(p)) return FP8MLP_EALIGN;
  if (((uintptr_t)sv->scales & 3u) || ((uintptr_t)bwd_scales & 3u)) return FP8MLP_EALIGN;
  size_t off[SB_COUNT];
  if (!ws || ws_bytes < layout_sg_bwd(M, d, h, off)) return FP8MLP_EWORKSPACE;
  if (!a16(ws)) return FP8MLP_EALIGN;
  uint8_t* w8 = (uint8_t*)ws;
  uint8_t* gq = w8 + off[SB_GQ];
  uint16_t* dg = (uint16_t*)(w8 + off[SB_DG]);
  uint16_t* du = (uint16_t*)(w8 + off[SB_DU]);
  uint8_t *dgq = w8 + off[SB_DGQ], *duq = w8 + off[SB_DUQ];
  float* dxf = (float*)(w8 + off[SB_DXF]);
  uint32_t *pdg = (uint32_t*)(w8 + off[SB_PDG]), *pdu = (uint32_t*)(w8 + off[SB_PDU]);
  float* bsc = bwd_scales ? bwd_scales : (float*)(w8 + off[SB_SC]);
  const float* sc = sv->scales;
  hipStream_t s = (hipStream_t)stream;

  // 1. Gq = quant(dY) (E5M2)
  QuantBatch b{};
  b.njobs = 1;
  b.job[0] = make_job(dy, M, d, d, FP8MLP_E5M2, gq, d, nullptr, 0, &bsc[0], nullptr, (uint32_t*)(w8 + off[SB_PG]),
                      amax_parts_for(M, d), kModePlain);
  if (launch_amax_cast(b, s) != hipSuccess) return FP8MLP_EHIP;

  // 2. dA = Gq . Wd (NN), and in its epilogue 3. dG, dU with their tile maxima
  GemmArgs ga = gemm_args(gq, d, FP8MLP_E5M2, &bsc[0], sv->wdq, h, FP8MLP_E4M3, &sc[3], M, h, d, kEpiSwiGLUBwd);
  ga.layout = kLayNN; ga.aux = sv->g; ga.aux2 = sv->u; ga.ldaux = h; ga.c = dg; ga.c2 = du; ga.ldc = h;
  ga.partials = pdg; ga.partials2 = pdu; ga.accum = accum;
  if (launch_gemm(ga, s) != hipSuccess) return FP8MLP_EHIP;

  // 4. the E5M2 codes of dG and dU (one cast launch)
  const int ptiles = (int)gemm_num_tiles(M, h);
  QuantBatch bg{};
  bg.njobs = 2;
  bg.job[0] = make_job(dg, M, h, h, FP8MLP_E5M2, dgq, h, nullptr, 0, &bsc[1], nullptr, pdg, ptiles, kModePlain);
  bg.job[1] = make_job(du, M, h, h, FP8MLP_E5M2, duq, h, nullptr, 0, &bsc[2], nullptr, pdu, ptiles, kModePlain);
  if (launch_cast(bg, s) != hipSuccess) return FP8MLP_EHIP;

  // 5. the three grad-weights in one launch, so that their tiles fill the
  // CUs together (TN, reduction over the M tokens):
  //    dW_down = Gq^T . Aq, dW_gate = dGq^T . Xq, dW_up = dUq^T . Xq
  GemmArgs gw = gemm_args(nullptr, 0, FP8MLP_E5M2, nullptr, nullptr, 0, FP8MLP_E4M3, nullptr, 0, 0, M,
                          kEpiStoreGroup);
  gw.layout = kLayTN; gw.accum = accum; gw.ngroup = 3;
  gw.grp[0] = GemmProblem{gq, sv->aq, &bsc[0], &sc[4], dw_down, d, h, h, d, h};
  gw.grp[1] = GemmProblem{dgq, sv->xq, &bsc[1], &sc[0], dw_gate, h, d, d, h, d};
  gw.grp[2] = GemmProblem{duq, sv->xq, &bsc[2], &sc[0], dw_up, h, d, d, h, d};
  if (launch_gemm(gw, s) != hipSuccess) return FP8MLP_EHIP;

  // 6. dX = dGq . Wg + dUq . Wu (NN), summed in fp32 and rounded once: one
  // launch over both products when h is a whole number of 128-deep stages,
  // else the first product stored in fp32 and the second added to it
  if (h % 128 == 0) {
    GemmArgs x = gemm_args(dgq, h, FP8MLP_E5M2, &bsc[1], sv->wgq, d, FP8MLP_E4M3, &sc[1], M, d, 2 * h, kEpiStore2);
    x.layout = kLayNN; x.a_2 = duq; x.b_2 = sv->wuq; x.sa_2 = &bsc[2]; x.sb_2 = &sc[2];
    x.c = dx; x.ldc = d; x.accum = accum;
    return launch_gemm(x, s) != hipSuccess ? FP8MLP_EHIP : FP8MLP_OK;
  }
  GemmArgs x1 = gemm_args(dgq, h, FP8MLP_E5M2, &bsc[1], sv->wgq, d, FP8MLP_E4M3, &sc[1], M, d, h, kEpiStoreF32);
  x1.layout = kLayNN; x1.cf = dxf; x1.ldc = d; x1.accum = accum;
  GemmArgs x2 = gemm_args(duq, h, FP8MLP_E5M2, &bsc[2], sv->wuq, d, FP8MLP_E4M3, &sc[2], M, d, h,
                          kEpiAccF32Bf16);  // adds to the first product and rounds once into dx
  x2.layout = kLayNN; x2.cf = dxf; x2.c = dx; x2.ldc = d; x2.accum = accum;
  if (launch_gemm(x1, s) != hipSuccess || launch_gemm(x2, s) != hipSuccess) return FP8MLP_EHIP;
  return FP8MLP_OK;
}

int bf16_gemm_nt(const uint16_t* a, int64_t lda, const uint16_t* b, int64_t ldb, int64_t M, int64_t N, int64_t K,
                 float alpha, float beta, const uint16_t* aux, int64_t ldaux, uint16_t* c, int64_t ldc,
                 uint16_t* ct, int64_t ldct, void* stream) {
  if (M < 0 || N < 0 || K < 0) return FP8MLP_EINVAL;
  if (M == 0 || N == 0) return FP8MLP_OK;
  if (!c || ldc < N || (aux && ldaux < N) || (ct && ldct < M)) return FP8MLP_EINVAL;
  if (!a2(c) || (aux && !a2(aux)) || (ct && !a2(ct))) return FP8MLP_EALIGN;
  if (K > 0) {
    if (!a || !b || lda < K || ldb < K) return FP8MLP_EINVAL;
    if (K % 8 != 0) return FP8MLP_ENOTSUP;
    if (!a16(a) || !a16(b) || lda % 8 || ldb % 8) return FP8MLP_EALIGN;
    if (!tile_range_ok(2 * lda, 2 * K) || !tile_range_ok(2 * ldb, 2 * K)) return FP8MLP_ENOTSUP;
  }
  if (M > INT32_MAX / 2 || N > INT32_MAX / 2) return FP8MLP_ENOTSUP;
  GemmArgs g{};
  g.a = (const uint8_t*)a; g.b = (const uint8_t*)b; g.lda = K > 0 ? lda : 0; g.ldb = K > 0 ? ldb : 0;
  g.fa = g.fb = kBF16; g.M = M; g.N = N; g.K = K; g.epi = kEpiAxpby;
  g.alpha = alpha; g.beta = beta; g.aux = aux; g.ldaux = ldaux; g.c = c; g.ldc = ldc; g.ct = ct; g.ldct = ldct;
  return hip_status(launch_gemm(g, (hipStream_t)stream));
}

size_t bf16_gemm_sym_workspace_bytes(int64_t M, int64_t K) {
  if (M < 0 || K < 0 || M % 16 || K % 8) return 0;
  return align_up(sym_partials_bytes(M, K) + 16);
}

int bf16_gemm_sym(const uint16_t* a, int64_t lda, int64_t M, int64_t K, float alpha, float beta,
                  const uint16_t* aux, int64_t ldaux, uint16_t* c, int64_t ldc, void* ws, size_t ws_bytes,
                  void* stream) {
  if (M < 0 || K < 0) return FP8MLP_EINVAL;
  if (M % 16 || K % 8) return FP8MLP_ENOTSUP;
  if (M == 0) return FP8MLP_OK;
  if (!c || ldc < M || (aux && ldaux < M) || (K > 0 && (!a || lda < K))) return FP8MLP_EINVAL;
  if (!a16(c) || ldc % 8 || (aux && !a2(aux)) || (K > 0 && (!a16(a) || lda % 8))) return FP8MLP_EALIGN;
  if (K > 0 && !tile_range_ok(2 * lda, 2 * K)) return FP8MLP_ENOTSUP;
  if (M > INT32_MAX / 2) return FP8MLP_ENOTSUP;
  if (!ws || ws_bytes < bf16_gemm_sym_workspace_bytes(M, K)) return FP8MLP_EWORKSPACE;
  if (!a16(ws)) return FP8MLP_EALIGN;
  return hip_status(launch_sym_gemm(a, K > 0 ? lda : 0, M, K, alpha, beta, aux, ldaux, c, ldc, (float*)ws,
                                    (hipStream_t)stream));
}

namespace {
// Newton-Schulz workspace: A, B [m, m]; T0, T1 [n, m]; the symmetric
// products' fp32 partial sums; norm partials.
enum NsSlot { NS_A, NS_B, NS_T0, NS_T1, NS_SP, NS_P, NS_COUNT };
int check_ns_dims(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return FP8MLP_EINVAL;
  if (rows % 16 || cols % 16) return FP8MLP_ENOTSUP;
  const int64_t m = rows < cols ? rows : cols, n = rows < cols ? cols : rows;
  if (m > 16384 || n > 1048576) return FP8MLP_ENOTSUP;
  return FP8MLP_OK;
}
size_t layout_ns(int64_t rows, int64_t cols, size_t* off) {
  const int64_t m = rows < cols ? rows : cols, n = rows < cols ? cols : rows;
  const size_t sp1 = sym_partials_bytes(m, n), sp2 = sym_partials_bytes(m, m);
  const size_t sz[NS_COUNT] = {(size_t)(m * m) * 2, (size_t)(m * m) * 2, (size_t)(n * m) * 2, (size_t)(n * m) * 2,
                               sp1 > sp2 ? sp1 : sp2, (size_t)ns_parts_for(rows * cols) * 8};
  size_t o = 0;
  for (int i = 0; i < NS_COUNT; ++i) { off[i] = o; o = align_up(o + sz[i]); }
  return o;
}
}  // namespace

size_t muon_ns_workspace_bytes(int64_t rows, int64_t cols) {
  if (check_ns_dims(rows, cols)) return 0;
  size_t off[NS_COUNT];
  return layout_ns(rows, cols, off);
}

int muon_newton_schulz(const uint16_t* g, int64_t rows, int64_t cols, int steps, const float* coeffs, float eps,
                       uint16_t* out, float* norm, void* ws, size_t ws_bytes, void* stream) {
  int st = check_ns_dims(rows, cols);
  if (st) return st;
  if (steps < 0 || steps > 100 || !(eps >= 0.0f)) return FP8MLP_EINVAL;
  if (rows == 0 || cols == 0) return FP8MLP_OK;
  if (!g || !out) return FP8MLP_EINVAL;
  const size_t bytes = (size_t)(rows * cols) * 2;
  if ((const uint8_t*)g < (const uint8_t*)out + bytes && (const uint8_t*)out < (const uint8_t*)g + bytes)
    return FP8MLP_EINVAL;  // out overlaps g
  if (!a16(g) || !a16(out) || ((uintptr_t)norm & 3u)) return FP8MLP_EALIGN;
  size_t off[NS_COUNT];
  if (!ws || ws_bytes < layout_ns(rows, cols, off)) return FP8MLP_EWORKSPACE;
  if (!a16(ws)) return FP8MLP_EALIGN;
  const float ca = coeffs ? coeffs[0] : 3.4445f, cb = coeffs ? coeffs[1] : -4.7750f, cc = coeffs ? coeffs[2] : 2.0315f;
  uint8_t* w8 = (uint8_t*)ws;
  uint16_t* A = (uint16_t*)(w8 + off[NS_A]);
  uint16_t* B = (uint16_t*)(w8 + off[NS_B]);
  float* sp = (float*)(w8 + off[NS_SP]);
  uint16_t* T0 = (uint16_t*)(w8 + off[NS_T0]);
  uint16_t* T1 = (uint16_t*)(w8 + off[NS_T1]);
  double* parts = (double*)(w8 + off[NS_P]);
  hipStream_t s = (hipStream_t)stream;
  const bool tall = rows > cols;
  const int64_t m = tall ? cols : rows, n = tall ? rows : cols;
  // X [m, n] is updated in place; X^T after k steps alternates between two
  // buffers, arranged for a tall G so that the last one is `out`.
  uint16_t* X = tall ? T1 : out;
  auto xt_buf = [&](int k) -> uint16_t* {
    if (tall) return (k % 2 == steps % 2) ? out : T0;
    return (k % 2 == 0) ? T0 : T1;
  };
  // X0: normalised G in G's own layout, then the other orientation
  if (tall) {
    if (launch_ns_normalise(g, rows * cols, eps, parts, xt_buf(0), norm, s) != hipSuccess) return FP8MLP_EHIP;
    if (launch_transpose_bf16(xt_buf(0), n, m, X, s) != hipSuccess) return FP8MLP_EHIP;
  } else {
    if (launch_ns_normalise(g, rows * cols, eps, parts, X, norm, s) != hipSuccess) return FP8MLP_EHIP;
    if (steps > 0 && launch_transpose_bf16(X, m, n, xt_buf(0), s) != hipSuccess) return FP8MLP_EHIP;
  }
  for (int k = 0; k < steps; ++k) {
    // A = X X^T and B = c A A + b A: symmetric, upper triangle only (A is its
    // own transpose, so A A = A A^T is an NT product of A with itself)
    if (launch_sym_gemm(X, n, m, n, 1.0f, 0.0f, nullptr, 0, A, m, sp, s) != hipSuccess ||
        launch_sym_gemm(A, m, m, m, cc, cb, A, m, B, m, sp, s) != hipSuccess)
      return FP8MLP_EHIP;
    GemmArgs g3{};  // X = B X + a X (in place), and X^T for the next step
    g3.a = (const uint8_t*)B; g3.b = (const uint8_t*)xt_buf(k); g3.lda = g3.ldb = m; g3.fa = g3.fb = kBF16;
    g3.M = m; g3.N = n; g3.K = m; g3.epi = kEpiAxpby; g3.alpha = 1.0f; g3.beta = ca; g3.aux = X; g3.ldaux = n;
    g3.c = X; g3.ldc = n;
    if (tall || k + 1 < steps) { g3.ct = xt_buf(k + 1); g3.ldct = m; }
    if (launch_gemm(g3, s) != hipSuccess) return FP8MLP_EHIP;
  }
  return FP8MLP_OK;
}

}  // extern "C"
