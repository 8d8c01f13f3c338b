/*
 * fp8mlp.h - C ABI of the MI355X (gfx950) FP8 tensorwise-scaled linear layer
 * and non-gated relu^2 MLP block.
 *
 * The method (decomputer.nl, "Het trainen van een 3.8B LLM tot 0.384 CORE
 * voor $998", section "Vroege experimenten" item 4 and the first bullet of
 * "Doorvoer verhogen"; the manulx.blog summary's FP8 paragraph): every
 * linear layer runs its three GEMMs - one forward, two backward - in FP8,
 * each operand carrying one scale per tensor that is recomputed from that
 * tensor on every call (dynamic tensorwise scaling), with bf16 tensors around
 * them.  The block is the page's non-gated relu2 MLP at 4x width (appendix
 * configuration: hidden_act relu2, gated_mlp false, intermediate 12288 for
 * hidden 3072).
 *
 * Numeric contract (the pages leave these open; this is the reading used):
 *   formats   OCP E4M3 ("fn", max 448) for activations and weights,
 *             OCP E5M2 (max 57344) for gradients;
 *   scale     s = RN32(amax / fmax), amax = max |x| over the tensor;
 *             s = 1 when amax == 0.  s is the dequantisation scale;
 *   codes     q = RNE_fp8( clamp( RN32(x / s), -fmax, +fmax ) ), the sign of
 *             zero kept (RN32 = binary32 round-to-nearest-even division);
 *   GEMM      out = RN_bf16( RN32(sa * sb) * sum_k a_k b_k ), fp32
 *             accumulation of exact fp8 products, bf16 output.
 *
 * Accumulation (`accum` argument of every entry point that runs an FP8
 * GEMM):
 *   FP8MLP_ACCUM_EXACT  the contract above: every product exact, fp32
 *             accumulation.  The codes are decoded to bf16 (exactly) and
 *             multiplied on the bf16 matrix cores, at about half the FP8 rate.
 *   FP8MLP_ACCUM_FAST   the FP8 matrix cores (v_mfma_*_f8f6f4).  They add the
 *             64 products of one instruction in aligned groups of 8 and
 *             truncate each product in a group to a multiple of 2^(e-13), e
 *             the exponent of the group's largest product, so a dot product
 *             of length K can differ from the exact one by up to
 *             7 * 2^-13 * sum_k |a_k b_k| (plus the fp32 accumulation).  This is
 *             the throughput path (the counterpart of a scaled matmul's
 *             "fast accumulation" option).
 * Any other value is rejected with FP8MLP_EINVAL.
 *
 * Conventions for every entry point:
 *   - Pointers to tensors are DEVICE pointers (hipMalloc'd or torch CUDA
 *     tensors) unless marked otherwise.  Matrices are row-major with an
 *     explicit leading dimension in elements (ld >= number of columns).
 *     bf16 values are passed as uint16_t bit patterns, FP8 values as
 *     uint8_t codes.  Scales are fp32 scalars in device memory.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on that stream: no host synchronisation, no device
 *     memory allocation, no host<->device copies.
 *   - Buffers are owned by the caller.  The library keeps no state between
 *     calls; calls on different streams must not share output or workspace
 *     buffers.
 *   - Errors: arguments are validated before anything is launched; an invalid
 *     call returns a non-zero status and touches no memory.  A failed launch
 *     returns FP8MLP_EHIP.  Faults inside kernels surface at the caller's
 *     next synchronisation.  Overflow is never an error (casts saturate).
 *   - Inputs and outputs must not overlap.
 */
#ifndef FP8MLP_H
#define FP8MLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Version 3: the gated block's backward workspace holds no dA buffer (its
 * grad-input GEMM applies the gate's derivative in the epilogue). */
#define FP8MLP_ABI_VERSION 3

/* FP8 GEMM accumulation modes (see the numeric contract above). */
#define FP8MLP_ACCUM_FAST 0
#define FP8MLP_ACCUM_EXACT 1

/* FP8 formats (OCP 8-bit floating point). */
#define FP8MLP_E4M3 0 /* 1-4-3, bias 7, no infinities, max 448        */
#define FP8MLP_E5M2 1 /* 1-5-2, bias 15, IEEE-like specials, max 57344 */

/* Status codes. */
#define FP8MLP_OK 0
#define FP8MLP_EINVAL 1     /* NULL pointer, size < 0, ld < cols, bad format or accumulation mode */
#define FP8MLP_EALIGN 2     /* pointer or leading dimension misaligned          */
#define FP8MLP_EWORKSPACE 3 /* workspace missing or smaller than the query      */
#define FP8MLP_EHIP 4       /* a HIP launch failed                              */
#define FP8MLP_ENOTSUP 5    /* shape outside what the library supports          */

int fp8mlp_abi_version(void);
/* Static string describing a status code (never NULL). */
const char* fp8mlp_status_string(int status);

/* ------------------------------------------------------------------------ */
/* Dynamic tensorwise quantisation (amax reduction + scale + cast).          */
/* ------------------------------------------------------------------------ */

/* Workspace bytes fp8_amax_quant needs for a rows x cols tensor. */
size_t fp8_amax_quant_workspace_bytes(int64_t rows, int64_t cols);

/*
 * x      [rows, cols] bf16, leading dim ldx.
 * fmt    FP8MLP_E4M3 or FP8MLP_E5M2.
 * q      [rows, cols] codes, leading dim ldq (may be NULL if qt is given).
 * qt     [cols, rows] codes of x transposed, leading dim ldqt (may be NULL).
 *        The GEMMs below read the row-major codes in all three layouts; qt
 *        is for callers that want the transposed operand itself (an NT
 *        product over the rows of x, for example).
 * scale  out: 1 float, s = RN32(amax/fmax) (1 when amax == 0).
 * amax   out: 1 float, max |x| (may be NULL).
 * ws     workspace of at least fp8_amax_quant_workspace_bytes(rows, cols)
 *        bytes, 16-byte aligned; its contents need no initialisation.
 * Requires x to be 2-byte aligned.  16-byte aligned q/qt with leading
 * dimensions that are multiples of 16 take the vectorised path; x rows that
 * are not 8-byte aligned are read with realigning loads; anything else (and
 * ragged edges) takes a correct element-wise path.
 * An empty tensor (rows == 0 or cols == 0) is valid: amax = 0, scale = 1,
 * no codes written.
 * A dense tensor (ldx == ldq == cols, x 16-byte aligned) that wants q only
 * and gives at least 256 work units (about 17 M elements) takes one pass:
 * one grid takes the amax, waits once grid-wide and casts, holding part of
 * x in registers across the wait; otherwise an amax launch and a cast
 * launch.  Both forms give the same bytes.  The single pass's wait is
 * bounded; should it ever give up (a fault, not a load condition), the
 * scale is NaN and the codes it could not finish are NaN (0x7F).  For
 * tests, the environment variable FP8MLP_QUANT_PATH=two|single forces a
 * form (single: an error where it cannot apply) and FP8MLP_QUANT_SPIN_LIMIT
 * sets the wait's bound.  Calls that share one workspace must not overlap.
 * Non-finite inputs are outside the numeric contract (the pages' tensors
 * are finite).  What is guaranteed: if x holds a NaN or an infinity, amax
 * and scale come out non-finite (NaN orders above infinity), so a caller can
 * detect an overflowed tensor from its scale; its codes are unspecified.
 */
int fp8_amax_quant(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                   uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt, float* scale,
                   float* amax, void* ws, size_t ws_bytes, void* stream);

/* fp8_amax_quant for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, results and errors as
 * fp8_amax_quant without ws / ws_bytes.  The amax partials live in a
 * library-owned static device array of 4 KB (1024 u32; no tensor needs
 * more), one per GPU, held until the process ends and found on the first
 * call on each GPU (hipGetSymbolAddress) with that GPU current.  The call
 * allocates nothing and always takes the amax launch and the cast launch.  Calls on one GPU share that array: calls that overlap
 * on one GPU (different streams, or host threads) race and must be
 * serialised by the caller.  Nothing in the array has to start at zero: each
 * call writes every partial it reads. */
int fp8_amax_quant_noalloc(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                           uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt, float* scale,
                           float* amax, void* stream);

/* RMSNorm fused with the dynamic tensorwise quantisation of its output (the
 * MLP input X is the RMSNorm of the residual stream; decomputer.nl, appendix:
 * Llama-style RMSNorm, rms_norm_eps 1.0e-6).  Each step in a stated precision:
 *   ms = RN32(RN64(sum_j x_j^2 / cols))  (sum in fp64)
 *   r  = RN32(1 / RN32(sqrt(RN32(ms + eps))))          -> rstd[row]
 *   X_j = RN_bf16(RN32(RN32(x_j r) gamma_j))           (gamma NULL: no weight)
 * then q / qt / scale / amax exactly as fp8_amax_quant of X.  X itself is not
 * stored: the statistics pass takes r and the amax, the cast pass recomputes
 * X from x, r and gamma.  Rows of at most 3072 columns (16-byte aligned,
 * q only, 4096 rows or more) take both in one pass, each block holding 16
 * rows in registers across one grid-wide wait, with the same results and
 * the same bounded-wait behaviour as fp8_amax_quant.
 * x [rows, cols] bf16 (ldx); gamma [cols] bf16 or NULL; rstd out [rows] fp32;
 * ws of fp8_rmsnorm_quant_workspace_bytes(rows, cols) bytes, 16-byte aligned.
 * Empty tensors are valid (scale 1, amax 0). */
size_t fp8_rmsnorm_quant_workspace_bytes(int64_t rows, int64_t cols);
int fp8_rmsnorm_quant(const uint16_t* x, const uint16_t* gamma, float eps, int64_t rows, int64_t cols,
                      int64_t ldx, int fmt, uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt,
                      float* scale, float* amax, float* rstd, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* The three FP8 GEMMs of one linear layer (decomputer.nl, "Doorvoer        */
/* verhogen", first bullet: the forward and both backward GEMMs in FP8),    */
/* on row-major codes as fp8_amax_quant writes them.  Weight W [N,K] is     */
/* stored [out, in], the input X [M,K] and the output gradient dY [M,N]     */
/* [tokens, features].                                                      */
/*   forward      Y  = X . W^T     NT  C[m,n] = sum_k A[m,k] B[n,k]          */
/*   grad-input   dX = dY . W      NN  C[m,n] = sum_k A[m,k] B[k,n]          */
/*   grad-weight  dW = dY^T . X    TN  C[m,n] = sum_k A[k,m] B[k,n]          */
/* Each computes RN_bf16(RN32(sa*sb) * sum) with the accumulation `accum`.  */
/* Requirements: operand pointers 16-byte aligned and their leading         */
/* dimensions multiples of 16; any M, N, K >= 0 (ragged edges are masked,   */
/* a reduction length that is not a multiple of 16 included; M == 0 or      */
/* N == 0 is a no-op, K == 0 writes zeros, the empty sum); y/dx/dw 2-byte    */
/* aligned (16-byte aligned with a leading dimension that is a multiple of  */
/* 8 for full-width stores).  The output is overwritten (no accumulation).  */
/* ------------------------------------------------------------------------ */

/* Forward  Y[M,N] = X[M,K] . W[N,K]^T.
 * xq [M,K] (ldx), wq [N,K] (ldw), y [M,N] bf16 (ldy). */
int fp8_linear_fwd(const uint8_t* xq, int64_t ldx, int fx, const float* sx, const uint8_t* wq,
                   int64_t ldw, int fw, const float* sw, int64_t M, int64_t N, int64_t K,
                   uint16_t* y, int64_t ldy, int accum, void* stream);

/* Grad-input  dX[M,K] = dY[M,N] . W[N,K], reduction over the N output
 * features.  dyq [M,N] (lddy), wq [N,K] (ldw) - the forward's weight codes;
 * dx [M,K] bf16 (lddx). */
int fp8_linear_dgrad(const uint8_t* dyq, int64_t lddy, int fdy, const float* sdy,
                     const uint8_t* wq, int64_t ldw, int fw, const float* sw, int64_t M,
                     int64_t N, int64_t K, uint16_t* dx, int64_t lddx, int accum, void* stream);

/* Grad-weight  dW[N,K] = dY[M,N]^T . X[M,K], reduction over the M tokens.
 * dyq [M,N] (lddy), xq [M,K] (ldx) - the forward's input codes; dw [N,K]
 * bf16 (lddw). */
int fp8_linear_wgrad(const uint8_t* dyq, int64_t lddy, int fdy, const float* sdy,
                     const uint8_t* xq, int64_t ldx, int fx, const float* sx, int64_t M,
                     int64_t N, int64_t K, uint16_t* dw, int64_t lddw, int accum, void* stream);

/* The forward of one FP8 linear layer from its bf16 tensors, the way the
 * pages run a linear's forward (decomputer.nl, "Vroege experimenten" item 4:
 * dynamic tensorwise scaling of input and weight on every call): X [M,K]
 * (ldx) and W [N,K] (ldw) bf16 are quantised to E4M3 with their own
 * tensorwise scales, then Y [M,N] = RN_bf16(RN32(sx*sw) Xq . Wq^T) (ldy).
 * Three launches: one amax pass over both tensors, one cast of both, the
 * GEMM.  Outputs, all caller-owned, for the backward to reuse: the codes xq
 * [M,K] (ldxq) and wq [N,K] (ldwq), and scales[0] = sx, scales[1] = sw
 * (device, 4-byte aligned).  Results are bit-identical to fp8_amax_quant of
 * X and of W followed by fp8_linear_fwd.  Requirements: x, w 2-byte
 * aligned; xq, wq as fp8_linear_fwd's operands (16-byte aligned, leading
 * dimensions multiples of 16), not overlapping each other or x, w; ws
 * 16-byte aligned with fp8_linear_fwd_bf16_workspace_bytes(M, N, K) bytes.
 * Empty X or W get scale 1; M == 0 or N == 0 writes no Y, K == 0 zeros. */
size_t fp8_linear_fwd_bf16_workspace_bytes(int64_t M, int64_t N, int64_t K);
int fp8_linear_fwd_bf16(const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw, int64_t M, int64_t N,
                        int64_t K, uint8_t* xq, int64_t ldxq, uint8_t* wq, int64_t ldwq, float* scales,
                        uint16_t* y, int64_t ldy, void* ws, size_t ws_bytes, int accum, void* stream);

/* ------------------------------------------------------------------------ */
/* Non-gated relu^2 MLP block: Y = relu(X W_up^T)^2 W_down^T, FP8 GEMMs     */
/* (decomputer.nl, "Doorvoer verhogen", non-gated MLP bullet; appendix:     */
/* hidden_act relu2, intermediate 12288 for hidden 3072).                   */
/*   X [M,d], W_up [h,d], W_down [d,h], Y [M,d], all bf16, densely packed.  */
/*   Forward (E4M3 everywhere):                                             */
/*     Xq,Uq,Dq = quant(X), quant(W_up), quant(W_down)                      */
/*     H  = NT(Xq, Uq)                       bf16 [M,h]                     */
/*     A  = RN_bf16(relu(H)^2)               (fused: never stored)          */
/*     Aq = quant(A);  Y = NT(Aq, Dq)                                       */
/*   Backward (gradients E5M2):                                             */
/*     Gq = quant(dY);  dW_down = TN(Gq, Aq)                                */
/*     dA = NN(Gq, Dq);  dH = RN_bf16(2 relu(H) dA)  (fused epilogue)       */
/*     Hq = quant(dH);  dW_up = TN(Hq, Xq);  dX = NN(Hq, Uq)                */
/* Requirements: M, d, h multiples of 16 (d, h >= 16; M == 0, no tokens, is  */
/* valid: Y and dX are empty, dW_up and dW_down zero, scales of X, A, dY    */
/* and dH are 1); all pointers 16-byte aligned.                             */
/* ------------------------------------------------------------------------ */

/* Forward quantities the backward pass reads: the row-major codes of every
 * GEMM operand of the forward, H and the scales.  Caller-allocated device
 * buffers, all densely packed; written by relu2_mlp_fwd. */
typedef struct {
  uint8_t* xq;   /* [M, d] E4M3 codes of X      */
  uint8_t* uq;   /* [h, d] E4M3 codes of W_up   */
  uint8_t* dq;   /* [d, h] E4M3 codes of W_down */
  uint8_t* aq;   /* [M, h] E4M3 codes of A      */
  uint16_t* h;   /* [M, h] bf16 pre-activation H */
  float* scales; /* [4]: sx, su, sd, sa         */
} relu2_mlp_saved;

size_t relu2_mlp_fwd_workspace_bytes(int64_t M, int64_t d, int64_t h);
size_t relu2_mlp_bwd_workspace_bytes(int64_t M, int64_t d, int64_t h);

/* Byte offsets of the regions inside the workspaces, for inspection.
 * Forward (n >= 4): the amax partials of X, W_up, W_down and the per-tile
 * max(H) partials.  Backward (n >= 6): Gq [M,d], dH [M,h] bf16, Hq [M,h],
 * the amax partials of dY and of dH, 2 floats of scales. */
int relu2_mlp_fwd_workspace_layout(int64_t M, int64_t d, int64_t h, size_t* offsets, int n);
int relu2_mlp_bwd_workspace_layout(int64_t M, int64_t d, int64_t h, size_t* offsets, int n);

int relu2_mlp_fwd(const uint16_t* x, const uint16_t* w_up, const uint16_t* w_down, int64_t M,
                  int64_t d, int64_t h, uint16_t* y, const relu2_mlp_saved* saved, void* ws,
                  size_t ws_bytes, int accum, void* stream);

/* dx [M,d], dw_up [h,d], dw_down [d,h] are overwritten.  `bwd_scales`
 * (may be NULL) receives 2 floats: sg (scale of dY), sh (scale of dH). */
int relu2_mlp_bwd(const uint16_t* dy, const relu2_mlp_saved* saved, int64_t M, int64_t d,
                  int64_t h, uint16_t* dx, uint16_t* dw_up, uint16_t* dw_down, float* bwd_scales,
                  void* ws, size_t ws_bytes, int accum, void* stream);

/* ------------------------------------------------------------------------ */
/* Gated (SwiGLU) MLP block through the same FP8 linears, the form the      */
/* pages replaced by relu^2 (decomputer.nl, "Doorvoer verhogen", non-gated   */
/* MLP bullet: three matmuls instead of two, intermediate ratio 2.75):       */
/*   X [M,d], W_gate [h,d], W_up [h,d], W_down [d,h], Y [M,d], bf16, dense.  */
/*   Forward (E4M3):  Xq, Wgq, Wuq, Wdq = quant(X, W_gate, W_up, W_down)     */
/*     G = NT(Xq, Wgq), U = NT(Xq, Wuq)           bf16 [M,h], kept for bwd   */
/*     A = RN_bf16(RN32(RN32(G sigmoid(G)) U))    (fp32 sigmoid)             */
/*     Aq = quant(A);  Y = NT(Aq, Wdq)                                       */
/*   Backward (gradients E5M2):                                              */
/*     Gq = quant(dY);  dW_down = TN(Gq, Aq);  dA = NN(Gq, Wdq), not stored: */
/*     dG = RN_bf16(dA U silu'(G)),  dU = RN_bf16(dA silu(G))  (fp32, in the  */
/*     epilogue of the dA GEMM; silu'(g) = s (1 + g (1 - s)), s = sigmoid(g)) */
/*     dGq, dUq = quant(dG), quant(dU)                                       */
/*     dW_gate = TN(dGq, Xq);  dW_up = TN(dUq, Xq)  (one launch with dW_down) */
/*     dX = RN_bf16(RN32(RN32(p_g NN(dGq,Wgq)) + RN32(p_u NN(dUq,Wuq))))      */
/*       (h a multiple of 128: one fp32 accumulation of both products,     */
/*       dX = RN_bf16(p_u (NN(dUq,Wuq) + RN32(p_g / p_u) NN(dGq,Wgq))))       */
/* Requirements as for the relu^2 block (M, d, h multiples of 16, M == 0    */
/* valid, 16-byte aligned pointers).                                        */
/* ------------------------------------------------------------------------ */
typedef struct {
  uint8_t* xq;     /* [M, d] codes of X                      */
  uint8_t* wgq;    /* [h, d] codes of W_gate                 */
  uint8_t* wuq;    /* [h, d] codes of W_up                   */
  uint8_t* wdq;    /* [d, h] codes of W_down                 */
  uint8_t* aq;     /* [M, h] codes of A                      */
  uint16_t* g;     /* [M, h] bf16 gate pre-activation G      */
  uint16_t* u;     /* [M, h] bf16 up projection U            */
  float* scales;   /* 5 floats: sx, s_gate, s_up, s_down, sa */
} swiglu_mlp_saved;

size_t swiglu_mlp_fwd_workspace_bytes(int64_t M, int64_t d, int64_t h);
size_t swiglu_mlp_bwd_workspace_bytes(int64_t M, int64_t d, int64_t h);
/* Byte offsets of the workspace regions.  Forward (n >= 6): A bf16, amax
 * partials of X, W_gate, W_up, W_down, A.  Backward (n >= 10): Gq, dG, dU,
 * dGq, dUq, dX fp32, amax partials of dY, dG, dU, scales. */
int swiglu_mlp_fwd_workspace_layout(int64_t M, int64_t d, int64_t h, size_t* offsets, int n);
int swiglu_mlp_bwd_workspace_layout(int64_t M, int64_t d, int64_t h, size_t* offsets, int n);
int swiglu_mlp_fwd(const uint16_t* x, const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                   int64_t M, int64_t d, int64_t h, uint16_t* y, const swiglu_mlp_saved* saved, void* ws,
                   size_t ws_bytes, int accum, void* stream);
/* bwd_scales (may be NULL): 3 floats, s_dY, s_dG, s_dU. */
int swiglu_mlp_bwd(const uint16_t* dy, const swiglu_mlp_saved* saved, int64_t M, int64_t d, int64_t h,
                   uint16_t* dx, uint16_t* dw_gate, uint16_t* dw_up, uint16_t* dw_down, float* bwd_scales,
                   void* ws, size_t ws_bytes, int accum, void* stream);

/* The gate and up projections of the gated block as one FP8 GEMM (the first
 * step of swiglu_mlp_fwd, usable on its own).  For E4M3 codes Xq [M,K] and
 * Wgq, Wuq [N,K] (one leading dimension ldw for both):
 *   G = RN_bf16(RN32(sx*sg) Xq.Wgq^T),   U = RN_bf16(RN32(sx*su) Xq.Wuq^T),
 *   A = RN_bf16(RN32(RN32(G sigmoid(G)) U))        (fp32 sigmoid),
 * all [M,N] bf16 with leading dimension ldo.  Each output tile pairs 128
 * rows of Wgq with the same rows of Wuq, so G, U and A leave one kernel.
 * Requirements as for fp8_linear_fwd (16-byte aligned operands with leading
 * dimensions that are multiples of 16), and K % 16 == 0; g, u and a 2-byte
 * aligned (16-byte aligned with ldo % 8 == 0 for full-width stores), not
 * overlapping each other or the operands.  M == 0 or N == 0 writes nothing;
 * K == 0 writes zeros. */
int fp8_gated_linear_fwd(const uint8_t* xq, int64_t ldx, const float* sx, const uint8_t* wgq, const float* sg,
                         const uint8_t* wuq, const float* su, int64_t ldw, int64_t M, int64_t N, int64_t K,
                         uint16_t* g, uint16_t* u, uint16_t* a, int64_t ldo, int accum, void* stream);

/* ------------------------------------------------------------------------ */
/* FP8 LM head fused with the softcapped cross-entropy, chunked over rows.  */
/*                                                                          */
/* decomputer.nl, "Doorvoer verhogen", fused linear cross-entropy bullet:   */
/* the head's matmul runs inside the loss, a chunk of rows at a time, so    */
/* the whole [M, V] logits tensor is never stored; the appendix caps the    */
/* logits at 15.0 (logit_softcap; loss LigerFusedLinearCrossEntropyLoss     */
/* with softcap 15.0).  With c = softcap, for every chunk of `chunk` rows:  */
/*   Z   = RN_bf16(RN32(sx*sw) Xq_k . Wq^T)        logits, bf16             */
/*   S   = c tanh(Z / c)                                                    */
/*   loss_r = log sum_j exp(S_rj) - S_r,t_r        over j < n_classes       */
/*   dZ  = RN_bf16((softmax(S) - onehot(t)) (1 - tanh^2(Z/c)) / n_valid)     */
/*   dZq, s_k = quant(dZ, E5M2)                    the chunk's own scale     */
/*   dX_k = RN_bf16(RN32(s_k*sw) dZq . Wq)         grad-input (bf16)         */
/*   dW  += RN32(s_k*sx) dZq^T . Xq_k              fp32, rounded once at end  */
/* with Xq, sx and Wq, sw the E4M3 tensorwise quantisations of X and W.      */
/* Two equal chunks (M == 2 chunk, chunk a multiple of 128, V a multiple of  */
/* 4, chunk x Vp bytes within the fp32 region) take dW in one product over   */
/* both chunks instead, with p_k = RN32(s_k*sx) and S_k the chunk's fp32     */
/* sum: dW = RN_bf16(p_2 (S_2 + RN32(p_1/p_2) S_1)); the first chunk's codes */
/* then sit at the start of the fp32 region.                                 */
/* Rows whose target lies outside [0, n_classes) are ignored; n_valid counts */
/* the others; loss = sum of row losses / n_valid (0 when n_valid == 0).     */
/* The softmax, tanh and exp run in fp32; sums in a fixed order, so results  */
/* are reproducible bit for bit.                                             */
/* ------------------------------------------------------------------------ */

/* Workspace for fp8_lm_head_ce (0 if the shape is not supported).  Holds Xq,
 * Wq, one chunk of logits (bf16, chunk x V rounded up to 16) and its codes,
 * the fp32 dW accumulator and small per-row / per-chunk arrays. */
size_t fp8_lm_head_ce_workspace_bytes(int64_t M, int64_t K, int64_t V, int64_t chunk);

/* Byte offsets (n >= 11) of the workspace regions, in this order: Xq [M,K],
 * Wq [V,K], logits/dZ of the last chunk (bf16 [chunk,Vp]), dZ codes of the
 * last chunk [chunk,Vp], dW fp32 [V,K] (with two equal chunks: the first
 * chunk's dZ codes), row losses [M] fp32, amax partials of X and W,
 * row partials, the valid-row count, scales; Vp = V rounded up to 16. */
int fp8_lm_head_ce_workspace_layout(int64_t M, int64_t K, int64_t V, int64_t chunk, size_t* offsets, int n);

/*
 * x        [M, K] bf16 hidden states (dense rows); w [V, K] bf16 head weight
 *          (V may include padding rows beyond n_classes).
 * targets  [M] int32 class ids (device); ids outside [0, n_classes) are ignored.
 * softcap  c > 0 (15.0 on the pages).
 * chunk    rows per chunk, a multiple of 16 (the logits buffer is chunk x V).
 * loss     out: 1 float (device), the mean loss over the counted rows.
 * dx       out: [M, K] bf16.  dw  out: [V, K] bf16 (rows >= n_classes are 0
 *          when the padded rows of w are zero).
 * scales   out (may be NULL): 2 + ceil(M / chunk) floats: sx, sw, then the
 *          dZ scale of every chunk.
 * Requirements: M, K multiples of 16 (M == 0 valid: loss 0, dw 0);
 *          1 <= n_classes <= V <= 4194304; x, w, dx, dw 16-byte aligned.
 */
int fp8_lm_head_ce(const uint16_t* x, const uint16_t* w, const int32_t* targets, int64_t M, int64_t K,
                   int64_t V, int64_t n_classes, float softcap, int64_t chunk, float* loss, uint16_t* dx,
                   uint16_t* dw, float* scales, void* ws, size_t ws_bytes, int accum, void* stream);

/* ------------------------------------------------------------------------ */
/* Muon's Newton-Schulz orthogonalisation of a bf16 matrix.                 */
/*                                                                          */
/* decomputer.nl, "Vroege experimenten" item 2 and the appendix: Muon for   */
/* the matrix parameters (lr 0.02, momentum 0.95); its Newton-Schulz        */
/* orthogonalisation costs about a quarter of a step.  The iteration is     */
/* Muon's published quintic one, on the wide orientation (X = G, or G^T     */
/* when rows > cols), each bf16 tensor formed with one rounding:            */
/*   X0 = RN_bf16(RN32(G / RN32(n + eps))),  n = RN32(||G||_F)  (fp64 sum)  */
/*   repeat `steps` times:                                                  */
/*     A = RN_bf16(X X^T)                          (symmetric, see below)    */
/*     B = RN_bf16(fma(c, A A, RN32(b A)))        (fp32 sum of the terms)    */
/*     X = RN_bf16(fma(1, B X, RN32(a X)))                                  */
/* with (a, b, c) = coeffs as fp32 numbers.  The products accumulate in     */
/* fp32 on the bf16 matrix cores; A and B are computed on their upper       */
/* triangle and mirrored (bf16_gemm_sym).                                   */
/* ------------------------------------------------------------------------ */

/* bf16 GEMM on the same matrix-core kernel as the FP8 linears:
 *   C[r, c] = RN_bf16(fma(alpha, sum_k A[r,k] B[c,k], RN32(beta aux[r, c])))
 * (aux NULL: RN_bf16(alpha sum)), and with ct non-NULL also ct[c, r] = C[r, c].
 * A [M,K] (lda), B [N,K] (ldb), aux / C [M,N] (ldaux / ldc), ct [N,M] (ldct),
 * all bf16, row-major.  aux may equal C (each element is read before it is
 * written, by the same thread); A, B and ct must not overlap C.
 * Requirements: K % 8 == 0; a, b 16-byte aligned, lda and ldb multiples of 8;
 * M, N >= 0 (ragged edges masked; K == 0 gives RN_bf16(RN32(beta aux))). */
int bf16_gemm_nt(const uint16_t* a, int64_t lda, const uint16_t* b, int64_t ldb, int64_t M, int64_t N, int64_t K,
                 float alpha, float beta, const uint16_t* aux, int64_t ldaux, uint16_t* c, int64_t ldc,
                 uint16_t* ct, int64_t ldct, void* stream);

/* Symmetric bf16 product C = RN_bf16(fma(alpha, A A^T, RN32(beta aux))) for
 * A [M,K] (lda) and aux [M,M] symmetric or NULL.  Only the upper triangle of
 * 256 x 256 tiles is multiplied, its K range split so that the tiles fill the
 * chip; the fp32 partial sums are added in a fixed order and each element
 * (i, j), i <= j, is written to both (i, j) and (j, i), so C is symmetric bit
 * for bit (aux contributes its (i, j) element to both).
 * Requirements: M % 16 == 0, K % 8 == 0; a, c 16-byte aligned, lda and ldc
 * multiples of 8; ws of bf16_gemm_sym_workspace_bytes(M, K) bytes, 16-byte
 * aligned; c must not overlap a, aux or ws. */
size_t bf16_gemm_sym_workspace_bytes(int64_t M, int64_t K);
int bf16_gemm_sym(const uint16_t* a, int64_t lda, int64_t M, int64_t K, float alpha, float beta,
                  const uint16_t* aux, int64_t ldaux, uint16_t* c, int64_t ldc, void* ws, size_t ws_bytes,
                  void* stream);

/* Workspace for muon_newton_schulz (0 if the shape is not supported): A and
 * B [m, m], two [n, m] buffers for X^T (one holds X for a tall G), the
 * symmetric products' partial sums and the norm's partial sums;
 * m = min(rows, cols), n = max(rows, cols). */
size_t muon_ns_workspace_bytes(int64_t rows, int64_t cols);

/*
 * g       [rows, cols] bf16, dense (row stride cols); not overwritten.
 * steps   0..100 (5 in Muon); steps == 0 returns X0.
 * coeffs  host pointer to {a, b, c}, or NULL for {3.4445, -4.7750, 2.0315}.
 * eps     added to the norm (1e-7 in Muon).
 * out     [rows, cols] bf16, dense; must not overlap g.
 * norm    out (device, may be NULL): 2 floats, n and the divisor RN32(n + eps).
 * Requirements: rows, cols multiples of 16 (0 valid: nothing to do);
 *               m <= 16384, n <= 1048576; g, out 16-byte aligned;
 *               ws of muon_ns_workspace_bytes(rows, cols) bytes, 16-byte aligned.
 */
int muon_newton_schulz(const uint16_t* g, int64_t rows, int64_t cols, int steps, const float* coeffs, float eps,
                       uint16_t* out, float* norm, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FP8MLP_H */
