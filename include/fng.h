/*
 * fng.h - C ABI of libfng.so: normalization fused into bf16 GEMM and attention
 * on AMD Instinct MI355X (gfx950).
 *
 * The operations follow "Towards Free Normalization: Fusing Normalization into
 * GEMM and Attention Kernels" (PyTorch blog):
 *   - section 2 (Lazy Pre-Norm): C = rmsnorm(A) @ B with the row statistic
 *     accumulated during the K loop and applied as an epilogue row scale;
 *   - sections 1 and 3 (naive full-N fusion, multi-CTA norm): C = norm(A @ B),
 *     LayerNorm or RMSNorm over each output row;
 *   - section 4 (FlashNormAttention): LayerNorm of the queries before the
 *     attention product and RMSNorm of its output after it.
 * Plus the unfused baselines those fusions replace (row norms, plain GEMM,
 * plain attention).
 *
 * Conventions for every entry point
 *   - Tensors are caller-owned device memory on the current HIP device,
 *     row-major and contiguous.  bf16 tensors are raw 16-bit bfloat16 bit
 *     patterns.  Statistics outputs are fp32.
 *   - Matrices: X is [M, K], W is [K, N] (N contiguous), Y is [M, N].
 *   - Attention tensors are [B, S, H, D] (D contiguous).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; no call synchronizes except fng_get_kernel_status.
 *   - Every call validates its arguments first and returns a status.  No call
 *     throws, prints, aborts or allocates device memory.  A failed validation
 *     enqueues nothing.
 *   - Inputs are never written.  Outputs are fully overwritten.  Outputs must
 *     not alias inputs, except Y == X for fng_rmsnorm / fng_layernorm.
 *   - Preconditions (checked): base pointers 16-byte aligned; for GEMM entry
 *     points K % 8 == 0 and N % 8 == 0 (rows are whole 16-byte vectors), K >= 1;
 *     for attention D == 128 and Skv >= 1; eps > 0.  M, N (GEMM) and B, Sq, H
 *     (attention) may be 0, which enqueues nothing and returns FNG_OK.  Tile
 *     tails in M, N, K and Sq, Skv are masked inside the kernels.
 *   - Optional outputs (rstd_out, mean_out, ...) may be NULL.
 *   - Accumulation and statistics are fp32; outputs are rounded to bf16 with
 *     round-to-nearest-even.
 */
#ifndef FNG_H
#define FNG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FNG_OK = 0,
  FNG_ERR_INVALID_ARG = 1, /* NULL required pointer, negative size, eps <= 0, ... */
  FNG_ERR_UNSUPPORTED = 2, /* shape outside what the kernels implement (e.g. D != 128) */
  FNG_ERR_MISALIGNED = 3,  /* pointer not 16-byte aligned, or K/N not a multiple of 8 */
  FNG_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than *_workspace_bytes() */
  FNG_ERR_HIP = 5,         /* the HIP runtime reported an error for a launch */
  FNG_ERR_TIMEOUT = 6      /* a split-N exchange wait hit its bound: 20 ms of real
                              time per wait (peers of one round are co-resident and
                              normally arrive within microseconds); see below */
} fng_status;

/* How a post-norm GEMM reduces statistics over N. */
typedef enum {
  FNG_PATH_AUTO = 0,    /* FULLN for N <= 256, and for N <= fng_fulln_max_n() when
                           K <= 512 or M >= 32768; else SPLITN when the grid fits,
                           else TWOPASS */
  FNG_PATH_FULLN = 1,   /* one workgroup owns whole output rows (section 1's naive
                           fusion); requires N <= fng_fulln_max_n() */
  FNG_PATH_SPLITN = 2,  /* N split over co-resident workgroups that exchange per-row
                           partial statistics through the workspace (section 3's
                           multi-CTA norm, without clusters) */
  FNG_PATH_TWOPASS = 3  /* GEMM kernel stores un-normalized bf16 Y plus partial
                           statistics, a second kernel normalizes Y in place
                           (the unfused IO the fusion removes; comparison/fallback) */
} fng_path;

/* ---------------------------------------------------------------------------
 * Lazy pre-RMSNorm GEMM (section 2, "Lazy Pre-Norm", the kernel pseudocode and
 * the row-scale commutation identity):
 *   rstd[m] = 1 / sqrt(mean_k X[m,k]^2 + eps)
 *   Y[m,n]  = rstd[m] * sum_k X[m,k] * gamma[k] * W[k,n]
 * i.e. Y = rmsnorm(X) * gamma @ W.  The statistic uses the raw X; gamma (bf16,
 * [K], optional: NULL means no affine) multiplies along K inside the product.
 * rstd_out: optional fp32 [M].  With rstd_out given (and no gain), a shape
 * that takes the big tiles in more than one round runs as two launches: the
 * one over the last partial round's columns (or the first round's columns)
 * accumulates each row's sum of squares beside its K loop and writes rstd,
 * the other applies it; without rstd_out every tile accumulates the
 * statistic beside its own K loop (the page's redundancy across CTAs).
 * ------------------------------------------------------------------------- */
int fng_prenorm_rms_gemm(const void* X, const void* W, const void* gamma, void* Y,
                         float* rstd_out, int64_t M, int64_t N, int64_t K, float eps,
                         void* stream);

/* The same operation with a caller workspace, for the two things the call
 * above cannot do without one:
 *   - with gamma (bf16 [K]), the gain is folded into the rows of W once per
 *     call by a streaming pass into the workspace (diag(gamma) W rounded to
 *     bf16, the rounding the in-loop fold makes), then the lazy kernel runs
 *     as without a gain; the in-loop fold of the call above scales each W
 *     value once per wave that reads it;
 *   - with rstd_out NULL, the statistic is still accumulated in one launch
 *     and handed to the other through the workspace (the call above then
 *     accumulates it beside every tile's K loop).
 * workspace: caller-owned device memory of
 * fng_prenorm_rms_gemm_workspace_bytes(M, N, K, gamma != NULL) bytes, no
 * initial contents needed, overwritten by each call (FNG_ERR_WORKSPACE if
 * NULL or smaller): rstd (M fp32, padded to 256 B), then diag(gamma) W when a
 * gain is given and the shape takes the big tiles.  Shapes, alignment,
 * limits and results as fng_prenorm_rms_gemm.  Up to three kernel launches
 * on `stream`. */
size_t fng_prenorm_rms_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int has_gamma);
int fng_prenorm_rms_gemm_ws(const void* X, const void* W, const void* gamma, void* Y,
                            float* rstd_out, int64_t M, int64_t N, int64_t K, float eps,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Lazy LayerNorm pre-norm (NOT on the page, which keeps lazy application to
 * RMSNorm because LayerNorm's elementwise part subtracts the mean): Y =
 * layernorm(X) @ W over K (biased variance, eps inside the root, no affine),
 * computed as diag(rstd) (X W - mean colsum(W)), a rank-1 correction in the
 * epilogue.  The row sums and sums of squares of the raw X are accumulated
 * beside the K loop (var = sumsq/K - mean^2, which loses digits when |mean|
 * is much larger than the row's spread); colsum(W) comes from a separate pass
 * over W (fixed-order fp32 partial sums).  Shapes, alignment and limits as
 * fng_prenorm_rms_gemm; optional fp32 [M] mean_out, rstd_out.  workspace:
 * caller-owned device memory of fng_prenorm_ln_workspace_bytes(N, K) bytes
 * (no initial contents needed; overwritten by each call), FNG_ERR_WORKSPACE if
 * NULL or smaller.  Two kernel launches (three with the tail split) on
 * `stream`; with both mean_out and rstd_out, as for fng_prenorm_rms_gemm, the
 * sums are taken by one launch over some column blocks and the other launch
 * applies diag(rstd) (X W - mean colsum(W)) from its mean_out / rstd_out. */
size_t fng_prenorm_ln_workspace_bytes(int64_t N, int64_t K);
int fng_prenorm_ln_gemm(const void* X, const void* W, void* Y, float* mean_out,
                        float* rstd_out, int64_t M, int64_t N, int64_t K, float eps,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * GEMM + post-norm (section 1 naive fusion and section 3 multi-CTA norm):
 *   Z = X @ W  (fp32 accumulation);  Y = norm(Z) over each row of N,
 * LayerNorm: Y = (Z - mean) / sqrt(var + eps), biased variance, no affine;
 * RMSNorm:   Y = Z / sqrt(mean(Z^2) + eps), no affine.
 * Statistics come from the fp32 accumulator, before the bf16 rounding.
 * mean_out (LN only) and rstd_out: optional fp32 [M].
 *
 * workspace: caller-owned device memory of at least
 * fng_gemm_postnorm_workspace_bytes(M, N, K, path) bytes, zero-filled ONCE
 * when allocated; the kernels keep it consistent for the next call.  It may
 * be NULL only when that size is 0.  Calls sharing one workspace must be
 * ordered (same stream).  The split-N grid is sized to what the GPU holds at
 * once (one workgroup per CU) and launched normally: its workgroups wait for
 * each other with a bounded wait.  On a GPU shared with other work that keeps
 * CUs busy past that bound, or after a fault, a call reports FNG_ERR_TIMEOUT
 * through fng_get_kernel_status; its Y is then invalid and the workspace must
 * be zero-filled again.  Between calls the workspace holds an epoch word
 * (bytes 4..7) that counts the split-N calls made on it.
 * ------------------------------------------------------------------------- */
size_t fng_gemm_postnorm_workspace_bytes(int64_t M, int64_t N, int64_t K, int path);
int64_t fng_fulln_max_n(void);

int fng_gemm_postnorm_ln(const void* X, const void* W, void* Y, float* mean_out,
                         float* rstd_out, int64_t M, int64_t N, int64_t K, float eps,
                         void* workspace, size_t workspace_bytes, int path, void* stream);

int fng_gemm_postnorm_rms(const void* X, const void* W, void* Y, float* rstd_out,
                          int64_t M, int64_t N, int64_t K, float eps, void* workspace,
                          size_t workspace_bytes, int path, void* stream);

/* The post-norm with its affine: Y = norm(X @ W) * gamma + beta over N
 * (gamma, beta bf16 [N], 16-byte aligned; beta may be NULL, gamma may not).
 * ln != 0: LayerNorm (mean_out used), else RMSNorm (mean_out ignored).  The
 * gain and bias are applied in fp32 in the same epilogue as the
 * normalization, before the single bf16 rounding (in the two-pass path, in its
 * second pass).  Paths, workspace and limits as fng_gemm_postnorm_ln. */
int fng_gemm_postnorm_affine(const void* X, const void* W, const void* gamma,
                             const void* beta, void* Y, float* mean_out, float* rstd_out,
                             int64_t M, int64_t N, int64_t K, float eps, int ln,
                             void* workspace, size_t workspace_bytes, int path, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * post-RMSNorm GEMM of fng_gemm_postnorm_rms without the workspace argument.
 * Its split-N / two-pass workspace is a fixed array of
 * FNG_NOALLOC_SCRATCH_BYTES (8 MiB) of device memory inside the library, one
 * per GPU, held until the process ends; the call allocates nothing.  Paths,
 * results and limits as fng_gemm_postnorm_rms, plus: a shape whose workspace
 * (fng_gemm_postnorm_workspace_bytes(M, N, K, path)) exceeds the array
 * returns FNG_ERR_WORKSPACE before anything is enqueued (the split-N path
 * fits M x N up to 16384 x 8192).  The first call on a device clears the
 * array (one small kernel on `stream`); every later call on that GPU reuses
 * it as the previous call left it.  All calls on one GPU share the one array:
 * calls that overlap in time (different streams, or other host threads)
 * race and give wrong results; order them.  A split-N wait that hits its
 * bound cannot be read back with fng_get_kernel_status (the caller has no
 * workspace pointer): the rows it concerns are written as NaN instead. */
#define FNG_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int fng_gemm_postnorm_rms_noalloc(const void* X, const void* W, void* Y, float* rstd_out,
                                  int64_t M, int64_t N, int64_t K, float eps, int path,
                                  void* stream);

/* Reads the status word a split-N call leaves in `workspace` (synchronizes
 * `stream`).  Returns FNG_OK, FNG_ERR_TIMEOUT, or a validation/HIP error. */
int fng_get_kernel_status(const void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Backward by fusion regrouping (section 3, "What about backward?"): the norm
 * backward is the epilogue of the GEMM that produces its upstream gradient,
 * so it stays an epilogue fusion (the forward's full-N and split-N paths).
 *   dZ = norm_backward(G @ Wt), rows of length N, with the forward's outputs:
 *     LayerNorm:  dZ = rstd * (g - mean(g) - Y * mean(g * Y))
 *     RMSNorm:    dZ = rstd * (g - Y * mean(g * Y))
 * G [M, K]: the gradient at the output of the layer after the norm; Wt [K, N]:
 * that layer's weight read as [K, N] (a torch Linear's weight [out, in] as
 * stored); Y [M, N]: the norm's forward output (bf16); rstd [M]: its forward
 * statistic (fp32).  dZ [M, N] is the gradient at the norm's input.  `path`:
 * FNG_PATH_AUTO, FULLN (N <= fng_fulln_max_n()) or SPLITN (workspace of
 * fng_gemm_postnorm_workspace_bytes(M, N, K, FNG_PATH_SPLITN) bytes, zeroed
 * once, as the forward's); TWOPASS returns FNG_ERR_UNSUPPORTED.  AUTO takes
 * the forward's choice, except that for N > 256 it takes split-N whenever
 * `workspace` holds at least the split-N size (faster there than the full-N
 * backward tiles), unless M >= 65536, N <= 512 and K <= 1024 (then full-N,
 * whose tiles for such tall inputs are faster); a smaller or NULL workspace
 * keeps the forward's choice.
 * M*N*2 must be below 2^31.  G, Wt, Y, dZ 16-byte aligned; rstd 4-byte
 * aligned.
 * ------------------------------------------------------------------------- */
int fng_gemm_postnorm_ln_bwd(const void* G, const void* Wt, const void* Y, const float* rstd, void* dZ,
                             int64_t M, int64_t N, int64_t K, void* workspace,
                             size_t workspace_bytes, int path, void* stream);
int fng_gemm_postnorm_rms_bwd(const void* G, const void* Wt, const void* Y, const float* rstd, void* dZ,
                              int64_t M, int64_t N, int64_t K, void* workspace,
                              size_t workspace_bytes, int path, void* stream);
/* Input gradient of the lazy pre-RMSNorm GEMM Y = rmsnorm(X) @ W (section 2;
 * the normalized X is rebuilt from X and the forward rstd, never stored):
 *   dX = rstd * (g - xhat * mean(g * xhat)),  g = dY @ Wt,  xhat = X * rstd
 * with the forward's sizes: dY [M, N], Wt [N, K] (W transposed, a torch
 * Linear's weight as stored), X and dX [M, K], rstd [M].  The norm runs over
 * K: paths and workspace as above with (M, K, N) in place of (M, N, K).  The
 * weight gradient is fng_prenorm_rms_bwd_dw below. */
int fng_prenorm_rms_bwd_dx(const void* dY, const void* Wt, const void* X, const float* rstd, void* dX,
                           int64_t M, int64_t N, int64_t K, void* workspace,
                           size_t workspace_bytes, int path, void* stream);

/* Weight gradient of the lazy pre-RMSNorm GEMM Y = (rmsnorm(X) * gamma) @ W
 * (section 2's limitations: the normalized X has to be rebuilt from X and rstd
 * for the gradients of both operands, not only dX):
 *   dW[k, n] = gamma[k] * sum_m X[m, k] * rstd[m] * dY[m, n]
 * i.e. dW = (rmsnorm(X) * gamma)^T @ dY with rstd applied along the
 * contraction (the batch rows) inside the product; rmsnorm(X) is never
 * written.  X [M, K] bf16 (the forward's input), rstd fp32 [M] (the forward's
 * rstd_out), dY [M, N] bf16, gamma bf16 [K] or NULL (the forward's gain),
 * dW [K, N] bf16 (W's layout), fully overwritten.  rstd NULL (gamma NULL
 * then too) computes the plain X^T @ dY: the product an unfused chain runs
 * after writing rmsnorm(X) out, here as its baseline.  X, dY, dW, gamma and rstd
 * 16-byte aligned; K % 8 == 0, N % 8 == 0; M >= 1 (FNG_ERR_INVALID_ARG for
 * M == 0: an empty batch has a zero gradient the call does not write);
 * K or N == 0 enqueues nothing.  Products are bf16 MFMAs with fp32
 * accumulation; each dY value is multiplied by its row's rstd in fp32 and
 * rounded to bf16 once before the product.  One kernel launch (two with the
 * tail split of the last partial round of tiles) on `stream`. */
int fng_prenorm_rms_bwd_dw(const void* X, const float* rstd, const void* dY, const void* gamma,
                           void* dW, int64_t M, int64_t N, int64_t K, void* stream);

/* ---------------------------------------------------------------------------
 * Norm-sandwiched attention (section 4, FlashNormAttention, in its per-head,
 * softmax, no-residual form):
 *   for each (b, h):  q^ = layernorm(Q[b,:,h,:]) over D   (eps_ln, no affine)
 *                     P  = softmax(q^ K[b,:,h,:]^T * sm_scale) over all keys
 *                     O  = P V[b,:,h,:]
 *                     out[b,:,h,:] = rmsnorm(O) over D    (eps_rms, no affine)
 * Q, out: [B, Sq, H, D]; K, V: [B, Skv, H, D]; D must be 128.  Non-causal.
 * sm_scale <= 0 selects 1/sqrt(D).  Optional fp32 [B, Sq, H] statistics outputs.
 * K and V magnitudes must be below 65504 (the kernel multiplies in fp16 with
 * fp32 accumulation; bf16 inputs in that range convert to fp16 exactly down to
 * 2^-14).  The normalized queries are pre-multiplied by sm_scale * log2(e)
 * before their fp16 rounding.
 * ------------------------------------------------------------------------- */
int fng_norm_attention(const void* Q, const void* K, const void* V, void* out,
                       float* ln_mean_out, float* ln_rstd_out, float* rms_rstd_out,
                       int64_t B, int64_t Sq, int64_t Skv, int64_t H, int64_t D,
                       float sm_scale, float eps_ln, float eps_rms, void* stream);

/* ---------------------------------------------------------------------------
 * Full FlashNormAttention (section 4, the fused short-KV kernel), on jagged
 * queries.  Q and out are [T, H, D] (rows of all batches back to back; batch
 * b owns rows q_offsets[b] .. q_offsets[b+1]-1); K and V are [B, Skv, H, D]
 * dense.  For every query row x (all H*D values of one row):
 *     ln  = layernorm(x) over all H*D values           (eps_ln, no affine)
 *     o_h = act(ln_h K[b,:,h,:]^T * sm_scale) V[b,:,h,:] + ln_h
 *     out = rmsnorm(o) over all H*D values + x         (eps_rms, no affine)
 * act: FNG_ACT_SOFTMAX (over the keys, non-causal) or FNG_ACT_GELU
 * (elementwise, tanh form).  sm_scale <= 0 selects 1/sqrt(D).
 * q_offsets: int32 DEVICE memory, [B + 1], non-decreasing, q_offsets[0] >= 0,
 *   q_offsets[B] <= T, every batch length <= max_len_q.  The contents are not
 *   checked on the host; the kernel never reads or writes outside Q, out and
 *   the statistics buffers whatever they hold, but rows a batch owns beyond
 *   max_len_q, and rows no batch owns, are left unwritten.
 * H must be 1, 2, 4 or 8 and D 128; Skv >= 1 (H = 8: one workgroup of eight
 * waves per 32 query rows, one wave per head).  Optional fp32 [T] statistics:
 * ln mean and rstd, rms rstd (the backward below takes them).  Products are
 * bf16 MFMAs with fp32 accumulation: K and V as stored, the normalized
 * queries (pre-multiplied by sm_scale, times log2(e) for softmax) and the
 * activations split into bf16 high and low parts (about 16 significant bits).
 * ------------------------------------------------------------------------- */
typedef enum { FNG_ACT_SOFTMAX = 0, FNG_ACT_GELU = 1 } fng_act_t;

int fng_flash_norm_attention(const void* Q, const int32_t* q_offsets, const void* K,
                             const void* V, void* out, float* ln_mean_out,
                             float* ln_rstd_out, float* rms_rstd_out, int64_t B,
                             int64_t T, int64_t max_len_q, int64_t Skv, int64_t H,
                             int64_t D, float sm_scale, float eps_ln, float eps_rms,
                             int act, void* stream);

/* Backward of fng_flash_norm_attention (section 4, "Backward implementation"):
 * given dout = d loss / d out [T, H, D], writes dQ [T, H, D] and dK, dV
 * [B, Skv, H, D] (bf16), the exact gradients of the forward above.  As on the
 * page only per-row statistics are kept from the forward: the LayerNorm
 * output is rebuilt from Q, ln_mean and ln_rstd and the RMSNorm output as
 * out - Q (out = the forward's output); the softmax's row term
 * sum_keys P * dP comes from the recomputed scores.
 *   Q, out, dout: [T, H, D] bf16; K, V: [B, Skv, H, D] bf16;
 *   ln_mean, ln_rstd, rms_rstd: fp32 [T], the forward's statistics outputs;
 *   q_offsets, B, T, max_len_q, H, D, sm_scale, act: as in the forward call.
 * dQ rows a batch owns beyond max_len_q, and rows no batch owns, are left
 * unwritten; those rows contribute nothing to dK and dV.  Every dK, dV entry
 * is written (zero for batches without rows).
 * workspace: caller-owned device memory of
 * fng_flash_norm_attention_bwd_workspace_bytes(T, H) bytes, no initial
 * contents needed (the first kernel writes per-row intermediates that the
 * second reads: the gradient at the RMSNorm input in fp16, and for the
 * softmax the log-sum-exp per (row, head)); FNG_ERR_WORKSPACE if NULL or
 * smaller.  Limits: H 1, 2, 4 or 8; D 128; 1 <= Skv <= 128 (the page's short-KV
 * case: a query row's scores over all keys stay in registers).  Products are
 * fp16 MFMAs with fp32 accumulation (K and V converted from bf16, so below
 * 65504 in magnitude).  Two kernel launches on `stream`. */
size_t fng_flash_norm_attention_bwd_workspace_bytes(int64_t T, int64_t H);

/* Backward of fng_jagged_attention (the attention step without norms or
 * residuals: the unfused chain's attention, whose backward the fused call
 * above replaces together with the norm and residual backward passes):
 * given dout [T, H, D], writes dQ [T, H, D] and dK, dV [B, Skv, H, D] (bf16),
 * with s = Q K^T sm_scale, P = act(s): dV = P^T dout, dS = act'(s, dout V^T)
 * sm_scale, dQ = dS K, dK = dS^T Q (summed over each batch's rows).  The
 * same two kernels as fng_flash_norm_attention_bwd without their norm and
 * residual terms.  Arguments, workspace
 * (fng_flash_norm_attention_bwd_workspace_bytes(T, H) bytes, no initial
 * contents needed), limits, unwritten rows and precision as there. */
int fng_jagged_attention_bwd(const void* Q, const int32_t* q_offsets, const void* K, const void* V,
                             const void* dout, void* dQ, void* dK, void* dV, void* workspace,
                             size_t workspace_bytes, int64_t B, int64_t T, int64_t max_len_q,
                             int64_t Skv, int64_t H, int64_t D, float sm_scale, int act, void* stream);
int fng_flash_norm_attention_bwd(const void* Q, const int32_t* q_offsets, const void* K,
                                 const void* V, const void* out, const void* dout,
                                 const float* ln_mean, const float* ln_rstd,
                                 const float* rms_rstd, void* dQ, void* dK, void* dV,
                                 void* workspace, size_t workspace_bytes, int64_t B,
                                 int64_t T, int64_t max_len_q, int64_t Skv, int64_t H,
                                 int64_t D, float sm_scale, int act, void* stream);

/* ---------------------------------------------------------------------------
 * Unfused baselines (the separate kernels the fusions replace; section 1
 * describes the standalone row norm that loads whole rows).
 * ------------------------------------------------------------------------- */
/* Y = rmsnorm(X) * gamma over rows of length N; gamma bf16 [N] or NULL. */
int fng_rmsnorm(const void* X, const void* gamma, void* Y, float* rstd_out, int64_t M,
                int64_t N, float eps, void* stream);
/* Y = layernorm(X) over rows of length N (biased variance, no affine). */
int fng_layernorm(const void* X, void* Y, float* mean_out, float* rstd_out, int64_t M,
                  int64_t N, float eps, void* stream);
/* Unfused norm backward over rows of length N (the regrouped GEMM's baseline):
 * dZ = rstd * (G - mean(G) - Y * mean(G * Y)) (LayerNorm), Y the forward output;
 * dZ = rstd * (G - xhat * mean(G * xhat)) (RMSNorm), xhat = H, or H * rstd when
 * h_is_input (H is then the norm's input).  G, H/Y, dZ [M, N] bf16, rstd [M]. */
int fng_layernorm_bwd(const void* G, const void* Y, const float* rstd, void* dZ, int64_t M,
                      int64_t N, void* stream);
int fng_rmsnorm_bwd(const void* G, const void* H, const float* rstd, void* dZ, int64_t M,
                    int64_t N, int h_is_input, void* stream);
/* Y = X @ W in bf16 with fp32 accumulation (same mainloop as the fused GEMMs). */
int fng_gemm(const void* X, const void* W, void* Y, int64_t M, int64_t N, int64_t K,
             void* stream);
/* out = softmax(Q K^T * sm_scale) V, BSHD, D == 128, same kernel as
 * fng_norm_attention without the two norms.  Q * sm_scale * log2(e), K and V
 * must stay below 65504 in magnitude (fp16 MFMA operands). */
int fng_attention(const void* Q, const void* K, const void* V, void* out, int64_t B,
                  int64_t Sq, int64_t Skv, int64_t H, int64_t D, float sm_scale,
                  void* stream);

/* out = act(Q K^T * sm_scale) V per head on jagged queries: the attention of
 * fng_flash_norm_attention without its norms and residuals (same layouts,
 * offsets contract, limits and kernel). */
int fng_jagged_attention(const void* Q, const int32_t* q_offsets, const void* K,
                         const void* V, void* out, int64_t B, int64_t T, int64_t max_len_q,
                         int64_t Skv, int64_t H, int64_t D, float sm_scale, int act,
                         void* stream);

/* ---------------------------------------------------------------------------
 * Misc.
 * ------------------------------------------------------------------------- */
const char* fng_status_string(int status);
int fng_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FNG_H */
