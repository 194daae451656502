// Internal interface between the C ABI (fng_api.cpp) and the kernel files.
// Arguments reaching these launchers have already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fng.h"

namespace fng {

struct GemmCall {
  const void* X;
  const void* W;
  const void* gamma;  // bf16 [K] or nullptr
  void* Y;
  float* mean_out;
  float* rstd_out;
  int64_t M, N, K;
  float eps;
  void* part;         // split-N / two-pass partials
  uint32_t* cnt;
  uint32_t* done;
  uint32_t* status;
  const void* beta;   // post-norm affine: bf16 [N] bias (with gamma [N] as gain), or nullptr
  bool poison_on_timeout = false;  // split-N: write NaN rows where an exchange wait timed out
};

// fng_gemm.hip
int launch_gemm(const GemmCall& c, hipStream_t s);
int launch_prenorm(const GemmCall& c, hipStream_t s);
// the same with a caller workspace (see fng_prenorm_rms_gemm_ws): [rstd, M fp32, 256-B aligned]
// [gamma-scaled W, K x N bf16, when prenorm_ws_needs_wg(M, N) and a gain is given]
int launch_prenorm_ws(const GemmCall& c, void* ws, hipStream_t s);
bool prenorm_ws_needs_wg(int64_t M, int64_t N);
// lazy LayerNorm pre-norm: colsum receives prenorm_ln_parts(K) x N fp32 partial column sums of W
int launch_prenorm_ln(const GemmCall& c, float* colsum, hipStream_t s);
int prenorm_ln_parts(int64_t K);
int launch_postnorm_fulln(const GemmCall& c, bool ln, hipStream_t s);
// fng_fulln.hip: the full-N post-norm for K <= 256 and N <= 256 (W resident in LDS)
bool fulln_small_fits(int64_t N, int64_t K);
int launch_postnorm_fulln_small(const GemmCall& c, bool ln, hipStream_t s);
int launch_postnorm_splitn(const GemmCall& c, bool ln, hipStream_t s);
int launch_postnorm_partial(const GemmCall& c, bool ln, hipStream_t s);
// norm backward epilogue inputs: H = xhat [M, N] (or the norm's input when
// h_raw, xhat = H * rstd), rstd [M] from the forward
struct NormBwdArgs {
  const void* H;
  const float* rstd;
  bool h_raw;
};
int launch_norm_bwd_fulln(const GemmCall& c, const NormBwdArgs& b, bool ln, hipStream_t s);
int launch_norm_bwd_splitn(const GemmCall& c, const NormBwdArgs& b, bool ln, hipStream_t s);
// weight gradient of the lazy pre-RMSNorm GEMM: dW [K, N] = (X * rstd (* gamma))^T dY
int launch_prenorm_dw(const void* X, const float* rstd, const void* dY, const void* gamma, void* dW, int64_t M,
                      int64_t N, int64_t K, hipStream_t s);
int splitn_feasible(int64_t M, int64_t N);
int64_t splitn_tiles_m(int64_t M);
int64_t splitn_tiles_n(int64_t N);
int64_t splitn_bm();
int64_t fulln_max_n();
// the norm backward's full-N tiles for >= 65536 rows (one row block per
// workgroup, 256 x <= 256 or 128 x 512)
bool bwd_fulln_tall(int64_t M);

// fng_norm.hip
int launch_rownorm_bwd(const void* G, const void* H, const float* rstd, void* dZ, int64_t M, int64_t N,
                       bool h_raw, bool ln, hipStream_t s);
int launch_rownorm(const void* X, const void* gamma, void* Y, float* mean_out, float* rstd_out,
                   int64_t M, int64_t N, float eps, bool ln, hipStream_t s);
// second pass of the two-pass post-norm: merge per-tile partials, normalize Y in place
int launch_postnorm_finalize(void* Y, const void* part, float* mean_out, float* rstd_out,
                             int64_t M, int64_t N, int64_t tiles_n, int64_t bm, int64_t bn,
                             float eps, bool ln, const void* gamma, const void* beta, hipStream_t s);

// fng_attention.hip
struct AttnCall {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* ln_mean_out;
  float* ln_rstd_out;
  float* rms_rstd_out;
  int64_t B, Sq, Skv, H, D;
  float sm_scale, eps_ln, eps_rms;
};
int launch_attention(const AttnCall& c, bool norm, hipStream_t s);

// fng_fna.hip
struct FnaCall {
  const void* Q;
  const int32_t* offsets;
  const void* K;
  const void* V;
  void* O;
  float* ln_mean_out;
  float* ln_rstd_out;
  float* rms_rstd_out;
  int64_t B, T, max_len, Skv, H;
  float sm_scale, eps_ln, eps_rms;
  int act;
};
int launch_fna(const FnaCall& c, bool norm, hipStream_t s);

// fng_fna_bwd.hip
struct FnaBwdCall {
  const void* Q;
  const int32_t* offsets;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  const float* ln_mean;
  const float* ln_rstd;
  const float* rms_rstd;
  void* dQ;
  void* dK;
  void* dV;
  void* workspace;   // fna_bwd_workspace_bytes(T, H) bytes
  int64_t B, T, max_len, Skv, H;
  float sm_scale;
  int act;
};
// norm = false: the plain jagged attention's backward (Q, K, V, dO; no statistics, no output)
int launch_fna_bwd(const FnaBwdCall& c, bool norm, hipStream_t s);
size_t fna_bwd_workspace_bytes(int64_t T, int64_t H);

}  // namespace fng
