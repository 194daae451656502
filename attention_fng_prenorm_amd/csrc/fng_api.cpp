// C ABI of libfng.so: argument validation and dispatch to the HIP kernels.
// Every entry point validates before touching the HIP runtime, so a rejected
// call enqueues nothing.  Semantics and conventions are documented in
// include/fng.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fng_internal.h"

#include <mutex>

#define FNG_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

using fng::GemmCall;

constexpr int kVersion = 1;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// common GEMM validation; returns FNG_OK or the error
int check_gemm(const void* X, const void* W, const void* Y, int64_t M, int64_t N, int64_t K, float eps,
               bool need_eps) {
  if (M < 0 || N < 0 || K < 1) return FNG_ERR_INVALID_ARG;
  if (need_eps && !(eps > 0.f && isfinite(eps))) return FNG_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return FNG_OK;
  if (!X || !W || !Y) return FNG_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(W) || !aligned16(Y)) return FNG_ERR_MISALIGNED;
  if (K % 8 != 0 || N % 8 != 0) return FNG_ERR_MISALIGNED;
  // 32-bit index and buffer-range limits of the kernels
  if (M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return FNG_ERR_UNSUPPORTED;
  if ((K + 256) * N * 2 >= (int64_t)INT32_MAX) return FNG_ERR_UNSUPPORTED;   // W (+ K-tile overrun) below 2 GiB
  if ((256 + 1) * K * 2 >= (int64_t)INT32_MAX) return FNG_ERR_UNSUPPORTED;  // one X row block below 2 GiB
  if (M * N >= ((int64_t)1 << 46)) return FNG_ERR_UNSUPPORTED;
  return FNG_OK;
}

bool m_or_n_empty(int64_t M, int64_t N) { return M == 0 || N == 0; }

struct Workspace {
  float* part;
  uint32_t* cnt;
  uint32_t* done;
  uint32_t* status;
  size_t bytes;
};

// layout: [status (256 B): timeout flag, epoch, finished workgroups] [cnt: tiles_m u32, unused]
// [done: tiles_m u32, unused] (256-B aligned) [partials]
size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

Workspace layout(void* base, int64_t M, int64_t N) {
  const int64_t tm = fng::splitn_tiles_m(M), tn = fng::splitn_tiles_n(N), bm = fng::splitn_bm();
  char* b = static_cast<char*>(base);
  Workspace w{};
  size_t off = 0;
  w.status = reinterpret_cast<uint32_t*>(b + off);
  off += 256;
  w.cnt = reinterpret_cast<uint32_t*>(b + off);
  off += align256((size_t)tm * 4);
  w.done = reinterpret_cast<uint32_t*>(b + off);
  off += align256((size_t)tm * 4);
  w.part = reinterpret_cast<float*>(b + off);
  // split-N: two 64-bit (value, epoch tag) entries per row and tile; the
  // two-pass path uses the same region as plain floats
  off += (size_t)tm * tn * bm * 2 * sizeof(uint64_t);
  w.bytes = off;
  return w;
}

// automatic choice, from the measured post-LayerNorm sweep over M = 256k rows
// and K, N in 64..2048: one workgroup across N wins up to N = 256, and at
// N = 512 with the 128 x 512 tiles (M >= 32768) at every K, with the 64 x 512
// tiles while K <= 512; beyond that the split-N exchange wins
bool auto_fulln(int64_t M, int64_t N, int64_t K) {
  return N <= 256 || (N <= fng::fulln_max_n() && (K <= 512 || M >= 32768));
}

int resolve_path(int path, int64_t M, int64_t N, int64_t K) {
  if (path == FNG_PATH_AUTO) {
    if (auto_fulln(M, N, K)) return FNG_PATH_FULLN;
    if (fng::splitn_feasible(M, N)) return FNG_PATH_SPLITN;
    return FNG_PATH_TWOPASS;
  }
  return path;
}

int postnorm(bool ln, const void* X, const void* W, void* Y, float* mean_out, float* rstd_out, int64_t M,
             int64_t N, int64_t K, float eps, void* workspace, size_t workspace_bytes, int path,
             void* stream, const void* gamma = nullptr, const void* beta = nullptr, bool poison = false) {
  int st = check_gemm(X, W, Y, M, N, K, eps, true);
  if (st != FNG_OK) return st;
  if (path < FNG_PATH_AUTO || path > FNG_PATH_TWOPASS) return FNG_ERR_INVALID_ARG;
  if (m_or_n_empty(M, N)) return FNG_OK;
  if ((mean_out && !aligned16(mean_out)) || (rstd_out && !aligned16(rstd_out))) return FNG_ERR_MISALIGNED;
  if ((gamma && !aligned16(gamma)) || (beta && !aligned16(beta))) return FNG_ERR_MISALIGNED;
  path = resolve_path(path, M, N, K);
  GemmCall c{X, W, gamma, Y, mean_out, rstd_out, M, N, K, eps, nullptr, nullptr, nullptr, nullptr, beta, poison};
  if (path == FNG_PATH_FULLN) {
    if (N > fng::fulln_max_n()) return FNG_ERR_UNSUPPORTED;
    return fng::launch_postnorm_fulln(c, ln, as_stream(stream));
  }
  const size_t need = fng_gemm_postnorm_workspace_bytes(M, N, K, path);
  if (!workspace || workspace_bytes < need) return FNG_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FNG_ERR_MISALIGNED;
  Workspace w = layout(workspace, M, N);
  c.part = w.part;
  c.cnt = w.cnt;
  c.done = w.done;
  c.status = w.status;
  if (path == FNG_PATH_SPLITN) {
    if (!fng::splitn_feasible(M, N)) return FNG_ERR_UNSUPPORTED;
    return fng::launch_postnorm_splitn(c, ln, as_stream(stream));
  }
  st = fng::launch_postnorm_partial(c, ln, as_stream(stream));
  if (st != FNG_OK) return st;
  return fng::launch_postnorm_finalize(Y, w.part, mean_out, rstd_out, M, N, fng::splitn_tiles_n(N),
                                       fng::splitn_bm(), 256, eps, ln, gamma, beta, as_stream(stream));
}

int check_attn(const void* Q, const void* K, const void* V, const void* O, int64_t B, int64_t Sq,
               int64_t Skv, int64_t H, int64_t D) {
  if (B < 0 || Sq < 0 || H < 0 || Skv < 1 || D < 1) return FNG_ERR_INVALID_ARG;
  if (D != 128) return FNG_ERR_UNSUPPORTED;
  if (B == 0 || Sq == 0 || H == 0) return FNG_OK;
  if (!Q || !K || !V || !O) return FNG_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return FNG_ERR_MISALIGNED;
  // per-batch 32-bit buffer ranges (with one tile of overrun: 256 query rows,
  // 64 key rows) and the grid size
  if ((Sq + 256) * H * D * 2 >= (int64_t)INT32_MAX) return FNG_ERR_UNSUPPORTED;
  if ((Skv + 64) * H * D * 2 >= (int64_t)INT32_MAX) return FNG_ERR_UNSUPPORTED;
  if (B * H * ((Sq + 255) / 256) >= (int64_t)INT32_MAX) return FNG_ERR_UNSUPPORTED;
  return FNG_OK;
}

int check_fna(const void* Q, const int32_t* off, const void* K, const void* V, const void* O,
              int64_t B, int64_t T, int64_t max_len, int64_t Skv, int64_t H, int64_t D, int act) {
  if (B < 0 || T < 0 || max_len < 0 || H < 0 || Skv < 1 || D < 1) return FNG_ERR_INVALID_ARG;
  if (act != FNG_ACT_SOFTMAX && act != FNG_ACT_GELU) return FNG_ERR_INVALID_ARG;
  if (D != 128) return FNG_ERR_UNSUPPORTED;
  if (B == 0 || T == 0 || max_len == 0 || H == 0) return FNG_OK;
  if (H != 1 && H != 2 && H != 4 && H != 8) return FNG_ERR_UNSUPPORTED;
  if (!Q || !off || !K || !V || !O) return FNG_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || (uintptr_t)off % 4 != 0)
    return FNG_ERR_MISALIGNED;
  // 32-bit row indices and per-batch buffer ranges (one block of query rows
  // and one 32-key tile of overrun), and the grid size
  if (T >= (int64_t)INT32_MAX || B >= (int64_t)INT32_MAX) return FNG_ERR_UNSUPPORTED;
  if ((max_len + 256) * H * D * 2 >= (int64_t)INT32_MAX) return FNG_ERR_UNSUPPORTED;
  if ((Skv + 32) * H * D * 2 >= (int64_t)INT32_MAX) return FNG_ERR_UNSUPPORTED;
  if (B * ((max_len + 255) / 32) >= (int64_t)INT32_MAX) return FNG_ERR_UNSUPPORTED;
  return FNG_OK;
}

}  // namespace

FNG_EXPORT int fng_version(void) { return kVersion; }

FNG_EXPORT const char* fng_status_string(int status) {
  switch (status) {
    case FNG_OK: return "ok";
    case FNG_ERR_INVALID_ARG: return "invalid argument";
    case FNG_ERR_UNSUPPORTED: return "unsupported shape or path";
    case FNG_ERR_MISALIGNED: return "misaligned pointer or dimension";
    case FNG_ERR_WORKSPACE: return "workspace missing or too small";
    case FNG_ERR_HIP: return "HIP runtime error";
    case FNG_ERR_TIMEOUT: return "split-N exchange wait timed out";
    default: return "unknown status";
  }
}

FNG_EXPORT int64_t fng_fulln_max_n(void) { return fng::fulln_max_n(); }

FNG_EXPORT size_t fng_gemm_postnorm_workspace_bytes(int64_t M, int64_t N, int64_t K, int path) {
  if (M <= 0 || N <= 0) return 0;
  if (path == FNG_PATH_FULLN) return 0;
  if (path == FNG_PATH_AUTO && auto_fulln(M, N, K)) return 0;
  return layout(nullptr, M, N).bytes;
}

FNG_EXPORT int fng_prenorm_rms_gemm(const void* X, const void* W, const void* gamma, void* Y,
                                    float* rstd_out, int64_t M, int64_t N, int64_t K, float eps,
                                    void* stream) {
  const int st = check_gemm(X, W, Y, M, N, K, eps, true);
  if (st != FNG_OK || m_or_n_empty(M, N)) return st;
  if ((gamma && !aligned16(gamma)) || (rstd_out && !aligned16(rstd_out))) return FNG_ERR_MISALIGNED;
  GemmCall c{X, W, gamma, Y, nullptr, rstd_out, M, N, K, eps, nullptr, nullptr, nullptr, nullptr};
  return fng::launch_prenorm(c, as_stream(stream));
}

FNG_EXPORT size_t fng_prenorm_rms_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int has_gamma) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  size_t b = ((size_t)M * 4 + 255) & ~(size_t)255;
  if (has_gamma && fng::prenorm_ws_needs_wg(M, N)) b += (size_t)K * (size_t)N * 2;
  return b;
}

FNG_EXPORT int fng_prenorm_rms_gemm_ws(const void* X, const void* W, const void* gamma, void* Y, float* rstd_out,
                                       int64_t M, int64_t N, int64_t K, float eps, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  const int st = check_gemm(X, W, Y, M, N, K, eps, true);
  if (st != FNG_OK || m_or_n_empty(M, N)) return st;
  if ((gamma && !aligned16(gamma)) || (rstd_out && !aligned16(rstd_out))) return FNG_ERR_MISALIGNED;
  if (!workspace || workspace_bytes < fng_prenorm_rms_gemm_workspace_bytes(M, N, K, gamma != nullptr))
    return FNG_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FNG_ERR_MISALIGNED;
  GemmCall c{X, W, gamma, Y, nullptr, rstd_out, M, N, K, eps, nullptr, nullptr, nullptr, nullptr};
  return fng::launch_prenorm_ws(c, workspace, as_stream(stream));
}

FNG_EXPORT size_t fng_prenorm_ln_workspace_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0) return 0;
  return (size_t)fng::prenorm_ln_parts(K) * (size_t)N * 4;
}

FNG_EXPORT int fng_prenorm_ln_gemm(const void* X, const void* W, void* Y, float* mean_out, float* rstd_out,
                                   int64_t M, int64_t N, int64_t K, float eps, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  const int st = check_gemm(X, W, Y, M, N, K, eps, true);
  if (st != FNG_OK || m_or_n_empty(M, N)) return st;
  if ((mean_out && !aligned16(mean_out)) || (rstd_out && !aligned16(rstd_out))) return FNG_ERR_MISALIGNED;
  if (!workspace || workspace_bytes < fng_prenorm_ln_workspace_bytes(N, K)) return FNG_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FNG_ERR_MISALIGNED;
  GemmCall c{X, W, nullptr, Y, mean_out, rstd_out, M, N, K, eps, nullptr, nullptr, nullptr, nullptr};
  return fng::launch_prenorm_ln(c, static_cast<float*>(workspace), as_stream(stream));
}

FNG_EXPORT int fng_gemm_postnorm_ln(const void* X, const void* W, void* Y, float* mean_out, float* rstd_out,
                                    int64_t M, int64_t N, int64_t K, float eps, void* workspace,
                                    size_t workspace_bytes, int path, void* stream) {
  return postnorm(true, X, W, Y, mean_out, rstd_out, M, N, K, eps, workspace, workspace_bytes, path, stream);
}

FNG_EXPORT int fng_gemm_postnorm_affine(const void* X, const void* W, const void* gamma, const void* beta,
                                        void* Y, float* mean_out, float* rstd_out, int64_t M, int64_t N,
                                        int64_t K, float eps, int ln, void* workspace, size_t workspace_bytes,
                                        int path, void* stream) {
  if (!gamma && M > 0 && N > 0) return FNG_ERR_INVALID_ARG;
  return postnorm(ln != 0, X, W, Y, ln ? mean_out : nullptr, rstd_out, M, N, K, eps, workspace, workspace_bytes,
                  path, stream, gamma, beta);
}

FNG_EXPORT int fng_gemm_postnorm_rms(const void* X, const void* W, void* Y, float* rstd_out, int64_t M,
                                     int64_t N, int64_t K, float eps, void* workspace,
                                     size_t workspace_bytes, int path, void* stream) {
  return postnorm(false, X, W, Y, nullptr, rstd_out, M, N, K, eps, workspace, workspace_bytes, path, stream);
}

namespace {

// dZ = norm_backward(G @ Wt) over rows of length N; xhat = H (h_raw: H * rstd)
int norm_bwd(bool ln, const void* G, const void* Wt, const void* H, const float* rstd, bool h_raw, void* dZ,
             int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes, int path, void* stream) {
  int st = check_gemm(G, Wt, dZ, M, N, K, 1.f, false);
  if (st != FNG_OK) return st;
  if (path < FNG_PATH_AUTO || path > FNG_PATH_TWOPASS) return FNG_ERR_INVALID_ARG;
  if (m_or_n_empty(M, N)) return FNG_OK;
  if (!H || !rstd) return FNG_ERR_INVALID_ARG;
  if (!aligned16(H) || reinterpret_cast<uintptr_t>(rstd) % 4 != 0) return FNG_ERR_MISALIGNED;
  if (M * N * 2 >= (int64_t)INT32_MAX) return FNG_ERR_UNSUPPORTED;  // the saved tensor's 32-bit copy offsets
  if (path == FNG_PATH_TWOPASS) return FNG_ERR_UNSUPPORTED;        // the backward has no two-pass path
  // automatic choice: above 256 columns the full-N backward tiles of 64 x 512
  // (four waves, one workgroup per CU) are slower than split-N's 256 x 256
  // tiles (regrouped LayerNorm backward at 262144 x 512, K = 256: 294 vs
  // 228 us), so split-N is taken there whenever the caller gave a workspace
  // of its size; tall inputs keep full-N up to 512 columns and K = 1024, where
  // their eight-wave 128 x 512 tiles are 0-7 % faster than split-N (262144
  // rows: N = 384, K = 64: 167.6 vs 180.0 us; N = 512, K = 512: 271.6 vs
  // 281.9 us; at K = 2048 split-N is 3-4 % faster)
  const bool tall_fulln = fng::bwd_fulln_tall(M) && N <= fng::fulln_max_n() && K <= 1024;
  if (path == FNG_PATH_AUTO && N > 256 && !tall_fulln && workspace &&
      workspace_bytes >= fng_gemm_postnorm_workspace_bytes(M, N, K, FNG_PATH_SPLITN) && fng::splitn_feasible(M, N))
    path = FNG_PATH_SPLITN;
  path = resolve_path(path, M, N, K);
  if (path == FNG_PATH_TWOPASS) return FNG_ERR_UNSUPPORTED;
  GemmCall c{G, Wt, nullptr, dZ, nullptr, nullptr, M, N, K, 1.f, nullptr, nullptr, nullptr, nullptr};
  const fng::NormBwdArgs b{H, rstd, h_raw};
  if (path == FNG_PATH_FULLN) {
    if (N > fng::fulln_max_n()) return FNG_ERR_UNSUPPORTED;
    return fng::launch_norm_bwd_fulln(c, b, ln, as_stream(stream));
  }
  const size_t need = fng_gemm_postnorm_workspace_bytes(M, N, K, FNG_PATH_SPLITN);
  if (!workspace || workspace_bytes < need) return FNG_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FNG_ERR_MISALIGNED;
  Workspace w = layout(workspace, M, N);
  c.part = w.part;
  c.cnt = w.cnt;
  c.done = w.done;
  c.status = w.status;
  if (!fng::splitn_feasible(M, N)) return FNG_ERR_UNSUPPORTED;
  return fng::launch_norm_bwd_splitn(c, b, ln, as_stream(stream));
}

int row_bwd(bool ln, const void* G, const void* H, const float* rstd, void* dZ, int64_t M, int64_t N, bool h_raw,
            void* stream) {
  if (M < 0 || N < 1) return FNG_ERR_INVALID_ARG;
  if (M == 0) return FNG_OK;
  if (!G || !H || !rstd || !dZ) return FNG_ERR_INVALID_ARG;
  if (!aligned16(G) || !aligned16(H) || !aligned16(dZ) || reinterpret_cast<uintptr_t>(rstd) % 4 != 0 || N % 8 != 0)
    return FNG_ERR_MISALIGNED;
  if (N > INT32_MAX / 4 || M > INT32_MAX) return FNG_ERR_UNSUPPORTED;
  return fng::launch_rownorm_bwd(G, H, rstd, dZ, M, N, h_raw, ln, as_stream(stream));
}

}  // namespace

FNG_EXPORT int fng_gemm_postnorm_ln_bwd(const void* G, const void* Wt, const void* Y, const float* rstd, void* dZ,
                                        int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                                        int path, void* stream) {
  return norm_bwd(true, G, Wt, Y, rstd, false, dZ, M, N, K, workspace, workspace_bytes, path, stream);
}

FNG_EXPORT int fng_gemm_postnorm_rms_bwd(const void* G, const void* Wt, const void* Y, const float* rstd, void* dZ,
                                         int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                                         int path, void* stream) {
  return norm_bwd(false, G, Wt, Y, rstd, false, dZ, M, N, K, workspace, workspace_bytes, path, stream);
}

FNG_EXPORT int fng_prenorm_rms_bwd_dx(const void* dY, const void* Wt, const void* X, const float* rstd, void* dX,
                                      int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                                      int path, void* stream) {
  // the product dY [M, N] @ Wt [N, K] has K columns: the norm axis
  return norm_bwd(false, dY, Wt, X, rstd, true, dX, M, K, N, workspace, workspace_bytes, path, stream);
}

FNG_EXPORT int fng_prenorm_rms_bwd_dw(const void* X, const float* rstd, const void* dY, const void* gamma, void* dW,
                                      int64_t M, int64_t N, int64_t K, void* stream) {
  if (M < 1 || N < 0 || K < 0) return FNG_ERR_INVALID_ARG;
  if (N == 0 || K == 0) return FNG_OK;
  if (!X || !dY || !dW || (gamma && !rstd)) return FNG_ERR_INVALID_ARG;
  if (!aligned16(X) || (rstd && !aligned16(rstd)) || !aligned16(dY) || !aligned16(dW) || (gamma && !aligned16(gamma)))
    return FNG_ERR_MISALIGNED;
  if (K % 8 != 0 || N % 8 != 0) return FNG_ERR_MISALIGNED;
  // 32-bit buffer ranges: X and dY (with one 256-row tile of overrun) below 2 GiB
  if (M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return FNG_ERR_UNSUPPORTED;
  if ((M + 256) * K * 2 >= (int64_t)INT32_MAX || (M + 256) * N * 2 >= (int64_t)INT32_MAX) return FNG_ERR_UNSUPPORTED;
  if (K * N >= ((int64_t)1 << 46)) return FNG_ERR_UNSUPPORTED;
  return fng::launch_prenorm_dw(X, rstd, dY, gamma, dW, M, N, K, as_stream(stream));
}

FNG_EXPORT int fng_layernorm_bwd(const void* G, const void* Y, const float* rstd, void* dZ, int64_t M, int64_t N,
                                 void* stream) {
  return row_bwd(true, G, Y, rstd, dZ, M, N, false, stream);
}

FNG_EXPORT int fng_rmsnorm_bwd(const void* G, const void* H, const float* rstd, void* dZ, int64_t M, int64_t N,
                               int h_is_input, void* stream) {
  return row_bwd(false, G, H, rstd, dZ, M, N, h_is_input != 0, stream);
}

// ---------------------------------------------------------------------------
// The post-RMSNorm GEMM without a caller workspace: the split-N / two-pass
// workspace lives in a file-scope device array of fixed size, one per GPU
// (each device that loads the library holds its own copy until the process
// ends).  Host code never passes the array's name to a kernel or a copy (on
// the host it is only a stand-in for the symbol): its device address comes
// from hipGetSymbolAddress, once per device, and is kept per device.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = FNG_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte blocks");
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// zero-fill of the array, in a kernel (not hipMemsetAsync, so that a caller
// capturing the call in a graph records only kernel nodes)
__global__ __launch_bounds__(256) void scratch_clear_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The array's device address on the current device; on the first call for a
// device it is looked up and the array cleared on `stream` (the split-N
// exchange needs a zeroed header once; afterwards each call leaves it
// consistent for the next).  nullptr on a HIP error.
void* device_scratch(hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev]) return g_scratch_ptr[dev];
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
  hipLaunchKernelGGL(scratch_clear_kernel, dim3(256), dim3(256), 0, stream, static_cast<uint4*>(ptr),
                     kScratchBytes / 16);
  if (hipGetLastError() != hipSuccess) return nullptr;
  g_scratch_ptr[dev] = ptr;
  return ptr;
}

}  // namespace

FNG_EXPORT int fng_gemm_postnorm_rms_noalloc(const void* X, const void* W, void* Y, float* rstd_out, int64_t M,
                                             int64_t N, int64_t K, float eps, int path, void* stream) {
  // validate everything that does not touch the device first
  int st = check_gemm(X, W, Y, M, N, K, eps, true);
  if (st != FNG_OK) return st;
  if (path < FNG_PATH_AUTO || path > FNG_PATH_TWOPASS) return FNG_ERR_INVALID_ARG;
  if (m_or_n_empty(M, N)) return FNG_OK;
  const size_t need = fng_gemm_postnorm_workspace_bytes(M, N, K, path);
  if (need > kScratchBytes) return FNG_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    ws = device_scratch(as_stream(stream));
    if (!ws) return FNG_ERR_HIP;
  }
  return postnorm(false, X, W, Y, nullptr, rstd_out, M, N, K, eps, ws, kScratchBytes, path, stream, nullptr,
                  nullptr, true);
}

FNG_EXPORT int fng_get_kernel_status(const void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || workspace_bytes < 256) return FNG_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FNG_ERR_MISALIGNED;
  uint32_t word = 0;
  if (hipMemcpyAsync(&word, workspace, sizeof(word), hipMemcpyDeviceToHost, as_stream(stream)) != hipSuccess)
    return FNG_ERR_HIP;
  if (hipStreamSynchronize(as_stream(stream)) != hipSuccess) return FNG_ERR_HIP;
  return word ? FNG_ERR_TIMEOUT : FNG_OK;
}

FNG_EXPORT int fng_norm_attention(const void* Q, const void* K, const void* V, void* out, float* ln_mean_out,
                                  float* ln_rstd_out, float* rms_rstd_out, int64_t B, int64_t Sq, int64_t Skv,
                                  int64_t H, int64_t D, float sm_scale, float eps_ln, float eps_rms,
                                  void* stream) {
  if (!(eps_ln > 0.f && isfinite(eps_ln)) || !(eps_rms > 0.f && isfinite(eps_rms))) return FNG_ERR_INVALID_ARG;
  if (!isfinite(sm_scale)) return FNG_ERR_INVALID_ARG;
  const int st = check_attn(Q, K, V, out, B, Sq, Skv, H, D);
  if (st != FNG_OK || B == 0 || Sq == 0 || H == 0) return st;
  fng::AttnCall c{Q, K, V, out, ln_mean_out, ln_rstd_out, rms_rstd_out, B, Sq, Skv, H, D,
                  sm_scale > 0.f ? sm_scale : 1.0f / sqrtf((float)D), eps_ln, eps_rms};
  return fng::launch_attention(c, true, as_stream(stream));
}

FNG_EXPORT int fng_flash_norm_attention(const void* Q, const int32_t* q_offsets, const void* K, const void* V,
                                        void* out, float* ln_mean_out, float* ln_rstd_out, float* rms_rstd_out,
                                        int64_t B, int64_t T, int64_t max_len_q, int64_t Skv, int64_t H, int64_t D,
                                        float sm_scale, float eps_ln, float eps_rms, int act, void* stream) {
  if (!(eps_ln > 0.f && isfinite(eps_ln)) || !(eps_rms > 0.f && isfinite(eps_rms))) return FNG_ERR_INVALID_ARG;
  if (!isfinite(sm_scale)) return FNG_ERR_INVALID_ARG;
  const int st = check_fna(Q, q_offsets, K, V, out, B, T, max_len_q, Skv, H, D, act);
  if (st != FNG_OK || B == 0 || T == 0 || max_len_q == 0 || H == 0) return st;
  fng::FnaCall c{Q, q_offsets, K, V, out, ln_mean_out, ln_rstd_out, rms_rstd_out, B, T, max_len_q, Skv, H,
                 sm_scale > 0.f ? sm_scale : 1.0f / sqrtf((float)D), eps_ln, eps_rms, act};
  return fng::launch_fna(c, true, as_stream(stream));
}

FNG_EXPORT size_t fng_flash_norm_attention_bwd_workspace_bytes(int64_t T, int64_t H) {
  if (T <= 0 || (H != 1 && H != 2 && H != 4 && H != 8)) return 0;
  return fng::fna_bwd_workspace_bytes(T, H);
}

namespace {
// the two backward entry points: norm = true is FlashNormAttention's (out and
// the three statistics are inputs), false the plain jagged attention's
int fna_bwd_call(bool norm, const void* Q, const int32_t* q_offsets, const void* K, const void* V, const void* out,
                 const void* dout, const float* ln_mean, const float* ln_rstd, const float* rms_rstd, void* dQ,
                 void* dK, void* dV, void* workspace, size_t workspace_bytes, int64_t B, int64_t T, int64_t max_len_q,
                 int64_t Skv, int64_t H, int64_t D, float sm_scale, int act, void* stream) {
  if (!isfinite(sm_scale)) return FNG_ERR_INVALID_ARG;
  int st = check_fna(Q, q_offsets, K, V, out, B, T, max_len_q, Skv, H, D, act);
  if (st != FNG_OK) return st;
  if (Skv > 128 || (H != 0 && H != 1 && H != 2 && H != 4 && H != 8)) return FNG_ERR_UNSUPPORTED;
  if (B == 0 || H == 0) return FNG_OK;
  // dK and dV are written for every batch, even when no query row is processed
  if (!dK || !dV) return FNG_ERR_INVALID_ARG;
  if (!aligned16(dK) || !aligned16(dV)) return FNG_ERR_MISALIGNED;
  const bool rows = T > 0 && max_len_q > 0;
  if (rows) {
    if (!dout || !dQ || (norm && (!ln_mean || !ln_rstd || !rms_rstd))) return FNG_ERR_INVALID_ARG;
    if (!aligned16(dout) || !aligned16(dQ)) return FNG_ERR_MISALIGNED;
    if (norm && ((uintptr_t)ln_mean % 4 || (uintptr_t)ln_rstd % 4 || (uintptr_t)rms_rstd % 4))
      return FNG_ERR_MISALIGNED;
    if (!workspace || workspace_bytes < fng::fna_bwd_workspace_bytes(T, H)) return FNG_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FNG_ERR_MISALIGNED;
  } else {
    // check_fna returned before its pointer checks; the key/value kernel still
    // reads the offsets, K and V
    if (!q_offsets || !K || !V) return FNG_ERR_INVALID_ARG;
    if (!aligned16(K) || !aligned16(V) || (uintptr_t)q_offsets % 4 != 0) return FNG_ERR_MISALIGNED;
    if (T >= (int64_t)INT32_MAX || B >= (int64_t)INT32_MAX || (Skv + 32) * H * D * 2 >= (int64_t)INT32_MAX)
      return FNG_ERR_UNSUPPORTED;
  }
  if (B * H >= (int64_t)INT32_MAX) return FNG_ERR_UNSUPPORTED;
  fng::FnaBwdCall c{Q, q_offsets, K, V, out, dout, ln_mean, ln_rstd, rms_rstd, dQ, dK, dV, workspace,
                    B, T, rows ? max_len_q : 0, Skv, H, sm_scale > 0.f ? sm_scale : 1.0f / sqrtf((float)D), act};
  return fng::launch_fna_bwd(c, norm, as_stream(stream));
}
}  // namespace

FNG_EXPORT int fng_flash_norm_attention_bwd(const void* Q, const int32_t* q_offsets, const void* K,
                                            const void* V, const void* out, const void* dout,
                                            const float* ln_mean, const float* ln_rstd, const float* rms_rstd,
                                            void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes,
                                            int64_t B, int64_t T, int64_t max_len_q, int64_t Skv, int64_t H,
                                            int64_t D, float sm_scale, int act, void* stream) {
  return fna_bwd_call(true, Q, q_offsets, K, V, out, dout, ln_mean, ln_rstd, rms_rstd, dQ, dK, dV, workspace,
                      workspace_bytes, B, T, max_len_q, Skv, H, D, sm_scale, act, stream);
}

FNG_EXPORT int fng_jagged_attention_bwd(const void* Q, const int32_t* q_offsets, const void* K, const void* V,
                                        const void* dout, void* dQ, void* dK, void* dV, void* workspace,
                                        size_t workspace_bytes, int64_t B, int64_t T, int64_t max_len_q,
                                        int64_t Skv, int64_t H, int64_t D, float sm_scale, int act, void* stream) {
  // no forward output is read: dout stands in for it in the shape checks
  return fna_bwd_call(false, Q, q_offsets, K, V, dout, dout, nullptr, nullptr, nullptr, dQ, dK, dV, workspace,
                      workspace_bytes, B, T, max_len_q, Skv, H, D, sm_scale, act, stream);
}

FNG_EXPORT int fng_rmsnorm(const void* X, const void* gamma, void* Y, float* rstd_out, int64_t M, int64_t N,
                           float eps, void* stream) {
  if (M < 0 || N < 1 || !(eps > 0.f && isfinite(eps))) return FNG_ERR_INVALID_ARG;
  if (M == 0) return FNG_OK;
  if (!X || !Y) return FNG_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(Y) || (gamma && !aligned16(gamma)) || N % 8 != 0) return FNG_ERR_MISALIGNED;
  if (N > INT32_MAX / 4 || M > INT32_MAX) return FNG_ERR_UNSUPPORTED;
  return fng::launch_rownorm(X, gamma, Y, nullptr, rstd_out, M, N, eps, false, as_stream(stream));
}

FNG_EXPORT int fng_layernorm(const void* X, void* Y, float* mean_out, float* rstd_out, int64_t M, int64_t N,
                             float eps, void* stream) {
  if (M < 0 || N < 1 || !(eps > 0.f && isfinite(eps))) return FNG_ERR_INVALID_ARG;
  if (M == 0) return FNG_OK;
  if (!X || !Y) return FNG_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(Y) || N % 8 != 0) return FNG_ERR_MISALIGNED;
  if (N > INT32_MAX / 4 || M > INT32_MAX) return FNG_ERR_UNSUPPORTED;
  return fng::launch_rownorm(X, nullptr, Y, mean_out, rstd_out, M, N, eps, true, as_stream(stream));
}

FNG_EXPORT int fng_gemm(const void* X, const void* W, void* Y, int64_t M, int64_t N, int64_t K, void* stream) {
  const int st = check_gemm(X, W, Y, M, N, K, 1.f, false);
  if (st != FNG_OK || m_or_n_empty(M, N)) return st;
  GemmCall c{X, W, nullptr, Y, nullptr, nullptr, M, N, K, 0.f, nullptr, nullptr, nullptr, nullptr};
  return fng::launch_gemm(c, as_stream(stream));
}

FNG_EXPORT int fng_attention(const void* Q, const void* K, const void* V, void* out, int64_t B, int64_t Sq,
                             int64_t Skv, int64_t H, int64_t D, float sm_scale, void* stream) {
  if (!isfinite(sm_scale)) return FNG_ERR_INVALID_ARG;
  const int st = check_attn(Q, K, V, out, B, Sq, Skv, H, D);
  if (st != FNG_OK || B == 0 || Sq == 0 || H == 0) return st;
  fng::AttnCall c{Q, K, V, out, nullptr, nullptr, nullptr, B, Sq, Skv, H, D,
                  sm_scale > 0.f ? sm_scale : 1.0f / sqrtf((float)D), 1e-5f, 1e-6f};
  return fng::launch_attention(c, false, as_stream(stream));
}

FNG_EXPORT int fng_jagged_attention(const void* Q, const int32_t* q_offsets, const void* K, const void* V,
                                    void* out, int64_t B, int64_t T, int64_t max_len_q, int64_t Skv, int64_t H,
                                    int64_t D, float sm_scale, int act, void* stream) {
  if (!isfinite(sm_scale)) return FNG_ERR_INVALID_ARG;
  const int st = check_fna(Q, q_offsets, K, V, out, B, T, max_len_q, Skv, H, D, act);
  if (st != FNG_OK || B == 0 || T == 0 || max_len_q == 0 || H == 0) return st;
  fng::FnaCall c{Q, q_offsets, K, V, out, nullptr, nullptr, nullptr, B, T, max_len_q, Skv, H,
                 sm_scale > 0.f ? sm_scale : 1.0f / sqrtf((float)D), 1e-5f, 1e-6f, act};
  return fng::launch_fna(c, false, as_stream(stream));
}
