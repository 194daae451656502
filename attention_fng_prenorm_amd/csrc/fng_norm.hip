// Standalone row normalizations (the unfused baseline the fusions replace) and
// the second kernel of the two-pass post-norm fallback.
//
// "Towards Free Normalization: Fusing Normalization into GEMM and Attention
// Kernels", section 1: a norm kernel tiles only the outer dimension and loads
// whole rows.  Here a group of LPR lanes owns one row, each lane holding CPL
// 16-byte chunks in registers, so the row is read from HBM once and written
// once.  Statistics are fp32; LayerNorm is two-pass over the registers
// (mean, then the sum of squared deviations), RMSNorm divides the sum of
// squares by the row length; eps is inside the square root.
#include "fng_device.h"
#include "fng_internal.h"

namespace fng {

struct RowNormParams {
  const uint16_t* X;
  const uint16_t* gamma;
  uint16_t* Y;
  float* mean_out;
  float* rstd_out;
  int64_t M;
  int N;
  float eps;
};

template <int LPR, int CPL, bool LN, bool GAMMA>
__global__ __launch_bounds__(256) void rownorm_kernel(RowNormParams p) {
  constexpr int RPB = 256 / LPR;  // rows per block
  const int tid = threadIdx.x;
  const int sub = tid % LPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR;
  const bool valid = row < p.M;
  const int N = p.N;
  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(p.X + (valid ? row : 0) * (int64_t)N, valid ? (uint32_t)N * 2u : 0u);

  u32x4_t v[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) v[c] = buffer_load16(xr, (uint32_t)((c * LPR + sub) * 16));

  float s = 0.f;
  float mean = 0.f;
  if constexpr (LN) {
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) s += bf16lo(v[c][e]) + bf16hi(v[c][e]);
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) s = xor_sum(s, m);
    mean = s / (float)N;
    s = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      if ((c * LPR + sub) * 8 < N) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = bf16lo(v[c][e]) - mean, b = bf16hi(v[c][e]) - mean;
          s += a * a + b * b;
        }
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < CPL; ++c) s = sumsq_bf16x8(v[c], s);
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) s = xor_sum(s, m);
  const float rstd = __builtin_amdgcn_rsqf(s / (float)N + p.eps);

  if (!valid) return;
  if (sub == 0) {
    if (p.rstd_out) p.rstd_out[row] = rstd;
    if constexpr (LN)
      if (p.mean_out) p.mean_out[row] = mean;
  }
  __amdgpu_buffer_rsrc_t gr;
  if constexpr (GAMMA) gr = make_rsrc(p.gamma, (uint32_t)N * 2u);
  uint16_t* y = p.Y + row * (int64_t)N;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int col = (c * LPR + sub) * 8;
    if (col >= N) continue;
    u32x4_t o;
    u32x4_t g;
    if constexpr (GAMMA) g = buffer_load16(gr, (uint32_t)col * 2u);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float a = (bf16lo(v[c][e]) - mean) * rstd;
      float b = (bf16hi(v[c][e]) - mean) * rstd;
      if constexpr (GAMMA) {
        a *= bf16lo(g[e]);
        b *= bf16hi(g[e]);
      }
      o[e] = pack_bf16(a, b);
    }
    *reinterpret_cast<u32x4_t*>(y + col) = o;
  }
}

// rows longer than the register-resident variants: one block per row, the row
// is read twice (statistics, then normalize)
template <bool LN, bool GAMMA>
__global__ __launch_bounds__(256) void rownorm_long_kernel(RowNormParams p) {
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int N = p.N;
  const uint16_t* x = p.X + row * (int64_t)N;
  uint16_t* y = p.Y + row * (int64_t)N;
  __shared__ float red[4];
  auto block_sum = [&](float v) {
    for (int m = 32; m >= 1; m >>= 1) v = xor_sum(v, m);
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
  };
  float mean = 0.f;
  if constexpr (LN) {
    float s = 0.f;
    for (int col = tid * 8; col < N; col += 256 * 8) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(x + col);
      for (int e = 0; e < 4; ++e) s += bf16lo(v[e]) + bf16hi(v[e]);
    }
    mean = block_sum(s) / (float)N;
  }
  float s = 0.f;
  for (int col = tid * 8; col < N; col += 256 * 8) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(x + col);
    for (int e = 0; e < 4; ++e) {
      const float a = bf16lo(v[e]) - mean, b = bf16hi(v[e]) - mean;
      s += a * a + b * b;
    }
  }
  const float rstd = __builtin_amdgcn_rsqf(block_sum(s) / (float)N + p.eps);
  if (tid == 0) {
    if (p.rstd_out) p.rstd_out[row] = rstd;
    if constexpr (LN)
      if (p.mean_out) p.mean_out[row] = mean;
  }
  // all reads of this row finish before any write (Y may alias X)
  __syncthreads();
  for (int col = tid * 8; col < N; col += 256 * 8) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(x + col);
    u32x4_t g = {0, 0, 0, 0};
    if constexpr (GAMMA) g = *reinterpret_cast<const u32x4_t*>(p.gamma + col);
    u32x4_t o;
    for (int e = 0; e < 4; ++e) {
      float a = (bf16lo(v[e]) - mean) * rstd, b = (bf16hi(v[e]) - mean) * rstd;
      if constexpr (GAMMA) {
        a *= bf16lo(g[e]);
        b *= bf16hi(g[e]);
      }
      o[e] = pack_bf16(a, b);
    }
    *reinterpret_cast<u32x4_t*>(y + col) = o;
  }
}

namespace {

template <int LPR, int CPL, bool LN>
int go(const RowNormParams& p, hipStream_t s) {
  constexpr int RPB = 256 / LPR;
  const int64_t grid = (p.M + RPB - 1) / RPB;
  if (p.gamma)
    hipLaunchKernelGGL((rownorm_kernel<LPR, CPL, LN, true>), dim3((unsigned)grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((rownorm_kernel<LPR, CPL, LN, false>), dim3((unsigned)grid), dim3(256), 0, s, p);
  return hipGetLastError() == hipSuccess ? FNG_OK : FNG_ERR_HIP;
}

template <bool LN>
int dispatch(const RowNormParams& p, hipStream_t s) {
  const int N = p.N;
  if (N <= 128) return go<16, 1, LN>(p, s);
  if (N <= 256) return go<32, 1, LN>(p, s);
  if (N <= 512) return go<64, 1, LN>(p, s);
  if (N <= 1024) return go<64, 2, LN>(p, s);
  if (N <= 2048) return go<64, 4, LN>(p, s);
  if (N <= 4096) return go<64, 8, LN>(p, s);
  if (N <= 8192) return go<64, 16, LN>(p, s);
  if (p.gamma)
    hipLaunchKernelGGL((rownorm_long_kernel<LN, true>), dim3((unsigned)p.M), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((rownorm_long_kernel<LN, false>), dim3((unsigned)p.M), dim3(256), 0, s, p);
  return hipGetLastError() == hipSuccess ? FNG_OK : FNG_ERR_HIP;
}

}  // namespace

int launch_rownorm(const void* X, const void* gamma, void* Y, float* mean_out, float* rstd_out,
                   int64_t M, int64_t N, float eps, bool ln, hipStream_t s) {
  RowNormParams p{static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(gamma),
                  static_cast<uint16_t*>(Y), mean_out, rstd_out, M, (int)N, eps};
  return ln ? dispatch<true>(p, s) : dispatch<false>(p, s);
}

// ---------------------------------------------------------------------------
// Standalone norm backward (the unfused baseline of the regrouped backward):
// per row, from the upstream gradient g, the normalized values xhat (the
// forward output, or x * rstd from the norm's input) and the forward rstd,
//   LayerNorm: dz = rstd (g - mean(g) - xhat mean(g xhat))
//   RMSNorm:   dz = rstd (g - xhat mean(g xhat)).
// Same row ownership as the forward kernel; both rows are held in registers.
// ---------------------------------------------------------------------------
struct RowBwdParams {
  const uint16_t* G;
  const uint16_t* H;   // xhat, or the norm's input when h_raw
  const float* rstd;
  uint16_t* dZ;
  int64_t M;
  int N;
  int h_raw;
};

template <int LPR, int CPL, bool LN>
__global__ __launch_bounds__(256) void rownorm_bwd_kernel(RowBwdParams p) {
  constexpr int RPB = 256 / LPR;
  const int tid = threadIdx.x;
  const int sub = tid % LPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR;
  const bool valid = row < p.M;
  const int N = p.N;
  const uint32_t bytes = valid ? (uint32_t)N * 2u : 0u;
  const __amdgpu_buffer_rsrc_t gr = make_rsrc(p.G + (valid ? row : 0) * (int64_t)N, bytes);
  const __amdgpu_buffer_rsrc_t hr = make_rsrc(p.H + (valid ? row : 0) * (int64_t)N, bytes);
  u32x4_t gv[CPL], hv[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    gv[c] = buffer_load16(gr, (uint32_t)((c * LPR + sub) * 16));
    hv[c] = buffer_load16(hr, (uint32_t)((c * LPR + sub) * 16));
  }
  const float r = valid ? p.rstd[row] : 1.f;
  const float hs = p.h_raw ? r : 1.f;
  float s1 = 0.f, s2 = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float g0 = bf16lo(gv[c][e]), g1 = bf16hi(gv[c][e]);
      if constexpr (LN) s1 += g0 + g1;
      s2 = fmaf(g0, bf16lo(hv[c][e]) * hs, s2);
      s2 = fmaf(g1, bf16hi(hv[c][e]) * hs, s2);
    }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) {
    if constexpr (LN) s1 = xor_sum(s1, m);
    s2 = xor_sum(s2, m);
  }
  if (!valid) return;
  const float c1 = s1 / (float)N, c2 = s2 / (float)N;
  uint16_t* dz = p.dZ + row * (int64_t)N;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int col = (c * LPR + sub) * 8;
    if (col >= N) continue;
    u32x4_t o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = r * (bf16lo(gv[c][e]) - c1 - bf16lo(hv[c][e]) * hs * c2);
      const float b = r * (bf16hi(gv[c][e]) - c1 - bf16hi(hv[c][e]) * hs * c2);
      o[e] = pack_bf16(a, b);
    }
    *reinterpret_cast<u32x4_t*>(dz + col) = o;
  }
}

// rows longer than 8192: one block per row, both rows read twice
template <bool LN>
__global__ __launch_bounds__(256) void rownorm_bwd_long_kernel(RowBwdParams p) {
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int N = p.N;
  const uint16_t* g = p.G + row * (int64_t)N;
  const uint16_t* h = p.H + row * (int64_t)N;
  uint16_t* dz = p.dZ + row * (int64_t)N;
  __shared__ float red[2][4];
  const float r = p.rstd[row];
  const float hs = p.h_raw ? r : 1.f;
  float s1 = 0.f, s2 = 0.f;
  for (int col = tid * 8; col < N; col += 256 * 8) {
    const u32x4_t gv = *reinterpret_cast<const u32x4_t*>(g + col);
    const u32x4_t hv = *reinterpret_cast<const u32x4_t*>(h + col);
    for (int e = 0; e < 4; ++e) {
      if constexpr (LN) s1 += bf16lo(gv[e]) + bf16hi(gv[e]);
      s2 = fmaf(bf16lo(gv[e]), bf16lo(hv[e]) * hs, s2);
      s2 = fmaf(bf16hi(gv[e]), bf16hi(hv[e]) * hs, s2);
    }
  }
  for (int m = 32; m >= 1; m >>= 1) {
    s1 = xor_sum(s1, m);
    s2 = xor_sum(s2, m);
  }
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = s1;
    red[1][tid >> 6] = s2;
  }
  __syncthreads();
  const float c1 = (red[0][0] + red[0][1] + red[0][2] + red[0][3]) / (float)N;
  const float c2 = (red[1][0] + red[1][1] + red[1][2] + red[1][3]) / (float)N;
  for (int col = tid * 8; col < N; col += 256 * 8) {
    const u32x4_t gv = *reinterpret_cast<const u32x4_t*>(g + col);
    const u32x4_t hv = *reinterpret_cast<const u32x4_t*>(h + col);
    u32x4_t o;
    for (int e = 0; e < 4; ++e)
      o[e] = pack_bf16(r * (bf16lo(gv[e]) - (LN ? c1 : 0.f) - bf16lo(hv[e]) * hs * c2),
                       r * (bf16hi(gv[e]) - (LN ? c1 : 0.f) - bf16hi(hv[e]) * hs * c2));
    *reinterpret_cast<u32x4_t*>(dz + col) = o;
  }
}

namespace {

template <int LPR, int CPL, bool LN>
int go_bwd(const RowBwdParams& p, hipStream_t s) {
  constexpr int RPB = 256 / LPR;
  const int64_t grid = (p.M + RPB - 1) / RPB;
  hipLaunchKernelGGL((rownorm_bwd_kernel<LPR, CPL, LN>), dim3((unsigned)grid), dim3(256), 0, s, p);
  return hipGetLastError() == hipSuccess ? FNG_OK : FNG_ERR_HIP;
}

template <bool LN>
int dispatch_bwd(const RowBwdParams& p, hipStream_t s) {
  const int N = p.N;
  if (N <= 128) return go_bwd<16, 1, LN>(p, s);
  if (N <= 256) return go_bwd<32, 1, LN>(p, s);
  if (N <= 512) return go_bwd<64, 1, LN>(p, s);
  if (N <= 1024) return go_bwd<64, 2, LN>(p, s);
  if (N <= 2048) return go_bwd<64, 4, LN>(p, s);
  if (N <= 4096) return go_bwd<64, 8, LN>(p, s);
  hipLaunchKernelGGL((rownorm_bwd_long_kernel<LN>), dim3((unsigned)p.M), dim3(256), 0, s, p);
  return hipGetLastError() == hipSuccess ? FNG_OK : FNG_ERR_HIP;
}

}  // namespace

int launch_rownorm_bwd(const void* G, const void* H, const float* rstd, void* dZ, int64_t M, int64_t N,
                       bool h_raw, bool ln, hipStream_t s) {
  RowBwdParams p{static_cast<const uint16_t*>(G), static_cast<const uint16_t*>(H), rstd,
                 static_cast<uint16_t*>(dZ), M, (int)N, h_raw ? 1 : 0};
  return ln ? dispatch_bwd<true>(p, s) : dispatch_bwd<false>(p, s);
}

// ---------------------------------------------------------------------------
// two-pass post-norm, second kernel: one wave per row merges the per-tile
// partials (fixed order; Chan et al. pairwise (count, mean, M2) merge for
// LayerNorm, plain sum of squares for RMSNorm) and normalizes the row of Y
// in place.
// ---------------------------------------------------------------------------
struct FinalizeParams {
  uint16_t* Y;
  const float* part;  // [tiles_m][tiles_n][bm][2]
  float* mean_out;
  float* rstd_out;
  int64_t M;
  int N, tiles_n, bm, bn;
  float eps;
  const uint16_t* gamma;  // post-norm affine gain [N] and bias [N] (each may be nullptr)
  const uint16_t* beta;
};

template <bool LN>
__global__ __launch_bounds__(256) void finalize_kernel(FinalizeParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.M) return;
  const int64_t tm = row / p.bm;
  const int r = (int)(row % p.bm);
  const float* pb = p.part + (size_t)tm * p.tiles_n * p.bm * 2;
  float mean = 0.f, rstd;
  if constexpr (LN) {
    float cn = 0.f, m2 = 0.f;
    for (int q = 0; q < p.tiles_n; ++q) {
      const float nb = (float)min(p.bn, p.N - q * p.bn);
      const float mb = pb[((size_t)q * p.bm + r) * 2 + 0];
      const float m2b = pb[((size_t)q * p.bm + r) * 2 + 1];
      const float tot = cn + nb;
      const float d = mb - mean;
      mean += d * (nb / tot);
      m2 += m2b + d * d * (cn * nb / tot);
      cn = tot;
    }
    rstd = __builtin_amdgcn_rsqf(m2 / (float)p.N + p.eps);
  } else {
    float s = 0.f;
    for (int q = 0; q < p.tiles_n; ++q) s += pb[((size_t)q * p.bm + r) * 2 + 1];
    rstd = __builtin_amdgcn_rsqf(s / (float)p.N + p.eps);
  }
  if (lane == 0) {
    if (p.rstd_out) p.rstd_out[row] = rstd;
    if constexpr (LN)
      if (p.mean_out) p.mean_out[row] = mean;
  }
  uint16_t* y = p.Y + row * (int64_t)p.N;
  for (int col = lane * 8; col < p.N; col += 64 * 8) {
    u32x4_t v = *reinterpret_cast<const u32x4_t*>(y + col);
    // LayerNorm intermediates were stored minus their tile mean
    float shift = -mean;
    if constexpr (LN) shift = pb[((size_t)(col / p.bn) * p.bm + r) * 2 + 0] - mean;
    u32x4_t g = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u}, b = {0u, 0u, 0u, 0u};
    if (p.gamma) g = *reinterpret_cast<const u32x4_t*>(p.gamma + col);
    if (p.beta) b = *reinterpret_cast<const u32x4_t*>(p.beta + col);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t ge = g[e], be = b[e];
      v[e] = pack_bf16(fmaf((bf16lo(v[e]) + shift) * rstd, bf16lo(ge), bf16lo(be)),
                       fmaf((bf16hi(v[e]) + shift) * rstd, bf16hi(ge), bf16hi(be)));
    }
    *reinterpret_cast<u32x4_t*>(y + col) = v;
  }
}

int launch_postnorm_finalize(void* Y, const void* part, float* mean_out, float* rstd_out, int64_t M,
                             int64_t N, int64_t tiles_n, int64_t bm, int64_t bn, float eps, bool ln,
                             const void* gamma, const void* beta, hipStream_t s) {
  FinalizeParams p{static_cast<uint16_t*>(Y), static_cast<const float*>(part), mean_out, rstd_out, M,
                   (int)N, (int)tiles_n, (int)bm, (int)bn, eps, static_cast<const uint16_t*>(gamma),
                   static_cast<const uint16_t*>(beta)};
  const int64_t grid = (M + 3) / 4;
  if (ln)
    hipLaunchKernelGGL(finalize_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(finalize_kernel<false>, dim3((unsigned)grid), dim3(256), 0, s, p);
  return hipGetLastError() == hipSuccess ? FNG_OK : FNG_ERR_HIP;
}

}  // namespace fng
