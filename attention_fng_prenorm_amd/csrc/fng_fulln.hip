// Small post-norm GEMM: Y = norm(X @ W) over each output row, for K <= 256
// and N <= 256 -- section 1 of "Towards Free Normalization: Fusing
// Normalization into GEMM and Attention Kernels" (naive fusion: one
// workgroup's tile spans all N, the row statistics come straight from the
// fp32 accumulators), laid out for gfx950.
//
// At these sizes the whole of W (<= 128 KB) and a 32-row slab of X (<= 16 KB)
// sit in LDS at once, so there is no ring: every copy of the workgroup is
// issued up front (X first, then W in four quarters of 64 rows) and the K
// loop waits for one quarter at a time.  Eight waves, two per SIMD, so one
// wave's MFMAs overlap the other's fragment reads; wave w owns output columns
// [32 w, 32 w + 32) for all 32 rows: one 32x32 MFMA accumulator, issued
// transposed (D = W_frag * X_frag) so that lane l holds row l % 32.
// The statistics take one LDS round: each wave reduces its 32 columns of a
// row to (mean, M2) (LayerNorm) or a sum of squares (RMSNorm), and every lane
// merges the eight in a fixed order (the parallel-variance combination of
// per-group means and M2 for LayerNorm), so the result is bitwise
// reproducible.  The normalized bf16 tile is staged in the freed X region and
// stored along rows.
#include "fng_device.h"
#include "fng_internal.h"

namespace fng {
namespace {

constexpr int kRows = 32;    // output rows per workgroup
constexpr int kWaves = 8;    // wave w: output columns [32 w, 32 w + 32)
constexpr int kMaxK = 256;
constexpr int kMaxN = 256;
constexpr int kWBytes = kMaxK * kMaxN * 2;  // W [k][n]: 512-byte rows
constexpr int kXBytes = kRows * kMaxK * 2;  // X [row][k]: 512-byte rows
constexpr int kRedBytes = kWaves * kRows * 2 * 4;

struct SmallParams {
  const uint16_t* X;
  const uint16_t* W;
  const uint16_t* gamma;  // affine gain [N] (AFF) or nullptr
  const uint16_t* beta;   // affine bias [N] or nullptr
  uint16_t* Y;
  float* mean_out;
  float* rstd_out;
  int M, N, K;
  float eps;
};

template <bool LN, bool AFF>
__global__ __launch_bounds__(64 * kWaves) void fulln_small_kernel(SmallParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[kWBytes + kXBytes + kRedBytes];
  FNG_LDS char* lds = (FNG_LDS char*)smem;
  // W: 16-byte chunk c of row k stored at chunk c ^ 4 (k % 4) (a transposing
  //    read covers rows k .. k + 3 and four consecutive chunks: each row lands
  //    on its own quarter of the 64 banks)
  // X: chunk c of row r stored at chunk c ^ (r % 16) (a fragment read covers
  //    16 rows at one chunk: 16 distinct bank groups)
  FNG_LDS char* wl = lds;
  FNG_LDS char* xl = lds + kWBytes;
  FNG_LDS float* red = (FNG_LDS float*)(lds + kWBytes + kXBytes);  // [wave][row][2]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int M = p.M, N = p.N, K = p.K;
  const int m0 = blockIdx.x * kRows;

  // ---- copies: X (16 x 1 KB, two per wave), then W by quarters of 64 rows
  //      (32 x 1 KB each, four per wave); out-of-range pieces read as zeros
  {
    const int64_t xrem = (int64_t)(M - m0) * K * 2;
    const uint32_t xbytes = (uint32_t)(xrem < (int64_t)kRows * K * 2 ? xrem : (int64_t)kRows * K * 2);
    const i32x4_t xr = dma_rsrc(p.X + (size_t)m0 * K, xbytes);
    const i32x4_t wr = dma_rsrc(p.W, (uint32_t)(K * N * 2));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int blk = wave * 2 + i;
      const int idx = blk * 1024 + lane * 16;
      const int r = idx / 512, c = ((idx % 512) / 16) ^ (r & 15);
      dma16(xr, xl + blk * 1024, c * 8 < K ? (uint32_t)(r * K + c * 8) * 2u : kOOB);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int blk = q * 32 + wave * 4 + i;
        const int idx = blk * 1024 + lane * 16;
        const int k = idx / 512, c = ((idx % 512) / 16) ^ ((k & 3) << 2);
        dma16(wr, wl + blk * 1024, (k < K && c * 8 < N) ? (uint32_t)(k * N + c * 8) * 2u : kOOB);
      }
  }

  // ---- fragment addresses (k16 slice s adds s * 16 rows of W, 32 bytes of X)
  //   W (MFMA A operand, 32 columns x 16 k): in each 16-lane group g, lane i
  //   receives column 16 (g % 2) + i of rows 8 (g / 2) .. + 3 and + 4 .. + 7
  //   X (B operand, 16 k x 32 rows): lane l reads 8 k of row l % 32
  const int g = lane >> 4, li = lane & 15;
  const int wn = wave * 32 + 16 * (g & 1) + 4 * (li & 3);
  const int wk = 8 * (g >> 1) + (li >> 2);
  const FNG_LDS char* wa = wl + wk * 512 + (((wn >> 3) ^ ((wk & 3) << 2)) * 16) + (wn & 7) * 2;
  const int nslices = (K + 15) / 16;

  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  auto quarter = [&](int q) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 4 * q; s < 4 * q + 4; ++s) {
      if (s < nslices) {
        const u32x2_t lo = lds_read_tr16(wa + s * 16 * 512);
        const u32x2_t h2 = lds_read_tr16(wa + s * 16 * 512 + 4 * 512);
        const int c = 2 * s + hi;
        const u32x4_t xf = lds_read16(xl + l32 * 512 + ((c ^ (l32 & 15)) * 16));
        acc = mfma_bf16(u32x4_t{lo[0], lo[1], h2[0], h2[1]}, xf, acc);
      }
    }
  };
  // this wave issued 2 + 4 x 4 copies in order: quarter q (and X) have landed
  // once at most 4 (3 - q) are outstanding; the barrier makes it every wave's
  wait_vmcnt<12>();
  lds_barrier();
  quarter(0);
  wait_vmcnt<8>();
  lds_barrier();
  quarter(1);
  wait_vmcnt<4>();
  lds_barrier();
  quarter(2);
  wait_vmcnt<0>();
  lds_barrier();
  quarter(3);

  // ---- statistics: lane holds row l32, columns col(r) = cb + 8 (r / 4) + r % 4
  // (No fp32 divisions: each is a dozen instructions, and this phase is on
  // every workgroup's critical path; the counts are small integers.)
  const int cb = wave * 32 + 4 * hi;
  const int cnt_w = N - wave * 32 < 0 ? 0 : (N - wave * 32 > 32 ? 32 : N - wave * 32);
  const float inv_n = __builtin_amdgcn_rcpf((float)N);
  float mean = 0.f, rstd;
  if constexpr (LN) {
    // per wave: the mean of its columns and M2 about it; merged as
    // mean = sum_w cnt_w mean_w / N, M2 = sum_w (M2_w + cnt_w (mean_w - mean)^2)
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (cb + 8 * (r >> 2) + (r & 3) < N) s += acc[r];
    s = half_swap_sum(s);
    const float mw = cnt_w > 0 ? s * __builtin_amdgcn_rcpf((float)cnt_w) : 0.f;
    float q2 = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (cb + 8 * (r >> 2) + (r & 3) < N) {
        const float d = acc[r] - mw;
        q2 = fmaf(d, d, q2);
      }
    q2 = half_swap_sum(q2);
    if (hi == 0) {
      red[(wave * kRows + l32) * 2 + 0] = mw;
      red[(wave * kRows + l32) * 2 + 1] = q2;
    }
    __syncthreads();
    float mb[kWaves], cw[kWaves], msum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int nb = N - w * 32 < 0 ? 0 : (N - w * 32 > 32 ? 32 : N - w * 32);
      cw[w] = (float)nb;
      mb[w] = nb > 0 ? red[(w * kRows + l32) * 2 + 0] : 0.f;
      msum = fmaf(cw[w], mb[w], msum);
    }
    mean = msum * inv_n;
    float m2 = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (cw[w] > 0.f) {
        const float d = mb[w] - mean;
        m2 += red[(w * kRows + l32) * 2 + 1] + cw[w] * d * d;
      }
    }
    rstd = __builtin_amdgcn_rsqf(m2 * inv_n + p.eps);
  } else {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (cb + 8 * (r >> 2) + (r & 3) < N) s = fmaf(acc[r], acc[r], s);
    s = half_swap_sum(s);
    if (hi == 0) red[(wave * kRows + l32) * 2] = s;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (w * 32 < N) t += red[(w * kRows + l32) * 2];
    rstd = __builtin_amdgcn_rsqf(t * inv_n + p.eps);
  }
  const int m = m0 + l32;
  if (wave == 0 && hi == 0 && m < M) {
    if (p.rstd_out) p.rstd_out[m] = rstd;
    if constexpr (LN)
      if (p.mean_out) p.mean_out[m] = mean;
  }

  // ---- normalize, stage the bf16 tile in the X region (every wave has read
  //      its last X fragment before the barrier above), store along rows.
  //      (Each lane storing its 8 B straight from registers issues faster but
  //      leaves partial lines: 12.5 against 7.8 us per call when the outputs
  //      are not in the caches, 7.4 against 7.4 us when they are.)
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const int n = cb + 8 * r4;
    u32x2_t gq = {0u, 0u}, bq = {0u, 0u};
    if constexpr (AFF) {
      if (n < N) {
        gq = *reinterpret_cast<const u32x2_t*>(p.gamma + n);
        if (p.beta) bq = *reinterpret_cast<const u32x2_t*>(p.beta + n);
      }
    }
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float a = (acc[4 * r4 + e] - mean) * rstd;
      if constexpr (AFF) {
        const uint32_t gw = gq[e >> 1], bw = bq[e >> 1];
        a = fmaf(a, (e & 1) ? bf16hi(gw) : bf16lo(gw), (e & 1) ? bf16hi(bw) : bf16lo(bw));
      }
      v[e] = a;
    }
    const int c = wave * 4 + r4;  // 16-byte chunk of columns wave*32 + 8 r4 .. + 7
    *reinterpret_cast<FNG_LDS u32x2_t*>(xl + l32 * 512 + (c ^ l32) * 16 + hi * 8) =
        u32x2_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + i * 64 * kWaves;  // 32 rows x 32 chunks
    const int row = c >> 5, ch = c & 31;
    const int mm = m0 + row, n = ch * 8;
    if (mm < M && n < N) {
      const u32x4_t v = lds_read16(xl + row * 512 + (ch ^ row) * 16);
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p.Y + (size_t)mm * N + n));
    }
  }
}

template <bool LN, bool AFF>
int launch_small(const SmallParams& p, hipStream_t s) {
  const unsigned grid = (unsigned)((p.M + kRows - 1) / kRows);
  hipLaunchKernelGGL((fulln_small_kernel<LN, AFF>), dim3(grid), dim3(64 * kWaves), 0, s, p);
  return hipGetLastError() == hipSuccess ? FNG_OK : FNG_ERR_HIP;
}

}  // namespace

bool fulln_small_fits(int64_t N, int64_t K) { return N <= kMaxN && K <= kMaxK; }

int launch_postnorm_fulln_small(const GemmCall& c, bool ln, hipStream_t s) {
  if (!fulln_small_fits(c.N, c.K)) return FNG_ERR_UNSUPPORTED;
  SmallParams p{};
  p.X = static_cast<const uint16_t*>(c.X);
  p.W = static_cast<const uint16_t*>(c.W);
  p.gamma = static_cast<const uint16_t*>(c.gamma);
  p.beta = static_cast<const uint16_t*>(c.beta);
  p.Y = static_cast<uint16_t*>(c.Y);
  p.mean_out = c.mean_out;
  p.rstd_out = c.rstd_out;
  p.M = (int)c.M;
  p.N = (int)c.N;
  p.K = (int)c.K;
  p.eps = c.eps;
  const bool aff = c.gamma != nullptr;
  if (ln) return aff ? launch_small<true, true>(p, s) : launch_small<true, false>(p, s);
  return aff ? launch_small<false, true>(p, s) : launch_small<false, false>(p, s);
}

}  // namespace fng
