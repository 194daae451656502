// Full FlashNormAttention for gfx950, after section 4 of "Towards Free
// Normalization: Fusing Normalization into GEMM and Attention Kernels" (the
// fused short-KV kernel): for every query row x of H heads x 128,
//   ln  = LayerNorm(x) across all H*128 values
//   o_h = act(ln_h K_h^T * scale) V_h + ln_h        (first residual)
//   out = RMSNorm(o) across all H*128 values + x     (second residual)
// with act the softmax over the keys or the elementwise GELU (tanh form).
// Queries are jagged (rows offsets[b] .. offsets[b+1]-1 of batch b); keys and
// values are dense and short (the page's short-KV case keeps them whole per
// batch; here they stream through LDS in tiles of 32 keys).  NORM=false gives
// the plain activation attention (no norms, no residuals): the unfused
// baseline's attention.
//
// Work split: one workgroup = 8 waves = (8/H row groups) x H heads; wave
// (g, h) owns 32 query rows of head h.  The page's norms run across heads, so
// where it exchanges statistics between the CTAs of a cluster, the waves of
// one workgroup exchange per-(row, head) partials through LDS: (mean, M2) of
// each head merged with the pairwise formula for the LayerNorm, sums of
// squares for the RMSNorm.
//
// Per key tile every wave computes S^T = K_h Q^T (its A rows loaded in the
// key order that hands P to the next MFMA without a shuffle, as in the
// norm-sandwiched attention kernel), the activation, and O^T += V_h^T P^T;
// fp16 MFMA operands, fp32 accumulation.  The raw query rows are read again
// in the epilogue for the two residuals rather than held in registers.
#include "fng_device.h"
#include "fng_internal.h"

namespace fng {

namespace {

constexpr int kD = 128;
constexpr int kKT = 32;                 // keys per tile
constexpr int kRowK = kD * 2 + 16;      // bytes per K row ([key][d]), padded
constexpr int kRowV = kKT * 2 + 16;     // bytes per V^T row ([d][key]), padded
constexpr int kTileK = kKT * kRowK;     // per head
constexpr int kTileV = kD * kRowV;      // per head
constexpr float kLazy = 8.0f;           // running-max hysteresis (log2 units)

enum : int { ACT_SOFTMAX = 0, ACT_GELU = 1 };

struct FnaParams {
  const uint16_t* Q;
  const int32_t* off;
  const uint16_t* K;
  const uint16_t* V;
  uint16_t* O;
  float* ln_mean_out;
  float* ln_rstd_out;
  float* rms_rstd_out;
  int B, max_len, Skv, T;
  int qblocks;
  float scale;   // softmax: sm_scale * log2(e); GELU: sm_scale
  float eps_ln, eps_rms;
};

__device__ __forceinline__ int kappa(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// GELU, tanh form: 0.5 s (1 + tanh(u)) with u = sqrt(2/pi) (s + 0.044715 s^3),
// evaluated as s * sigmoid(2u) = s / (1 + 2^w), w = -2 u log2(e): one exp2 and
// one reciprocal; saturates to s (w -> -inf) and to -0 (w -> +inf, 2^w = inf)
constexpr float kGeluC0 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;
constexpr float kGeluC1 = kGeluC0 * 0.044715f;
__device__ __forceinline__ float gelu_tanh(float s) {
  const float w = s * fmaf(kGeluC1, s * s, kGeluC0);
  return s * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(w));
}

template <int H, bool NORM, int ACT>
__global__ __launch_bounds__(512, 1) void fna_kernel(FnaParams p) {
  constexpr int G = 8 / H;            // row groups
  constexpr int BM = 32 * G;          // query rows per workgroup
  constexpr int STAGE = H * (kTileK + kTileV);
  constexpr int NST = 2;
  static_assert(NST * STAGE + BM * H * 2 * 4 <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) char smem[NST * STAGE + BM * H * 2 * 4];
  FNG_LDS char* lds = (FNG_LDS char*)smem;
  FNG_LDS float* xch = (FNG_LDS float*)(lds + NST * STAGE);  // [BM][H][2] statistics exchange

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = wave % H;
  const int g = wave / H;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const uint32_t t0 = xcd_remap(blockIdx.x, gridDim.x);
  const int b = (int)(t0 / (uint32_t)p.qblocks);
  const int qb = (int)(t0 % (uint32_t)p.qblocks);
  const int r0 = p.off[b];
  const int len = min(p.off[b + 1] - r0, p.max_len);
  if (r0 < 0 || qb * BM >= len) return;  // whole workgroup: no work in this block

  const int lrow = g * 32 + l32;           // row within the block
  const int qi = qb * BM + lrow;           // row within the batch
  const int row = r0 + qi;                 // global query row
  const bool valid = qi < len && row < p.T;
  // query rows of this batch, beyond its length read as zero
  const uint32_t qbytes = (uint32_t)(max(0, min(len, p.T - r0)) * H * kD * 2);
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(p.Q + (size_t)r0 * H * kD, qbytes);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(p.K + (size_t)b * p.Skv * H * kD, (uint32_t)(p.Skv * H * kD * 2));
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(p.V + (size_t)b * p.Skv * H * kD, (uint32_t)(p.Skv * H * kD * 2));
  const uint32_t qrow_off = (uint32_t)(((size_t)qi * H + h) * kD * 2);

  // ---- K/V staging, all heads of one 32-key tile ---------------------------
  // K: chunk c = tid + 512 i (i < H) is head i, key (tid / 16), d 8 (tid % 16)..
  // V: item j = tid + 512 i (i < H / 2, or tid < 256 for one head) is head
  //    j / 256, keys 2p, 2p+1 (p = j % 16), d 8 ((j / 16) % 16).., written
  //    transposed as one 4-byte word per d row.
  constexpr int VIT = H >= 2 ? H / 2 : 1;
  u32x4_t rk[H], rv[VIT][2];
  auto gload = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < H; ++i) {
      const int key = kt * kKT + (tid >> 4), dc = tid & 15;
      rk[i] = buffer_load16(kr, (uint32_t)((((size_t)key * H + i) * kD + dc * 8) * 2));
    }
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int j = tid + 512 * i;
      if (H == 1 && j >= 256) continue;
      const int hv = j >> 8, pp = j & 15, dc = (j >> 4) & 15;
      const int key = kt * kKT + 2 * pp;
#pragma unroll
      for (int u = 0; u < 2; ++u)
        rv[i][u] = buffer_load16(vr, (uint32_t)((((size_t)(key + u) * H + hv) * kD + dc * 8) * 2));
    }
  };
  auto sstore = [&](int buf) __attribute__((always_inline)) {
    FNG_LDS char* st = lds + buf * STAGE;
#pragma unroll
    for (int i = 0; i < H; ++i) {
      u32x4_t v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = bf16x2_to_f16x2(rk[i][e]);
      lds_write16(st + i * kTileK + (tid >> 4) * kRowK + (tid & 15) * 16, v);
    }
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int j = tid + 512 * i;
      if (H == 1 && j >= 256) continue;
      const int hv = j >> 8, pp = j & 15, dc = (j >> 4) & 15;
      FNG_LDS char* dst = st + H * kTileK + hv * kTileV + (dc * 8) * kRowV + pp * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        *reinterpret_cast<FNG_LDS uint32_t*>(dst + (2 * e) * kRowV) = pack_f16(bf16lo(rv[i][0][e]), bf16lo(rv[i][1][e]));
        *reinterpret_cast<FNG_LDS uint32_t*>(dst + (2 * e + 1) * kRowV) =
            pack_f16(bf16hi(rv[i][0][e]), bf16hi(rv[i][1][e]));
      }
    }
  };

  gload(0);  // the first key tile's loads overlap the query prologue

  // ---- prologue: query fragments (lane holds d = 16kk + 8hi + 0..7) -------
  u32x4_t qf[8];
  float mu = 0.f, rstd = 1.f;
  {
    u32x4_t raw[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) raw[kk] = buffer_load16(qr, qrow_off + (uint32_t)(16 * kk + 8 * hi) * 2u);
    if constexpr (NORM) {
      // this head's sum and sum of squares over its 128 values (exact bf16
      // products, fp32 accumulation), then (mean, M2) merged across heads
      const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
      float s[2] = {0.f, 0.f}, s2[2] = {0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = raw[kk][e];
          const bf16x2_t v = __builtin_bit_cast(bf16x2_t, w);
          s[e & 1] = __builtin_amdgcn_fdot2_f32_bf16(v, ones, s[e & 1], false);
          s2[e & 1] = __builtin_amdgcn_fdot2_f32_bf16(v, v, s2[e & 1], false);
        }
      const float sh = half_swap_sum(s[0] + s[1]);
      const float mh = sh * (1.0f / kD);
      const float m2h = fmaxf(half_swap_sum(s2[0] + s2[1]) - sh * mh, 0.f);
      if (hi == 0) {
        xch[(lrow * H + h) * 2 + 0] = mh;
        xch[(lrow * H + h) * 2 + 1] = m2h;
      }
      __syncthreads();
      float msum = 0.f;
#pragma unroll
      for (int j = 0; j < H; ++j) msum += xch[(lrow * H + j) * 2 + 0];
      mu = msum * (1.0f / H);
      float m2 = 0.f;
#pragma unroll
      for (int j = 0; j < H; ++j) {
        const float dm = xch[(lrow * H + j) * 2 + 0] - mu;
        m2 += xch[(lrow * H + j) * 2 + 1] + (float)kD * dm * dm;
      }
      rstd = __builtin_amdgcn_rsqf(m2 * (1.0f / (H * kD)) + p.eps_ln);
      if (h == 0 && hi == 0 && valid) {
        if (p.ln_mean_out) p.ln_mean_out[row] = mu;
        if (p.ln_rstd_out) p.ln_rstd_out[row] = rstd;
      }
    }
    const float mul = rstd * p.scale, add = -mu * mul;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = raw[kk][e];
        qf[kk][e] = pack_f16(fmaf(bf16lo(w), mul, add), fmaf(bf16hi(w), mul, add));
      }
  }

  // fragment offsets: K row kappa(l32), chunk hi; V^T row l32, keys 8hi..
  const int koff = h * kTileK + kappa(l32) * kRowK + hi * 16;
  const int voff = H * kTileK + h * kTileV + l32 * kRowV + hi * 16;

  // lane (l32, hi) holds, in register 4 r4 + e of o[dt], d = 32 dt + 8 r4 + 4 hi + e
  u32x2_t xq[4][4];
  auto xload = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        xq[dt][r4] = buffer_load8(qr, qrow_off + (uint32_t)(32 * dt + 8 * r4 + 4 * hi) * 2u);
  };

  f32x16_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;

  const int ntiles = (p.Skv + kKT - 1) / kKT;
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < ntiles; ++kt) {
    const bool more = kt + 1 < ntiles;
    if (more) gload(kt + 1);
    else if constexpr (NORM) xload();  // raw query rows for the residuals
    const FNG_LDS char* st = lds + (kt & 1) * STAGE;

    // S^T (32 keys x 32 queries): register r <-> key 16(r/8) + 8hi + r%8
    f32x16_t sa;
#pragma unroll
    for (int r = 0; r < 16; ++r) sa[r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) sa = mfma_f16(lds_read16(st + koff + kk * 32), qf[kk], sa);
    float sc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = sa[r];
    const int kvalid = p.Skv - kt * kKT;
    if (kvalid < kKT) {  // ragged last tile only
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (16 * (r >> 3) + 8 * hi + (r & 7) >= kvalid) sc[r] = (ACT == ACT_SOFTMAX) ? -INFINITY : 0.f;
    }
    float pr[16];
    if constexpr (ACT == ACT_SOFTMAX) {
      float mx = sc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
      mx = half_swap_max(mx);
      const float mnew = mx > mrun + kLazy ? mx : mrun;
      const float alpha = (mnew == mrun || mrun == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(mrun - mnew);
      mrun = mnew;
      lrun *= alpha;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(sc[r] - mrun);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) pr[r] = gelu_tanh(sc[r]);
    }
    // P^T operand, k16 step c: keys 16c + 8hi + (0..7); row sum over the
    // same fp16 values (softmax)
    u32x4_t pf[2];
    const f16x2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
    float ls[2] = {0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f16x2_t h2 = {(_Float16)pr[8 * c + 2 * e], (_Float16)pr[8 * c + 2 * e + 1]};
        pf[c][e] = __builtin_bit_cast(uint32_t, h2);
        if constexpr (ACT == ACT_SOFTMAX) ls[e & 1] = __builtin_amdgcn_fdot2(h2, ones, ls[e & 1], false);
      }
    if constexpr (ACT == ACT_SOFTMAX) lrun += ls[0] + ls[1];
    // O^T += V^T P^T
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        o[dt] = mfma_f16(lds_read16(st + voff + c * 32 + dt * 32 * kRowV), pf[c], o[dt]);
    if (more) sstore((kt + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue ------------------------------------------------------------
  const float inv = (ACT == ACT_SOFTMAX) ? 1.0f / half_swap_sum(lrun) : 1.0f;
  float rstd2 = 1.f;
  if constexpr (NORM) {
    float ss = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float x[4] = {bf16lo(xq[dt][r4][0]), bf16hi(xq[dt][r4][0]), bf16lo(xq[dt][r4][1]), bf16hi(xq[dt][r4][1])};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = fmaf(o[dt][4 * r4 + e], inv, (x[e] - mu) * rstd);  // + ln (residual 1)
          o[dt][4 * r4 + e] = v;
          ss = fmaf(v, v, ss);
        }
      }
    ss = half_swap_sum(ss);
    __syncthreads();  // the prologue's statistics have been read
    if (hi == 0) xch[(lrow * H + h) * 2] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int j = 0; j < H; ++j) tot += xch[(lrow * H + j) * 2];
    rstd2 = __builtin_amdgcn_rsqf(tot * (1.0f / (H * kD)) + p.eps_rms);
    if (h == 0 && hi == 0 && valid && p.rms_rstd_out) p.rms_rstd_out[row] = rstd2;
  }
  if (!valid) return;
  uint16_t* orow = p.O + ((size_t)row * H + h) * kD;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float v[4];
      if constexpr (NORM) {
        const float x[4] = {bf16lo(xq[dt][r4][0]), bf16hi(xq[dt][r4][0]), bf16lo(xq[dt][r4][1]), bf16hi(xq[dt][r4][1])};
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fmaf(o[dt][4 * r4 + e], rstd2, x[e]);  // + x (residual 2)
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = o[dt][4 * r4 + e] * inv;
      }
      *reinterpret_cast<u32x2_t*>(orow + 32 * dt + 8 * r4 + 4 * hi) =
          u32x2_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
    }
}

template <int H>
int launch_h(const FnaParams& p, bool norm, int act, hipStream_t s) {
  const dim3 grid((unsigned)(p.B * p.qblocks)), block(512);
  if (norm) {
    if (act == ACT_GELU) hipLaunchKernelGGL((fna_kernel<H, true, ACT_GELU>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((fna_kernel<H, true, ACT_SOFTMAX>), grid, block, 0, s, p);
  } else {
    if (act == ACT_GELU) hipLaunchKernelGGL((fna_kernel<H, false, ACT_GELU>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((fna_kernel<H, false, ACT_SOFTMAX>), grid, block, 0, s, p);
  }
  return hipGetLastError() == hipSuccess ? FNG_OK : FNG_ERR_HIP;
}

}  // namespace

int launch_fna(const FnaCall& c, bool norm, hipStream_t s) {
  FnaParams p{};
  p.Q = static_cast<const uint16_t*>(c.Q);
  p.off = c.offsets;
  p.K = static_cast<const uint16_t*>(c.K);
  p.V = static_cast<const uint16_t*>(c.V);
  p.O = static_cast<uint16_t*>(c.O);
  p.ln_mean_out = c.ln_mean_out;
  p.ln_rstd_out = c.ln_rstd_out;
  p.rms_rstd_out = c.rms_rstd_out;
  p.B = (int)c.B;
  p.max_len = (int)c.max_len;
  p.Skv = (int)c.Skv;
  p.T = (int)c.T;
  p.scale = c.act == FNG_ACT_SOFTMAX ? c.sm_scale * 1.4426950408889634f : c.sm_scale;
  p.eps_ln = c.eps_ln;
  p.eps_rms = c.eps_rms;
  const int bm = 32 * (8 / (int)c.H);
  p.qblocks = (int)((c.max_len + bm - 1) / bm);
  const int act = c.act == FNG_ACT_GELU ? ACT_GELU : ACT_SOFTMAX;
  switch (c.H) {
    case 1: return launch_h<1>(p, norm, act, s);
    case 2: return launch_h<2>(p, norm, act, s);
    case 4: return launch_h<4>(p, norm, act, s);
    default: return FNG_ERR_UNSUPPORTED;
  }
}

}  // namespace fng
