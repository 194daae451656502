// Norm-sandwiched attention for gfx950, after section 4 (FlashNormAttention) of
// "Towards Free Normalization: Fusing Normalization into GEMM and Attention
// Kernels": the query rows are LayerNorm-ed in the kernel's prologue, the
// attention output rows are RMSNorm-ed in its epilogue, so neither norm makes
// its own trip through HBM.  Both norms run over head_dim (128) of one head;
// softmax is the activation; there are no residual adds.  NORM=false gives the
// plain attention baseline from the same code.
//
// Work split: one workgroup = 4 waves = 128 query rows of one (batch, head);
// each wave owns 32 query rows for the whole kernel and loops over the keys in
// tiles of 64 with an online (running max / running sum) softmax.
//
// Orientation: the score MFMA is issued as S^T = K * Q^T and the output MFMA as
// O^T = V^T * P^T, so lane l always holds query row l % 32: the softmax row
// max/sum, the LayerNorm and the RMSNorm are all in-lane sums plus one
// exchange with lane l ^ 32.  The probabilities P stay in registers between
// the two MFMAs: the key order in which a lane holds them is matched by the
// rows the V fragment is read from (ds_read_b64_tr_b16 on V kept [key][d]).
//
// Precision: MFMA operands are fp16 (K and V converted from bf16 while staged
// into LDS, the normalized queries and the probabilities rounded to fp16),
// accumulation and all statistics are fp32.  fp16 keeps three more mantissa
// bits than bf16 for the two operands the kernel itself produces (normalized
// q and P), which is what keeps the RMSNorm-amplified output error at the
// bf16 output-rounding level.
#include "fng_device.h"
#include "fng_internal.h"

namespace fng {

struct AttnParams {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  uint16_t* O;
  float* ln_mean_out;
  float* ln_rstd_out;
  float* rms_rstd_out;
  int B, Sq, Skv, H;
  float scale_log2;  // sm_scale * log2(e)
  float eps_ln, eps_rms;
  int tiles_q;
  int total;
};

constexpr int kD = 128;
constexpr int kBQ = 128;  // query rows per workgroup
constexpr int kBK = 64;   // keys per tile
constexpr int kTileBytes = kBK * kD * 2;

// LDS chunk swizzles (16-byte chunks, 16 per 256-byte row, 64 banks of 4 B):
// a K fragment read covers 16 consecutive keys at one chunk; a transposing V
// read covers keys k..k+3 and four consecutive chunks.
__device__ __forceinline__ int swz_k(int key) { return key & 15; }
__device__ __forceinline__ int swz_v(int key) { return (key & 3) << 2; }

template <bool NORM>
__global__ __launch_bounds__(256, 2) void attention_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) char smem[4 * kTileBytes];  // K, V x 2 stages
  FNG_LDS char* lds = (FNG_LDS char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const uint32_t t = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = (int)(t % (uint32_t)p.tiles_q);
  const int bh = (int)(t / (uint32_t)p.tiles_q);
  const int h = bh % p.H;
  const int b = bh / p.H;
  const int H = p.H, Sq = p.Sq, Skv = p.Skv;

  // per-batch buffer resources: rows past the sequence end read as zero
  const size_t qbase = (size_t)b * Sq * H * kD;
  const size_t kbase = (size_t)b * Skv * H * kD;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(p.Q + qbase, (uint32_t)((size_t)Sq * H * kD * 2));
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(p.K + kbase, (uint32_t)((size_t)Skv * H * kD * 2));
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(p.V + kbase, (uint32_t)((size_t)Skv * H * kD * 2));

  // ---- queries: lane holds d = 16*kk + 8*hi + e of query row q -------------
  const int q = qt * kBQ + wave * 32 + l32;
  const uint32_t qoff = (uint32_t)(((size_t)q * H + h) * kD * 2);
  u32x4_t qf[8];
  {
    u32x4_t raw[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) raw[kk] = buffer_load16(qr, qoff + (uint32_t)(16 * kk + 8 * hi) * 2u);
    if constexpr (NORM) {
      float s = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int e = 0; e < 4; ++e) s += bf16lo(raw[kk][e]) + bf16hi(raw[kk][e]);
      const float mean = xor_sum(s, 32) * (1.0f / kD);
      float s2 = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = bf16lo(raw[kk][e]) - mean, c = bf16hi(raw[kk][e]) - mean;
          s2 += a * a + c * c;
        }
      const float rstd = __builtin_amdgcn_rsqf(xor_sum(s2, 32) * (1.0f / kD) + p.eps_ln);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          qf[kk][e] = pack_f16((bf16lo(raw[kk][e]) - mean) * rstd, (bf16hi(raw[kk][e]) - mean) * rstd);
      if (hi == 0 && q < Sq) {
        const size_t si = ((size_t)b * Sq + q) * H + h;
        if (p.ln_mean_out) p.ln_mean_out[si] = mean;
        if (p.ln_rstd_out) p.ln_rstd_out[si] = rstd;
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int e = 0; e < 4; ++e) qf[kk][e] = bf16x2_to_f16x2(raw[kk][e]);
    }
  }

  // ---- K/V staging: 1024 chunks of 8 elements per tile, 4 per thread --------
  u32x4_t rk[4], rv[4];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int key = kt * kBK + (c >> 4), dc = c & 15;
      const uint32_t off = (uint32_t)((((size_t)key * H + h) * kD + dc * 8) * 2);
      rk[i] = buffer_load16(kr, off);
      rv[i] = buffer_load16(vr, off);
    }
  };
  auto sstore = [&](int stage) {
    FNG_LDS char* ks = lds + stage * (2 * kTileBytes);
    FNG_LDS char* vs = ks + kTileBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int key = c >> 4, dc = c & 15;
      u32x4_t k16, v16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        k16[e] = bf16x2_to_f16x2(rk[i][e]);
        v16[e] = bf16x2_to_f16x2(rv[i][e]);
      }
      lds_write16(ks + key * (kD * 2) + ((dc ^ swz_k(key)) & 15) * 16, k16);
      lds_write16(vs + key * (kD * 2) + ((dc ^ swz_v(key)) & 15) * 16, v16);
    }
  };

  f32x16_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float mrun = -INFINITY;  // running max (log2 domain) of query row q
  float lrun = 0.f;        // this lane's share of the running sum

  const int ntiles = (Skv + kBK - 1) / kBK;
  gload(0);
  sstore(0);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int stage = kt & 1;
    const bool more = kt + 1 < ntiles;
    if (more) gload(kt + 1);
    const FNG_LDS char* ks = lds + stage * (2 * kTileBytes);
    const FNG_LDS char* vs = ks + kTileBytes;

    // S^T for keys 32*u + (0..31): register r <-> key 32u + 8(r/4) + 4hi + r%4
    f32x16_t s[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[u][r] = 0.f;
      const int key = 32 * u + l32;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int dc = 2 * kk + hi;
        const u32x4_t kf = lds_read16(ks + key * (kD * 2) + ((dc ^ swz_k(key)) & 15) * 16);
        s[u] = mfma_f16(kf, qf[kk], s[u]);
      }
    }

    // online softmax in the log2 domain
    const int kvalid = Skv - kt * kBK;  // >= 1
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * u + 8 * (r >> 2) + 4 * hi + (r & 3);
        float v = s[u][r] * p.scale_log2;
        if (key >= kvalid) v = -INFINITY;
        s[u][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = xor_max(mx, 32);
    const float mnew = fmaxf(mrun, mx);
    const float alpha = exp2f(mrun - mnew);
    mrun = mnew;
    float ls = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = exp2f(s[u][r] - mnew);
        s[u][r] = e;
        ls += e;
      }
    lrun = lrun * alpha + ls;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] *= alpha;

    // P^T as the B operand: k16 step c holds keys 16c + 4hi + (0..3) in slots
    // 0..3 and 16c + 8 + 4hi + (0..3) in slots 4..7
    u32x4_t pf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int u = c >> 1, r0 = 8 * (c & 1);
      pf[c] = u32x4_t{pack_f16(s[u][r0 + 0], s[u][r0 + 1]), pack_f16(s[u][r0 + 2], s[u][r0 + 3]),
                      pack_f16(s[u][r0 + 4], s[u][r0 + 5]), pack_f16(s[u][r0 + 6], s[u][r0 + 7])};
    }
    // O^T += V^T P^T; V fragment rows are the same keys, read transposed
    const int g = lane >> 4, li = lane & 15;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int key0 = 16 * c + 4 * (g >> 1) + (li >> 2);
      const int key1 = key0 + 8;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int d = 32 * dt + 16 * (g & 1) + 4 * (li & 3);
        const int dc = d >> 3, db = (d & 7) * 2;
        const u32x2_t a = lds_read_tr16(vs + key0 * (kD * 2) + ((dc ^ swz_v(key0)) & 15) * 16 + db);
        const u32x2_t bb = lds_read_tr16(vs + key1 * (kD * 2) + ((dc ^ swz_v(key1)) & 15) * 16 + db);
        o[dt] = mfma_f16(u32x4_t{a[0], a[1], bb[0], bb[1]}, pf[c], o[dt]);
      }
    }
    if (more) sstore(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: 1/l, RMSNorm over d, bf16 store -------------------------
  const float inv = 1.0f / xor_sum(lrun, 32);
  float rstd = 1.f;
  if constexpr (NORM) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float v = o[i][r] * inv;
        ss += v * v;
      }
    rstd = __builtin_amdgcn_rsqf(xor_sum(ss, 32) * (1.0f / kD) + p.eps_rms);
    if (hi == 0 && q < Sq && p.rms_rstd_out) p.rms_rstd_out[((size_t)b * Sq + q) * H + h] = rstd;
  }
  if (q >= Sq) return;
  uint16_t* orow = p.O + (((size_t)b * Sq + q) * H + h) * kD;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * dt + 8 * r4 + 4 * hi;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = o[dt][4 * r4 + e] * inv;
        if constexpr (NORM) v[e] = (v[e]) * rstd;
      }
      *reinterpret_cast<u32x2_t*>(orow + d) = u32x2_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
    }
}

int launch_attention(const AttnCall& c, bool norm, hipStream_t s) {
  AttnParams p{};
  p.Q = static_cast<const uint16_t*>(c.Q);
  p.K = static_cast<const uint16_t*>(c.K);
  p.V = static_cast<const uint16_t*>(c.V);
  p.O = static_cast<uint16_t*>(c.O);
  p.ln_mean_out = c.ln_mean_out;
  p.ln_rstd_out = c.ln_rstd_out;
  p.rms_rstd_out = c.rms_rstd_out;
  p.B = (int)c.B;
  p.Sq = (int)c.Sq;
  p.Skv = (int)c.Skv;
  p.H = (int)c.H;
  p.scale_log2 = c.sm_scale * 1.4426950408889634f;
  p.eps_ln = c.eps_ln;
  p.eps_rms = c.eps_rms;
  p.tiles_q = (p.Sq + kBQ - 1) / kBQ;
  p.total = p.tiles_q * p.H * p.B;
  if (norm)
    hipLaunchKernelGGL(attention_kernel<true>, dim3(p.total), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(attention_kernel<false>, dim3(p.total), dim3(256), 0, s, p);
  return hipGetLastError() == hipSuccess ? FNG_OK : FNG_ERR_HIP;
}

}  // namespace fng
