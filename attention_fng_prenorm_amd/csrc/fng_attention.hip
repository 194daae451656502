// Norm-sandwiched attention for gfx950, after section 4 (FlashNormAttention) of
// "Towards Free Normalization: Fusing Normalization into GEMM and Attention
// Kernels": the query rows are LayerNorm-ed in the kernel's prologue, the
// attention output rows are RMSNorm-ed in its epilogue, so neither norm makes
// its own trip through HBM.  Both norms run over head_dim (128) of one head;
// softmax is the activation; there are no residual adds.  NORM=false gives the
// plain attention baseline from the same code.
//
// Work split: one workgroup = 8 waves (two per SIMD, so one wave's softmax
// can issue while the other's MFMAs run) = 256 query rows of one (batch,
// head); each wave owns 32 query rows for the whole kernel and loops over the
// keys in tiles of 64 with an online (running max / running sum) softmax.
//
// Orientation: the score MFMA is issued as S^T = K * Q^T and the output MFMA as
// O^T = V^T * P^T, so lane l always holds query row l % 32: the softmax row
// max/sum, the LayerNorm and the RMSNorm are all in-lane sums plus one
// exchange with lane l ^ 32.  The probabilities P stay in registers between
// the two MFMAs: the score MFMA's rows are loaded in a permuted key order so
// that a lane holds them in the order the output MFMA consumes them, and V is
// staged transposed so its fragments are plain row reads.
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
constexpr int kWaves = 8;              // 2 per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kBQ = 32 * kWaves;       // query rows per workgroup, 32 per wave
constexpr int kBK = 64;                // keys per tile
constexpr int kRowK = kD * 2 + 16;     // bytes per K row ([key][d]) in LDS, padded
constexpr int kRowV = kBK * 2 + 16;    // bytes per V^T row ([d][key]) in LDS, padded
constexpr int kTileK = kBK * kRowK;
constexpr int kTileV = kD * kRowV;
constexpr int kOffV = 2 * kTileK;      // LDS: K buffers 0/1, then V^T buffers 0/1
constexpr int kChunks = kBK * kD / 8 / kThreads;  // 16-byte chunks per thread per tile
// The running max of a row is only moved when a tile's max exceeds it by more
// than this (log2 domain), so most tiles skip the accumulator rescale; the
// probabilities stay below 2^kLazy, well inside fp16.
constexpr float kLazy = 8.0f;

// LDS layouts (64 banks of 4 B).  K is kept [key][d] and V transposed,
// [d][key], both in fp16 and with every row padded by 16 bytes: a fragment
// read (16 lanes on 16 consecutive rows at one 16-byte column) then covers all
// banks, and a lane's offsets for the different fragments differ by constants.
//
// Key order: the score MFMA's A operand row m is loaded with key kappa(m)
// (bits 2 and 3 of m swapped), which leaves lane (q, hi) of S^T holding, in
// registers 8i..8i+7 of key block w, the eight consecutive keys
// 32w + 16i + 8hi + (0..7): exactly the k-slots the output MFMA takes its
// P^T operand in, so the probabilities go from one MFMA to the next without a
// shuffle and V^T fragments are plain 16-byte row reads.
__device__ __forceinline__ int kappa(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

template <bool B>
using flag = std::integral_constant<bool, B>;

template <bool NORM>
__global__ __launch_bounds__(kThreads, 1) void attention_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kTileK + 2 * kTileV];
  static_assert(kWaves * 32 * kD * 2 <= 2 * kTileK + 2 * kTileV, "the output rows are staged over the K/V buffers");
  FNG_LDS char* lds = (FNG_LDS char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const uint32_t t0 = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = (int)(t0 % (uint32_t)p.tiles_q);
  const int bh = (int)(t0 / (uint32_t)p.tiles_q);
  const int h = bh % p.H;
  const int b = bh / p.H;
  const int H = p.H, Sq = p.Sq, Skv = p.Skv;

  // per-batch buffer resources: rows past the sequence end read as zero
  const size_t qbase = (size_t)b * Sq * H * kD;
  const size_t kbase = (size_t)b * Skv * H * kD;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(p.Q + qbase, (uint32_t)((size_t)Sq * H * kD * 2));
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(p.K + kbase, (uint32_t)((size_t)Skv * H * kD * 2));
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(p.V + kbase, (uint32_t)((size_t)Skv * H * kD * 2));

  // ---- queries: lane holds d = 16*kk + 8*hi + e of query row q, normalized
  // (NORM) and pre-multiplied by sm_scale * log2(e) ---------------------------
  const int q = qt * kBQ + wave * 32 + l32;
  u32x4_t qf[8];
  {
    const uint32_t qoff = (uint32_t)(((size_t)q * H + h) * kD * 2);
    u32x4_t raw[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) raw[kk] = buffer_load16(qr, qoff + (uint32_t)(16 * kk + 8 * hi) * 2u);
    float shift = 0.f, mul = p.scale_log2;
    if constexpr (NORM) {
      float s = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int e = 0; e < 4; ++e) s += bf16lo(raw[kk][e]) + bf16hi(raw[kk][e]);
      const float mean = half_swap_sum(s) * (1.0f / kD);
      float s2 = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = bf16lo(raw[kk][e]) - mean, x1 = bf16hi(raw[kk][e]) - mean;
          s2 += x0 * x0 + x1 * x1;
        }
      const float rstd = __builtin_amdgcn_rsqf(half_swap_sum(s2) * (1.0f / kD) + p.eps_ln);
      shift = mean;
      mul = rstd * p.scale_log2;
      if (hi == 0 && q < Sq) {
        const size_t si = ((size_t)b * Sq + q) * H + h;
        if (p.ln_mean_out) p.ln_mean_out[si] = mean;
        if (p.ln_rstd_out) p.ln_rstd_out[si] = rstd;
      }
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        qf[kk][e] = pack_f16((bf16lo(raw[kk][e]) - shift) * mul, (bf16hi(raw[kk][e]) - shift) * mul);
  }

  // ---- lane-constant LDS offsets -------------------------------------------
  // K fragment (kk, w): key 32w + kappa(l32), d = 16kk + 8hi + (0..7)
  const int koff = kappa(l32) * kRowK + hi * 16;
  // V^T fragment (c, dt): d = 32dt + l32, keys 16c + 8hi + (0..7)
  const int voff = l32 * kRowV + hi * 16;

  // ---- K/V staging: 1024 chunks of 8 elements per tile and tensor ---------
  // K: chunk c = tid + 512i is key c/16, d 8(c%16)..+7, stored as it is.
  // V: thread holds keys 2p, 2p+1 (p = tid%32) at d 8(tid/32)..+7 and writes
  // the transposed pairs, one 4-byte word per d row.
  u32x4_t rk[kChunks], rv[kChunks];
  auto gload_k = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + kThreads * i;
      const int key = kt * kBK + (c >> 4), dc = c & 15;
      rk[i] = buffer_load16(kr, (uint32_t)((((size_t)key * H + h) * kD + dc * 8) * 2));
    }
  };
  auto gload_v = [&](int kt) __attribute__((always_inline)) {
    const int key = kt * kBK + 2 * (tid & 31), dc = tid >> 5;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      rv[i] = buffer_load16(vr, (uint32_t)((((size_t)(key + i) * H + h) * kD + dc * 8) * 2));
  };
  auto sstore_k = [&](int buf) __attribute__((always_inline)) {
    FNG_LDS char* dst = lds + buf * kTileK;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + kThreads * i;
      u32x4_t v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = bf16x2_to_f16x2(rk[i][e]);
      lds_write16(dst + (c >> 4) * kRowK + (c & 15) * 16, v);
    }
  };
  auto sstore_v = [&](int buf) __attribute__((always_inline)) {
    FNG_LDS char* dst = lds + kOffV + buf * kTileV + (tid >> 5) * 8 * kRowV + (tid & 31) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      *reinterpret_cast<FNG_LDS uint32_t*>(dst + (2 * e) * kRowV) = pack_f16(bf16lo(rv[0][e]), bf16lo(rv[1][e]));
      *reinterpret_cast<FNG_LDS uint32_t*>(dst + (2 * e + 1) * kRowV) = pack_f16(bf16hi(rv[0][e]), bf16hi(rv[1][e]));
    }
  };

  // ---- running state -------------------------------------------------------
  f32x16_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float mrun = -INFINITY;  // running max (log2 domain) of row q
  float lrun = 0.f;        // this lane's share of the running sum

  // S^T = K Q^T for keys 32w + (0..31): register r <-> key 32w + 16(r/8) + 8hi + r%8.
  // Fragment i = 2kk + w; reads run kPre fragments ahead of the MFMAs.
  constexpr int kPre = 4;
  auto qk = [&](int t, f32x16_t(&s)[2]) __attribute__((always_inline)) {
    const FNG_LDS char* kb = lds + (t & 1) * kTileK + koff;
    auto rd = [&](int i) { return lds_read16(kb + (i >> 1) * 32 + (i & 1) * 32 * kRowK); };
#pragma unroll
    for (int w = 0; w < 2; ++w)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[w][r] = 0.f;
    u32x4_t kf[kPre];
#pragma unroll
    for (int i = 0; i < kPre; ++i) kf[i] = rd(i);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i & 1] = mfma_f16(kf[i % kPre], qf[i >> 1], s[i & 1]);
      if (i + kPre < 16) kf[i % kPre] = rd(i + kPre);
    }
  };
  // O^T += V^T P^T; fragment i = 4c + dt, read kPre fragments ahead
  auto pv = [&](int t, const u32x4_t(&pf)[4]) __attribute__((always_inline)) {
    const FNG_LDS char* vb = lds + kOffV + (t & 1) * kTileV + voff;
    auto rd = [&](int i) { return lds_read16(vb + (i >> 2) * 32 + (i & 3) * 32 * kRowV); };
    u32x4_t vf[kPre];
#pragma unroll
    for (int i = 0; i < kPre; ++i) vf[i] = rd(i);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      o[i & 3] = mfma_f16(vf[i % kPre], pf[i >> 2], o[i & 3]);
      if (i + kPre < 16) vf[i % kPre] = rd(i + kPre);
    }
  };
  // softmax, first half: mask the keys past the end, row max, running max
  // update, rescale of l and o when the max moved
  auto sm_max = [&](f32x16_t(&s)[2], int t, bool mask) __attribute__((always_inline)) {
    if (mask) {
      const int kvalid = Skv - t * kBK;
#pragma unroll
      for (int w = 0; w < 2; ++w)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * w + 16 * (r >> 3) + 8 * hi + (r & 7) >= kvalid) s[w][r] = -INFINITY;
    }
    float mx = s[0][0];
#pragma unroll
    for (int w = 0; w < 2; ++w)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[w][r]);
    mx = half_swap_max(mx);
    const float mold = mrun;
    const float mnew = mx > mold + kLazy ? mx : mold;
    const float alpha = (mnew == mold || mold == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(mold - mnew);
    mrun = mnew;
    lrun *= alpha;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
    }
  };
  // softmax, second half: probabilities relative to the running max, row sum,
  // fp16 pack as the B operand: k16 step c holds keys 16c + 8hi + (0..7)
  auto sm_exp = [&](f32x16_t(&s)[2], u32x4_t(&pf)[4]) __attribute__((always_inline)) {
    // row sum over the fp16 probabilities the output MFMA consumes, two per
    // v_dot2 (the operand is taken from the fp16 pair itself, not re-read out
    // of the packed vector)
    const f16x2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int w = c >> 1, r0 = 8 * (c & 1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f16x2_t h2 = {(_Float16)__builtin_amdgcn_exp2f(s[w][r0 + 2 * e] - mrun),
                            (_Float16)__builtin_amdgcn_exp2f(s[w][r0 + 2 * e + 1] - mrun)};
        pf[c][e] = __builtin_bit_cast(uint32_t, h2);
        ls[e] = __builtin_amdgcn_fdot2(h2, ones, ls[e], false);
      }
    }
    lrun += (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };

  const int ntiles = (Skv + kBK - 1) / kBK;
  const bool ragged = (Skv % kBK) != 0;

  // Software pipeline over key tiles: iteration t computes the scores of tile
  // t and the softmax and output update of tile t - 1.  K(t) and V(t - 1) are
  // resident together; K(t + 1) and V(t) are staged during iteration t into
  // the buffers freed by iteration t - 1.
  //
  // The two waves that share a SIMD (w and w + 4) run the iteration's phases
  // in different orders, so that while one is in its VALU-heavy softmax the
  // other issues MFMAs:
  //   waves 0-3: softmax(t - 1), O += V(t - 1) P(t - 1), S(t) = K(t) Q^T
  //   waves 4-7: S(t) = K(t) Q^T, softmax(t - 1), O += V(t - 1) P(t - 1)
  // (next_known: tile t + 1 is known to exist.)
  f32x16_t sa[2], sb[2];
  u32x4_t pf[4];
  auto iter = [&](auto order_a, auto has_prev, auto has_cur, auto maskable, auto next_known, int t,
                  f32x16_t(&s_prev)[2], f32x16_t(&s_cur)[2]) __attribute__((always_inline)) {
    constexpr bool A = decltype(order_a)::value;
    constexpr bool PREV = decltype(has_prev)::value;
    constexpr bool CUR = decltype(has_cur)::value;
    constexpr bool MASKABLE = decltype(maskable)::value;
    const bool next_k = decltype(next_known)::value || (CUR && t + 1 < ntiles);
    const bool mask_prev = MASKABLE && ragged && t - 1 == ntiles - 1;
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
    if (next_k) gload_k(t + 1);
    if constexpr (CUR) gload_v(t);
    if constexpr (!A && CUR) {
      qk(t, s_cur);
      fence();
    }
    if constexpr (PREV) {
      sm_max(s_prev, t - 1, mask_prev);
      sm_exp(s_prev, pf);
      fence();
      pv(t - 1, pf);
      fence();
    }
    if constexpr (A && CUR) {
      qk(t, s_cur);
      fence();
    }
    if constexpr (CUR) {
      if (next_k) sstore_k((t + 1) & 1);
      sstore_v(t & 1);
      __syncthreads();
    }
  };

  auto pipeline = [&](auto order_a) __attribute__((always_inline)) {
    iter(order_a, flag<false>{}, flag<true>{}, flag<true>{}, flag<false>{}, 0, sb, sa);
    int t = 1;
    for (; t + 1 < ntiles - 1; t += 2) {
      iter(order_a, flag<true>{}, flag<true>{}, flag<false>{}, flag<true>{}, t, sa, sb);
      iter(order_a, flag<true>{}, flag<true>{}, flag<false>{}, flag<true>{}, t + 1, sb, sa);
    }
    if (t < ntiles - 1) {
      iter(order_a, flag<true>{}, flag<true>{}, flag<false>{}, flag<true>{}, t, sa, sb);
#pragma unroll
      for (int w = 0; w < 2; ++w) sa[w] = sb[w];
      ++t;
    }
    if (t == ntiles - 1) {
      iter(order_a, flag<true>{}, flag<true>{}, flag<true>{}, flag<false>{}, t, sa, sb);
      iter(order_a, flag<true>{}, flag<false>{}, flag<true>{}, flag<false>{}, t + 1, sb, sa);
    } else {  // a single key tile: its scores are in sa
      iter(order_a, flag<true>{}, flag<false>{}, flag<true>{}, flag<false>{}, t, sa, sb);
    }
  };

  gload_k(0);
  sstore_k(0);
  __syncthreads();
  if (wave < 4)
    pipeline(flag<true>{});
  else
    pipeline(flag<false>{});

  // ---- epilogue: 1/l, RMSNorm over d, bf16 store -------------------------
  const float inv = 1.0f / half_swap_sum(lrun);
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
    rstd = __builtin_amdgcn_rsqf(half_swap_sum(ss) * (1.0f / kD) + p.eps_rms);
    if (hi == 0 && q < Sq && p.rms_rstd_out) p.rms_rstd_out[((size_t)b * Sq + q) * H + h] = rstd;
  }
  // The wave's 32 output rows go through LDS (the K/V buffers are free once
  // every wave is past its last key tile) and out as whole 256-byte rows,
  // 16 bytes per lane: the lane's own values are 8-byte pieces of its row,
  // which stored directly cost more than the staging.  Chunk c of row r sits
  // at chunk c ^ (r % 16) of the row's 256 bytes (the 32 rows of one write
  // spread over the banks).
  __syncthreads();
  FNG_LDS char* stg = lds + wave * (32 * kD * 2);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = o[dt][4 * r4 + e] * inv * rstd;
      const int c = 4 * dt + r4;  // 16-byte chunk of d = 8c .. 8c + 7; this lane's half: hi
      *reinterpret_cast<FNG_LDS u32x2_t*>(stg + l32 * (kD * 2) + ((c ^ (l32 & 15)) * 16) + hi * 8) =
          u32x2_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
    }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 32 * 16 / 64; ++it) {
    const int idx = it * 64 + lane;  // 16 chunks per row, 32 rows
    const int r = idx >> 4, c = idx & 15;
    const int qq = qt * kBQ + wave * 32 + r;
    if (qq < Sq) {
      const u32x4_t v = lds_read16(stg + r * (kD * 2) + ((c ^ (r & 15)) * 16));
      *reinterpret_cast<u32x4_t*>(p.O + (((size_t)b * Sq + qq) * H + h) * kD + 8 * c) = v;
    }
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
    hipLaunchKernelGGL(attention_kernel<true>, dim3(p.total), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(attention_kernel<false>, dim3(p.total), dim3(kThreads), 0, s, p);
  return hipGetLastError() == hipSuccess ? FNG_OK : FNG_ERR_HIP;
}

}  // namespace fng
