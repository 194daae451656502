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
// Work split: one workgroup = max(4, H) waves = (waves/H row groups) x H
// heads; wave (g, h) owns 32 query rows of head h (H = 8: one row group of
// 32 rows, eight waves, one workgroup per CU).  The page's norms run across heads, so
// where it exchanges statistics between the CTAs of a cluster, the waves of
// one workgroup exchange per-(row, head) partials through LDS: (mean, M2) of
// each head merged with the pairwise formula for the LayerNorm, sums of
// squares for the RMSNorm.
//
// Data movement: every global read is an HBM -> LDS copy of whole rows
// (buffer_load ... lds, 16 B per lane, 16-B chunks XOR-swizzled per row so
// the fragment reads below are bank-conflict free): the block's query rows
// (all heads, contiguous in memory), key and value tiles of 32 keys for all
// heads, and the raw query rows again for the residuals while the last tile
// is computed.  One K region and one V region are recycled separately: the
// next K tile is copied while this tile's activation and P V run, the next V
// tile while the next scores are computed.  At 65 KB of LDS two workgroups
// share a CU, so one's MFMAs overlap the other's vector work and copies.
// The output goes back through LDS so that it is stored as whole rows.
//
// Arithmetic: K and V stay bf16 as stored.  The normalized queries and the
// activations P are split into bf16 high and low parts (x = hi + lo to about
// 16 significant bits), so every product is a bf16 MFMA with fp32
// accumulation: S^T = K_h (q_hi + q_lo)^T, O^T += V_h^T (P_hi + P_lo)^T.  K
// fragments are read with ds_read_b128 in the key order that hands P to the
// next MFMA without a shuffle; V^T fragments come from V [key][d] through the
// transposing read ds_read_b64_tr_b16.
#include <type_traits>

#include "fng_device.h"
#include "fng_internal.h"

namespace fng {

namespace {

constexpr int kD = 128;
constexpr int kKT = 32;                 // keys per tile
constexpr int kRowB = kD * 2;           // bytes of one head's row
constexpr int kTileB = kKT * kRowB;     // one head's K (or V) tile, [key][d]
constexpr float kLazy = 8.0f;           // running-max hysteresis (log2 units)

enum : int { ACT_SOFTMAX = 0, ACT_GELU = 1 };

template <bool B>
using flag = std::integral_constant<bool, B>;

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

template <int H>
constexpr int fna_waves() { return H <= 4 ? 4 : H; }

template <int H, bool NORM, int ACT>
__global__ __launch_bounds__(64 * fna_waves<H>(), H <= 4 ? 2 : 1) void fna_kernel(FnaParams p) {
  constexpr int NW = fna_waves<H>();       // waves per workgroup
  constexpr int NT = 64 * NW;
  constexpr int G = NW / H;                // row groups
  constexpr int BM = 32 * G;               // query rows per workgroup
  constexpr int RB = H * kRowB;            // bytes per query row (all heads)
  constexpr int QSB = BM * RB;             // the block's query rows
  constexpr int KVB = H * kTileB;          // one K (or V) tile of every head
  constexpr int NK = KVB / (1024 * NW);    // 1 KB copies per wave for one K or V tile
  constexpr int NQ = QSB / (1024 * NW);    // ... for the block's query rows
  // LDS: K tile | V tile | query rows (their own region unless they fit the V
  // region, H >= 4) | statistics exchange
  constexpr bool QV = KVB == QSB;          // query rows fill the V (prologue) and K (epilogue) regions
  constexpr int KREG = 0, VREG = KVB;
  constexpr int QPRO = QV ? VREG : 2 * KVB;      // query rows in the prologue
  constexpr int QEPI = QV ? KREG : 2 * KVB;      // residual rows / output
  constexpr int MAIN = QV ? 2 * KVB : 2 * KVB + QSB;
  static_assert(H != 4 || QV, "H = 4: the query block fills the K or V region");
  static_assert(H <= 4 || (QV && NK * 1024 * NW == KVB && NQ * 1024 * NW == QSB), "H = 8 layout");
  static_assert(H > 4 || MAIN + BM * H * 8 <= 80 * 1024, "two workgroups per CU");
  static_assert(MAIN + BM * H * 8 <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) char smem[MAIN + BM * H * 8];
  FNG_LDS char* lds = (FNG_LDS char*)smem;
  FNG_LDS float* xch = (FNG_LDS float*)(lds + MAIN);  // [BM][H][2] statistics exchange

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  // the batch's query rows that exist; rows past them copy as zeros
  const int brows = max(0, min(len, p.T - r0));
  const i32x4_t qr = dma_rsrc(p.Q + (size_t)r0 * H * kD, (uint32_t)(brows * RB));
  const i32x4_t kr = dma_rsrc(p.K + (size_t)b * p.Skv * H * kD, (uint32_t)(p.Skv * RB));
  const i32x4_t vr = dma_rsrc(p.V + (size_t)b * p.Skv * H * kD, (uint32_t)(p.Skv * RB));
  const uint32_t qblk = (uint32_t)(qb * BM) * (uint32_t)RB;

  // ---- HBM -> LDS copies ---------------------------------------------------
  // Rows keep their global layout; the 16-B chunk c of row r sits at chunk
  // c ^ (r % 16) (query rows, K) or c ^ 4 (r % 4) (V).  Wave w copies 1 KB
  // blocks; lane l's 16 B are block byte 16 l.
  auto copy_q = [&](FNG_LDS char* qs) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int blk = wave * NQ + i;
      const int idx = blk * 1024 + lane * 16;
      const int r = idx / RB, pc = (idx % RB) / 16;
      dma16(qr, qs + blk * 1024, qblk + (uint32_t)(r * RB + (pc ^ (r & 15)) * 16));
    }
  };
  // K or V tile kt of every head: block j is head j / 8, keys 4 (j % 8) ..
  auto copy_kv = [&](bool isv, int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int blk = wave * NK + i;
      const int hd = blk / 8, r = 4 * (blk % 8) + (lane >> 4), pc = lane & 15;
      const uint32_t base = (uint32_t)((((kt * kKT + r) * H + hd) * kD) * 2);
      if (isv) dma16(vr, lds + VREG + blk * 1024, base + (uint32_t)((pc ^ (4 * (r & 3))) * 16));
      else dma16(kr, lds + KREG + blk * 1024, base + (uint32_t)((pc ^ (r & 15)) * 16));
    }
  };

  // ---- prologue: the block's query rows and the first key tile -------------
  copy_q(lds + QPRO);
  copy_kv(false, 0);
  if constexpr (!QV) copy_kv(true, 0);
  wait_vmcnt<(QV ? NK : 2 * NK)>();  // this wave's query copies have landed
  lds_barrier();

  // lane holds d = 16kk + 8hi + 0..7 of its row and head: the MFMA B operand
  u32x4_t qh[8], ql[8];
  float mu = 0.f, rstd = 1.f;
  {
    u32x4_t raw[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      raw[kk] = lds_read16(lds + QPRO + lrow * RB + (((16 * h + 2 * kk + hi) ^ (lrow & 15)) * 16));
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
    }
    // normalized (and pre-scaled) query, split into bf16 high and low parts.
    // The mean is subtracted before the scale: x - mu is exact for the
    // values near the mean (and 0 on a constant row, whose normalized row is
    // then exactly 0); x * mul - mu * mul would leave the rounding of mu * mul,
    // which the output RMSNorm amplifies by up to 1/sqrt(eps) when the
    // attention output is that small.
    const float mul = rstd * p.scale;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = raw[kk][e];
        const float x0 = (bf16lo(w) - mu) * mul, x1 = (bf16hi(w) - mu) * mul;
        const uint32_t hw = pack_bf16(x0, x1);
        qh[kk][e] = hw;
        ql[kk][e] = pack_bf16(x0 - bf16lo(hw), x1 - bf16hi(hw));
      }
  }
  if constexpr (QV) {
    lds_barrier();  // every wave has read its query rows: the V region is free
    copy_kv(true, 0);
  }

  // ---- main loop over key tiles ----------------------------------------------
  // K fragment (A operand of S^T): row kappa(l32), 16 B at d = 16kk + 8hi.
  const int krow = kappa(l32);
  int koff[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) koff[kk] = KREG + h * kTileB + krow * kRowB + (((2 * kk + hi) ^ (krow & 15)) * 16);
  // V^T fragment (A operand of O^T) through two transposing reads: lane
  // (group g4 = lane / 16, li = lane % 16) addresses key 8 (g4 / 2) + li / 4
  // (+4 for the second read) and d = 32 dt + 16 (g4 % 2) + 4 (li % 4)
  const int g4 = lane >> 4, li = lane & 15;
  const int vkey = 8 * (g4 >> 1) + (li >> 2);
  int voff[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int d = 32 * dt + 16 * (g4 & 1) + 4 * (li & 3);
    voff[dt] = VREG + h * kTileB + vkey * kRowB + ((((d >> 3) ^ (4 * (vkey & 3)))) * 16) + (d & 7) * 2;
  }

  f32x16_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;
  const int ntiles = (p.Skv + kKT - 1) / kKT;

  // S^T (32 keys x 32 queries) of tile kt: register r <-> key 16(r/8) + 8hi + r%8
  auto scores = [&](f32x16_t& sa) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sa[r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const u32x4_t kf = lds_read16(lds + koff[kk]);
      sa = mfma_bf16(kf, qh[kk], sa);
      sa = mfma_bf16(kf, ql[kk], sa);
    }
  };
  // activation of tile kt's scores -> the P^T operand (k16 step c: keys
  // 16c + 8hi + 0..7) as bf16 high and low parts.  Branch-free, so that it
  // interleaves with the next tile's score MFMAs.  Keys past Skv have zero K
  // rows (the copies zero-fill), hence score 0: GELU(0) = 0 needs no mask;
  // softmax masks them (only the last tile, RAGGED).  Softmax keeps a running
  // max and sum and returns the factor O must be rescaled by (rescale()).
  auto activate = [&](auto ragged, const f32x16_t& sa, int kt, u32x4_t (&ph)[2], u32x4_t (&pl)[2])
      __attribute__((always_inline)) {
    constexpr bool RAGGED = decltype(ragged)::value;
    float pr[16];
    float alpha = 1.f;
    if constexpr (ACT == ACT_SOFTMAX) {
      float sc[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = sa[r];
      if constexpr (RAGGED) {
        const int kvalid = p.Skv - kt * kKT;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (16 * (r >> 3) + 8 * hi + (r & 7) >= kvalid) sc[r] = -INFINITY;
      }
      float mx = sc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
      mx = half_swap_max(mx);
      const float mnew = mx > mrun + kLazy ? mx : mrun;
      alpha = (mnew == mrun || mrun == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(mrun - mnew);
      mrun = mnew;
      float ls[2] = {0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pr[r] = __builtin_amdgcn_exp2f(sc[r] - mrun);
        ls[r & 1] += pr[r];
      }
      lrun = fmaf(lrun, alpha, ls[0] + ls[1]);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) pr[r] = gelu_tanh(sa[r]);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a0 = pr[8 * c + 2 * e], a1 = pr[8 * c + 2 * e + 1];
        const uint32_t hw = pack_bf16(a0, a1);
        ph[c][e] = hw;
        pl[c][e] = pack_bf16(a0 - bf16lo(hw), a1 - bf16hi(hw));
      }
    return alpha;
  };
  auto rescale = [&](float alpha) __attribute__((always_inline)) {
    if constexpr (ACT == ACT_SOFTMAX) {
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
      }
    }
  };
  // O^T += V^T P^T with the V tile in the V region
  auto pv = [&](const u32x4_t (&ph)[2], const u32x4_t (&pl)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const FNG_LDS char* va = lds + voff[dt] + c * 16 * kRowB;
        const u32x2_t lo = lds_read_tr16(va);
        const u32x2_t hi2 = lds_read_tr16(va + 4 * kRowB);
        const u32x4_t vf = {lo[0], lo[1], hi2[0], hi2[1]};
        o[dt] = mfma_bf16(vf, ph[c], o[dt]);
        o[dt] = mfma_bf16(vf, pl[c], o[dt]);
      }
  };
  // after the K region is read: the next K tile
  auto next_k = [&](int kt) __attribute__((always_inline)) {
    if (kt + 1 < ntiles) copy_kv(false, kt + 1);
  };
  // wait for the V tile, which is older than the copy next_k(kt) issued
  auto wait_v = [&](int kt) __attribute__((always_inline)) {
    if (kt + 1 < ntiles) wait_vmcnt<NK>();
    else wait_vmcnt<0>();
  };

  // Software pipeline: the scores of tile kt are computed while the
  // activation of tile kt - 1 runs (MFMA and vector work of one wave
  // overlap), then tile kt - 1's P V product.  K is one tile ahead of V:
  // the K region holds tile kt while the V region still holds tile kt - 1.
  // Copies in flight, oldest first: K(kt), V(kt - 1) before tile kt's scores
  // (V(0), K(1) at kt = 1); V(kt - 1), then K(kt + 1) before tile kt - 1's
  // P V product.
  f32x16_t scur, sprev;
  u32x4_t ph[2], pl[2];
  wait_vmcnt<NK>();
  lds_barrier();  // K tile 0 is in LDS
  scores(scur);
  lds_barrier();  // every wave has read K tile 0
  next_k(0);
  for (int kt = 1; kt < ntiles; ++kt) {
    sprev = scur;
    if (kt == 1) wait_vmcnt<0>();
    else wait_vmcnt<NK>();
    lds_barrier();  // K tile kt is in LDS
    scores(scur);
    float alpha = activate(flag<false>{}, sprev, kt - 1, ph, pl);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);  // ten vector ops
    }
    // the operands are produced here, beside the MFMAs, not sunk past the
    // barrier to their use
    asm volatile("" : "+v"(ph[0]), "+v"(ph[1]), "+v"(pl[0]), "+v"(pl[1]), "+v"(alpha));
    lds_barrier();  // every wave has read K tile kt
    next_k(kt);
    wait_v(kt);
    rescale(alpha);
    lds_barrier();  // V tile kt - 1 is in LDS
    pv(ph, pl);
    lds_barrier();  // every wave has read V tile kt - 1
    copy_kv(true, kt);
  }
  const float alpha = activate(flag<true>{}, scur, ntiles - 1, ph, pl);
  rescale(alpha);
  wait_vmcnt<0>();
  lds_barrier();  // the last V tile (and the residual rows) are in LDS
  pv(ph, pl);

  // ---- epilogue ------------------------------------------------------------
  lds_barrier();  // every wave is done with the last tile
  FNG_LDS char* qs = lds + QEPI;
  // lane (l32, hi) holds, in register 4 r4 + e of o[dt], d = 32 dt + 8 r4 + 4 hi + e:
  // 8 B at chunk 16h + 4dt + r4 (swizzled), byte 8hi of the chunk
  auto epi_addr = [&](int dt, int r4) __attribute__((always_inline)) {
    return qs + lrow * RB + (((16 * h + 4 * dt + r4) ^ (lrow & 15)) * 16) + hi * 8;
  };
  const float inv = (ACT == ACT_SOFTMAX) ? 1.0f / half_swap_sum(lrun) : 1.0f;
  float rstd2 = 1.f;
  // the residuals come from the split query still in registers: qh + ql is
  // (x - mu) rstd scale to about 2^-17 relative, so ln = (qh + ql) / scale and
  // x = (qh + ql) / (scale rstd) + mu.  Its lane layout (d = 16kk + 8hi + ..)
  // is moved to O's (d = 32dt + 8r4 + 4hi + ..) by swapping the words the
  // lane halves exchange (v_permlane32_swap): word pair e, e + 2 of kk gives
  // d = 8(2kk) + 4hi + 2e .. in the first result and d = 8(2kk + 1) + 4hi + 2e
  // .. in the second.
  float xres[4][4][4];  // [dt][r4][e] residual-1 term ln and x, see below
  if constexpr (NORM) {
    const float to_ln = 1.0f / p.scale;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const auto sh = __builtin_amdgcn_permlane32_swap(qh[kk][e], qh[kk][e + 2], false, false);
        const auto sl = __builtin_amdgcn_permlane32_swap(ql[kk][e], ql[kk][e + 2], false, false);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int m = 2 * kk + half;  // 8-block of d: dt = m / 4, r4 = m % 4
          const uint32_t wh = half ? sh[1] : sh[0], wl = half ? sl[1] : sl[0];
          xres[m >> 2][m & 3][2 * e] = (bf16lo(wh) + bf16lo(wl)) * to_ln;
          xres[m >> 2][m & 3][2 * e + 1] = (bf16hi(wh) + bf16hi(wl)) * to_ln;
        }
      }
    float ss = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = fmaf(o[dt][4 * r4 + e], inv, xres[dt][r4][e]);  // + ln (residual 1)
          o[dt][4 * r4 + e] = v;
          ss = fmaf(v, v, ss);
        }
    ss = half_swap_sum(ss);
    if (hi == 0) xch[(lrow * H + h) * 2] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int j = 0; j < H; ++j) tot += xch[(lrow * H + j) * 2];
    rstd2 = __builtin_amdgcn_rsqf(tot * (1.0f / (H * kD)) + p.eps_rms);
    if (h == 0 && hi == 0 && valid) {
      if (p.ln_mean_out) p.ln_mean_out[row] = mu;
      if (p.ln_rstd_out) p.ln_rstd_out[row] = rstd;
      if (p.rms_rstd_out) p.rms_rstd_out[row] = rstd2;
    }
  }
  // the output goes to LDS, then back to HBM as whole rows
  const float inv_rstd = 1.0f / rstd;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float v[4];
      if constexpr (NORM) {
#pragma unroll
        for (int e = 0; e < 4; ++e)  // + x (residual 2), x = ln / rstd + mu
          v[e] = fmaf(o[dt][4 * r4 + e], rstd2, fmaf(xres[dt][r4][e], inv_rstd, mu));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = o[dt][4 * r4 + e] * inv;
      }
      *reinterpret_cast<FNG_LDS u32x2_t*>(epi_addr(dt, r4)) = u32x2_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
    }
  lds_barrier();
  // whole rows back to HBM: 16 B per lane, rows of the batch only, non-temporal
  // (written once; streaming them keeps the batches' K/V lines in the L2:
  // 224 -> 219 us on the 768-batch workload; the same hint on the 8-byte
  // stores of the per-head attention kernel made it 1.5x slower)
#pragma unroll
  for (int i = 0; i < QSB / (16 * NT); ++i) {
    const int c = tid + NT * i;
    const int r = c / (RB / 16), lc = c % (RB / 16);
    const int q = qb * BM + r;
    if (q < len && r0 + q < p.T) {
      const u32x4_t v = lds_read16(qs + r * RB + ((lc ^ (r & 15)) * 16));
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p.O + (size_t)(r0 + q) * H * kD + lc * 8));
    }
  }
}

template <int H>
int launch_h(const FnaParams& p, bool norm, int act, hipStream_t s) {
  const dim3 grid((unsigned)(p.B * p.qblocks)), block(64 * fna_waves<H>());
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
  const int bm = c.H <= 4 ? 32 * (4 / (int)c.H) : 32;
  p.qblocks = (int)((c.max_len + bm - 1) / bm);
  const int act = c.act == FNG_ACT_GELU ? ACT_GELU : ACT_SOFTMAX;
  switch (c.H) {
    case 1: return launch_h<1>(p, norm, act, s);
    case 2: return launch_h<2>(p, norm, act, s);
    case 4: return launch_h<4>(p, norm, act, s);
    case 8: return launch_h<8>(p, norm, act, s);
    default: return FNG_ERR_UNSUPPORTED;
  }
}

}  // namespace fng
