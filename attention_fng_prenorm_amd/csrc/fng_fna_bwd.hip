// FlashNormAttention backward for gfx950, after section 4 of "Towards Free
// Normalization: Fusing Normalization into GEMM and Attention Kernels"
// ("Backward implementation").  Forward, for every query row x (H heads x 128):
//   n   = LayerNorm(x) across all H*128 values      (mean mu, rstd r1 saved)
//   s_h = n_h K_h^T * scale,  p_h = act(s_h)         (softmax or tanh GELU)
//   o_h = p_h V_h + n_h,  y = RMSNorm(o) (rstd r2 saved),  out = y + x
// Backward, given g = d out:
//   do  = r2 (g - y * mean(g y))                     (RMSNorm backward)
//   dp_h = do_h V_h^T,  ds_h = act'(dp_h) * scale
//   dn  = do + sum_h ds_h K_h                        (first residual)
//   dq  = g + r1 (dn - mean(dn) - n * mean(dn n))    (LayerNorm backward, second residual)
//   dV_h = sum over the batch's rows of p_h^T do_h,  dK_h = sum of ds_h^T n_h
// As on the page, nothing beyond the three per-row statistics is saved: n is
// rebuilt from x, mu and r1 and the RMSNorm output as y = out - x.  The
// softmax's row term delta = sum_keys p dp comes from the recomputed P and dP
// (the page rebuilds the attention output for it, which here would carry the
// bf16 output's rounding into every ds).
//
// Two kernels.  The norms couple all heads of a row and the key/value
// gradients sum over all rows of a batch; a batch's dK and dV for every head
// (512 KB in fp32) do not fit one compute unit, so:
//  * fna_bwd_rows_kernel: one workgroup = 32 x (4/H) rows of every head (wave
//    (g, h) owns 32 rows of head h, as in the forward), so the cross-head sums
//    are LDS exchanges.  Key and value tiles of 32 keys stream through LDS;
//    the softmax first makes one pass for the row's log-sum-exp and delta.
//    Writes dq, and do (fp16) and the log-sum-exp for the second kernel.
//  * fna_bwd_kv_kernel: one workgroup per (batch, head) with that head's K
//    and V in LDS (fp16); 8 waves in two groups that take alternate 32-row
//    blocks (one group's loads overlap the other's products); wave w of a
//    group owns keys 32w .. 32w + 31 and accumulates dK^T, dV^T over its
//    blocks, whose n and do are staged in LDS; the groups' sums are added at
//    the end.  Its softmax terms are made consistent within the kernel: per
//    row it sums L = sum_keys p and W = sum_keys p dp of its own P and dP
//    (across the key lanes, then the four waves) and uses p / L and
//    delta = W / L, so its ds sums to zero over the keys up to fp32 rounding,
//    as the exact one does (with one key the exact dK is zero).
//
// Arithmetic: MFMA 32x32x16 with fp32 accumulation.  The rows kernel takes K
// and V as stored (bf16, copied HBM -> LDS) and rounds n * scale, do and ds to
// bf16, for GELU split into high and low parts (x = hi + lo to about 16
// significant bits; one MFMA per part, as the forward does); its epilogue
// re-reads q and takes do in fp16, so the LayerNorm backward sees them at full
// precision.  The key/value kernel
// multiplies in fp16 (n, do, p and ds are O(1) quantities; K and V converted
// from bf16, exact in the fp16 normal range).  Every 32 x 256-byte tile in LDS stores 16-byte chunk c
// of row r at chunk c ^ swz(r % 16), swz(r) = 4 (r % 4) + (r / 4) % 4: both
// the 16-byte fragment reads (16 rows, one chunk) and the transposing reads
// (4 rows x 4 chunks per 16 lanes) then hit distinct banks.
#include "fng_device.h"
#include "fng_internal.h"

namespace fng {

namespace {

constexpr int kD = 128;
constexpr int kKT = 32;                 // keys (or rows) per tile
constexpr int kRowB = kD * 2;           // bytes of one head's row
constexpr int kTileB = kKT * kRowB;     // one head's 32-row tile

enum : int { ACT_SOFTMAX = 0, ACT_GELU = 1 };

struct FnaBwdParams {
  const uint16_t* Q;
  const int32_t* off;
  const uint16_t* K;
  const uint16_t* V;
  const uint16_t* O;
  const uint16_t* dO;
  const float* ln_mean;
  const float* ln_rstd;
  const float* rms_rstd;
  uint16_t* dQ;
  uint16_t* dK;
  uint16_t* dV;
  uint16_t* do16;   // [T, H, 128] fp16: the RMSNorm input gradient
  float* lse;       // [T, H] log2-domain log-sum-exp of the scores (softmax)
  int B, H, max_len, Skv, T;
  int qblocks;
  float scale;
};

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// query/key order of an MFMA operand whose result registers must hand rows
// 16c + 8hi + j to the next MFMA's B operand: bits 2 and 3 swapped
__device__ __forceinline__ int kappa(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// tanh-form GELU through sigma = 0.5 (1 + tanh u) = 1 / (1 + 2^w),
// u = sqrt(2/pi) (s + 0.044715 s^3), w = -2 u log2(e); with 1 - tanh^2 u =
// 4 sigma (1 - sigma) its derivative is
//   sigma + 2 s sigma (1 - sigma) sqrt(2/pi) (1 + 3 * 0.044715 s^2)
constexpr float kK0 = 0.7978845608028654f;
constexpr float kK1 = 3.0f * 0.044715f * kK0;
constexpr float kG0 = -2.0f * kK0 * 1.4426950408889634f;
constexpr float kG1 = kG0 * 0.044715f;
__device__ __forceinline__ float gelu_sigma(float s) {
  const float w = s * fmaf(kG1, s * s, kG0);
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(w));
}
__device__ __forceinline__ float gelu_grad(float s, float sg) {
  return fmaf(2.0f * s * sg * (1.0f - sg), fmaf(kK1, s * s, kK0), sg);
}

__device__ __forceinline__ float f16lo(uint32_t w) {
  const f16x2_t v = __builtin_bit_cast(f16x2_t, w);
  return (float)v[0];
}
__device__ __forceinline__ float f16hi(uint32_t w) {
  const f16x2_t v = __builtin_bit_cast(f16x2_t, w);
  return (float)v[1];
}

// ---------------------------------------------------------------------------
// rows: dq, do, log-sum-exp, delta
// ---------------------------------------------------------------------------
// rows kernel: 4 waves = (4 / H) row groups x H heads, two workgroups per CU
// (one workgroup's copies overlap the other's products).  With four heads every
// wave copies, and alone reads, its own head's K and V tiles, so the tile loop
// needs no workgroup barrier: the waves only meet at the two cross-head
// exchanges.
// waves of a rows workgroup: four (two workgroups per CU) up to four heads,
// one per head for eight (one workgroup per CU, the same eight waves per CU)
template <int H>
constexpr int bwd_rows_waves() { return H <= 4 ? 4 : H; }

// NORM = false: the plain jagged attention's backward (the unfused chain's
// attention step): no norms and no residuals, so the gradient at the
// attention output is dout itself, the scores' operand is q * scale, and dq
// is the accumulated ds K
template <int H, int ACT, bool NORM>
__global__ __launch_bounds__(64 * bwd_rows_waves<H>(), H <= 4 ? 2 : 1) void fna_bwd_rows_kernel(FnaBwdParams p) {
  constexpr int NW = bwd_rows_waves<H>();
  constexpr int G = NW / H;                // row groups
  constexpr int BM = 32 * G;               // query rows per workgroup
  constexpr int RB = H * kRowB;            // bytes per query row (all heads)
  constexpr int KVB = H * kTileB;          // one K (or V) tile of every head
  constexpr int NK = KVB / (1024 * NW);    // 1 KB copies per wave for one tile
  constexpr bool OWN = H == NW;            // wave w copies exactly head w's tiles
  // bf16 high + low parts of the computed operands for GELU, whose dS = dP
  // GELU'(S) passes their rounding on at full weight; with the softmax the
  // rounding reaches dS scaled by P (about 1/Skv) and single parts keep dQ
  // within 3e-5 of the bf16 rounding floor (measured on the full workload)
  constexpr bool SPLIT = ACT == ACT_GELU;
  constexpr int XCH = 2 * KVB;
  static_assert(XCH + BM * H * 16 <= (H <= 4 ? 80 : 160) * 1024, "two workgroups per CU up to four heads");
  // hand-off of the K / V tiles: workgroup barrier, or for OWN this wave's
  // own LDS reads done (the copies' own wait is its vmcnt)
  auto tile_sync = [&]() __attribute__((always_inline)) {
    if constexpr (OWN) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    else lds_barrier();
  };
  __shared__ __attribute__((aligned(1024))) char smem[XCH + BM * H * 16];
  FNG_LDS char* lds = (FNG_LDS char*)smem;
  FNG_LDS float* xch = (FNG_LDS float*)(lds + XCH);  // [BM][H][4] per-head partial sums

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

  const int lrow = g * 32 + l32;
  const int qi = qb * BM + lrow;
  const int row = r0 + qi;
  const bool valid = qi < len && row < p.T;
  const int brows = max(0, min(len, p.T - r0));
  const uint32_t rbytes = (uint32_t)(brows * RB);
  const auto qrs = make_rsrc_uniform(p.Q + (size_t)r0 * H * kD, rbytes);
  const auto ors = make_rsrc_uniform(p.O + (size_t)r0 * H * kD, rbytes);
  const auto grs = make_rsrc_uniform(p.dO + (size_t)r0 * H * kD, rbytes);
  const i32x4_t kr = dma_rsrc(p.K + (size_t)b * p.Skv * H * kD, (uint32_t)(p.Skv * RB));
  const i32x4_t vr = dma_rsrc(p.V + (size_t)b * p.Skv * H * kD, (uint32_t)(p.Skv * RB));

  // key and value tile kt of every head into LDS (K at 0, V at KVB): block j
  // is head j / 8, keys 4 (j % 8) .. +3; position c of row r holds the row's
  // chunk c ^ swz(r)
  auto tile_src = [&](int kt, int i) __attribute__((always_inline)) {
    const int blk = wave * NK + i;
    const int hd = blk / 8, r = 4 * (blk % 8) + (lane >> 4), pc = lane & 15;
    return (uint32_t)((((kt * kKT + r) * H + hd) * kD) * 2 + ((pc ^ swz(r)) * 16));
  };
  auto copy_tiles = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      dma16(kr, lds + (wave * NK + i) * 1024, tile_src(kt, i));
      dma16(vr, lds + KVB + (wave * NK + i) * 1024, tile_src(kt, i));
    }
  };
  // four heads: each wave's own K and V slices, copied separately (V first)
  auto copy_k = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NK; ++i) dma16(kr, lds + (wave * NK + i) * 1024, tile_src(kt, i));
  };
  auto copy_v = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NK; ++i) dma16(vr, lds + KVB + (wave * NK + i) * 1024, tile_src(kt, i));
  };
  auto copy_first = [&]() __attribute__((always_inline)) {
    if constexpr (OWN) {
      copy_v(0);
      copy_k(0);
    } else {
      copy_tiles(0);
    }
  };
  copy_first();

  // ---- prologue: the row's values for this head, lane layout of the MFMA B
  // operand (lane holds d = 16kk + 8hi + 0..7 of its row) --------------------
  const float mu = NORM && valid ? p.ln_mean[row] : 0.f;
  const float r1 = NORM ? (valid ? p.ln_rstd[row] : 0.f) : 1.f;
  const float r2 = NORM && valid ? p.rms_rstd[row] : 0.f;
  const uint32_t rbase = (uint32_t)(qi * RB + h * kRowB + hi * 16);
  float gy = 0.f;
  {
    u32x4_t xq[8], xo[8], xg[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      xq[kk] = buffer_load16(qrs, rbase + kk * 32);
      xo[kk] = NORM ? buffer_load16(ors, rbase + kk * 32) : u32x4_t{0u, 0u, 0u, 0u};
      xg[kk] = buffer_load16(grs, rbase + kk * 32);
    }
    float c2 = 0.f;
    if constexpr (NORM) {
      // sum of g * y over this head, y = out - x (the RMSNorm output)
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t wq = xq[kk][e], wo = xo[kk][e], wg = xg[kk][e];
          gy = fmaf(bf16lo(wg), bf16lo(wo) - bf16lo(wq), gy);
          gy = fmaf(bf16hi(wg), bf16hi(wo) - bf16hi(wq), gy);
        }
      gy = half_swap_sum(gy);
      if (hi == 0) xch[(lrow * H + h) * 4 + 0] = gy;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < H; ++j) c2 += xch[(lrow * H + j) * 4 + 0];
      c2 *= 1.0f / (H * kD);
    }
    // do = r2 (g - y c2).  do goes to the MFMA as bf16 high and low parts and
    // to the key/value kernel (and this kernel's epilogue) as fp16
    u32x4_t dob[8], dol[8];
    uint16_t* dodst = p.do16 + (size_t)row * H * kD + h * kD + hi * 8;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      u32x4_t df;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t wq = xq[kk][e], wo = xo[kk][e], wg = xg[kk][e];
        float d2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const float x = u ? bf16hi(wq) : bf16lo(wq);
          const float y = (u ? bf16hi(wo) : bf16lo(wo)) - x;
          const float gv = u ? bf16hi(wg) : bf16lo(wg);
          d2[u] = NORM ? r2 * fmaf(-y, c2, gv) : gv;
        }
        const uint32_t hw = pack_bf16(d2[0], d2[1]);
        dob[kk][e] = hw;
        if constexpr (SPLIT) dol[kk][e] = pack_bf16(d2[0] - bf16lo(hw), d2[1] - bf16hi(hw));
        df[e] = pack_f16(d2[0], d2[1]);
      }
      if (valid) *reinterpret_cast<u32x4_t*>(dodst + 16 * kk) = df;
    }

    // ---- the scores' B operand: n * scale (* log2 e for the softmax), bf16
    // high and low parts --------------------------------------------------------
    const float cq = (ACT == ACT_SOFTMAX) ? p.scale * 1.4426950408889634f : p.scale;
    u32x4_t nb[8], nl[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t wq = xq[kk][e];
        const float a0 = (bf16lo(wq) - mu) * r1 * cq, a1 = (bf16hi(wq) - mu) * r1 * cq;
        const uint32_t hw = pack_bf16(a0, a1);
        nb[kk][e] = hw;
        if constexpr (SPLIT) nl[kk][e] = pack_bf16(a0 - bf16lo(hw), a1 - bf16hi(hw));
      }

    // ---- fragment addresses ------------------------------------------------
    // 16-byte reads (A operand of S^T = K n^T and dP^T = V do^T): key row
    // kappa(l32), chunk 2kk + hi
    const int krow = kappa(l32);
    // koff(kk) = base + ((2kk + hi) ^ swz) * 16 = kb + 32 (kk ^ kx).  With the
    // GELU's high and low operand parts the kernel holds two more sets of
    // loop operands: there the sums are formed at each use from two registers
    // (the empty asm keeps the compiler from hoisting all eight out of the
    // loops); held in registers they made the allocator spill a loop operand
    // and reload it inside the key loop, behind a wait for every copy in
    // flight.
    // With the softmax (single bf16 operand parts, no spill) the eight
    // precomputed addresses are cheaper than the per-use arithmetic (measured).
    constexpr bool LEAN = SPLIT;
    const int kb = h * kTileB + krow * kRowB + 16 * (hi ^ (swz(krow) & 1));
    const int kx = swz(krow) >> 1;
    int koffa[LEAN ? 1 : 8];
    if constexpr (!LEAN) {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) koffa[kk] = kb + 32 * (kk ^ kx);
    }
    auto koff = [&](int kk) __attribute__((always_inline)) {
      if constexpr (LEAN) {
        int b = kb, x = kx;
        asm volatile("" : "+v"(b), "+v"(x));
        return b + 32 * (kk ^ x);
      } else {
        return koffa[kk];
      }
    };
    // transposing reads (A operand of dn^T = K^T ds^T): lane (g4, li) reads
    // key 16c + 8 (g4 / 2) + li / 4 (+4 for the second read), d = 32 dt +
    // 16 (g4 % 2) + 4 (li % 4)
    const int g4 = lane >> 4, li = lane & 15;
    const int tkey = 8 * (g4 >> 1) + (li >> 2);
    // toff(dt, s2) = base + ((d >> 3) ^ swz(kq)) * 16 + (d & 7) * 2 with
    // d >> 3 = 4 dt + c, c = 2 (g4 % 2) + (li % 4) / 2, (d & 7) * 2 = 8 (li % 2):
    // = tb[s2] + 64 (dt ^ tx[s2])
    int tb[2], tx[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int kq = tkey + 4 * s2;
      const int c = 2 * (g4 & 1) + ((li & 3) >> 1);
      tb[s2] = h * kTileB + kq * kRowB + 16 * (c ^ (swz(kq) & 3)) + 8 * (li & 1);
      tx[s2] = swz(kq) >> 2;
    }
    int toffa[LEAN ? 1 : 4][2];
    if constexpr (!LEAN) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) toffa[dt][s2] = tb[s2] + 64 * (dt ^ tx[s2]);
    }
    auto toff = [&](int dt, int s2) __attribute__((always_inline)) {
      if constexpr (LEAN) {
        int b = tb[s2], x = tx[s2];
        asm volatile("" : "+v"(b), "+v"(x));
        return b + 64 * (dt ^ x);
      } else {
        return toffa[dt][s2];
      }
    };
    const int ntiles = (p.Skv + kKT - 1) / kKT;

    auto scores = [&](f32x16_t& sa, int reg) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sa[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const u32x4_t kf = lds_read16(lds + reg + koff(kk));
        sa = mfma_bf16(kf, nb[kk], sa);
        if constexpr (SPLIT) sa = mfma_bf16(kf, nl[kk], sa);
      }
    };

    auto dprod = [&](f32x16_t& dp, int reg) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const u32x4_t vf = lds_read16(lds + reg + koff(kk));
        dp = mfma_bf16(vf, dob[kk], dp);
        if constexpr (SPLIT) dp = mfma_bf16(vf, dol[kk], dp);
      }
    };

    // ---- pass 1 (softmax): the row's log-sum-exp over all keys and the row
    // term delta = sum_keys p dp, both accumulated online (running max m,
    // l = sum 2^(s - m), w = sum 2^(s - m) dp; delta = w / l).  delta from the
    // recomputed P and dP, not from the attention output rebuilt out of the
    // bf16 forward output: that one carries the output's rounding (with one
    // key, p = 1 and the exact ds is zero, the rebuilt one is not).
    float lse2 = 0.f, dl = 0.f;
    if constexpr (ACT == ACT_SOFTMAX) {
      float mrun = -INFINITY, lrun = 0.f, wrun = 0.f;
      for (int kt = 0; kt < ntiles; ++kt) {
        const bool more = kt + 1 < ntiles;
        f32x16_t sa, dp;
        if constexpr (OWN) {
          // V(kt) landed (K(kt) may still be in flight); once V(kt) is read
          // the next V is copied, then wait for K(kt)
          wait_vmcnt<NK>();
          dprod(dp, KVB);
          tile_sync();
          if (more) {
            copy_v(kt + 1);
            wait_vmcnt<NK>();
          } else {
            wait_vmcnt<0>();
          }
          scores(sa, 0);
        } else {
          wait_vmcnt<0>();
          tile_sync();  // K and V tile kt are in LDS
          scores(sa, 0);
          dprod(dp, KVB);
        }
        const int kvalid = p.Skv - kt * kKT;
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (16 * (r >> 3) + 8 * hi + (r & 7) >= kvalid) sa[r] = -INFINITY;
          mx = fmaxf(mx, sa[r]);
        }
        // a lane whose keys are all masked so far keeps mrun = -inf, l = w = 0
        const float mnew = fmaxf(mrun, mx);
        const float msafe = mnew == -INFINITY ? 0.f : mnew;
        float ls = 0.f, ws = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(sa[r] - msafe);
          ls += e;
          ws = fmaf(e, dp[r], ws);
        }
        const float alpha = mrun == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun - msafe);
        lrun = fmaf(lrun, alpha, ls);
        wrun = fmaf(wrun, alpha, ws);
        mrun = mnew;
        tile_sync();  // K (and V) tile kt have been read
        if constexpr (OWN) {
          if (more) copy_k(kt + 1);
        } else {
          if (more) copy_tiles(kt + 1);
        }
      }
      copy_first();  // tile 0 again for the second pass
      const float m = half_swap_max(mrun);
      const float a = mrun == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun - m);
      const float l = half_swap_sum(lrun * a);
      dl = half_swap_sum(wrun * a) / l;
      lse2 = m + __builtin_amdgcn_logf(l);  // v_log_f32: log2
      if (valid && hi == 0) p.lse[(size_t)row * H + h] = lse2;
    }

    // ---- pass 2: dP, ds and dn^T += K^T ds^T over the key tiles -------------
    f32x16_t dn[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) dn[i][r] = 0.f;
    for (int kt = 0; kt < ntiles; ++kt) {
      const bool more = kt + 1 < ntiles;
      f32x16_t sa, dp;
      if constexpr (OWN) {
        wait_vmcnt<NK>();  // V(kt) landed
        dprod(dp, KVB);
        tile_sync();
        if (more) {
          copy_v(kt + 1);
          wait_vmcnt<NK>();  // K(kt) landed
        } else {
          wait_vmcnt<0>();
        }
        scores(sa, 0);
      } else {
        wait_vmcnt<0>();
        tile_sync();  // K and V tile kt are in LDS
        scores(sa, 0);
        dprod(dp, KVB);
      }
      const int kvalid = p.Skv - kt * kKT;
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (ACT == ACT_SOFTMAX) {
          const float pr = (16 * (r >> 3) + 8 * hi + (r & 7) < kvalid) ? __builtin_amdgcn_exp2f(sa[r] - lse2) : 0.f;
          ds[r] = pr * (dp[r] - dl) * p.scale;
        } else {
          // keys past Skv: zero V rows give dp = 0
          ds[r] = dp[r] * gelu_grad(sa[r], gelu_sigma(sa[r])) * p.scale;
        }
      }
      u32x4_t dsb[2], dsl[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a0 = ds[8 * c + 2 * e], a1 = ds[8 * c + 2 * e + 1];
          const uint32_t hw = pack_bf16(a0, a1);
          dsb[c][e] = hw;
          if constexpr (SPLIT) dsl[c][e] = pack_bf16(a0 - bf16lo(hw), a1 - bf16hi(hw));
        }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const u32x2_t lo = lds_read_tr16(lds + toff(dt, 0) + c * 16 * kRowB);
          const u32x2_t hi2 = lds_read_tr16(lds + toff(dt, 1) + c * 16 * kRowB);
          const u32x4_t kf = {lo[0], lo[1], hi2[0], hi2[1]};
          dn[dt] = mfma_bf16(kf, dsb[c], dn[dt]);
          if constexpr (SPLIT) dn[dt] = mfma_bf16(kf, dsl[c], dn[dt]);
        }
      tile_sync();  // K (and V) tile kt have been read
      if constexpr (OWN) {
        if (more) copy_k(kt + 1);
      } else {
        if (more) copy_tiles(kt + 1);
      }
    }

    // ---- epilogue: LayerNorm backward across heads, dq = g + dx -------------
    // dn^T holds, in register 4 r4 + e of dn[dt], d = 32 dt + 8 r4 + 4 hi + e;
    // swapping lane halves (v_permlane32_swap) of the 8-blocks 2kk and 2kk + 1
    // gives the B layout d = 16kk + 8hi + j: j = e from the first result, 4 + e
    // from the second
    // q and the fp16 do again (L2 hits): n and do at full precision, not
    // from the bf16 MFMA operands
    u32x4_t dof[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      xq[kk] = NORM ? buffer_load16(qrs, rbase + kk * 32) : u32x4_t{0u, 0u, 0u, 0u};
      dof[kk] = (NORM && valid) ? *reinterpret_cast<const u32x4_t*>(dodst + 16 * kk) : u32x4_t{0u, 0u, 0u, 0u};
    }
    float s1 = 0.f, s2 = 0.f;
    float dnb[8][8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int m0 = 2 * kk, m1 = 2 * kk + 1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(dn[m0 >> 2][4 * (m0 & 3) + e]),
                                                         __float_as_uint(dn[m1 >> 2][4 * (m1 & 3) + e]), false, false);
        dnb[kk][e] = __uint_as_float(sw[0]);
        dnb[kk][4 + e] = __uint_as_float(sw[1]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t wq = xq[kk][e], wd = dof[kk][e];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int j = 2 * e + u;
          const float v = NORM ? dnb[kk][j] + (u ? f16hi(wd) : f16lo(wd)) : dnb[kk][j];
          const float n = ((u ? bf16hi(wq) : bf16lo(wq)) - mu) * r1;
          dnb[kk][j] = v;
          s1 += v;
          s2 = fmaf(v, n, s2);
        }
      }
    }
    float m1 = 0.f, m2 = 0.f;
    if constexpr (NORM) {
      s1 = half_swap_sum(s1);
      s2 = half_swap_sum(s2);
      if (hi == 0) {
        xch[(lrow * H + h) * 4 + 1] = s1;
        xch[(lrow * H + h) * 4 + 2] = s2;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < H; ++j) {
        m1 += xch[(lrow * H + j) * 4 + 1];
        m2 += xch[(lrow * H + j) * 4 + 2];
      }
      m1 *= 1.0f / (H * kD);
      m2 *= 1.0f / (H * kD);
    }
    // dQ goes through LDS (every wave is past its key loops: the K/V tiles are
    // free) and out as whole rows of all heads, where the block's rows fit
    // there; a lane's own values are 16-byte pieces of its row and head.
    // Measured at four heads 1 % faster; at eight (one workgroup per CU, no
    // other to cover the extra barrier) 1 % slower, so not there.
    constexpr bool STG = H <= 4 && BM * H * kRowB <= XCH;
    // without the norms' exchange above, a barrier of its own: every wave is
    // past its key loops before the staging overwrites the K/V tiles
    if constexpr (!NORM && STG) __syncthreads();
    if (STG || valid) {
      uint16_t* dst = p.dQ + (size_t)row * H * kD + h * kD + hi * 8;
      // dout again (an L2 hit, cheaper than holding it in 32 registers throughout)
      if constexpr (NORM) {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) xg[kk] = buffer_load16(grs, rbase + kk * 32);
      }
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        u32x4_t w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t wq = xq[kk][e], wg = xg[kk][e];
          float v[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            if constexpr (NORM) {
              const float n = ((u ? bf16hi(wq) : bf16lo(wq)) - mu) * r1;
              const float dx = r1 * (dnb[kk][2 * e + u] - m1 - n * m2);
              v[u] = (u ? bf16hi(wg) : bf16lo(wg)) + dx;
            } else {
              v[u] = dnb[kk][2 * e + u];
            }
          }
          w[e] = pack_bf16(v[0], v[1]);
        }
        // 16-byte chunk 2 kk + hi of the row's head h, chunks XOR-ed with the row
        if constexpr (STG) lds_write16(lds + lrow * RB + h * kRowB + (((2 * kk + hi) ^ (lrow & 15)) * 16), w);
        else *reinterpret_cast<u32x4_t*>(dst + 16 * kk) = w;
      }
    }
    if constexpr (STG) {
      __syncthreads();
      constexpr int CH = BM * H * 16;  // 16-byte chunks of the block's rows
#pragma unroll
      for (int i = 0; i < CH / (64 * NW); ++i) {
        const int idx = tid + 64 * NW * i;
        const int r = idx / (H * 16), cc = idx % (H * 16);
        const int qr = qb * BM + r;
        if (qr < len && r0 + qr < p.T) {
          const u32x4_t v = lds_read16(lds + r * RB + (cc >> 4) * kRowB + (((cc & 15) ^ (r & 15)) * 16));
          *reinterpret_cast<u32x4_t*>(p.dQ + (size_t)(r0 + qr) * H * kD + cc * 8) = v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// keys and values: dK, dV for one (batch, head)
// ---------------------------------------------------------------------------
// sum over the 32 key lanes (same lane half) of 16 per-row values v[r] (row
// 16 (r / 8) + 8 hi + r % 8): a butterfly that halves the values at each step;
// afterwards lanes l32 and l32 ^ 1 both hold the sum for register
// j = (l32 / 2) % 16
__device__ __forceinline__ float key_lane_sum(const float (&v)[16], int l32) {
  float a[8], b[4], c[2];
  const bool b4 = (l32 >> 4) & 1, b3 = (l32 >> 3) & 1, b2 = (l32 >> 2) & 1, b1 = (l32 >> 1) & 1;
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = (b4 ? v[i + 8] : v[i]) + __shfl_xor(b4 ? v[i] : v[i + 8], 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = (b3 ? a[i + 4] : a[i]) + __shfl_xor(b3 ? a[i] : a[i + 4], 8);
#pragma unroll
  for (int i = 0; i < 2; ++i) c[i] = (b2 ? b[i + 2] : b[i]) + __shfl_xor(b2 ? b[i] : b[i + 2], 4);
  const float d = (b1 ? c[1] : c[0]) + __shfl_xor(b1 ? c[0] : c[1], 2);
  return d + __shfl_xor(d, 1);
}

// 8 waves = two groups of four; group q takes the row blocks q, q + 2, ...
// and wave w of a group owns keys 32 w .. 32 w + 31.  K and V of the (batch,
// head) sit in LDS as fp16 for the whole loop.
template <int ACT, bool NORM>
__global__ __launch_bounds__(512, 1) void fna_bwd_kv_kernel(FnaBwdParams p) {
  constexpr int KVT = 128 * kRowB;                   // K (or V) of one head, 128 keys
  constexpr int KREG = 0, VREG = KVT;                // fp16 [key][d], rows swizzled
  constexpr int GREG = 2 * KVT;                      // per group: n tile, do tile, row data
  // (after the loop a group's region stages half of its output tensor: 128 keys
  // x 144-byte rows)
  constexpr int GTILES = 2 * kTileB + 3 * 32 * 4 + 2 * 32 * 4 * 4, GOUT = 128 * 144;
  constexpr int GSZ = GTILES > GOUT ? GTILES : GOUT;
  __shared__ __attribute__((aligned(1024))) char smem[GREG + 2 * GSZ];
  FNG_LDS char* lds = (FNG_LDS char*)smem;

  const int H = p.H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, kw = wave & 3;
  const int gtid = tid & 255;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int b = (int)(blockIdx.x / (uint32_t)H);
  const int h = (int)(blockIdx.x % (uint32_t)H);
  const int r0 = p.off[b];
  const int len = r0 < 0 ? 0 : max(0, min(p.off[b + 1] - r0, p.max_len));
  const int brows = max(0, min(len, p.T - r0));
  const int key = 32 * kw + l32;           // this lane's key (result column)
  const bool active = 32 * kw < p.Skv;     // wave-uniform

  FNG_LDS char* gl = lds + GREG + grp * GSZ;
  FNG_LDS char* nt = gl;                   // n tile [32 rows][128 d] fp16, swizzled
  FNG_LDS char* dt_ = gl + kTileB;         // do tile
  FNG_LDS float* lse_s = (FNG_LDS float*)(gl + 2 * kTileB);  // [32] log-sum-exp
  FNG_LDS float* il_s = lse_s + 32;        // [32] 1 / L
  FNG_LDS float* dl_s = lse_s + 64;        // [32] delta = W / L
  FNG_LDS float* part = lse_s + 96;        // [32 rows][4 waves][2] per-wave L, W

  // staging split within a group: thread covers row gtid / 8, d = 16 (gtid % 8) .. + 15
  const int srow = gtid >> 3, spart = gtid & 7;
  const size_t qstride = (size_t)H * kD;
  const int nblk = (brows + 31) / 32;
  const int npair = (nblk + 1) / 2;
  // the next block's raw values (register prefetch)
  u32x4_t pq[2], pd[2];
  float pmu = 0.f, pr1 = 0.f, plse = INFINITY;
  auto fetch = [&](int blk) __attribute__((always_inline)) {
    const int qrow = blk * 32 + srow;
    const bool ok = blk < nblk && qrow < brows;
    pq[0] = pq[1] = pd[0] = pd[1] = u32x4_t{0u, 0u, 0u, 0u};
    pmu = 0.f;
    pr1 = 0.f;
    plse = INFINITY;
    if (ok) {
      const size_t grow = (size_t)(r0 + qrow);
      const uint16_t* qs = p.Q + grow * qstride + h * kD + spart * 16;
      const uint16_t* ds = p.do16 + grow * qstride + h * kD + spart * 16;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        pq[u] = *reinterpret_cast<const u32x4_t*>(qs + 8 * u);
        pd[u] = *reinterpret_cast<const u32x4_t*>(ds + 8 * u);
      }
      pmu = NORM ? p.ln_mean[grow] : 0.f;
      pr1 = NORM ? p.ln_rstd[grow] : 1.f;
      if (ACT == ACT_SOFTMAX && spart == 0) plse = p.lse[grow * H + h];
    }
  };
  fetch(grp);

  // ---- K and V of this (batch, head) to LDS as fp16 ------------------------
  {
    const uint32_t kvbytes = (uint32_t)(p.Skv * H * kRowB);
    const auto krs = make_rsrc_uniform(p.K + (size_t)b * p.Skv * H * kD, kvbytes);
    const auto vrs = make_rsrc_uniform(p.V + (size_t)b * p.Skv * H * kD, kvbytes);
    const int kr_ = tid >> 2, q4 = tid & 3;  // key row, quarter of the row
    const uint32_t base = (uint32_t)((kr_ * H + h) * kRowB + q4 * 64);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x4_t a = buffer_load16(krs, base + u * 16);
      const u32x4_t v = buffer_load16(vrs, base + u * 16);
      u32x4_t ka, va;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ka[e] = bf16x2_to_f16x2(a[e]);
        va[e] = bf16x2_to_f16x2(v[e]);
      }
      const int pos = kr_ * kRowB + (((4 * q4 + u) ^ swz(kr_)) * 16);
      lds_write16(lds + KREG + pos, ka);
      lds_write16(lds + VREG + pos, va);
    }
  }

  f32x16_t dk[4], dv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[i][r] = 0.f;
      dv[i][r] = 0.f;
    }

  // fragment addresses: n / do tiles (A of S and dP: row kappa(l32), chunk
  // 2kk + hi; transposing reads for dV^T, dK^T), K / V (B of S and dP: key row,
  // chunk 2kk + hi)
  const int arow = kappa(l32);
  int aoff[8], boff[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    aoff[kk] = arow * kRowB + (((2 * kk + hi) ^ swz(arow)) * 16);
    boff[kk] = key * kRowB + (((2 * kk + hi) ^ swz(key)) * 16);
  }
  const int g4 = lane >> 4, li = lane & 15;
  const int trow = 8 * (g4 >> 1) + (li >> 2);
  int toff[4][2];
#pragma unroll
  for (int d4 = 0; d4 < 4; ++d4) {
    const int d = 32 * d4 + 16 * (g4 & 1) + 4 * (li & 3);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int rq = trow + 4 * s2;
      toff[d4][s2] = rq * kRowB + (((d >> 3) ^ swz(rq)) * 16) + (d & 7) * 2;
    }
  }
  const float cq = (ACT == ACT_SOFTMAX) ? p.scale * 1.4426950408889634f : p.scale;


  for (int it = 0; it < npair; ++it) {
    const int blk = 2 * it + grp;
    const bool has = blk < nblk;  // wave-uniform (per group)
    // the prefetched block to the group's LDS tiles (rows past the batch are
    // zeros, log-sum-exp +inf: p = 0)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      u32x4_t nq;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = pq[u][e];
        nq[e] = pack_f16((bf16lo(w) - pmu) * pr1, (bf16hi(w) - pmu) * pr1);
      }
      const int pos = srow * kRowB + (((2 * spart + u) ^ swz(srow)) * 16);
      lds_write16(nt + pos, nq);
      lds_write16(dt_ + pos, pd[u]);
    }
    if (spart == 0) lse_s[srow] = plse;
    __syncthreads();  // tiles (and, the first time, K and V) are in LDS
    fetch(blk + 2);   // overlaps with this block's products

    f32x16_t sa, dp;
    if (has && active) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sa[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        sa = mfma_f16(lds_read16(nt + aoff[kk]), lds_read16(lds + KREG + boff[kk]), sa);
        dp = mfma_f16(lds_read16(dt_ + aoff[kk]), lds_read16(lds + VREG + boff[kk]), dp);
      }
    }
    if constexpr (ACT == ACT_SOFTMAX) {
      // p unnormalized (the rows kernel's log-sum-exp), then per row
      // L = sum_keys p and W = sum_keys p dp over the four waves
      if (has && active) {
        float ev[16], wv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qr = 16 * (r >> 3) + 8 * hi + (r & 7);
          sa[r] = key < p.Skv ? __builtin_amdgcn_exp2f(sa[r] * cq - lse_s[qr]) : 0.f;
          ev[r] = sa[r];
          wv[r] = sa[r] * dp[r];
        }
        const float ls = key_lane_sum(ev, l32), ws = key_lane_sum(wv, l32);
        if ((l32 & 1) == 0) {
          // the row index is formed here from the lane id (a loop-invariant
          // address held across the loop was spilled, and its reload inside
          // the loop waited for the next row block's loads in flight)
          int ln = lane;
          asm volatile("" : "+v"(ln));
          const int j = ((ln & 31) >> 1) & 15;
          const int qr = 16 * (j >> 3) + 8 * (ln >> 5) + (j & 7);
          part[(qr * 4 + kw) * 2 + 0] = ls;
          part[(qr * 4 + kw) * 2 + 1] = ws;
        }
      }
      __syncthreads();
      if (has && gtid < 32) {
        float l = 0.f, w = 0.f;
        for (int k = 0; k < 4; ++k)
          if (32 * k < p.Skv) {
            l += part[(gtid * 4 + k) * 2 + 0];
            w += part[(gtid * 4 + k) * 2 + 1];
          }
        const float il = l > 0.f ? 1.0f / l : 0.f;
        il_s[gtid] = il;
        dl_s[gtid] = w * il;
      }
      __syncthreads();
    }
    if (has && active) {
      float pr[16], ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = 16 * (r >> 3) + 8 * hi + (r & 7);
        if constexpr (ACT == ACT_SOFTMAX) {
          pr[r] = sa[r] * il_s[qr];
          ds[r] = pr[r] * (dp[r] - dl_s[qr]) * p.scale;
        } else {
          const float s = sa[r] * cq;
          const float sg = gelu_sigma(s);
          pr[r] = s * sg;
          ds[r] = dp[r] * gelu_grad(s, sg) * p.scale;
        }
      }
      u32x4_t pb[2], dsb[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pb[c][e] = pack_f16(pr[8 * c + 2 * e], pr[8 * c + 2 * e + 1]);
          dsb[c][e] = pack_f16(ds[8 * c + 2 * e], ds[8 * c + 2 * e + 1]);
        }
      // dV^T += do^T P, dK^T += n^T dS (d x keys), A operands by transposing reads
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int d4 = 0; d4 < 4; ++d4) {
          const int o0 = toff[d4][0] + c * 16 * kRowB, o1 = toff[d4][1] + c * 16 * kRowB;
          const u32x2_t a0 = lds_read_tr16(dt_ + o0), a1 = lds_read_tr16(dt_ + o1);
          dv[d4] = mfma_f16(u32x4_t{a0[0], a0[1], a1[0], a1[1]}, pb[c], dv[d4]);
          const u32x2_t n0 = lds_read_tr16(nt + o0), n1 = lds_read_tr16(nt + o1);
          dk[d4] = mfma_f16(u32x4_t{n0[0], n0[1], n1[0], n1[1]}, dsb[c], dk[d4]);
        }
    }
    __syncthreads();  // the tiles are rewritten by the next pair of blocks
  }

  // ---- the two groups' sums, through LDS (the K / V region is free now), in
  // two halves of d: group 1 puts out its dK, group 0 its dV; group 0 stores
  // dK = its own + group 1's, group 1 stores dV = group 0's + its own (fixed
  // order: bitwise reproducible)
  // per group and half: [wave][8 chunks of 4 floats][64 lanes] (consecutive
  // lanes at consecutive 16 bytes: no bank conflicts)
  auto xoff = [&](int g_, int i, int r) { return g_ * (256 * 32) + ((kw * 8 + i * 4 + r / 4) * 64 + lane) * 4; };
  FNG_LDS float* xf = (FNG_LDS float*)lds;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    __syncthreads();  // the region is free (K / V, or the previous half, read)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int d4 = 2 * half + i;
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const f32x16_t& src = grp ? dk[d4] : dv[d4];
        *reinterpret_cast<FNG_LDS f32x4_t*>(xf + xoff(grp, i, r)) = f32x4_t{src[r], src[r + 1], src[r + 2], src[r + 3]};
      }
    }
    __syncthreads();
    // the sum in bf16 to this group's region, [key][64 d] with 144-byte rows
    // (keys 16 apart land 16 banks apart), then stored as whole 16-byte chunks
    FNG_LDS char* const stg = lds + GREG + grp * GSZ;
    constexpr int SROW = 144;
    static_assert(128 * SROW <= GSZ, "output staging fits the group region");
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int d4 = 2 * half + i;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4_t o = *reinterpret_cast<const FNG_LDS f32x4_t*>(xf + xoff(1 - grp, i, 4 * r4));
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = grp ? o[e] + dv[d4][4 * r4 + e] : dk[d4][4 * r4 + e] + o[e];
        // register r of tile d4 holds d = 32 d4 + 8 (r / 4) + 4 hi + r % 4
        *reinterpret_cast<FNG_LDS u32x2_t*>(stg + key * SROW + (32 * i + 8 * r4 + 4 * hi) * 2) =
            u32x2_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
      }
    }
    __syncthreads();
    uint16_t* const out = grp ? p.dV : p.dK;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int ch = gtid + 256 * c;  // 128 keys x 8 chunks of 16 bytes
      const int k = ch >> 3, q = ch & 7;
      if (k < p.Skv) {
        const u32x4_t v = *reinterpret_cast<const FNG_LDS u32x4_t*>(stg + k * SROW + q * 16);
        *reinterpret_cast<u32x4_t*>(out + (((size_t)b * p.Skv + k) * H + h) * kD + 64 * half + 8 * q) = v;
      }
    }
  }
}

template <int H>
void launch_rows_h(const FnaBwdParams& p, int act, bool norm, hipStream_t s) {
  const dim3 grid((unsigned)(p.B * p.qblocks)), block(64 * bwd_rows_waves<H>());
  if (norm) {
    if (act == ACT_GELU) hipLaunchKernelGGL((fna_bwd_rows_kernel<H, ACT_GELU, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((fna_bwd_rows_kernel<H, ACT_SOFTMAX, true>), grid, block, 0, s, p);
  } else {
    if (act == ACT_GELU) hipLaunchKernelGGL((fna_bwd_rows_kernel<H, ACT_GELU, false>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((fna_bwd_rows_kernel<H, ACT_SOFTMAX, false>), grid, block, 0, s, p);
  }
}

}  // namespace

int launch_fna_bwd(const FnaBwdCall& c, bool norm, hipStream_t s) {
  FnaBwdParams p{};
  p.Q = static_cast<const uint16_t*>(c.Q);
  p.off = c.offsets;
  p.K = static_cast<const uint16_t*>(c.K);
  p.V = static_cast<const uint16_t*>(c.V);
  p.O = static_cast<const uint16_t*>(c.O);
  p.dO = static_cast<const uint16_t*>(c.dO);
  p.ln_mean = c.ln_mean;
  p.ln_rstd = c.ln_rstd;
  p.rms_rstd = c.rms_rstd;
  p.dQ = static_cast<uint16_t*>(c.dQ);
  p.dK = static_cast<uint16_t*>(c.dK);
  p.dV = static_cast<uint16_t*>(c.dV);
  char* ws = static_cast<char*>(c.workspace);
  p.do16 = reinterpret_cast<uint16_t*>(ws);
  p.lse = reinterpret_cast<float*>(ws + (size_t)c.T * c.H * kD * 2);
  p.B = (int)c.B;
  p.H = (int)c.H;
  p.max_len = (int)c.max_len;
  p.Skv = (int)c.Skv;
  p.T = (int)c.T;
  p.scale = c.sm_scale;
  const int bm = c.H <= 4 ? 32 * (4 / (int)c.H) : 32;  // query rows per rows workgroup
  p.qblocks = (int)((c.max_len + bm - 1) / bm);
  const int act = c.act == FNG_ACT_GELU ? ACT_GELU : ACT_SOFTMAX;
  if (p.qblocks > 0 && p.T > 0) {  // else no query row: dK = dV = 0 from the second kernel alone
    switch (c.H) {
      case 1: launch_rows_h<1>(p, act, norm, s); break;
      case 2: launch_rows_h<2>(p, act, norm, s); break;
      case 4: launch_rows_h<4>(p, act, norm, s); break;
      case 8: launch_rows_h<8>(p, act, norm, s); break;
      default: return FNG_ERR_UNSUPPORTED;
    }
    if (hipGetLastError() != hipSuccess) return FNG_ERR_HIP;
  }
  const dim3 grid((unsigned)(c.B * c.H)), block(512);
  if (norm) {
    if (act == ACT_GELU) hipLaunchKernelGGL((fna_bwd_kv_kernel<ACT_GELU, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((fna_bwd_kv_kernel<ACT_SOFTMAX, true>), grid, block, 0, s, p);
  } else {
    if (act == ACT_GELU) hipLaunchKernelGGL((fna_bwd_kv_kernel<ACT_GELU, false>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((fna_bwd_kv_kernel<ACT_SOFTMAX, false>), grid, block, 0, s, p);
  }
  return hipGetLastError() == hipSuccess ? FNG_OK : FNG_ERR_HIP;
}

size_t fna_bwd_workspace_bytes(int64_t T, int64_t H) { return (size_t)(T * H) * (kD * 2 + 4); }

}  // namespace fng
