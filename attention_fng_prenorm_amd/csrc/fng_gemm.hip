// bf16 GEMM Y[M,N] = X[M,K] @ W[K,N] on gfx950 MFMA, with the normalization
// epilogues of "Towards Free Normalization: Fusing Normalization into GEMM and
// Attention Kernels":
//   EPI_PLAIN    the unfused GEMM baseline
//   EPI_PRENORM  section 2, Lazy Pre-Norm: the sum of squares of the raw X rows
//                is accumulated beside the K loop from the X fragments already
//                in registers for the MFMA, and rstd = 1/sqrt(ss/K + eps) is
//                applied as a row scale in the epilogue (the row-scale
//                commutation identity of that section).  An optional gain
//                gamma[k] is folded into the W fragments (the statistic uses
//                the raw X).
//   EPI_FULLN    section 1, naive fusion: one workgroup's tile spans all N, the
//                row statistics come straight from the fp32 accumulators.
//   EPI_SPLITN   section 3, multi-CTA norm without clusters: each workgroup
//                publishes per-row partial statistics of its N slice, the
//                workgroups of one row block (all co-resident: a persistent
//                grid no larger than the GPU holds at once) wait for each
//                other, merge the partials in a fixed order and normalize
//                their accumulators in place.
//   EPI_PARTIAL  first kernel of the two-pass fallback: un-normalized bf16 Y
//                plus the same per-row partials; fng_norm.hip finishes it.
//   EPI_ROWSCALE the lazy pre-norm's columns that reuse the statistic: another
//                launch of the same call (EPI_PRENORM, on other columns of the
//                same rows) accumulated each row's sum of squares beside its
//                K loop and wrote rstd (and, for the lazy LayerNorm, the mean);
//                these tiles only apply it (with LN: rstd (acc - mean colsum)).
//   EPI_DW       the lazy pre-norm's weight gradient dW = X^T diag(rstd) dY
//                (section 2's limitations: the normalized X is rebuilt from X
//                and rstd for the gradients of both operands): the output
//                rows are X's columns, the contraction runs over X's rows, so
//                X is kept [contraction][out] in LDS exactly as in memory and
//                read with transposing reads like W; rstd scales the dY
//                fragments along the contraction; an optional gain scales the
//                output rows.
//
// Block: 64 * WAVES_M * WAVES_N threads (4 or 8 waves).  Each wave owns a
// (BM/WAVES_M) x (BN/WAVES_N) sub-tile built from 32x32 MFMA tiles.  The MFMA
// is issued as D = W_frag * X_frag, so D is the transposed tile: lane l holds
// output row m = l % 32 and 16 columns, which keeps every row reduction of the
// norm epilogues inside a lane plus one lane-pair exchange.
//
// Staging: X and W tiles are copied HBM -> LDS directly (buffer_load ... lds,
// out-of-range rows and tails read as 0) through a 4-stage ring.  The 8-wave
// tiles run a ping-pong schedule: the two waves of each SIMD alternate
// between reading a K tile's fragments and multiplying them, two barriers
// per K tile; the other tiles use one barrier per K tile.  X is kept [m][k]
// (k contiguous) and read with ds_read_b128; W is kept [k][n] exactly as in
// memory and read k-contiguous per lane with ds_read_b64_tr_b16.  16-byte
// chunks are XOR-swizzled per row so fragment reads are bank-conflict free.
// In the plain, row-scale and 128-row lazy pre-norm tiles the X rows of two
// consecutive K tiles are copied together, one 128-byte line per row.
// Split-N places each round's tiles as rectangles of row blocks x 8 column
// tiles per XCD (splitn_placement).
#include <algorithm>

#include "fng_device.h"
#include "fng_internal.h"

namespace fng {

enum : int {
  EPI_PLAIN = 0, EPI_PRENORM = 1, EPI_FULLN = 2, EPI_SPLITN = 3, EPI_PARTIAL = 4,
  EPI_BWD_FULLN = 5,   // norm backward over whole rows held by one workgroup
  EPI_BWD_SPLITN = 6,  // norm backward, row sums exchanged like EPI_SPLITN
  EPI_DW = 7,          // weight gradient of the lazy pre-norm (see the header)
  EPI_TN = 8,          // the same product without the rstd scale: X^T dY (its unfused baseline)
  EPI_ROWSCALE = 9     // lazy pre-norm, second launch: rstd read from the first launch's output
};

struct GemmParams {
  const uint16_t* X;
  const uint16_t* W;
  const uint16_t* gamma;
  uint16_t* Y;
  float* mean_out;
  float* rstd_out;
  float* part;       // [tiles_m][tiles_n][BM][2] per-row partials (split-N, two-pass)
  uint32_t* cnt;     // [tiles_m] arrivals (split-N)
  uint32_t* done;    // [tiles_m] unused (kept in the workspace layout)
  uint32_t* status;  // split-N timeout flag
  int M, N, K;
  float eps;
  int tiles_m, tiles_n, total_tiles;
  int n_off, n_end;  // this launch's output columns [n_off, n_end) (plain and lazy GEMM)
  const uint16_t* H;     // norm backward: xhat [M, N], or the norm's input when h_raw
  const float* rstd_in;  // norm backward: the forward rstd [M]; weight gradient: the contraction scale [K];
                         // lazy pre-norm row scale: rstd [M] from the statistic launch
  const float* mean_in;  // lazy LayerNorm row scale: mean [M] from the statistic launch
  int h_raw;
  int group_m;       // row blocks per tile group (L2 locality of the tile order)
  uint32_t wait_ticks;     // split-N: bound of one exchange wait, in 100 MHz real-time ticks
  int poison_on_timeout;   // split-N: rows whose wait timed out are written as NaN
  const float* colsum;  // lazy LayerNorm: [N] column sums of W
  const uint16_t* beta;  // post-norm affine: bias [N] (gamma [N] is the gain), or nullptr
  // split-N placement: each XCD's tiles of a round form sn_rh row blocks x
  // sn_cw column tiles, sn_g XCDs sharing the row blocks (sn_cw 0: every
  // column tile of a row block on one XCD)
  int sn_cw, sn_rh, sn_g;
};

// LDS layout: the W parts of all ring stages, then the X parts, then the
// gamma slices.  A fragment address is one lane-dependent base register plus
// a compile-time (stage, k16 slice) offset in the instruction's 16-bit offset
// field.
template <int BM, int BN, int BK, int STAGES, bool GAMMA>
struct Smem {
  static constexpr int A_STAGE = BM * BK * 2;
  static constexpr int B_STAGE = BK * BN * 2;
  static constexpr int B_OFF = 0;
  static constexpr int A_OFF = STAGES * B_STAGE;
  static constexpr int G_OFF = A_OFF + STAGES * A_STAGE;
  static constexpr int BYTES = G_OFF + (GAMMA ? STAGES * 256 : 0);
  static constexpr int a(int s) { return A_OFF + s * A_STAGE; }
  static constexpr int b(int s) { return B_OFF + s * B_STAGE; }
  static constexpr int gm(int s) { return G_OFF + s * 256; }
};

// swizzles of the 16-byte chunk index inside one LDS row.  The LDS serves
// 256 B per cycle (64 banks of 4 B): a ds_read_b128 is served 16 lanes per
// cycle, a ds_read_b64_tr_b16 32 lanes per cycle, and each group must touch
// 64 distinct banks.
//   X rows (BK*2 bytes; a fragment read covers 16 consecutive rows at one
//   logical chunk): XOR the chunk with the row's index among the rows that
//   share a 256 B bank window, so the 16 rows land on distinct units.
//   W rows (BN*2 bytes; a transposing read covers rows k..k+3 and four
//   consecutive chunks): XOR with 4*(k % 4) moves each row to its own
//   quarter of the window.
template <int KC>
__device__ __forceinline__ int swz_a(int row) {
  constexpr int ROWS_PER_WINDOW = 256 / (KC * 16);
  return (row / ROWS_PER_WINDOW) & (KC - 1);
}
template <int NC>
__device__ __forceinline__ int swz_b(int krow) { return ((krow & 3) << 2) & (NC - 1); }
//   Paired X rows (two K tiles of one row, 2*BK*2 = 128 B at BK 32; two rows
//   share a window): XOR the 8-chunk index with (row / 2) % 8, so the 8 even
//   and the 8 odd rows of a read each cover all 8 units of their half.  The
//   XOR may flip chunk bit 2, so the second K tile's address is the first's
//   XOR 64, not a constant offset.
__device__ __forceinline__ int swz_px(int row) { return (row >> 1) & 7; }

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int EPI, bool LN, bool GAMMA>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_kernel(GemmParams p) {
  constexpr int NWAVES = WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M;
  constexpr int WN = BN / WAVES_N;
  constexpr int FM = WM / 32;
  constexpr int FN = WN / 32;
  constexpr int KC = BK / 8;    // 16-byte chunks per X row of a K tile
  constexpr int NC = BN / 8;    // 16-byte chunks per W row of a K tile
  constexpr int STAGES = 4;
  // HBM -> LDS copies: one wave instruction moves 64 lanes x 16 B = 1 KB
  constexpr int A_PER_WAVE = BM * BK * 2 / 1024 / NWAVES;
  constexpr int B_PER_WAVE = BK * BN * 2 / 1024 / NWAVES;
  constexpr int LOADS = A_PER_WAVE + B_PER_WAVE;  // per wave per stage (wave 0: +1 with gamma)
  // lazy pre-norm: the WAVES_N waves that share rows split the sums of squares.
  // Each wave visits its X fragments in a rotated order so that the ones it
  // sums are its first SS_SLOTS register slots (no run-time indexing).
  constexpr int SS_SLOTS = FM >= WAVES_N ? FM / WAVES_N : 1;
  static_assert(FM < WAVES_N || FM % WAVES_N == 0, "row fragments split evenly");
  static_assert(NWAVES == 4 || NWAVES == 8, "4 or 8 waves per workgroup");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile is a multiple of 32x32");
  static_assert(BK == 32 || BK == 64, "BK in {32, 64}");
  static_assert(A_PER_WAVE >= 1 && B_PER_WAVE >= 1, "whole 1 KB copies per wave");
  static_assert(A_PER_WAVE * NWAVES * 1024 == BM * BK * 2 && B_PER_WAVE * NWAVES * 1024 == BK * BN * 2,
                "tile bytes split evenly over the waves");
  static_assert(NC >= 8, "BN >= 64 for the W swizzle");
  // GAMMA: with the lazy pre-norm, the RMSNorm gain folded along K (PG); with
  // the post-norms, their affine (per-column gain and bias) in the epilogue
  constexpr bool PG = GAMMA && EPI == EPI_PRENORM;
  constexpr bool AFF = GAMMA && (EPI == EPI_FULLN || EPI == EPI_SPLITN);
  // weight gradient: X transposed in LDS (XT), fp32 scale along the
  // contraction folded into the W-side fragments (KS), gain on output rows
  constexpr bool XT = EPI == EPI_DW || EPI == EPI_TN;
  constexpr bool KS = EPI == EPI_DW;
  constexpr bool DWG = GAMMA && EPI == EPI_DW;
  static_assert(!GAMMA || PG || AFF || DWG, "GAMMA only with the lazy pre-norm, the post-norms or dW");
  constexpr int MC = BM / 8;    // 16-byte chunks per transposed X row of a K tile
  static_assert(!XT || MC >= 8, "BM >= 64 for the transposed X swizzle");
  using S = Smem<BM, BN, BK, STAGES, PG || KS>;
  static_assert(S::BYTES <= 160 * 1024, "LDS budget");
  static_assert(STAGES == 4, "the ring below is written out for 4 stages");

  // the norm backward stages the saved [BM, BN] tile over the whole ring and
  // keeps its row reductions in an extra region after it
  constexpr bool IS_BWD = EPI == EPI_BWD_FULLN || EPI == EPI_BWD_SPLITN;
  constexpr bool IS_SPLIT = EPI == EPI_SPLITN || EPI == EPI_BWD_SPLITN;
  // ping-pong mainloop: 8 waves in two row halves, two k16 slices per K tile.
  // The lazy pre-norm with the gain keeps the single-phase loop: its fold
  // (about 50 vector instructions per slice) would make the memory phase the
  // longer one (measured slower).
  constexpr bool PP = NWAVES == 8 && WAVES_M == 2 && BK == 32 && !PG;
  // X copied two K tiles at a time (ping-pong loop of the plain, lazy pre-norm
  // and row-scale GEMMs): with BK 32 one K tile of an X row is 64 B, and
  // copies of 64-byte row pieces cost half-line L2 requests (1.5x the
  // requests of the same product on 512-byte rows, measured: 37.6 M vs 25.2 M
  // per 4096 x 4096 x 12288 launch, with 16x the address stalls).  Paired,
  // each group of 8 lanes reads one whole 128-byte line: the X copies of
  // tiles 2j and 2j+1 ride with the issue of tile 2j+1 into the stages of
  // both, laid out [row][2 tiles x 4 chunks] (swz_px).  The split-N, full-N
  // and 256-row lazy pre-norm kernels keep the single-tile layout: the second
  // set of fragment addresses made their allocator spill, and split-N was
  // slower (measured).
  constexpr bool PX = PP && (EPI == EPI_PLAIN || EPI == EPI_ROWSCALE || (EPI == EPI_PRENORM && BM <= 128));
  constexpr int AX = PX ? 2 * A_PER_WAVE : A_PER_WAVE;  // X copies per wave per (odd) issue
  static_assert(!PX || (STAGES == 4 && BK * 4 == 128), "paired X rows are 128 B in a 4-stage ring");
  // the backward's row reductions: an extra region after the ring, or, where
  // that would pass the 160 KB of LDS (the 128 x 512 tile fills it), the
  // ring's tail beyond the saved tile, free once the epilogue starts
  constexpr int RED_BYTES = IS_BWD ? (WAVES_N * BM * 4 > BM * 8 ? WAVES_N * BM * 4 : BM * 8) : 0;
  constexpr bool RED_IN_RING = IS_BWD && S::BYTES + RED_BYTES > 160 * 1024;
  constexpr int RED = !IS_BWD ? 0 : RED_IN_RING ? BM * BN * 2 : S::BYTES;
  constexpr int EXTRA = RED_IN_RING ? 0 : RED_BYTES;
  static_assert(!RED_IN_RING || BM * BN * 2 + RED_BYTES <= S::BYTES, "reductions fit beside the saved tile");
  static_assert(S::BYTES + EXTRA <= 160 * 1024, "LDS budget with the backward's reductions");
  __shared__ __attribute__((aligned(1024))) char smem[S::BYTES + EXTRA];
  FNG_LDS char* lds = (FNG_LDS char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int rot = FM >= WAVES_N ? wn * SS_SLOTS : wn;
  const bool ss_owner = FM >= WAVES_N || wn < FM;
  // row (within the tile) of this lane's fragment slot i
  auto lrow = [&](int i) { return wm * WM + 32 * ((i + rot) % FM) + l32; };

  // Lane-dependent LDS base addresses of the fragment reads; every other part
  // of an address (ring stage, k16 slice, second transposed half) is a
  // compile-time offset.  The empty asm keeps each base in one register so
  // the compiler does not fold the large region offsets into per-stage copies.
  //   X slot i, k16 slice kk: row lrow(i), logical chunk 2*kk + hi, swizzled
  //   (an XOR, so one base per slot and slice).
  //   W column block j: rows kk*16 + 8*(g/2) + (li/4) (+4 for the second
  //   half), columns 16*(g%2) + 4*(li%4) of the block; the row swizzle only
  //   depends on li/4, so slices and halves are plain offsets.
  FNG_LDS char* xaddr[FM][BK / 16];
  FNG_LDS char* waddr[FN];
  {
    const int g = lane >> 4, li = lane & 15;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int q = 0; q < BK / 16; ++q) {
        uint32_t a;
        if constexpr (XT) {
          // transposed X: the same transposing-read pattern as W, over BM
          // output rows (slice q is a plain offset, added at the read)
          const int n = wm * WM + 32 * ((i + rot) % FM) + 16 * (g & 1) + 4 * (li & 3);
          const int k0 = 8 * (g >> 1) + (li >> 2);
          a = (uint32_t)reinterpret_cast<uintptr_t>(lds + S::A_OFF + k0 * (BM * 2) + ((n >> 3) ^ swz_b<MC>(k0)) * 16 +
                                                    (n & 7) * 2);
        } else if constexpr (PX) {
          // the first tile of a pair; the second is this address XOR 64
          const int row = lrow(i);
          const int kc = 2 * q + hi;
          a = (uint32_t)reinterpret_cast<uintptr_t>(lds + S::A_OFF + row * (BK * 4) + (kc ^ swz_px(row)) * 16);
        } else {
          const int row = lrow(i);
          const int kc = 2 * q + hi;
          a = (uint32_t)reinterpret_cast<uintptr_t>(lds + S::A_OFF + row * (BK * 2) + (kc ^ swz_a<KC>(row)) * 16);
        }
        asm volatile("" : "+v"(a));
        xaddr[i][q] = reinterpret_cast<FNG_LDS char*>(static_cast<uintptr_t>(a));
      }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = wn * WN + 32 * j + 16 * (g & 1) + 4 * (li & 3);
      const int k0 = 8 * (g >> 1) + (li >> 2);
      uint32_t a = (uint32_t)reinterpret_cast<uintptr_t>(lds + k0 * (BN * 2) + ((n >> 3) ^ swz_b<NC>(k0)) * 16 + (n & 7) * 2);
      asm volatile("" : "+v"(a));
      waddr[j] = reinterpret_cast<FNG_LDS char*>(static_cast<uintptr_t>(a));
    }
  }

  const int M = p.M, N = p.N, K = p.K;
  const int ktiles = (K + BK - 1) / BK;
  // the epilogues scale by reciprocals (v_rcp_f32, within 1 ulp): an fp32
  // division is a dozen instructions, and the split-N merge made two per
  // column tile on the thread that merges a row, on every tile's critical path
  const float inv_k = __builtin_amdgcn_rcpf((float)K);
  const float inv_n = __builtin_amdgcn_rcpf((float)N);

  // split-N: this call's tag = the last call's epoch + 1 (constant during the
  // call: the epoch only advances after every row block has been merged)
  uint32_t ep = 0;
  if constexpr (IS_SPLIT) ep = __hip_atomic_load(p.status + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;

  // persistent loop for split-N, one tile per workgroup otherwise
  const uint32_t G = gridDim.x;
  const uint32_t slot = xcd_remap(blockIdx.x, G);
  for (int t = (int)slot; t < p.total_tiles; t += (int)G) {
    int tm, tn;
    if constexpr (IS_SPLIT) {
      // a round is G consecutive tiles = whole row blocks, so every wait is
      // on a peer of the same round
      if (p.sn_cw > 0) {
        const int r = t / (int)G, s = t - r * (int)G;
        const int per = (int)G / 8;  // slots per XCD (slot -> XCD as in xcd_remap)
        const int x = s / per, j = s % per;
        tm = r * ((int)G / p.tiles_n) + (x / p.sn_g) * p.sn_rh + j % p.sn_rh;
        tn = (x % p.sn_g) * p.sn_cw + j / p.sn_rh;
      } else {
        tm = t / p.tiles_n;
        tn = t % p.tiles_n;
      }
    } else {
      const int per_group = p.group_m * p.tiles_n;
      const int g = t / per_group;
      const int first_m = g * p.group_m;
      const int gsize = min(p.group_m, p.tiles_m - first_m);
      const int r = t - g * per_group;
      tm = first_m + r % gsize;
      tn = r / gsize;
    }
    const int m0 = tm * BM;
    const int n0 = p.n_off + tn * BN;

    // rows of X past M and K/N tails of W read as zero; X's range is capped
    // below kOOB so that kOOB offsets are always out of range
    const int64_t xrem = (int64_t)(M - m0) * K * 2;
    const uint32_t xbytes = xrem > 0x7ffffff0LL ? 0x7ffffff0u : (uint32_t)xrem;
    const i32x4_t xr = XT ? dma_rsrc(p.X + m0, (uint32_t)((int64_t)K * M * 2 - (int64_t)m0 * 2))
                          : dma_rsrc(p.X + (size_t)m0 * K, xbytes);
    const i32x4_t wr = dma_rsrc(p.W + n0, (uint32_t)((int64_t)K * N * 2 - (int64_t)n0 * 2));
    i32x4_t gr;
    if constexpr (PG) gr = dma_rsrc(p.gamma, (uint32_t)K * 2);
    if constexpr (KS) gr = dma_rsrc(p.rstd_in, (uint32_t)K * 4);

    // ---- this lane's share of each K tile's copies ------------------------
    // X: copy i of this wave fills LDS bytes [(wave*A_PER_WAVE + i) KB, +1 KB)
    //    of the stage; lane l writes the 16 B at +16 l, i.e. row r, physical
    //    chunk pc, which holds logical chunk pc ^ swz(r).
    uint32_t a_off[AX];
    int a_k[AX];  // XT: 0 (chunk in range) or kOOB (past M), else the chunk's k offset
#pragma unroll
    for (int i = 0; i < AX; ++i) {
      const int idx = (wave * AX + i) * 1024 + lane * 16;
      if constexpr (PX) {
        // paired: 8 rows of 128 B per copy; lanes 8r .. 8r+7 read one row's
        // 128-byte line (each group of 4 lanes one contiguous half)
        const int row = idx / (BK * 4), pc = (idx % (BK * 4)) / 16;
        const int c = pc ^ swz_px(row);
        a_k[i] = c * 8;
        a_off[i] = (uint32_t)(row * K + c * 8) * 2u;
      } else if constexpr (XT) {
        // transposed X tile [BK][BM]: k row krow, out-row chunk mc (the W scheme)
        const int krow = idx / (BM * 2), pc = (idx % (BM * 2)) / 16;
        const int mc = pc ^ swz_b<MC>(krow);
        a_k[i] = m0 + mc * 8 < M ? 0 : (int)kOOB;
        a_off[i] = (uint32_t)(krow * M + mc * 8) * 2u;
      } else {
        const int row = idx / (BK * 2), pc = (idx % (BK * 2)) / 16;
        const int kc = pc ^ swz_a<KC>(row);
        a_k[i] = kc * 8;
        a_off[i] = (uint32_t)(row * K + kc * 8) * 2u;
      }
    }
    uint32_t b_off[B_PER_WAVE];
    bool b_ok[B_PER_WAVE];
#pragma unroll
    for (int i = 0; i < B_PER_WAVE; ++i) {
      const int idx = (wave * B_PER_WAVE + i) * 1024 + lane * 16;
      const int krow = idx / (BN * 2), pc = (idx % (BN * 2)) / 16;
      const int nc = pc ^ swz_b<NC>(krow);
      b_ok[i] = n0 + nc * 8 < N;
      b_off[i] = (uint32_t)(krow * N + nc * 8) * 2u;
    }
    // Out-of-range copies (K tail, N tail, tiles past the end) set bit 31 of
    // the offset: both descriptors' ranges are below 2^31, so they read zeros.
    // norm backward: the refills past the last K tile bring in the saved
    // [BM, BN] tile instead of zeros -- each LDS block of a freed stage gets
    // the block of the tile (output staging layout) that lives at that
    // address, so the tile is in LDS when the mainloop ends.  Same number of
    // copies per refill, so the vmcnt accounting does not change.
    i32x4_t hr;
    if constexpr (IS_BWD) hr = dma_rsrc(p.H, (uint32_t)((int64_t)M * N * 2));
    auto saved_block = [&](int off) __attribute__((always_inline)) {
      constexpr int NCH = BN / 8;
      constexpr int TB = BM * BN * 2 / 1024;  // blocks of the saved tile
      const int blk = off / 1024;
      if (blk >= TB) return kOOB;
      const int idx = blk * 1024 + lane * 16;
      const int row = idx / (BN * 2), pc = (idx % (BN * 2)) / 16;
      const int ch = (pc ^ row) & (NCH - 1);
      return (uint32_t)(((int64_t)(m0 + row) * N + n0 + ch * 8) * 2);
    };
    auto issue = [&](int kt, int s) {
      if constexpr (PX) {
        // odd tiles first copy X of the pair (kt - 1, kt) into pair slot s / 2
        // (both its stages are free: this issue refills the stage of the tile
        // before the current one, and the pair's other stage held the tile
        // before that), then W of kt; even tiles copy only their W
        if (kt & 1) {
          const int k0 = (kt - 1) * BK;
          FNG_LDS char* xs = lds + S::A_OFF + (s / 2) * (2 * S::A_STAGE);
          if (kt - 1 < ktiles && k0 + 2 * BK <= K) {
#pragma unroll
            for (int i = 0; i < AX; ++i) dma16_so(xr, xs + (wave * AX + i) * 1024, a_off[i], (uint32_t)(k0 * 2));
          } else {
            const uint32_t live = kt - 1 < ktiles ? 0u : kOOB;
#pragma unroll
            for (int i = 0; i < AX; ++i) {
              const uint32_t dead = (k0 + a_k[i] < K) ? live : kOOB;
              dma16(xr, xs + (wave * AX + i) * 1024, (a_off[i] + (uint32_t)(k0 * 2)) | dead);
            }
          }
        }
        if (kt < ktiles && (kt + 1) * BK <= K) {
#pragma unroll
          for (int i = 0; i < B_PER_WAVE; ++i)
            dma16_so(wr, lds + S::b(s) + (wave * B_PER_WAVE + i) * 1024, b_off[i] | (b_ok[i] ? 0u : kOOB),
                     (uint32_t)(kt * BK) * (uint32_t)N * 2u);
        } else {
          const uint32_t kt_live = kt < ktiles ? 0u : kOOB;
#pragma unroll
          for (int i = 0; i < B_PER_WAVE; ++i) {
            const uint32_t dead = b_ok[i] ? kt_live : kOOB;
            dma16(wr, lds + S::b(s) + (wave * B_PER_WAVE + i) * 1024,
                  (b_off[i] + (uint32_t)(kt * BK) * (uint32_t)N * 2u) | dead);
          }
        }
        return;
      }
      if constexpr (IS_BWD) {
        if (kt >= ktiles) {
#pragma unroll
          for (int i = 0; i < A_PER_WAVE; ++i) {
            const int off = S::a(s) + (wave * A_PER_WAVE + i) * 1024;
            dma16(hr, lds + off, saved_block(off));
          }
#pragma unroll
          for (int i = 0; i < B_PER_WAVE; ++i) {
            const int off = S::b(s) + (wave * B_PER_WAVE + i) * 1024;
            dma16(hr, lds + off, saved_block(off));
          }
          return;
        }
      }
      if (kt < ktiles && (kt + 1) * BK <= K) {
        // a whole K tile in range: the per-lane offsets are the tile's
        // constants, the K step goes in the scalar offset (no vector work)
#pragma unroll
        for (int i = 0; i < A_PER_WAVE; ++i) {
          if constexpr (XT)
            dma16_so(xr, lds + S::a(s) + (wave * A_PER_WAVE + i) * 1024, a_off[i] | (uint32_t)a_k[i],
                     (uint32_t)(kt * BK) * (uint32_t)M * 2u);
          else
            dma16_so(xr, lds + S::a(s) + (wave * A_PER_WAVE + i) * 1024, a_off[i], (uint32_t)(kt * BK * 2));
        }
#pragma unroll
        for (int i = 0; i < B_PER_WAVE; ++i)
          dma16_so(wr, lds + S::b(s) + (wave * B_PER_WAVE + i) * 1024, b_off[i] | (b_ok[i] ? 0u : kOOB),
                   (uint32_t)(kt * BK) * (uint32_t)N * 2u);
        if constexpr (PG) {
          if (wave == 0 && lane < KC) dma16(gr, lds + S::gm(s), (uint32_t)(kt * BK + lane * 8) * 2u);
        }
        if constexpr (KS) {
          if (wave == 0 && lane < BK / 4) dma16(gr, lds + S::gm(s), (uint32_t)(kt * BK + lane * 4) * 4u);
        }
        return;
      }
      const uint32_t kt_live = kt < ktiles ? 0u : kOOB;
#pragma unroll
      for (int i = 0; i < A_PER_WAVE; ++i) {
        if constexpr (XT) {
          // rows past K lie beyond the buffer range: zeros
          dma16(xr, lds + S::a(s) + (wave * A_PER_WAVE + i) * 1024,
                (a_off[i] + (uint32_t)(kt * BK) * (uint32_t)M * 2u) | (uint32_t)a_k[i] | kt_live);
        } else {
          const uint32_t dead = (kt * BK + a_k[i] < K) ? kt_live : kOOB;
          dma16(xr, lds + S::a(s) + (wave * A_PER_WAVE + i) * 1024, (a_off[i] + (uint32_t)(kt * BK * 2)) | dead);
        }
      }
#pragma unroll
      for (int i = 0; i < B_PER_WAVE; ++i) {
        const uint32_t dead = b_ok[i] ? kt_live : kOOB;
        dma16(wr, lds + S::b(s) + (wave * B_PER_WAVE + i) * 1024,
              (b_off[i] + (uint32_t)(kt * BK) * (uint32_t)N * 2u) | dead);
      }
      if constexpr (PG) {
        if (wave == 0 && lane < KC)
          dma16(gr, lds + S::gm(s), ((uint32_t)(kt * BK + lane * 8) * 2u) | kt_live);
      }
      if constexpr (KS) {
        if (wave == 0 && lane < BK / 4)
          dma16(gr, lds + S::gm(s), ((uint32_t)(kt * BK + lane * 4) * 4u) | kt_live);
      }
    };

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    float ss[SS_SLOTS][2];  // two partial sums per slot: two short dependency chains
    float sx[SS_SLOTS][2];  // lazy LayerNorm: the plain sums
#pragma unroll
    for (int s = 0; s < SS_SLOTS; ++s) ss[s][0] = ss[s][1] = sx[s][0] = sx[s][1] = 0.f;

    // one k16 slice of fragments: X rows of this wave, W columns of this wave
    // (and the matching gamma slice)
    struct Frags {
      u32x4_t x[FM];
      u32x4_t w[FN];
      u32x4_t g;
      f32x4_t s0, s1;  // KS: the contraction scale of this lane's 8 k values
    };
    auto load = [&](int s, int kk, Frags& f) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if constexpr (XT) {
          const FNG_LDS char* xa = xaddr[i][0] + (S::a(s) - S::A_OFF) + kk * 16 * (BM * 2);
          const u32x2_t lo = lds_read_tr16(xa);
          const u32x2_t hi2 = lds_read_tr16(xa + 4 * (BM * 2));
          f.x[i] = u32x4_t{lo[0], lo[1], hi2[0], hi2[1]};
        } else if constexpr (PX) {
          // the second tile of a pair at the first's address XOR 64
          const uint32_t a = (uint32_t)reinterpret_cast<uintptr_t>(xaddr[i][kk]) ^ ((s & 1) ? 64u : 0u);
          f.x[i] = lds_read16(reinterpret_cast<FNG_LDS char*>(static_cast<uintptr_t>(a)) + (s / 2) * (2 * S::A_STAGE));
        } else {
          f.x[i] = lds_read16(xaddr[i][kk] + (S::a(s) - S::A_OFF));
        }
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const FNG_LDS char* wa = waddr[j] + S::b(s) + kk * 16 * (BN * 2);
        const u32x2_t lo = lds_read_tr16(wa);
        const u32x2_t hi2 = lds_read_tr16(wa + 4 * (BN * 2));
        f.w[j] = u32x4_t{lo[0], lo[1], hi2[0], hi2[1]};
      }
      if constexpr (PG) f.g = lds_read16(lds + S::gm(s) + kk * 32 + hi * 16);
      if constexpr (KS) {
        f.s0 = __builtin_bit_cast(f32x4_t, lds_read16(lds + S::gm(s) + kk * 64 + hi * 32));
        f.s1 = __builtin_bit_cast(f32x4_t, lds_read16(lds + S::gm(s) + kk * 64 + hi * 32 + 16));
      }
    };
    // the vector work on one slice's fragments (ping-pong memory phase; the
    // gain fold never runs there)
    auto fold_ks = [&](Frags& f) {
      // weight gradient: rstd of the lane's 8 contraction rows scales its
      // dY values (words 0..3 hold rows 2e, 2e + 1), once per fragment
      float sc[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sc[e] = f.s0[e];
        sc[4 + e] = f.s1[e];
      }
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = f.w[j][e];
          f.w[j][e] = pack_bf16(bf16lo(w) * sc[2 * e], bf16hi(w) * sc[2 * e + 1]);
        }
    };
    auto vec = [&](Frags& f) {
      if constexpr (KS) fold_ks(f);
      if constexpr (EPI == EPI_PRENORM) {
        if (ss_owner) {
#pragma unroll
          for (int s = 0; s < SS_SLOTS; ++s) {
            sumsq_bf16x8_2(f.x[s], ss[s][0], ss[s][1]);
            if constexpr (LN) sum_bf16x8_2(f.x[s], sx[s][0], sx[s][1]);
          }
        }
      }
    };
    auto mfmas = [&](Frags& f) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma_bf16(f.w[j], f.x[i], acc[i][j]);
    };
    auto mma = [&](Frags& f) {
      if constexpr (EPI == EPI_PRENORM) {
        if (ss_owner) {
#pragma unroll
          for (int s = 0; s < SS_SLOTS; ++s) {
            sumsq_bf16x8_2(f.x[s], ss[s][0], ss[s][1]);
            if constexpr (LN) sum_bf16x8_2(f.x[s], sx[s][0], sx[s][1]);
          }
        }
      }
      if constexpr (PG) {
        // the gain multiplies along K; the lane's 8 W values and its 8 X
        // values share the same k, so it is folded into the W fragments
        // (the statistic above used the raw X)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            f.w[j][e] = pack_bf16(bf16lo(f.w[j][e]) * bf16lo(f.g[e]), bf16hi(f.w[j][e]) * bf16hi(f.g[e]));
      }
      if constexpr (KS) fold_ks(f);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma_bf16(f.w[j], f.x[i], acc[i][j]);
      if constexpr (EPI == EPI_PRENORM && !PG) {
        // the sum-of-squares dots go ahead of the slice's MFMAs: placed
        // between MFMAs they cost more (measured on gfx950, where a dot
        // issued behind an MFMA stalls the next MFMA of the wave)
        __builtin_amdgcn_sched_group_barrier(0x002, (LN ? 8 : 4) * SS_SLOTS, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, FM * FN, 0);
      }
    };

    // ---- mainloop: 4-deep ring of K tiles, one barrier per tile ------------
    // Step kt (its first k16 fragments already in registers): read the rest of
    // tile kt's fragments, multiply all but the last slice, then wait for this
    // wave's copies of tile kt+1 (at most those of tiles kt+2, kt+3 may still
    // be in flight) and barrier: every wave has finished reading tile kt and
    // tile kt+1 has landed.  Refill tile kt's stage with tile kt+4, read the
    // first fragments of tile kt+1, and only then multiply the last slice of
    // tile kt, which covers the latency of those reads.  The refill is issued
    // unconditionally (past the last tile it writes zeros nobody reads), so
    // the number of copies in flight is the same at every step.
    constexpr int KK = BK / 16;
    // sched_barrier(0) fences keep the compiler from sinking the next slice's
    // fragment reads down to their consumers: each slice's reads are issued
    // as a block ahead of the previous slice's MFMAs, which cover their latency.
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
    auto step = [&](int kt, int cur, int next, Frags& fa) {
      Frags fb;
#pragma unroll
      for (int kk = 1; kk < KK; ++kk) {
        if (kk % 2 == 1) { load(cur, kk, fb); fence(); mma(fa); fence(); }
        else { load(cur, kk, fa); fence(); mma(fb); fence(); }
      }
      wait_vmcnt<2 * LOADS>();
      lds_barrier();
      issue(kt + STAGES, cur);
      if constexpr (KK % 2 == 0) { load(next, 0, fa); fence(); mma(fb); fence(); }
      else { Frags fc; load(next, 0, fc); fence(); mma(fa); fence(); fa = fc; }
    };
    __syncthreads();  // the previous tile's epilogue may still read LDS
    // The loop-invariant address and offset registers pass through an empty
    // asm here: if the allocator spilled one of them, its reload (and the
    // compiler's wait for it) lands before the loop.  Otherwise the wait for
    // the reload sits inside the loop, where the compiler -- which does not
    // count the copies issued by inline asm -- makes it a wait for every
    // memory operation in flight, i.e. for all the copies of the next tiles
    // (measured: the split-N LayerNorm mainloop took 85 instead of ~56 us per
    // tile of 256 x 256 x 2048).
#pragma unroll
    for (int i = 0; i < AX; ++i) asm volatile("" : "+v"(a_off[i]), "+v"(a_k[i]));
#pragma unroll
    for (int i = 0; i < B_PER_WAVE; ++i) asm volatile("" : "+v"(b_off[i]));
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int q = 0; q < BK / 16; ++q) {
        uint32_t a = (uint32_t)reinterpret_cast<uintptr_t>(xaddr[i][q]);
        asm volatile("" : "+v"(a));
        xaddr[i][q] = reinterpret_cast<FNG_LDS char*>(static_cast<uintptr_t>(a));
      }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      uint32_t a = (uint32_t)reinterpret_cast<uintptr_t>(waddr[j]);
      asm volatile("" : "+v"(a));
      waddr[j] = reinterpret_cast<FNG_LDS char*>(static_cast<uintptr_t>(a));
    }
    if constexpr (PP) {
      // Ping-pong: the two waves of each SIMD (one per row half) alternate
      // between a memory phase M(t) -- read all of K tile t's fragments,
      // issue the copies of tile t+3 into the stage tile t-1 used, wait until
      // this wave's copies of tile t+1 have landed, and the vector work on
      // the fragments (the lazy pre-norm's sums of squares) -- and a compute
      // phase C(t) of the tile's MFMAs back to back.  The row-half-0 waves
      // run M(t) while the row-half-1 waves run C(t-1), then the roles swap;
      // a workgroup barrier separates the phases, so the matrix core of a
      // SIMD is fed by one wave while the other waits on LDS.
      //   stage reuse: tile t-1's stage is refilled in M(t), after the
      //   barrier that ends both halves' reads of tile t-1;
      //   data: every wave has waited for its copies of tile t+1 before the
      //   barrier that precedes the first read of tile t+1.
      Frags f0, f1;
      const bool first = wm == 0;
      auto mem = [&](int t, int st) {
        load(st, 0, f0);
        load(st, 1, f1);
        issue(t + 3, (st + 3) & 3);
        // this wave's copies of tile t+1 have landed; with paired X an even
        // tile's X came with the issue of the odd tile after it, so only the
        // W copies of two issues may still be in flight
        if (PX && (st & 1)) wait_vmcnt<2 * B_PER_WAVE>();
        else wait_vmcnt<2 * LOADS>();
        // the sums of squares wait for their fragments: after the copies are
        // issued, so the copies do not wait behind the LDS reads (measured)
        fence();
        vec(f0);
        vec(f1);
      };
      auto comp = [&] {
        fence();
        mfmas(f0);
        mfmas(f1);
        fence();
      };
      issue(0, 0);
      issue(1, 1);
      issue(2, 2);
      wait_vmcnt<PX ? 2 * B_PER_WAVE : 2 * LOADS>();
      lds_barrier();
      // every wave runs M(t), C(t) with a barrier after each; the second
      // half starts one barrier late and the first half ends one barrier
      // later, so both pass the same number of barriers
      if (!first) lds_barrier();
      auto tile = [&](int t, int st) {
        mem(t, st);
        fence();
        lds_barrier();
        comp();
        lds_barrier();
        fence();
      };
      // unrolled over the ring so that each stage is a compile-time constant
      // (LDS addresses in the instructions' offset fields, no address adds in
      // the memory phase): 2-3 % faster (split-N post-RMSNorm: 142.2 -> 138.9
      // us at 16384 x 1024 x 4096); with the norm backward, the weight
      // gradient and the 128 x 512 full-N tile the unrolled loop makes the
      // allocator spill and the kernels slower (measured)
      constexpr bool UNROLL = EPI == EPI_PLAIN || EPI == EPI_PRENORM || EPI == EPI_ROWSCALE || EPI == EPI_SPLITN ||
                              EPI == EPI_PARTIAL || EPI == EPI_TN || (EPI == EPI_FULLN && BN <= 256);
      if constexpr (UNROLL) {
        for (int t = 0; t < ktiles; t += 4) {
          tile(t, 0);
          if (t + 1 < ktiles) tile(t + 1, 1);
          if (t + 2 < ktiles) tile(t + 2, 2);
          if (t + 3 < ktiles) tile(t + 3, 3);
        }
      } else {
        for (int t = 0; t < ktiles; ++t) tile(t, t & 3);
      }
      if (first) lds_barrier();
      // the norm backward: the refills of tiles ktiles .. ktiles+2 (past the
      // last K tile) brought the saved tile into three stages; the fourth,
      // the last K tile's stage, read by both halves before the last
      // barrier, gets its part now
      if constexpr (IS_BWD) issue(ktiles + 3, (ktiles + 3) & 3);
    } else {
      issue(0, 0);
      issue(1, 1);
      issue(2, 2);
      issue(3, 3);
      wait_vmcnt<3 * LOADS>();
      lds_barrier();
      Frags fr;
      load(0, 0, fr);
      for (int kt = 0; kt < ktiles; kt += 4) {
        step(kt, 0, 1, fr);
        if (kt + 1 < ktiles) step(kt + 1, 1, 2, fr);
        if (kt + 2 < ktiles) step(kt + 2, 2, 3, fr);
        if (kt + 3 < ktiles) step(kt + 3, 3, 0, fr);
      }
    }
    // drain the trailing zero-fill copies before the epilogue reuses the LDS
    wait_vmcnt<0>();
    __syncthreads();

    // ---- epilogues -------------------------------------------------------
    // lane l of wave (wm, wn) holds rows  wm*WM + 32*i + l32          (i < FM)
    // and columns                         wn*WN + 32*j + 8*(r/4) + 4*hi + r%4
    auto col_of = [&](int j, int r4) { return n0 + wn * WN + 32 * j + 8 * r4 + 4 * hi; };
    auto row_of = [&](int i) { return m0 + lrow(i); };

    float rs_mean[FM], rs_rstd[FM];
    if constexpr (EPI == EPI_ROWSCALE) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int m = row_of(i);
        rs_rstd[i] = m < M ? p.rstd_in[m] : 0.f;
        if constexpr (LN) rs_mean[i] = m < M ? p.mean_in[m] : 0.f;
      }
    }
    if constexpr (EPI == EPI_PRENORM) {
      // lazy LayerNorm: mean = sum / K, var = sumsq / K - mean^2 (both sums of
      // the raw X; the subtraction loses digits only when |mean| >> spread)
      FNG_LDS float* red = (FNG_LDS float*)lds;
#pragma unroll
      for (int s = 0; s < SS_SLOTS; ++s) {
        const float tot = xor_sum(ss[s][0] + ss[s][1], 32);
        if (ss_owner && hi == 0) red[lrow(s)] = tot;
        if constexpr (LN) {
          const float t1 = xor_sum(sx[s][0] + sx[s][1], 32);
          if (ss_owner && hi == 0) red[BM + lrow(s)] = t1;
        }
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if constexpr (LN) {
          rs_mean[i] = red[BM + lrow(i)] * inv_k;
          const float var = fmaxf(red[lrow(i)] * inv_k - rs_mean[i] * rs_mean[i], 0.f);
          rs_rstd[i] = __builtin_amdgcn_rsqf(var + p.eps);
        } else {
          rs_mean[i] = 0.f;
          rs_rstd[i] = __builtin_amdgcn_rsqf(red[lrow(i)] * inv_k + p.eps);
        }
      }
    }
    // lazy LayerNorm: the column sums of W at this lane's columns, the
    // partials merged in a fixed order
    constexpr bool LAZY_LN = (EPI == EPI_PRENORM || EPI == EPI_ROWSCALE) && LN;
    float csum[LAZY_LN ? FN : 1][4][4];
    if constexpr (LAZY_LN) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int c = col_of(j, r4);
          f32x4_t v = {0.f, 0.f, 0.f, 0.f};
          if (c < N) v = *reinterpret_cast<const f32x4_t*>(p.colsum + c);
#pragma unroll
          for (int e = 0; e < 4; ++e) csum[j][r4][e] = v[e];
        }
    }

    // norm backward: the saved tile (xhat or the norm's input) is in LDS in
    // the output staging layout (copied by the last refills); the forward
    // rstd goes to registers
    float bw_r[FM], bw_hs[FM];
    if constexpr (IS_BWD) {
      static_assert(S::A_STAGE % 1024 == 0 && S::B_STAGE % 1024 == 0, "whole 1 KB blocks per stage");
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int m = row_of(i);
        bw_r[i] = m < M ? p.rstd_in[m] : 1.f;
        bw_hs[i] = p.h_raw ? bw_r[i] : 1.f;
      }
    }
    // weight gradient with the forward's gain: a scale per output row
    float dwg[DWG ? FM : 1];
    if constexpr (DWG) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int m = row_of(i);
        dwg[i] = m < M ? bf16lo((uint32_t)p.gamma[m]) : 0.f;
      }
    }
    // 8 B of the staged tile at this lane's (row slot i, columns col_of(j, r4) ..)
    auto stage_addr = [&](int i, int j, int r4) __attribute__((always_inline)) {
      constexpr int NCH = BN / 8;
      const int row = lrow(i);
      const int ch = (wn * WN + 32 * j + 8 * r4) / 8;
      return lds + row * (BN * 2) + ((ch ^ row) & (NCH - 1)) * 16 + hi * 8;
    };

    if constexpr (EPI == EPI_FULLN || EPI == EPI_SPLITN || EPI == EPI_PARTIAL || IS_BWD) {
      // per-row statistics of this tile's valid columns, fp32 accumulators
      // red: [WAVES_N][BM] floats in LDS (the stage buffers are free now, or
      // hold the backward's saved tile: then the extra region)
      FNG_LDS float* red = (FNG_LDS float*)(lds + RED);
      const int nvalid = min(BN, N - n0);
      auto row_reduce = [&](float (&v)[FM], float (&out)[FM]) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const float s = xor_sum(v[i], 32);
          if (hi == 0) red[wn * BM + lrow(i)] = s;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          float s = 0.f;
#pragma unroll
          for (int w = 0; w < WAVES_N; ++w) s += red[w * BM + lrow(i)];
          out[i] = s;
        }
        __syncthreads();
      };
      float part[FM], s1[FM], s2[FM];
      if constexpr (IS_BWD) {
        // s1 = sum of g (LayerNorm), s2 = sum of g * xhat over the tile's columns
        float p1[FM], p2[FM];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          float a1 = 0.f, a2 = 0.f;
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
              if (col_of(j, r4) < N) {
                const u32x2_t hv = *reinterpret_cast<const FNG_LDS u32x2_t*>(stage_addr(i, j, r4));
                const float x[4] = {bf16lo(hv[0]), bf16hi(hv[0]), bf16lo(hv[1]), bf16hi(hv[1])};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const float gv = acc[i][j][4 * r4 + e];
                  if constexpr (LN) a1 += gv;
                  a2 = fmaf(gv, x[e] * bw_hs[i], a2);
                }
              }
          p1[i] = a1;
          p2[i] = a2;
        }
        if constexpr (LN) row_reduce(p1, s1);
        else {
#pragma unroll
          for (int i = 0; i < FM; ++i) s1[i] = 0.f;
        }
        row_reduce(p2, s2);
      } else if constexpr (LN) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          float s = 0.f;
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
              if (col_of(j, r4) < N)
#pragma unroll
                for (int e = 0; e < 4; ++e) s += acc[i][j][4 * r4 + e];
          part[i] = s;
        }
        row_reduce(part, s1);  // tile row sums
        float tmean[FM];
        const float inv_valid = __builtin_amdgcn_rcpf((float)nvalid);
#pragma unroll
        for (int i = 0; i < FM; ++i) tmean[i] = s1[i] * inv_valid;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          float s = 0.f;
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
              if (col_of(j, r4) < N)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const float d = acc[i][j][4 * r4 + e] - tmean[i];
                  s += d * d;
                }
          part[i] = s;
        }
        row_reduce(part, s2);  // tile M2 about the tile mean
#pragma unroll
        for (int i = 0; i < FM; ++i) s1[i] = tmean[i];
      } else {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          float s = 0.f;
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
              if (col_of(j, r4) < N)
#pragma unroll
                for (int e = 0; e < 4; ++e) s += acc[i][j][4 * r4 + e] * acc[i][j][4 * r4 + e];
          part[i] = s;
        }
        row_reduce(part, s2);
#pragma unroll
        for (int i = 0; i < FM; ++i) s1[i] = 0.f;
      }
      // s1 = tile mean (LN) / 0 (RMS); s2 = tile M2 (LN) / tile sum of squares (RMS)

      if constexpr (EPI == EPI_FULLN) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          rs_mean[i] = s1[i];
          rs_rstd[i] = __builtin_amdgcn_rsqf(s2[i] * inv_n + p.eps);
        }
      } else if constexpr (EPI == EPI_BWD_FULLN) {
        // backward: rs_mean = mean(g), rs_rstd = mean(g * xhat)
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          rs_mean[i] = s1[i] * inv_n;
          rs_rstd[i] = s2[i] * inv_n;
        }
      } else {
        if constexpr (EPI == EPI_PARTIAL) {
          // two-pass: plain float partials part[tm][tn][row][2] for the finalize kernel
#pragma unroll
          for (int i = 0; i < FM; ++i) rs_mean[i] = s1[i];
          float* pp = p.part + ((size_t)tm * p.tiles_n + tn) * (BM * 2);
          if (wn == 0 && hi == 0) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
              const int row = lrow(i);
              pp[row * 2 + 0] = s1[i];
              pp[row * 2 + 1] = s2[i];
            }
          }
        }
        if constexpr (IS_SPLIT) {
          // Exchange (section 3's multi-CTA reduction, without clusters).
          // Each partial is one 64-bit device-scope store of (value, tag): the
          // tag is this call's epoch, so a reader that sees the tag has the
          // value, and readers poll the partials themselves -- one memory
          // round trip when the peers are done, no counter on the critical
          // path.  Device-scope accesses are performed at the device-coherent
          // level (past the per-XCD L2s): no cache-wide write-back needed.
          // part: [tm][tn][row][2] x 64 bit; status[1]: epoch of the last call.
          constexpr bool NEED1 = LN;  // LayerNorm needs the first partial too
          uint64_t* pt = reinterpret_cast<uint64_t*>(p.part);
          if (wn == 0 && hi == 0) {
            uint64_t* q = pt + ((size_t)tm * p.tiles_n + tn) * (BM * 2);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
              const int row = lrow(i);
              if constexpr (NEED1)
                __hip_atomic_store(q + row * 2 + 0, ((uint64_t)ep << 32) | __float_as_uint(s1[i]), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
              __hip_atomic_store(q + row * 2 + 1, ((uint64_t)ep << 32) | __float_as_uint(s2[i]), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
            }
          }
          FNG_LDS float* stats = (FNG_LDS float*)(lds + RED);  // [BM][2]
          // merge the tiles_n slices of row tid in a fixed order (bitwise
          // reproducible); loads in batches of 8 independent loads, a batch
          // re-polled until every tag in it is this call's
          if (tid < BM) {
            const uint64_t* pb = pt + (size_t)tm * p.tiles_n * (BM * 2) + tid * 2;
            const int nt = p.tiles_n;
            constexpr int BATCH = (NEED1 || IS_BWD) ? 8 : 16;  // RMS forward: one round trip for 16 column tiles
            float cn = 0.f, mean = 0.f, m2 = 0.f, ssum = 0.f, gsum = 0.f;
            // the wait is bounded in time (the real-time counter runs at a
            // fixed 100 MHz whatever the shader clock), not in polls
            const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
            bool timed_out = false;
            for (int q0 = 0; q0 < nt; q0 += BATCH) {
              uint64_t mb[BATCH], vb[BATCH];
              for (;;) {
#pragma unroll
                for (int u = 0; u < BATCH; ++u) {
                  const int q = min(q0 + u, nt - 1);  // clamped: always a valid slice
                  const uint64_t* a = pb + (size_t)q * BM * 2;
                  if constexpr (NEED1) mb[u] = __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                  vb[u] = __hip_atomic_load(a + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                bool ready = true;
#pragma unroll
                for (int u = 0; u < BATCH; ++u) {
                  if constexpr (NEED1) ready = ready && (uint32_t)(mb[u] >> 32) == ep;
                  ready = ready && (uint32_t)(vb[u] >> 32) == ep;
                }
                if (ready) break;
                if (__builtin_amdgcn_s_memrealtime() - t_start > (uint64_t)p.wait_ticks) {
                  __hip_atomic_fetch_or(p.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                  timed_out = true;
                  break;
                }
                __builtin_amdgcn_s_sleep(1);
              }
#pragma unroll
              for (int u = 0; u < BATCH; ++u) {
                if (q0 + u >= nt) break;
                const float v1 = NEED1 ? __uint_as_float((uint32_t)mb[u]) : 0.f;
                const float v2 = __uint_as_float((uint32_t)vb[u]);
                if constexpr (IS_BWD) {
                  // backward: plain sums of g and g * xhat
                  gsum += v1;
                  ssum += v2;
                } else if constexpr (LN) {
                  // Chan et al. pairwise merge of (count, mean, M2)
                  const float nb = (float)min(BN, N - (q0 + u) * BN);
                  const float w = nb * __builtin_amdgcn_rcpf(cn + nb);  // nb / (cn + nb)
                  const float d = v1 - mean;
                  mean += d * w;
                  m2 += v2 + d * d * (cn * w);
                  cn += nb;
                } else {
                  ssum += v2;
                }
              }
            }
            if constexpr (IS_BWD) {
              stats[tid * 2 + 0] = gsum * inv_n;
              stats[tid * 2 + 1] = ssum * inv_n;
            } else if constexpr (LN) {
              stats[tid * 2 + 0] = mean;
              stats[tid * 2 + 1] = __builtin_amdgcn_rsqf(m2 * inv_n + p.eps);
            } else {
              stats[tid * 2 + 0] = 0.f;
              stats[tid * 2 + 1] = __builtin_amdgcn_rsqf(ssum * inv_n + p.eps);
            }
            if (timed_out && p.poison_on_timeout) stats[tid * 2 + 1] = __builtin_nanf("");
          }
          __syncthreads();
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            rs_mean[i] = stats[lrow(i) * 2 + 0];
            rs_rstd[i] = stats[lrow(i) * 2 + 1];
          }
        }
      }
    }

    // statistics outputs (one writer per row)
    if constexpr (EPI == EPI_PRENORM || EPI == EPI_FULLN || EPI == EPI_SPLITN) {
      if (n0 == p.n_off && wn == 0 && hi == 0) {  // the launch's first column tile
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int m = row_of(i);
          if (m < M) {
            if (p.rstd_out) p.rstd_out[m] = rs_rstd[i];
            if constexpr (LN)
              if (p.mean_out) p.mean_out[m] = rs_mean[i];
          }
        }
      }
    }

    // ---- store bf16 through LDS: fragments -> swizzled LDS tile -> full rows
    // A lane holds 4 consecutive columns of one row per register quad; lanes l
    // and l + 32 hold the two halves of one 16-byte chunk.  The tile is staged
    // in LDS (chunk index XOR-ed with the row so the 32 rows of one write land
    // on distinct banks) and written back with 16-byte stores along rows.
    {
      static_assert(BM * BN * 2 <= S::BYTES, "output tile fits in the ring");
      constexpr int NCH = BN / 8;  // 16-byte chunks per tile row
      // post-norm affine (gain and optional bias per column, applied in fp32
      // before the single rounding): 4 bf16 of each at this lane's columns
      u32x2_t gq[AFF ? FN : 1][4], bq[AFF ? FN : 1][4];
      if constexpr (AFF) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int c = col_of(j, r4);
            const bool in = c < N;
            gq[j][r4] = in ? *reinterpret_cast<const u32x2_t*>(p.gamma + c) : u32x2_t{0u, 0u};
            bq[j][r4] = (in && p.beta) ? *reinterpret_cast<const u32x2_t*>(p.beta + c) : u32x2_t{0u, 0u};
          }
      }
      __syncthreads();             // statistics in LDS have been read
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = lrow(i);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            float v[4];
            float xh[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (IS_BWD) {  // this lane's staged xhat, about to be overwritten
              const u32x2_t hv = *reinterpret_cast<const FNG_LDS u32x2_t*>(stage_addr(i, j, r4));
              xh[0] = bf16lo(hv[0]) * bw_hs[i];
              xh[1] = bf16hi(hv[0]) * bw_hs[i];
              xh[2] = bf16lo(hv[1]) * bw_hs[i];
              xh[3] = bf16hi(hv[1]) * bw_hs[i];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float a = acc[i][j][4 * r4 + e];
              // dz = rstd (g - mean(g) - xhat mean(g xhat))
              if constexpr (IS_BWD) a = bw_r[i] * (a - rs_mean[i] - xh[e] * rs_rstd[i]);
              if constexpr (DWG) a *= dwg[i];
              if constexpr (LAZY_LN) a = (a - rs_mean[i] * csum[j][r4][e]) * rs_rstd[i];
              else if constexpr (EPI == EPI_PRENORM || EPI == EPI_ROWSCALE) a *= rs_rstd[i];
              if constexpr (EPI == EPI_FULLN || EPI == EPI_SPLITN) {
                a = (a - rs_mean[i]) * rs_rstd[i];
                if constexpr (AFF) {
                  const uint32_t gw = gq[j][r4][e >> 1], bw = bq[j][r4][e >> 1];
                  a = fmaf(a, (e & 1) ? bf16hi(gw) : bf16lo(gw), (e & 1) ? bf16hi(bw) : bf16lo(bw));
                }
              }
              // two-pass LayerNorm keeps the bf16 intermediate centred on the tile
              // mean, so rows whose mean dwarfs their spread keep their precision
              if constexpr (EPI == EPI_PARTIAL && LN) a -= rs_mean[i];
              v[e] = a;
            }
            const int ch = (wn * WN + 32 * j + 8 * r4) / 8;
            *reinterpret_cast<FNG_LDS u32x2_t*>(lds + row * (BN * 2) + ((ch ^ row) & (NCH - 1)) * 16 + hi * 8) =
                u32x2_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
          }
        }
      }
      __syncthreads();
      constexpr int NT = 64 * NWAVES;
#pragma unroll 4
      for (int c = tid; c < BM * NCH; c += NT) {
        const int row = c / NCH, ch = c % NCH;
        const int m = m0 + row, n = n0 + ch * 8;
        const u32x4_t v = lds_read16(lds + row * (BN * 2) + ((ch ^ row) & (NCH - 1)) * 16);
        // non-temporal: the output is not read again here, and streaming it
        // past the L2 keeps the operands' lines there (measured 0.5-1.5 %
        // faster on 4096 x 4096 x 14336 and 16384 x 1024 x 4096)
        if (m < M && n < N) __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p.Y + (size_t)m * N + n));
      }
    }
  }
  if constexpr (IS_SPLIT) {
    // The epoch advances once every workgroup of the grid has finished all
    // its tiles (each read the old epoch at its start and has merged every
    // partial it waited for): status[2] counts the finished workgroups, the
    // last one resets it and publishes this call's epoch for the next call
    // on the workspace.  One atomic per workgroup per call, after its last
    // store, so no tile's epilogue waits on it.
    if (tid == 0) {
      const uint32_t f = __hip_atomic_fetch_add(p.status + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (f == G - 1u) {
        __hip_atomic_store(p.status + 2, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.status + 1, ep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host side: configurations and launch
// ---------------------------------------------------------------------------
namespace {

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int EPI, bool LN, bool GAMMA>
int launch(const GemmParams& p0, int grid, bool cooperative, hipStream_t stream) {
  GemmParams p = p0;
  p.tiles_m = (p.M + BM - 1) / BM;
  p.tiles_n = (p.n_end - p.n_off + BN - 1) / BN;
  p.total_tiles = p.tiles_m * p.tiles_n;
  auto kern = gemm_kernel<BM, BN, BK, WAVES_M, WAVES_N, EPI, LN, GAMMA>;
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  if (grid <= 0) grid = p.total_tiles;
  if (cooperative) {
    void* args[] = {&p};
    if (hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kern), dim3(grid), dim3(NT), args, 0,
                                   stream) != hipSuccess)
      return FNG_ERR_HIP;
  } else {
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), 0, stream, p);
  }
  return hipGetLastError() == hipSuccess ? FNG_OK : FNG_ERR_HIP;
}

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int EPI, bool LN, bool GAMMA>
int max_coresident_grid() {
  int per_cu = 0, dev = 0, cus = 0;
  auto kern = gemm_kernel<BM, BN, BK, WAVES_M, WAVES_N, EPI, LN, GAMMA>;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern),
                                                   64 * WAVES_M * WAVES_N, 0) !=
      hipSuccess)
    return -1;
  return per_cu * cus;
}

GemmParams base_params(const GemmCall& c) {
  GemmParams p{};
  p.X = static_cast<const uint16_t*>(c.X);
  p.W = static_cast<const uint16_t*>(c.W);
  p.gamma = static_cast<const uint16_t*>(c.gamma);
  p.Y = static_cast<uint16_t*>(c.Y);
  p.mean_out = c.mean_out;
  p.rstd_out = c.rstd_out;
  p.beta = static_cast<const uint16_t*>(c.beta);
  p.M = (int)c.M;
  p.N = (int)c.N;
  p.K = (int)c.K;
  p.eps = c.eps;
  p.n_off = 0;
  p.n_end = p.N;
  p.group_m = 4;
  p.wait_ticks = 2000000u;  // 20 ms: peers of a round are co-resident, their waits take microseconds
  p.poison_on_timeout = c.poison_on_timeout ? 1 : 0;
  return p;
}

// tile choice for the MFMA-bound mainloop (large M and N)
constexpr int kBigBM = 256, kBigBN = 256, kBigBK = 32, kBigWM = 2, kBigWN = 4;

bool small_problem(const GemmCall& c) { return c.M * c.N <= 256LL * 256 * 64; }

int device_cus() {
  static int cached[64] = {0};
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cached[dev] = cus;
  return cus;
}

// The big tiles' last round often fills only part of the GPU (4096 x 14336 is
// 896 tiles of 256 x 256 on 256 CUs: 3.5 rounds, the last one half empty).
// Then the trailing column blocks run as a second launch of 128 x 256 tiles,
// chosen so that the first launch is a whole number of rounds and the tail
// has twice as many half-size tiles: 3 rounds + 1 round at half cost.
// Returns the first tail column (N when no split pays off).
int64_t tail_split_column(int64_t M, int64_t N) {
  const int cus = device_cus();
  const int64_t tm = (M + 255) / 256, tn = (N + 255) / 256;
  if (cus <= 0 || tn < 2 || (tm * tn) % cus == 0) return N;
  // main column blocks: a multiple of the blocks per whole round of CUs
  int64_t g = tm, c = cus;
  while (c) { const int64_t t = g % c; g = c; c = t; }
  const int64_t per_round = cus / g;  // column blocks whose tiles fill whole rounds
  const int64_t nb_main = (tn / per_round) * per_round;
  if (nb_main == 0 || nb_main == tn) return N;
  // estimated time in units of one 256 x 256 tile per CU
  const double single = (double)((tm * tn + cus - 1) / cus);
  const double split = (double)(tm * nb_main / cus) + 0.5 * (double)((2 * tm * (tn - nb_main) + cus - 1) / cus);
  return split + 0.25 < single ? nb_main * 256 : N;
}

// post-norm launches: LayerNorm or RMSNorm, with or without the affine
template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int EPI>
int launch_norm(const GemmParams& p, bool ln, bool aff, int grid, hipStream_t s) {
  if (ln) return aff ? launch<BM, BN, BK, WAVES_M, WAVES_N, EPI, true, true>(p, grid, false, s)
                     : launch<BM, BN, BK, WAVES_M, WAVES_N, EPI, true, false>(p, grid, false, s);
  return aff ? launch<BM, BN, BK, WAVES_M, WAVES_N, EPI, false, true>(p, grid, false, s)
             : launch<BM, BN, BK, WAVES_M, WAVES_N, EPI, false, false>(p, grid, false, s);
}

template <int EPI, bool GAMMA, bool LN = false>
int launch_big(const GemmParams& p0, hipStream_t s) {
  const int64_t ns = tail_split_column(p0.M, p0.N);
  GemmParams p = p0;
  p.n_end = (int)ns;
  int st = launch<kBigBM, kBigBN, kBigBK, kBigWM, kBigWN, EPI, LN, GAMMA>(p, 0, false, s);
  if (st != FNG_OK || ns >= p0.N) return st;
  p.n_off = (int)ns;
  p.n_end = p0.N;
  // half-size tiles for the tail: 128 x 256 (64 x 64 per wave) measured 5-8 %
  // faster than 256 x 128 (128 x 32 per wave) on the last 2048 columns of
  // 4096 x 14336
  return launch<kBigBM / 2, kBigBN, kBigBK, kBigWM, kBigWN, EPI, LN, GAMMA>(p, 0, false, s);
}

// column sums of W [K, N] for the lazy LayerNorm, in fixed order: block
// (x, y) sums rows [y kchunk, (y + 1) kchunk) of columns [256 x, 256 x + 256)
// into part[y][n] (32 row lanes per column chunk, then the lanes in order).
// 1024 threads with 4 rows in flight each keep 64 KB of W in flight per
// block: with 256 threads the pass ran at half the HBM bandwidth.
constexpr int kColsumLanes = 32;
__global__ __launch_bounds__(1024) void colsum_kernel(const uint16_t* W, float* part, int K, int N, int kchunk) {
  __shared__ float red[kColsumLanes][256];
  const int t = threadIdx.x;
  const int c8 = t & 31, rl = t >> 5;
  const int n = blockIdx.x * 256 + c8 * 8;
  const int k0 = blockIdx.y * kchunk, k1 = min(K, k0 + kchunk);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (n < N) {  // N % 8 == 0: the whole 8-column chunk is in range
#pragma unroll 4
    for (int k = k0 + rl; k < k1; k += kColsumLanes) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(W + (size_t)k * N + n);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = v[e];
        acc[2 * e] += bf16lo(w);
        acc[2 * e + 1] += bf16hi(w);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) red[rl][c8 * 8 + j] = acc[j];
  __syncthreads();
  if (t < 256) {
    const int col = blockIdx.x * 256 + t;
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < kColsumLanes; ++r) s += red[r][t];
    if (col < N) part[(size_t)blockIdx.y * N + col] = s;
  }
}

// the column-sum partials merged in place: part[0][n] = sum_q part[q][n],
// so that the GEMM's epilogue reads one sum per column (reading all the
// partials in every tile of the call cost ~16 us on 4096 x 4096 x 14336,
// this pass ~1 us).
__global__ __launch_bounds__(256) void colsum_merge_kernel(float* part, int N, int parts) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  float v = 0.f;
  for (int q = 0; q < parts; ++q) v += part[(size_t)q * N + n];
  part[n] = v;
}

}  // namespace

// split-N geometry shared with the workspace size computation
int64_t splitn_tiles_m(int64_t M) { return (M + kBigBM - 1) / kBigBM; }
int64_t splitn_tiles_n(int64_t N) { return (N + kBigBN - 1) / kBigBN; }
int64_t splitn_bm() { return kBigBM; }
int64_t fulln_max_n() { return 512; }

int launch_gemm(const GemmCall& c, hipStream_t s) {
  GemmParams p = base_params(c);
  if (small_problem(c)) return launch<64, 64, 64, 2, 2, EPI_PLAIN, false, false>(p, 0, false, s);
  // narrow outputs with many rows: the same tall tiles as the full-N post-norm,
  // so the unfused baseline is not handicapped by 256-wide tiles on N <= 128
  if (c.M >= 256 * 256 && c.N <= 64) return launch<256, 64, 64, 4, 2, EPI_PLAIN, false, false>(p, 0, false, s);
  if (c.M >= 256 * 256 && c.N <= 128) return launch<256, 128, 32, 2, 4, EPI_PLAIN, false, false>(p, 0, false, s);
  return launch_big<EPI_PLAIN, false>(p, s);
}

int launch_prenorm(const GemmCall& c, hipStream_t s) {
  GemmParams p = base_params(c);
  const bool g = c.gamma != nullptr;
  if (small_problem(c)) {
    return g ? launch<64, 64, 64, 2, 2, EPI_PRENORM, false, true>(p, 0, false, s)
             : launch<64, 64, 64, 2, 2, EPI_PRENORM, false, false>(p, 0, false, s);
  }
  if (g || !c.rstd_out) return g ? launch_big<EPI_PRENORM, true>(p, s) : launch_big<EPI_PRENORM, false>(p, s);
  // With rstd_out to hand the statistic over, a row's sum of squares is
  // accumulated beside the K loop of one launch only (section 2 accepts the
  // redundancy across CTAs as overlapped work; here it would be 56 sums per
  // row on 4096 x 14336, each lengthening its tile's memory phase): launch A
  // covers some column blocks of every row block with EPI_PRENORM and writes
  // rstd_out from its first column tile; launch B, after it on the stream,
  // covers the other columns with EPI_ROWSCALE, reading rstd_out.
  //   A = the half-size tiles of the last partial round (tail_split_column),
  //       run first; B = the whole rounds of 256 x 256 tiles;
  //   without a partial round and with at least two rounds of tiles: A = the
  //       first round's worth of column blocks, B = the rest.
  const int64_t ns = tail_split_column(p.M, p.N);
  GemmParams a = p, b = p;
  b.rstd_in = c.rstd_out;
  if (ns < p.N) {
    a.n_off = (int)ns;
    a.n_end = p.N;
    b.n_off = 0;
    b.n_end = (int)ns;
    const int st = launch<kBigBM / 2, kBigBN, kBigBK, kBigWM, kBigWN, EPI_PRENORM, false, false>(a, 0, false, s);
    if (st != FNG_OK) return st;
    return launch<kBigBM, kBigBN, kBigBK, kBigWM, kBigWN, EPI_ROWSCALE, false, false>(b, 0, false, s);
  }
  const int cus = device_cus();
  const int64_t tm = (p.M + kBigBM - 1) / kBigBM, tn = (p.N + kBigBN - 1) / kBigBN;
  if (cus <= 0 || tm * tn < 2 * cus) return launch_big<EPI_PRENORM, false>(p, s);
  const int64_t na = std::max<int64_t>(1, std::min<int64_t>(tn - 1, cus / tm));
  a.n_end = (int)(na * kBigBN);
  b.n_off = a.n_end;
  const int st = launch<kBigBM, kBigBN, kBigBK, kBigWM, kBigWN, EPI_PRENORM, false, false>(a, 0, false, s);
  if (st != FNG_OK) return st;
  return launch<kBigBM, kBigBN, kBigBK, kBigWM, kBigWN, EPI_ROWSCALE, false, false>(b, 0, false, s);
}

// the gain folded into the rows of W once per call: Wg[k, n] = bf16(gamma[k] * W[k, n]),
// one rounding, as the in-loop fold makes it.  grid (ceil(N/8 / 1024), K):
// block (x, k) scales 16-byte chunks x*1024 + t + 256 j (j < 4) of row k.
__global__ __launch_bounds__(256) void scale_rows_kernel(const uint16_t* W, const uint16_t* gamma, uint16_t* Wg,
                                                         int K, int N8) {
  const int k = blockIdx.y;
  const float g = bf16lo((uint32_t)gamma[k]);
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(W + (size_t)k * N8 * 8);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(Wg + (size_t)k * N8 * 8);
  const int c0 = blockIdx.x * 1024 + threadIdx.x;
  u32x4_t v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (c0 + 256 * j < N8) v[j] = src[c0 + 256 * j];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (c0 + 256 * j >= N8) break;
    u32x4_t o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t w = v[j][e];
      o[e] = pack_bf16(bf16lo(w) * g, bf16hi(w) * g);
    }
    dst[c0 + 256 * j] = o;
  }
}

// lazy pre-norm with a caller workspace: the gain folded into W by one
// streaming pass (the in-loop fold would scale each W value once per wave
// that reads it), and the statistic handed between the two launches through
// rstd_out or the workspace
bool prenorm_ws_needs_wg(int64_t M, int64_t N) {
  GemmCall c{};
  c.M = M;
  c.N = N;
  return !small_problem(c);
}

int launch_prenorm_ws(const GemmCall& c, void* ws, hipStream_t s) {
  GemmCall d = c;
  char* base = static_cast<char*>(ws);
  const size_t rbytes = ((size_t)c.M * 4 + 255) & ~(size_t)255;
  if (!d.rstd_out) d.rstd_out = reinterpret_cast<float*>(base);
  if (c.gamma && !small_problem(c)) {
    uint16_t* wg = reinterpret_cast<uint16_t*>(base + rbytes);
    const int n8 = (int)(c.N / 8);
    hipLaunchKernelGGL(scale_rows_kernel, dim3((unsigned)((n8 + 1023) / 1024), (unsigned)c.K), dim3(256), 0, s,
                       static_cast<const uint16_t*>(c.W), static_cast<const uint16_t*>(c.gamma), wg, (int)c.K, n8);
    if (hipGetLastError() != hipSuccess) return FNG_ERR_HIP;
    d.W = wg;
    d.gamma = nullptr;
  }
  return launch_prenorm(d, s);
}

int prenorm_ln_parts(int64_t K) { return K >= 8 * 64 ? 8 : (int)((K + 63) / 64); }

int launch_prenorm_ln(const GemmCall& c, float* colsum, hipStream_t s) {
  const int parts = prenorm_ln_parts(c.K);
  const int kchunk = (int)((c.K + parts - 1) / parts);
  hipLaunchKernelGGL(colsum_kernel, dim3((unsigned)((c.N + 255) / 256), (unsigned)parts), dim3(1024), 0, s,
                     static_cast<const uint16_t*>(c.W), colsum, (int)c.K, (int)c.N, kchunk);
  if (hipGetLastError() != hipSuccess) return FNG_ERR_HIP;
  if (parts > 1) {
    hipLaunchKernelGGL(colsum_merge_kernel, dim3((unsigned)((c.N + 255) / 256)), dim3(256), 0, s, colsum, (int)c.N,
                       parts);
    if (hipGetLastError() != hipSuccess) return FNG_ERR_HIP;
  }
  GemmParams p = base_params(c);
  p.colsum = colsum;
  if (small_problem(c)) return launch<64, 64, 64, 2, 2, EPI_PRENORM, true, false>(p, 0, false, s);
  if (!c.mean_out || !c.rstd_out) return launch_big<EPI_PRENORM, false, true>(p, s);
  // with mean_out and rstd_out to hand the statistics over: the split of
  // launch_prenorm, the row-scale launch applying diag(rstd) (acc - mean colsum)
  const int64_t ns = tail_split_column(p.M, p.N);
  GemmParams a = p, b = p;
  b.rstd_in = c.rstd_out;
  b.mean_in = c.mean_out;
  b.rstd_out = nullptr;
  b.mean_out = nullptr;
  if (ns < p.N) {
    a.n_off = (int)ns;
    a.n_end = p.N;
    b.n_end = (int)ns;
    const int st = launch<kBigBM / 2, kBigBN, kBigBK, kBigWM, kBigWN, EPI_PRENORM, true, false>(a, 0, false, s);
    if (st != FNG_OK) return st;
    return launch<kBigBM, kBigBN, kBigBK, kBigWM, kBigWN, EPI_ROWSCALE, true, false>(b, 0, false, s);
  }
  const int cus = device_cus();
  const int64_t tm = (p.M + kBigBM - 1) / kBigBM, tn = (p.N + kBigBN - 1) / kBigBN;
  if (cus <= 0 || tm * tn < 2 * cus) return launch_big<EPI_PRENORM, false, true>(p, s);
  const int64_t na = std::max<int64_t>(1, std::min<int64_t>(tn - 1, cus / tm));
  a.n_end = (int)(na * kBigBN);
  b.n_off = a.n_end;
  const int st = launch<kBigBM, kBigBN, kBigBK, kBigWM, kBigWN, EPI_PRENORM, true, false>(a, 0, false, s);
  if (st != FNG_OK) return st;
  return launch<kBigBM, kBigBN, kBigBK, kBigWM, kBigWN, EPI_ROWSCALE, true, false>(b, 0, false, s);
}

int launch_postnorm_fulln(const GemmCall& c, bool ln, hipStream_t s) {
  GemmParams p = base_params(c);
  // one workgroup spans all N.  With enough rows for >= 256 workgroups of 256
  // rows, tall tiles (W is re-read from L2 once per row block, so tall tiles
  // keep that traffic small): N <= 64: 256 x 64, BK 64; N <= 128: 256 x 128;
  // N <= 256: 256 x 256.  Fewer rows: 32 x 256 tiles, so the grid still fills
  // the GPU.  N <= 512: 128 x 512 from 32768 rows on, else 64 x 512 (taller
  // accumulators would not fit).
  const bool tall = c.M >= 256 * 256;
  if (tall && c.N <= 64)
    return launch_norm<256, 64, 64, 4, 2, EPI_FULLN>(p, ln, c.gamma != nullptr, 0, s);
  if (tall && c.N <= 128)
    return launch_norm<256, 128, 32, 2, 4, EPI_FULLN>(p, ln, c.gamma != nullptr, 0, s);
  if (tall && c.N <= 256)
    return launch_norm<kBigBM, kBigBN, kBigBK, kBigWM, kBigWN, EPI_FULLN>(p, ln, c.gamma != nullptr, 0, s);
  // K, N <= 256: all of W resident in LDS, eight waves (fng_fulln.hip)
  if (fulln_small_fits(c.N, c.K)) return launch_postnorm_fulln_small(c, ln, s);
  if (c.N <= 256)
    return launch_norm<32, 256, 64, 1, 4, EPI_FULLN>(p, ln, c.gamma != nullptr, 0, s);
  // N <= 512: 128 x 512 tiles of 8 waves (64 x 128 each, the ping-pong mainloop;
  // the 4-stage ring fills the 160 KB of LDS) once there are >= 256 of them
  if (c.M >= 256 * 128)
    return launch_norm<128, 512, 32, 2, 4, EPI_FULLN>(p, ln, c.gamma != nullptr, 0, s);
  return launch_norm<64, 512, 32, 1, 4, EPI_FULLN>(p, ln, c.gamma != nullptr, 0, s);
}

// Split-N placement.  With all column tiles of a row block on one XCD (16 at
// N = 4096), an XCD's tiles of a round read all of W (8 MiB at K = 1024)
// through its 4 MB L2.  Rectangles of 8 column tiles x (slots / 8) row blocks
// per XCD, two or more XCDs sharing a row block, cut the XCD's unique bytes
// per round (4 x 0.5 + 8 x 0.5 MB instead of 2 x 0.5 + 16 x 0.5 MB at
// 16384 x 1024 x 4096).  Only for whole rounds on a grid of 8 equal XCD
// shares; the merge order is by column tile, so the output is bitwise the same.
void splitn_placement(GemmParams& p, int grid, int total, int tn) {
  constexpr int cw = 8;
  if (grid % 8 != 0 || total % grid != 0 || tn % cw != 0) return;
  const int per = grid / 8;
  if (per % cw != 0 || 8 % (tn / cw) != 0) return;
  p.sn_cw = cw;
  p.sn_rh = per / cw;
  p.sn_g = tn / cw;
}

int splitn_feasible(int64_t M, int64_t N) {
  const int cap = max_coresident_grid<kBigBM, kBigBN, kBigBK, kBigWM, kBigWN, EPI_SPLITN, false, false>();
  if (cap <= 0) return 0;
  return splitn_tiles_n(N) <= cap ? 1 : 0;
}

int launch_postnorm_splitn(const GemmCall& c, bool ln, hipStream_t s) {
  GemmParams p = base_params(c);
  p.part = static_cast<float*>(c.part);
  p.cnt = c.cnt;
  p.done = c.done;
  p.status = c.status;
  // co-resident capacity of the variant that runs
  const bool aff = c.gamma != nullptr;
  const int cap =
      ln ? (aff ? max_coresident_grid<kBigBM, kBigBN, kBigBK, kBigWM, kBigWN, EPI_SPLITN, true, true>()
                : max_coresident_grid<kBigBM, kBigBN, kBigBK, kBigWM, kBigWN, EPI_SPLITN, true, false>())
         : (aff ? max_coresident_grid<kBigBM, kBigBN, kBigBK, kBigWM, kBigWN, EPI_SPLITN, false, true>()
                : max_coresident_grid<kBigBM, kBigBN, kBigBK, kBigWM, kBigWN, EPI_SPLITN, false, false>());
  const int tn = (int)splitn_tiles_n(c.N);
  const int total = (int)(splitn_tiles_m(c.M) * tn);
  if (cap <= 0 || tn > cap) return FNG_ERR_UNSUPPORTED;
  // a whole number of row blocks per round, so every wait is on a co-resident peer
  int grid = (cap / tn) * tn;
  if (grid > total) grid = total;
  splitn_placement(p, grid, total, tn);
  // A plain launch: the grid fits the GPU at once (the occupancy above, one
  // workgroup per CU), so every workgroup is dispatched while its peers wait.
  // A cooperative launch would guarantee it even on a GPU shared with other
  // work, but costs ~19 us per call on MI355X (measured); here a peer kept
  // out by other work only delays the wait, which is bounded and reports
  // FNG_ERR_TIMEOUT through the workspace status word.
  return launch_norm<kBigBM, kBigBN, kBigBK, kBigWM, kBigWN, EPI_SPLITN>(p, ln, aff, grid, s);
}

// norm backward by regrouping: dZ = norm_bwd(G @ Wt), whole rows per
// workgroup (the forward full-N tiles) or split-N with the exchange
bool bwd_fulln_tall(int64_t M) { return M >= 256 * 256; }

int launch_norm_bwd_fulln(const GemmCall& c, const NormBwdArgs& b, bool ln, hipStream_t s) {
  GemmParams p = base_params(c);
  p.H = static_cast<const uint16_t*>(b.H);
  p.rstd_in = b.rstd;
  p.h_raw = b.h_raw ? 1 : 0;
  const bool tall = bwd_fulln_tall(c.M);
  // (the forward's 256 x 64 tile with BK 64 fills all 160 KB of LDS; the
  // backward needs room for its row reductions)
  if (tall && c.N <= 64)
    return ln ? launch<256, 64, 32, 2, 2, EPI_BWD_FULLN, true, false>(p, 0, false, s)
              : launch<256, 64, 32, 2, 2, EPI_BWD_FULLN, false, false>(p, 0, false, s);
  if (tall && c.N <= 128)
    return ln ? launch<256, 128, 32, 2, 4, EPI_BWD_FULLN, true, false>(p, 0, false, s)
              : launch<256, 128, 32, 2, 4, EPI_BWD_FULLN, false, false>(p, 0, false, s);
  if (tall && c.N <= 256)
    return ln ? launch<kBigBM, kBigBN, kBigBK, kBigWM, kBigWN, EPI_BWD_FULLN, true, false>(p, 0, false, s)
              : launch<kBigBM, kBigBN, kBigBK, kBigWM, kBigWN, EPI_BWD_FULLN, false, false>(p, 0, false, s);
  // whole 512-column rows in eight waves for tall inputs (the forward's
  // full-N tile), so no row sums cross workgroups
  if (tall && c.N <= 512)
    return ln ? launch<128, 512, 32, 2, 4, EPI_BWD_FULLN, true, false>(p, 0, false, s)
              : launch<128, 512, 32, 2, 4, EPI_BWD_FULLN, false, false>(p, 0, false, s);
  if (c.N <= 256)
    return ln ? launch<32, 256, 64, 1, 4, EPI_BWD_FULLN, true, false>(p, 0, false, s)
              : launch<32, 256, 64, 1, 4, EPI_BWD_FULLN, false, false>(p, 0, false, s);
  return ln ? launch<64, 512, 32, 1, 4, EPI_BWD_FULLN, true, false>(p, 0, false, s)
            : launch<64, 512, 32, 1, 4, EPI_BWD_FULLN, false, false>(p, 0, false, s);
}

int launch_norm_bwd_splitn(const GemmCall& c, const NormBwdArgs& b, bool ln, hipStream_t s) {
  GemmParams p = base_params(c);
  p.H = static_cast<const uint16_t*>(b.H);
  p.rstd_in = b.rstd;
  p.h_raw = b.h_raw ? 1 : 0;
  p.part = static_cast<float*>(c.part);
  p.cnt = c.cnt;
  p.done = c.done;
  p.status = c.status;
  const int cap = ln ? max_coresident_grid<kBigBM, kBigBN, kBigBK, kBigWM, kBigWN, EPI_BWD_SPLITN, true, false>()
                     : max_coresident_grid<kBigBM, kBigBN, kBigBK, kBigWM, kBigWN, EPI_BWD_SPLITN, false, false>();
  const int tn = (int)splitn_tiles_n(c.N);
  const int total = (int)(splitn_tiles_m(c.M) * tn);
  if (cap <= 0 || tn > cap) return FNG_ERR_UNSUPPORTED;
  int grid = (cap / tn) * tn;
  if (grid > total) grid = total;
  splitn_placement(p, grid, total, tn);
  // plain launch of a grid the GPU holds at once, as the forward split-N
  return ln ? launch<kBigBM, kBigBN, kBigBK, kBigWM, kBigWN, EPI_BWD_SPLITN, true, false>(p, grid, false, s)
            : launch<kBigBM, kBigBN, kBigBK, kBigWM, kBigWN, EPI_BWD_SPLITN, false, false>(p, grid, false, s);
}

// weight gradient of the lazy pre-norm: dW [K, N] = X^T diag(rstd) dY with
// X [M, K], dY [M, N]; the kernel's rows are X's columns (K), its
// contraction X's rows (M)
int launch_prenorm_dw(const void* X, const float* rstd, const void* dY, const void* gamma, void* dW, int64_t M,
                      int64_t N, int64_t K, hipStream_t s) {
  GemmCall c{};
  c.X = X;
  c.W = dY;
  c.gamma = gamma;
  c.Y = dW;
  c.M = K;
  c.N = N;
  c.K = M;
  GemmParams p = base_params(c);
  p.rstd_in = rstd;
  const bool g = gamma != nullptr;
  if (small_problem(c)) {
    if (!rstd) return launch<64, 64, 64, 2, 2, EPI_TN, false, false>(p, 0, false, s);
    return g ? launch<64, 64, 64, 2, 2, EPI_DW, false, true>(p, 0, false, s)
             : launch<64, 64, 64, 2, 2, EPI_DW, false, false>(p, 0, false, s);
  }
  if (!rstd) return launch_big<EPI_TN, false>(p, s);
  return g ? launch_big<EPI_DW, true>(p, s) : launch_big<EPI_DW, false>(p, s);
}

int launch_postnorm_partial(const GemmCall& c, bool ln, hipStream_t s) {
  GemmParams p = base_params(c);
  p.part = static_cast<float*>(c.part);
  return ln ? launch<kBigBM, kBigBN, kBigBK, kBigWM, kBigWN, EPI_PARTIAL, true, false>(p, 0, false, s)
            : launch<kBigBM, kBigBN, kBigBK, kBigWM, kBigWN, EPI_PARTIAL, false, false>(p, 0, false, s);
}

}  // namespace fng
