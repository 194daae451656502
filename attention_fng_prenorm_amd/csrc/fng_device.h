// Device-side building blocks shared by the fng kernels (gfx950 / CDNA4).
//
// MFMA lane layouts used throughout (v_mfma_f32_32x32x16_{bf16,f16}):
//   operand A (32 x 16): lane l holds A[l % 32][8 * (l / 32) + j], j = 0..7
//   operand B (16 x 32): lane l holds B[8 * (l / 32) + j][l % 32], j = 0..7
//   result  D (32 x 32): lane l, register r holds
//                        D[8 * (r / 4) + 4 * (l / 32) + (r % 4)][l % 32]
// ds_read_b64_tr_b16: in each group of 16 lanes, lanes 4r..4r+3 address row r
// (4 consecutive 16-bit elements each, 16 columns in total); lane i of the
// group receives column i of rows 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fng {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define FNG_LDS __attribute__((address_space(3)))

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// buffer resources: hardware range checking turns out-of-range loads into 0
// ---------------------------------------------------------------------------
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // dword3 0x00020000: raw (untyped) 32-bit data format, as used for gfx9 buffers.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// the same, for values that are uniform across the wave but computed in vector
// registers: readfirstlane keeps the descriptor in scalar registers (a buffer
// descriptor held in vector registers makes every access a waterfall loop)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_uniform(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo),
                   __builtin_amdgcn_readfirstlane(bytes));
}

__device__ __forceinline__ u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ u32x2_t buffer_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// two fp32 -> packed bf16x2, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// two fp32 -> packed fp16x2, round to nearest even
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  f16x2_t v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// packed bf16x2 word -> packed fp16x2 word (exact for |x| in fp16 normal range)
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return pack_f16(bf16lo(w), bf16hi(w));
}

// ---------------------------------------------------------------------------
// MFMA wrappers
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16_t mfma_bf16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma_f16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// sum of squares of 8 bf16 held in a 16-byte vector, accumulated into acc:
// one v_dot2_f32_bf16 per pair (products exact in fp32, fp32 accumulation;
// measured on gfx950 to agree with an fp32 FMA chain to 3e-6 relative over
// 4096 terms).  Each word is first copied to a scalar: a bit-cast applied
// directly to an element of the vector was compiled as element 0 for every
// element (this toolchain), which silently drops 3/4 of the sum.
__device__ __forceinline__ float sumsq_bf16x8(u32x4_t v, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = v[i];
    const bf16x2_t p = __builtin_bit_cast(bf16x2_t, w);
    acc = __builtin_amdgcn_fdot2_f32_bf16(p, p, acc, false);
  }
  return acc;
}

// the same into two accumulators (words 0, 2 -> a0; 1, 3 -> a1)
__device__ __forceinline__ void sumsq_bf16x8_2(u32x4_t v, float& a0, float& a1) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = v[i];
    const bf16x2_t p = __builtin_bit_cast(bf16x2_t, w);
    if (i % 2 == 0) a0 = __builtin_amdgcn_fdot2_f32_bf16(p, p, a0, false);
    else a1 = __builtin_amdgcn_fdot2_f32_bf16(p, p, a1, false);
  }
}

// the same for the plain sum (dots with ones; exact products, fp32 accumulation)
__device__ __forceinline__ void sum_bf16x8_2(u32x4_t v, float& a0, float& a1) {
  const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = v[i];
    const bf16x2_t p = __builtin_bit_cast(bf16x2_t, w);
    if (i % 2 == 0) a0 = __builtin_amdgcn_fdot2_f32_bf16(p, ones, a0, false);
    else a1 = __builtin_amdgcn_fdot2_f32_bf16(p, ones, a1, false);
  }
}

// ---------------------------------------------------------------------------
// LDS access
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4_t lds_read16(const FNG_LDS char* p) {
  return *reinterpret_cast<const FNG_LDS u32x4_t*>(p);
}
__device__ __forceinline__ void lds_write16(FNG_LDS char* p, u32x4_t v) {
  *reinterpret_cast<FNG_LDS u32x4_t*>(p) = v;
}
// transposing read of 4 x 16-bit (see header comment)
__device__ __forceinline__ u32x2_t lds_read_tr16(const FNG_LDS char* p) {
  s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<FNG_LDS s16x4_t*>(const_cast<FNG_LDS char*>(p)));
  return __builtin_bit_cast(u32x2_t, v);
}

// ---------------------------------------------------------------------------
// HBM -> LDS copies and the waits around them
// ---------------------------------------------------------------------------
// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// workgroup barrier for LDS hand-offs: waits for this wave's LDS operations
// only (global copies are waited for explicitly with wait_vmcnt), and is a
// compiler memory barrier
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// HBM -> LDS copy of 16 bytes per lane (buffer_load_dwordx4 ... lds): lane l
// writes LDS bytes [base + 16 l, +16).  Written as inline asm so that the
// compiler does not model the LDS write: it would otherwise wait for every
// copy in flight before each LDS read.  The ring's explicit vmcnt waits and
// barriers are the synchronization.  The descriptor words and the LDS base
// are wave-uniform scalars.
typedef int i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4_t dma_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return i32x4_t{(int)__builtin_amdgcn_readfirstlane((uint32_t)b),
                 (int)(__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) & 0xffff),
                 (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000};
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(i32x4_t rsrc, const FNG_LDS char* lds_wave_base, uint32_t off) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds_wave_base));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(m0), "v"(off), "s"(rsrc) : "memory", "m0");
}
// the same with a wave-uniform byte offset in the instruction's scalar offset
// field (the buffer range check applies to the sum)
__device__ __forceinline__ void dma16_so(i32x4_t rsrc, const FNG_LDS char* lds_wave_base, uint32_t off,
                                         uint32_t soff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds_wave_base));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(m0), "v"(off), "s"(rsrc), "s"(soff) : "memory", "m0");
}
#pragma clang diagnostic pop

constexpr uint32_t kOOB = 0x80000000u;  // beyond every buffer range: DMA writes zeros

// ---------------------------------------------------------------------------
// cross-lane reductions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float xor_sum(float v, int mask) { return v + __shfl_xor(v, mask); }
__device__ __forceinline__ float xor_max(float v, int mask) { return fmaxf(v, __shfl_xor(v, mask)); }

// combine lane l with lane l ^ 32 without going through LDS
// (v_permlane32_swap exchanges the upper half of one operand with the lower
// half of the other; with both operands equal, the two results hold v[l] and
// v[l ^ 32], so both lanes of a pair get the same combined value)
__device__ __forceinline__ float half_swap_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float half_swap_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ---------------------------------------------------------------------------
// workgroup -> tile remap so that consecutive logical tiles run on one XCD.
// Workgroups are dispatched round-robin over the 8 XCDs; slot s of XCD x
// receives logical index x * (G / 8) + s.  A bijection on [0, G).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t xcd_remap(uint32_t wg, uint32_t G) {
  const uint32_t per = G / 8u;
  if (wg < per * 8u) return (wg % 8u) * per + wg / 8u;
  return wg;
}

}  // namespace fng
