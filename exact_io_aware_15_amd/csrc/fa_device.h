// Device-side helpers shared by the gfx950 attention kernels: vector types,
// bf16 packing and wave64 cross-lane reductions built on DPP and the gfx950
// permlane swaps (no LDS round trip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Reinterpret one 32-bit word as two bf16.  Takes the word by value: a bit cast
// applied directly to an element of a vector register is lowered as a cast of
// element 0, so vector elements must be copied out first.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

// Two fp32 -> two bf16 (RNE) in one v_cvt_pk_bf16_f32; a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ---- debug-sync build ----------------------------------------------------------
// Built with FA_DEBUG_SYNC=1 (libfa_debugsync.so), the tiled kernels wait for every
// HBM -> LDS copy and fence it with a workgroup barrier as soon as it is issued, and
// wait for every group of LDS fragment reads before the next stage.  The fast build
// relies on its per-tile waits alone; the two builds must give bitwise equal results,
// which a GPU test checks.
#ifndef FA_DEBUG_SYNC
#define FA_DEBUG_SYNC 0
#endif
// After a workgroup-uniform copy issue point: this wave's copies have landed, and so
// have every other wave's (barrier).
__device__ __forceinline__ void debug_copy_fence() {
  if constexpr (FA_DEBUG_SYNC) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  }
}
// After a stage of LDS reads (per wave): every read has returned.
__device__ __forceinline__ void debug_read_fence() {
  if constexpr (FA_DEBUG_SYNC) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---- DPP / permlane cross-lane moves ------------------------------------------
// DPP control words (gfx9): quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E,
// row_half_mirror = 0x141, row_ror:8 = 0x128.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Value held by lane (l ^ 16): permlane16_swap exchanges odd/even 16-lane rows.
__device__ __forceinline__ float xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // After the swap, r[0] holds rows (0,0,2,2) and r[1] rows (1,1,3,3) of x.
  const int lane = __lane_id();
  return __uint_as_float(((lane >> 4) & 1) ? r[0] : r[1]);
}
// Value held by lane (l ^ 32).
__device__ __forceinline__ float xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // r[0] = (lo, lo), r[1] = (hi, hi) halves of x.
  const int lane = __lane_id();
  return __uint_as_float((lane >> 5) ? r[0] : r[1]);
}

// Whole-pair reductions: after a swap of x with itself, r[0] and r[1] hold the two
// halves being combined, so op(r[0], r[1]) is the reduced value in every lane.
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Reductions over the 8 lanes {l ^ 1, l ^ 2, l ^ 4} (aligned groups of 8).
__device__ __forceinline__ float sum8(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  return x;
}
// Reductions across the lanes that share (l % 8): xor 8, 16, 32.
__device__ __forceinline__ float sum_stride8(float x) {
  x += dpp<0x128>(x);
  x = sum_xor16(x);
  return sum_xor32(x);
}
__device__ __forceinline__ float max_stride8(float x) {
  x = fmaxf(x, dpp<0x128>(x));
  x = max_xor16(x);
  return max_xor32(x);
}

}  // namespace fa
