// Shared helpers of the DSpark HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>

#include "../../include/dspark.h"

namespace dspark {

// ------------------------------------------------------------------ vectors
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// bf16 halves of a packed 32-bit word, as exact float32 values.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Two float32 values -> packed bf16 pair {b : a}, round to nearest even, in
// one v_cvt_pk_bf16_f32.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// gfx950 bf16 matrix-core products (fp32 accumulate).
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Byte permute: result byte i = byte sel[i] of the 8-byte value {hi:lo}.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// Low bf16 of a and low bf16 of b packed as {b.lo : a.lo}; same for high halves.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return perm(b, a, 0x07060302u); }

// Order-preserving map float -> uint32 (larger float -> larger integer);
// -0 is folded onto +0 so that equal values compare equal.
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float float_from_order_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// (value, index) -> 64-bit key whose maximum is the largest value with the
// lowest index among ties.
__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t idx) {
  return ((uint64_t)float_order_key(v) << 32) | (uint64_t)(0xffffffffu - idx);
}
__device__ __forceinline__ uint32_t argmax_key_index(uint64_t k) {
  return 0xffffffffu - (uint32_t)(k & 0xffffffffu);
}

// DPP lane moves inside rows of 16 lanes (gfx9 encodings).
constexpr int kDppQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppRowMirror = 0x140;  // lane 15 - l inside each row
constexpr int kDppHalfMirror = 0x141; // lane 7 - l inside each half row
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, false));
}

__device__ __forceinline__ void status_or(int32_t* st, int32_t bits) {
  if (st) atomicOr(st, bits);
}

// Wait until at most N of this wave's vector memory operations are pending
// (they complete in issue order).  Needed for global -> LDS copies, which the
// compiler does not track against later LDS reads.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Workgroup barrier without the waits __syncthreads() adds: the caller has
// made its own writes visible (wait_vmcnt for copies into LDS).
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace dspark

// ---------------------------------------------------------------- host side
namespace dspark_host {

// Record the reason of a failure for dspark_last_error() and return `code`.
int fail(int code, const char* fmt, ...);
// Clear the thread's last error and return DSPARK_OK.
int ok();
// Check the last HIP launch; returns DSPARK_OK or DSPARK_ERR_HIP.
int check_launch(const char* what);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace dspark_host
