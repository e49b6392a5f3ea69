// Matrix-core and cross-lane helpers of the chunked WKV kernels (gfx950).
//
// MFMA operand layout used throughout (v_mfma_f32_32x32x16_bf16, C += A B):
// lane l supplies row l % 32 of A (32 x 16) and column l % 32 of B (16 x 32),
// each as the 8 bf16 values k = 8 (l / 32) .. +7; the 32 x 32 fp32 result
// leaves column n = l % 32 in lane l, rows m = 8 (e / 4) + 4 (l / 32) + e % 4
// in its 16 accumulator elements e.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace wkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

static __device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Split two floats into packed hi and lo bf16 pairs.
static __device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
  hi = pack_bf16(a, b);
  uint32_t h = hi;
  asm("" : "+v"(h));  // widen the packed halves as they are, not by converting a again
  lo = pack_bf16(a - __uint_as_float(h << 16), b - __uint_as_float(h & 0xffff0000u));
}

static __device__ __forceinline__ bf16x8 ld8(const uint16_t *p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(p));
}
static __device__ __forceinline__ bf16x8 ld4x2(const uint16_t *p0, const uint16_t *p1) {
  const uint2 a = *reinterpret_cast<const uint2 *>(p0);
  const uint2 b = *reinterpret_cast<const uint2 *>(p1);
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}
// ds_read_b64_tr_b16: within each group of 16 lanes, source lane 4a + b
// points at 4 consecutive bf16 values; result lane i receives element i % 4
// of source lanes 4e + i / 4 (e = 0..3).  With source lane 4a + b at
// &M[t0 + a][c0 + 4b] of a row-major M, lane i gets M[t0 + e][c0 + i]: a
// column of four rows, i.e. a transposed read.
typedef short v4i16 __attribute__((ext_vector_type(4)));
static __device__ __forceinline__ uint2 ld_tr(const uint16_t *p) {
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)(p));
  return __builtin_bit_cast(uint2, r);
}
static __device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(bf16x8, make_uint4(a, b, c, d));
}

static __device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
static __device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Cross-lane helpers without address arithmetic: quad permutes on DPP, other
// xor distances inside 32-lane groups on the LDS swizzle crossbar.
static __device__ __forceinline__ float xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
static __device__ __forceinline__ float xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}
static __device__ __forceinline__ float mirror8(float x) {  // lane i of each 8-lane group reads lane 7 - i
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));
}
template <int M>
static __device__ __forceinline__ float xor_swz(float x) {  // M in {4, 8, 16}
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1F | (M << 10)));
}

// A wave-uniform 64-bit value the compiler cannot rewrite into per-lane
// induction variables (keeps per-chunk bases in scalar registers).
static __device__ __forceinline__ long uniform64(long x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((unsigned long)x >> 32));
  return (long)(((unsigned long)hi << 32) | lo);
}

// Keeps the compiler from moving work on a prefetched register above this
// point, so the wait for the load lands here.
static __device__ __forceinline__ void pin(uint32_t &x) { asm volatile("" : "+v"(x)); }

}  // namespace wkv
