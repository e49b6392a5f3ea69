// Device helpers shared by the WKV kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace wkv {

constexpr int kHead = 64;  // head size N the kernels are specialised for
static_assert(kHead == kHeadSize, "one head size");

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// Four consecutive input elements starting at element `idx`, widened to fp32.
// bf16 reads 8 bytes, fp32 reads 16 bytes; idx must be a multiple of 4.
// Two floats -> packed bf16 pair (round to nearest even): low half = a.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = static_cast<__bf16>(a);
  v[1] = static_cast<__bf16>(b);
  return __builtin_bit_cast(uint32_t, v);
}

// One float -> bf16 bits (round to nearest even).
__device__ __forceinline__ uint16_t bf16_bits(float a) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(a)); }

template <bool BF16>
__device__ __forceinline__ float4 load4(const void *base, long idx) {
  if constexpr (BF16) {
    uint2 p = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(base) + idx);
    return make_float4(bf16_lo(p.x), bf16_hi(p.x), bf16_lo(p.y), bf16_hi(p.y));
  } else {
    return *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + idx);
  }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void *base, long idx) {
  if constexpr (BF16) {
    return bf16_lo(static_cast<const uint16_t *>(base)[idx]);
  } else {
    return static_cast<const float *>(base)[idx];
  }
}

// e^x through the hardware base-2 exponential (v_exp_f32).
__device__ __forceinline__ float fast_exp(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// Per-step decay factor exp(-exp(x)) of the v5/v6 recurrences.
__device__ __forceinline__ float decay_of(float x) { return fast_exp(-fast_exp(x)); }

__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ float4 f4(float a, float b, float c, float d) { return make_float4(a, b, c, d); }

}  // namespace wkv
