// The few-token v6 recurrence of one (slot, head) on one wave, shared by the few-token
// varlen kernel and the varlen scan kernel (which hands it the slots of a call that
// consume at most kShortMax tokens).  The recurrence (the token-sequential scan's):
//   y_t[j] = sum_i r_t[i] (S[i][j] + u[i] k_t[i] v_t[j])
//   S[i][j] <- d_t[i] S[i][j] + k_t[i] v_t[j],   d_t[i] = exp(-exp(w_t[i]))
// Lane j holds column j of the state (S[0..63][j]), so every state load and store is a
// fully coalesced 256-byte row, and y_t[j] is a sum inside the lane; the row factors
// r_t[i], k_t[i], d_t[i] reach all lanes through LDS, four at a time as broadcast reads.
// Token rows are read one token ahead.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace wkv {

static __device__ __forceinline__ float wave_sum_f(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

// LDS the routine needs: three rows of 64 floats (r, k, d of one token), 16-byte aligned.
constexpr int kShortLdsFloats = 3 * kHead;

// s: this lane's state column, already loaded; off: the slot's first packed token row;
// row_out: the state row written at the end (nothing when the slot is empty and the state
// is updated in place).  Only the calling wave may reach this function's barriers (it is
// alone in its workgroup, or the other waves have exited).
template <bool BF16>
__device__ __forceinline__ void short_slot_wave(const ScanParams &p, int h, int lane, long off, int ntok,
                                                int row_out, float (&s)[kHead], float *lds) {
  const long C = (long)p.H * kHead;
  const float ui = p.u[h * kHead + lane];
  float *s_r = lds, *s_k = lds + kHead, *s_d = lds + 2 * kHead;
  // token rows one token ahead
  const long e0 = off * C + h * kHead + lane;
  float nr = 0.f, nk = 0.f, nv = 0.f, nx = 0.f;
  if (ntok > 0) {
    nr = load1<BF16>(p.r, e0); nk = load1<BF16>(p.k, e0); nv = load1<BF16>(p.v, e0); nx = load1<BF16>(p.w, e0);
  }
  for (int t = 0; t < ntok; ++t) {
    const long e = e0 + (long)t * C;
    const float rj = nr, kj = nk, vj = nv, dj = decay_of(nx);
    if (t + 1 < ntok) {
      nr = load1<BF16>(p.r, e + C); nk = load1<BF16>(p.k, e + C); nv = load1<BF16>(p.v, e + C); nx = load1<BF16>(p.w, e + C);
    }
    float yj = wave_sum_f(rj * ui * kj) * vj;  // bonus: (r_t . (u * k_t)) v_t[j]
    s_r[lane] = rj;
    s_k[lane] = kj;
    s_d[lane] = dj;
    __syncthreads();  // orders the row factors' stores before the broadcast reads
#pragma unroll
    for (int i4 = 0; i4 < kHead / 4; ++i4) {
      const float4 r4 = *reinterpret_cast<const float4 *>(&s_r[4 * i4]);
      const float4 k4 = *reinterpret_cast<const float4 *>(&s_k[4 * i4]);
      const float4 d4 = *reinterpret_cast<const float4 *>(&s_d[4 * i4]);
      const float rr[4] = {r4.x, r4.y, r4.z, r4.w}, kk[4] = {k4.x, k4.y, k4.z, k4.w};
      const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        // decay in place, then add k v in place: both update the state register itself
        yj = fmaf(rr[e4], s[4 * i4 + e4], yj);
        s[4 * i4 + e4] = fmaf(kk[e4], vj, s[4 * i4 + e4] * dd[e4]);
      }
    }
    __syncthreads();  // the reads finish before the next token's factors are stored
    if (p.y_bf16) static_cast<uint16_t *>(p.y)[e] = bf16_bits(yj);
    else static_cast<float *>(p.y)[e] = yj;
  }

  if (p.state_out) {
    if (ntok == 0 && p.state_out == p.state_in) return;  // empty slot: untouched
    float *sp = p.state_out + ((long)row_out * p.H + h) * (kHead * kHead) + lane;
#pragma unroll
    for (int i = 0; i < kHead; ++i) sp[i * kHead] = s[i];
  }
}

}  // namespace wkv
