// Few-token WKV v6 varlen calls: T = 1 decode steps, or a token budget spread
// over many slots.  The recurrence (the token-sequential scan's):
//   y_t[j] = sum_i r_t[i] (S[i][j] + u[i] k_t[i] v_t[j])
//   S[i][j] <- d_t[i] S[i][j] + k_t[i] v_t[j],   d_t[i] = exp(-exp(w_t[i]))
// (the rwkv_ops page's RWKV6_OP call with state_map; the standard RWKV-6
// recurrence).
//
// Such calls are bound by streaming the 16 KiB state of every (slot, head) in
// and out.  Each (slot, head) gets one wave: lane j holds column j of the
// state (S[0..63][j]), so every state load and store is a fully coalesced
// 256-byte row, the output y_t[j] = sum_i r_t[i] S[i][j] +
// (r_t . (u * k_t)) v_t[j] is a sum inside the lane, and the row factors
// r_t[i], k_t[i], d_t[i] reach all lanes through LDS, four at a time as
// broadcast reads.  The state is requested as soon as the slot's row is known
// (clamped; an invalid row is rejected before anything is written), and the
// slot offset is a wave reduction.
#include "common.hpp"
#include "kernels.hpp"
#include "wkv.h"

namespace wkv {
namespace {

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
  return x;
}
__device__ __forceinline__ float wave_sum_f(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

template <bool BF16>
__global__ void __launch_bounds__(64) wkv6_varlen_short_kernel(ScanParams p) {
  const int h = blockIdx.x;
  const int unit = blockIdx.y;
  const int lane = threadIdx.x;  // value column j for the state and y; channel i for r, k, d
  const long C = (long)p.H * kHead;

  const int my_len = p.lengths[unit];
  const int my_row = p.state_map ? p.state_map[unit] : unit;
  // the other slots' lengths and rows (64 per pass) first, then the state column of the
  // (clamped) row, so that waiting for the former does not wait for the latter
  int sum = 0, bad = 0, dup = 0;
  {
    const bool in = lane < p.units;
    const int L = in ? p.lengths[lane] : 0;
    const int m = (p.state_map && in) ? p.state_map[lane] : 0;
    if (lane < unit) { sum = L; bad = L < 0; }
    dup = p.state_map && in && lane != unit && m == my_row;
  }
  const int row_c = min(max(my_row, 0), p.n_state - 1);
  float s[kHead];
  {
    const float *sp = p.state_in + ((long)row_c * p.H + h) * (kHead * kHead) + lane;
#pragma unroll
    for (int i = 0; i < kHead; ++i) s[i] = sp[i * kHead];
  }
  for (int i = lane + 64; i < p.units; i += 64) {
    const int L = p.lengths[i];
    if (i < unit) { sum += L; bad |= (L < 0); }
    if (p.state_map && i != unit && p.state_map[i] == my_row) dup = 1;
  }
  const int off = wave_sum_i(sum);
  const bool any_bad = __any(bad), any_dup = __any(dup);
  int status = 0;
  if (my_len < 0 || my_len > p.max_len || any_bad) status |= WKV_DEV_BAD_LENGTH;
  if (my_row < 0 || my_row >= p.n_state) status |= WKV_DEV_BAD_STATE_MAP;
  if (any_dup) status |= WKV_DEV_DUPLICATE_ROW;
  if (!(status & WKV_DEV_BAD_LENGTH) && (long)off + my_len > (long)p.total_tokens)
    status |= WKV_DEV_TOKEN_OVERFLOW;
  if (status) {
    if (lane == 0 && p.dev_status) atomicOr(p.dev_status, status);
    return;
  }
  const int ntok = my_len;
  const float ui = p.u[h * kHead + lane];
  // the token's row factors r[i], k[i], d[i], read back by every lane as 16-byte broadcasts
  __shared__ __align__(16) float s_r[kHead], s_k[kHead], s_d[kHead];

  // token rows one token ahead
  const long e0 = (long)off * C + h * kHead + lane;
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
    __syncthreads();  // one wave: orders the row factors' stores before the broadcast reads
#pragma unroll
    for (int i4 = 0; i4 < kHead / 4; ++i4) {
      const float4 r4 = *reinterpret_cast<const float4 *>(&s_r[4 * i4]);
      const float4 k4 = *reinterpret_cast<const float4 *>(&s_k[4 * i4]);
      const float4 d4 = *reinterpret_cast<const float4 *>(&s_d[4 * i4]);
      const float rr[4] = {r4.x, r4.y, r4.z, r4.w}, kk[4] = {k4.x, k4.y, k4.z, k4.w};
      const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // decay in place, then add k v in place: both update the state register itself
        yj = fmaf(rr[e], s[4 * i4 + e], yj);
        s[4 * i4 + e] = fmaf(kk[e], vj, s[4 * i4 + e] * dd[e]);
      }
    }
    __syncthreads();  // the reads finish before the next token's factors are stored
    if (p.y_bf16) static_cast<uint16_t *>(p.y)[e] = bf16_bits(yj);
    else static_cast<float *>(p.y)[e] = yj;
  }

  if (p.state_out) {
    if (ntok == 0 && p.state_out == p.state_in) return;  // empty slot: untouched
    float *sp = p.state_out + ((long)my_row * p.H + h) * (kHead * kHead) + lane;
#pragma unroll
    for (int i = 0; i < kHead; ++i) sp[i * kHead] = s[i];
  }
}

}  // namespace

hipError_t launch_wkv6_varlen_short(const ScanParams &p, bool bf16, hipStream_t s) {
  dim3 grid(p.H, p.units);
  if (bf16) hipLaunchKernelGGL((wkv6_varlen_short_kernel<true>), grid, dim3(64), 0, s, p);
  else hipLaunchKernelGGL((wkv6_varlen_short_kernel<false>), grid, dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace wkv
