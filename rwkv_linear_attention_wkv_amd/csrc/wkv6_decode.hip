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
#include "varlen_short.hpp"
#include "wkv.h"

namespace wkv {
namespace {

__device__ __forceinline__ long wave_sum_l(long x) {
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
  // 64-bit offset sum (65535 slots of up to 2^31 - 1 tokens cannot wrap it); one
  // invalid length anywhere rejects every slot, whose offsets it makes meaningless
  long sum = 0;
  int bad = 0, dup = 0;
  {
    const bool in = lane < p.units;
    const int L = in ? p.lengths[lane] : 0;
    const int m = (p.state_map && in) ? p.state_map[lane] : 0;
    if (lane < unit) sum = L;
    bad = (L < 0) | (L > p.max_len);
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
    if (i < unit) sum += L;
    bad |= (L < 0) | (L > p.max_len);
    if (p.state_map && i != unit && p.state_map[i] == my_row) dup = 1;
  }
  const long off = wave_sum_l(sum);
  const bool any_bad = __any(bad), any_dup = __any(dup);
  int status = 0;
  if (my_len < 0 || my_len > p.max_len || any_bad) status |= WKV_DEV_BAD_LENGTH;
  if (my_row < 0 || my_row >= p.n_state) status |= WKV_DEV_BAD_STATE_MAP;
  if (any_dup) status |= WKV_DEV_DUPLICATE_ROW;
  if (!(status & WKV_DEV_BAD_LENGTH) && off + my_len > (long)p.total_tokens)
    status |= WKV_DEV_TOKEN_OVERFLOW;
  if (status) {
    if (lane == 0 && p.dev_status) atomicOr(p.dev_status, status);
    return;
  }
  __shared__ __align__(16) float lds[kShortLdsFloats];
  short_slot_wave<BF16>(p, h, lane, off, my_len, my_row, s, lds);
}

}  // namespace

hipError_t launch_wkv6_varlen_short(const ScanParams &p, bool bf16, hipStream_t s) {
  dim3 grid(p.H, p.units);
  if (bf16) hipLaunchKernelGGL((wkv6_varlen_short_kernel<true>), grid, dim3(64), 0, s, p);
  else hipLaunchKernelGGL((wkv6_varlen_short_kernel<false>), grid, dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace wkv
