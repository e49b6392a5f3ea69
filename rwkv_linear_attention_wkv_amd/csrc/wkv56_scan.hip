// Token-sequential WKV v5 / v6 scan on the vector ALUs (dense rows, varlen
// slots and T = 1 decode share this kernel).
//
// Recurrence per (row or slot, head), with S indexed [key i][value j]:
//   y_t[j] = sum_i r_t[i] (S[i][j] + u[i] k_t[i] v_t[j])
//   S[i][j] <- d_t[i] S[i][j] + k_t[i] v_t[j],   d_t[i] = exp(-exp(w_t[i]))
// (the rwkv_ops page's RWKV6_OP call: r, k, v, w, u, init_state, state_map ->
// y, y_state; the standard RWKV-5/6 recurrence).
//
// Work decomposition: one 256-thread workgroup per (head, unit).  Thread
// (rg, cq) owns the 4x4 block of the fp32 state with rows 4rg..4rg+3 and
// columns 4cq..4cq+3 in registers for the whole call, so the state is read
// once and written once.  Tokens are staged 16 at a time through LDS as fp32
// (decay already exponentiated); each thread forms partial outputs over its
// four key rows, the four row groups of a wave are summed with lane
// shuffles, and the four waves are summed through LDS in a fixed order, so
// results are deterministic.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "wkv.h"

namespace wkv {
namespace {

constexpr int kThreads = 256;
constexpr int kTB = 16;  // tokens staged per block

template <bool V6, bool BF16, bool VARLEN>
__global__ void __launch_bounds__(kThreads) wkv56_scan_kernel(ScanParams p) {
  const int h = blockIdx.x;
  const int unit = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rg = tid >> 4;  // key rows 4rg .. 4rg+3
  const int cq = tid & 15;  // value columns 4cq .. 4cq+3
  const long C = (long)p.H * kHead;

  __shared__ float4 s_r[kTB][16];
  __shared__ float4 s_k[kTB][16];
  __shared__ float4 s_d[kTB][16];
  __shared__ float4 s_v[kTB][16];
  __shared__ float4 s_y[kTB][4][16];
  __shared__ int s_meta[3];

  long tok0;
  int ntok;
  int row_in = -1;
  int row_out;

  if constexpr (VARLEN) {
    // Offset of this slot = sum of earlier lengths; validate the slot.
    if (tid == 0) { s_meta[0] = 0; s_meta[1] = 0; s_meta[2] = 0; }
    __syncthreads();
    const int my_row = p.state_map ? p.state_map[unit] : unit;
    int sum = 0, bad = 0, dup = 0;
    for (int i = tid; i < p.units; i += kThreads) {
      const int L = p.lengths[i];
      if (i < unit) { sum += L; bad |= (L < 0); }
      if (p.state_map && i != unit && p.state_map[i] == my_row) dup = 1;
    }
    if (sum) atomicAdd(&s_meta[0], sum);
    if (bad) atomicOr(&s_meta[1], 1);
    if (dup) atomicOr(&s_meta[2], 1);
    __syncthreads();
    const int off = s_meta[0];
    const int my_len = p.lengths[unit];
    int status = 0;
    if (my_len < 0 || my_len > p.max_len || s_meta[1]) status |= WKV_DEV_BAD_LENGTH;
    if (my_row < 0 || my_row >= p.n_state) status |= WKV_DEV_BAD_STATE_MAP;
    if (s_meta[2]) status |= WKV_DEV_DUPLICATE_ROW;
    if (!(status & WKV_DEV_BAD_LENGTH) && (long)off + my_len > (long)p.total_tokens)
      status |= WKV_DEV_TOKEN_OVERFLOW;
    if (status) {
      if (tid == 0 && p.dev_status) atomicOr(p.dev_status, status);
      return;
    }
    tok0 = off;
    ntok = my_len;
    row_in = my_row;
    row_out = my_row;
  } else {
    tok0 = (long)unit * p.T;
    ntok = p.T;
    row_out = unit;
    if (p.state_in) {
      row_in = p.state_map ? p.state_map[unit] : (p.n_state == 1 ? 0 : unit);
      if (row_in < 0 || row_in >= p.n_state) {
        if (tid == 0 && p.dev_status) atomicOr(p.dev_status, WKV_DEV_BAD_STATE_MAP);
        return;
      }
    }
  }

  // ---- state block in registers
  float s[4][4];
  if (row_in >= 0 && p.state_in) {
    const float *sp = p.state_in + ((long)row_in * p.H + h) * (kHead * kHead);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float4 t = *reinterpret_cast<const float4 *>(sp + (4 * rg + a) * kHead + 4 * cq);
      s[a][0] = t.x; s[a][1] = t.y; s[a][2] = t.z; s[a][3] = t.w;
    }
  } else {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) s[a][c] = 0.f;
  }

  float ur[4], dstat[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    ur[a] = p.u[h * kHead + 4 * rg + a];
    dstat[a] = V6 ? 0.f : decay_of(static_cast<const float *>(p.w)[h * kHead + 4 * rg + a]);
  }

  for (int t0 = 0; t0 < ntok; t0 += kTB) {
    const int nb = min(kTB, ntok - t0);
    {  // stage kTB tokens of this head as fp32
      const int tt = tid >> 4, q = tid & 15;
      if (tt < nb) {
        const long e = (tok0 + t0 + tt) * C + h * kHead + 4 * q;
        s_r[tt][q] = load4<BF16>(p.r, e);
        s_k[tt][q] = load4<BF16>(p.k, e);
        s_v[tt][q] = load4<BF16>(p.v, e);
        if constexpr (V6) {
          const float4 x = load4<BF16>(p.w, e);
          s_d[tt][q] = f4(decay_of(x.x), decay_of(x.y), decay_of(x.z), decay_of(x.w));
        }
      }
    }
    __syncthreads();

    float yp[kTB][4];
#pragma unroll
    for (int tt = 0; tt < kTB; ++tt) {
      if (tt < nb) {
        const float4 r4 = s_r[tt][rg], k4 = s_k[tt][rg], v4 = s_v[tt][cq];
        const float rr[4] = {r4.x, r4.y, r4.z, r4.w};
        const float kk[4] = {k4.x, k4.y, k4.z, k4.w};
        const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
        float dd[4];
        if constexpr (V6) {
          const float4 d4 = s_d[tt][rg];
          dd[0] = d4.x; dd[1] = d4.y; dd[2] = d4.z; dd[3] = d4.w;
        } else {
#pragma unroll
          for (int a = 0; a < 4; ++a) dd[a] = dstat[a];
        }
        float ruk = 0.f;
#pragma unroll
        for (int a = 0; a < 4; ++a) ruk = fmaf(rr[a] * ur[a], kk[a], ruk);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float acc = ruk * vv[c];
#pragma unroll
          for (int a = 0; a < 4; ++a) acc = fmaf(rr[a], s[a][c], acc);
          yp[tt][c] = acc;
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int c = 0; c < 4; ++c) s[a][c] = fmaf(dd[a], s[a][c], kk[a] * vv[c]);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) yp[tt][c] = 0.f;
      }
    }
    // sum the wave's four row groups (lanes differing in bits 4 and 5)
#pragma unroll
    for (int tt = 0; tt < kTB; ++tt)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float x = yp[tt][c];
        x += __shfl_xor(x, 16);
        x += __shfl_xor(x, 32);
        yp[tt][c] = x;
      }
    if (lane < 16) {
#pragma unroll
      for (int tt = 0; tt < kTB; ++tt)
        if (tt < nb) s_y[tt][wave][cq] = f4(yp[tt][0], yp[tt][1], yp[tt][2], yp[tt][3]);
    }
    __syncthreads();
    {  // sum the four waves in a fixed order and store fp32 outputs
      const int tt = tid >> 4, q = tid & 15;
      if (tt < nb) {
        const float4 a0 = s_y[tt][0][q], a1 = s_y[tt][1][q], a2 = s_y[tt][2][q], a3 = s_y[tt][3][q];
        const float4 o = f4(((a0.x + a1.x) + a2.x) + a3.x, ((a0.y + a1.y) + a2.y) + a3.y,
                            ((a0.z + a1.z) + a2.z) + a3.z, ((a0.w + a1.w) + a2.w) + a3.w);
        *reinterpret_cast<float4 *>(p.y + (tok0 + t0 + tt) * C + h * kHead + 4 * q) = o;
      }
    }
    // The next staging writes s_r..s_v, which nobody reads any more; the
    // next write of s_y happens after the next staging barrier.
  }

  if (p.state_out) {
    if (VARLEN && ntok == 0 && p.state_out == p.state_in) return;  // empty slot: untouched
    float *sp = p.state_out + ((long)row_out * p.H + h) * (kHead * kHead);
#pragma unroll
    for (int a = 0; a < 4; ++a)
      *reinterpret_cast<float4 *>(sp + (4 * rg + a) * kHead + 4 * cq) = f4(s[a][0], s[a][1], s[a][2], s[a][3]);
  }
}

// Varlen calls whose slots consume only a few tokens (T = 1 decode steps, or a
// token budget spread over many slots) are bound by streaming the 16 KiB
// state of every (slot, head) in and out.  This variant gives each
// (slot, head) one wave: lane j holds column j of the state (S[0..63][j]), so
// every state load and store is a fully coalesced 256-byte row, the output
// y_t[j] = sum_i r_t[i] S[i][j] + (r_t . (u * k_t)) v_t[j] is a sum inside the
// lane, and the row factors r_t[i], k_t[i], d_t[i] reach all lanes as scalar
// operands (v_readlane).  No workgroup barrier: the state is requested as soon
// as the slot's row is known (clamped; an invalid row is rejected before
// anything is written), and the slot offset is a wave reduction.
constexpr int kShortMax = 8;

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
#pragma unroll
    for (int i = 0; i < kHead; ++i) {
      const float ri = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rj), i));
      const float ki = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(kj), i));
      const float di = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dj), i));
      yj = fmaf(ri, s[i], yj);
      s[i] = fmaf(di, s[i], ki * vj);
    }
    p.y[e] = yj;
  }

  if (p.state_out) {
    if (ntok == 0 && p.state_out == p.state_in) return;  // empty slot: untouched
    float *sp = p.state_out + ((long)my_row * p.H + h) * (kHead * kHead) + lane;
#pragma unroll
    for (int i = 0; i < kHead; ++i) sp[i * kHead] = s[i];
  }
}

template <bool V6, bool BF16, bool VARLEN>
hipError_t launch(const ScanParams &p, hipStream_t s) {
  dim3 grid(p.H, p.units);
  hipLaunchKernelGGL((wkv56_scan_kernel<V6, BF16, VARLEN>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_wkv56_scan(const ScanParams &p, bool v6, bool bf16, bool varlen, hipStream_t s) {
  if (varlen) {
    // varlen always carries a per-token decay
    if (p.max_len <= kShortMax) {
      dim3 grid(p.H, p.units);
      if (bf16) hipLaunchKernelGGL((wkv6_varlen_short_kernel<true>), grid, dim3(64), 0, s, p);
      else hipLaunchKernelGGL((wkv6_varlen_short_kernel<false>), grid, dim3(64), 0, s, p);
      return hipGetLastError();
    }
    return bf16 ? launch<true, true, true>(p, s) : launch<true, false, true>(p, s);
  }
  if (v6) return bf16 ? launch<true, true, false>(p, s) : launch<true, false, false>(p, s);
  return bf16 ? launch<false, true, false>(p, s) : launch<false, false, false>(p, s);
}

}  // namespace wkv
