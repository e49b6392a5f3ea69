// Token-sequential WKV v5 / v6 scan on the vector ALUs (dense rows, varlen
// slots and T = 1 decode share this kernel).
//
// Recurrence per (row or slot, head), with S indexed [key i][value j]:
//   y_t[j] = sum_i r_t[i] (S[i][j] + u[i] k_t[i] v_t[j])
//   S[i][j] <- d_t[i] S[i][j] + k_t[i] v_t[j],   d_t[i] = exp(-exp(w_t[i]))
// (the rwkv_ops page's RWKV6_OP call: r, k, v, w, u, init_state, state_map ->
// y, y_state; the standard RWKV-5/6 recurrence).
//
// Work decomposition: one 512-thread workgroup per (head, unit).  Wave w owns
// key rows 8w..8w+7 of the fp32 state and lane j owns value column j, so the
// state is read and written as coalesced 256-byte rows and stays in
// registers for the whole call (8 values per lane).  Tokens are staged 32 at
// a time through LDS as fp32 (decay already exponentiated), together with
// each token's bonus r . (u * k); the raw words of the next block are loaded
// into registers while the current one is computed.  Per token a lane updates its 8 state
// values and forms its wave's partial output over the wave's rows, reading
// the row factors r, k, d as LDS broadcasts; the eight partials and the bonus
// term are then summed through LDS in a fixed order, so results are
// deterministic.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "wkv.h"

namespace wkv {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kRows = kHead / kWaves;  // key rows per wave
constexpr int kTB = 32;                 // tokens staged per block
static_assert(16 * kTB == kThreads, "one staging thread per (token, channel quad)");

template <bool V6, bool BF16, bool VARLEN>
__global__ void __launch_bounds__(kThreads) wkv56_scan_kernel(ScanParams p) {
  const int h = blockIdx.x;
  const int unit = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;  // value column j
  const int wave = tid >> 6;  // key rows kRows*wave ..
  const long C = (long)p.H * kHead;

  __shared__ float4 s_r[kTB][16], s_k[kTB][16], s_d[kTB][16];  // per token, channels 4q..4q+3
  __shared__ float s_v[kTB][kHead];
  __shared__ float s_bon[kTB];                 // r . (u * k) per token
  __shared__ float s_y[kTB][kWaves][kHead];    // per-wave partial outputs
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

  // ---- this lane's column of the wave's key rows, in registers
  float s[kRows];
  if (row_in >= 0 && p.state_in) {
    const float *sp = p.state_in + ((long)row_in * p.H + h) * (kHead * kHead) + lane;
#pragma unroll
    for (int a = 0; a < kRows; ++a) s[a] = sp[(kRows * wave + a) * kHead];
  } else {
#pragma unroll
    for (int a = 0; a < kRows; ++a) s[a] = 0.f;
  }
  // staging role: thread (token tt, channel quad q)
  const int st_tt = tid >> 4, st_q = tid & 15;
  float4 u4 = make_float4(0.f, 0.f, 0.f, 0.f), dst4 = make_float4(0.f, 0.f, 0.f, 0.f);
  {
    u4 = *reinterpret_cast<const float4 *>(p.u + h * kHead + 4 * st_q);
    if constexpr (!V6) {
      const float4 x = *reinterpret_cast<const float4 *>(static_cast<const float *>(p.w) + h * kHead + 4 * st_q);
      dst4 = f4(decay_of(x.x), decay_of(x.y), decay_of(x.z), decay_of(x.w));
    }
  }

  // staged token rows are loaded one block ahead, as raw words
  typedef typename std::conditional<BF16, uint2, float4>::type Raw;
  auto load_raw = [&](const void *base, long idx) -> Raw {
    if constexpr (BF16) return *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(base) + idx);
    else return *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + idx);
  };
  auto widen = [&](Raw w) -> float4 {
    if constexpr (BF16) return make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
    else return w;
  };
  Raw pr{}, pk{}, pv{}, px{};
  auto fetch = [&](int t0) {
    if (t0 + st_tt < ntok) {
      const long e = (tok0 + t0 + st_tt) * C + h * kHead + 4 * st_q;
      pr = load_raw(p.r, e);
      pk = load_raw(p.k, e);
      pv = load_raw(p.v, e);
      if constexpr (V6) px = load_raw(p.w, e);
    }
  };
  fetch(0);
  for (int t0 = 0; t0 < ntok; t0 += kTB) {
    const int nb = min(kTB, ntok - t0);
    {  // stage kTB tokens of this head as fp32, with each token's bonus
      float bon = 0.f;
      if (st_tt < nb) {
        const float4 r4 = widen(pr), k4 = widen(pk), v4 = widen(pv);
        s_r[st_tt][st_q] = r4;
        s_k[st_tt][st_q] = k4;
        *reinterpret_cast<float4 *>(&s_v[st_tt][4 * st_q]) = v4;
        if constexpr (V6) {
          const float4 x = widen(px);
          s_d[st_tt][st_q] = f4(decay_of(x.x), decay_of(x.y), decay_of(x.z), decay_of(x.w));
        } else {
          s_d[st_tt][st_q] = dst4;
        }
        bon = fmaf(r4.x * u4.x, k4.x, fmaf(r4.y * u4.y, k4.y, fmaf(r4.z * u4.z, k4.z, r4.w * u4.w * k4.w)));
      }
      // sum over the 16 channel quads of the token (lanes differing in bits 0..3)
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) bon += __shfl_xor(bon, m);
      if (st_q == 0) s_bon[st_tt] = bon;
    }
    fetch(t0 + kTB);  // the next block, in flight during this one
    __syncthreads();

#pragma unroll
    for (int tt = 0; tt < kTB; ++tt) {
      if (tt < nb) {
        const float vj = s_v[tt][lane];
        float yp = 0.f;
#pragma unroll
        for (int g = 0; g < kRows / 4; ++g) {
          const float4 r4 = s_r[tt][2 * wave + g], k4 = s_k[tt][2 * wave + g], d4 = s_d[tt][2 * wave + g];
          const float rr[4] = {r4.x, r4.y, r4.z, r4.w}, kk[4] = {k4.x, k4.y, k4.z, k4.w};
          const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            yp = fmaf(rr[a], s[4 * g + a], yp);
            s[4 * g + a] = fmaf(dd[a], s[4 * g + a], kk[a] * vj);
          }
        }
        s_y[tt][wave][lane] = yp;
      }
    }
    __syncthreads();
    {  // sum the wave partials in a fixed order, add the bonus term, store fp32 outputs
      const int tt = tid >> 4, j = 4 * (tid & 15);
      if (tt < nb) {
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float4 a = *reinterpret_cast<const float4 *>(&s_y[tt][w][j]);
          o.x += a.x; o.y += a.y; o.z += a.z; o.w += a.w;
        }
        const float b = s_bon[tt];
        const float4 v4 = *reinterpret_cast<const float4 *>(&s_v[tt][j]);
        o = f4(fmaf(b, v4.x, o.x), fmaf(b, v4.y, o.y), fmaf(b, v4.z, o.z), fmaf(b, v4.w, o.w));
        *reinterpret_cast<float4 *>(p.y + (tok0 + t0 + tt) * C + h * kHead + j) = o;
      }
    }
    // The next staging writes s_r..s_bon after this block's reads (ordered by the barrier
    // above); s_y is written again only after the next staging barrier.
    __syncthreads();
  }

  if (p.state_out) {
    if (VARLEN && ntok == 0 && p.state_out == p.state_in) return;  // empty slot: untouched
    float *sp = p.state_out + ((long)row_out * p.H + h) * (kHead * kHead) + lane;
#pragma unroll
    for (int a = 0; a < kRows; ++a) sp[(kRows * wave + a) * kHead] = s[a];
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
  if (varlen)  // varlen always carries a per-token decay
    return bf16 ? launch<true, true, true>(p, s) : launch<true, false, true>(p, s);
  if (v6) return bf16 ? launch<true, true, false>(p, s) : launch<true, false, false>(p, s);
  return bf16 ? launch<false, true, false>(p, s) : launch<false, false, false>(p, s);
}

}  // namespace wkv
