// WKV v7 (the generalized delta rule of the rwkv_ops page's generalized_delta_rule
// operator: r, w, k, v, a, b of shape [B, T, H, K], w the decay in log space, state
// [.., K, V]).  Per (batch row, head), with the state h[key i][value j]:
//   sa[j]    = sum_i a_t[i] h[i][j]
//   h[i][j] <- exp(w_t[i]) h[i][j] + b_t[i] sa[j] + k_t[i] v_t[j]
//   y_t[j]   = sum_i r_t[i] h[i][j]        (with the updated state)
// (the standard RWKV-7 recurrence; the page gives the interface only).
//
// Value columns j evolve independently, so one 256-thread workgroup per (row, head)
// gives each wave 16 columns, and each lane 8 key rows of 2 columns (16 state values
// in registers): lane 8m + g of wave w holds rows 8g .. 8g+7 of columns 16w + 2m and
// 16w + 2m + 1.  The two sums over key rows (a^T h before the update, r^T h after it)
// are sums over the 8 lanes of a column pair, formed on DPP (half-row mirror, then
// two quad permutes), so the token loop needs no barrier.  Tokens are staged through
// LDS in blocks of 16 (r, exp(w), k, a, b per key row; v per column), read back as
// 16-byte broadcasts, and the next block's tokens are loaded while one is computed.
#include "common.hpp"
#include "kernels.hpp"
#include "wkv.h"

namespace wkv {
namespace {

constexpr int kThreads = 256;
constexpr int kTB = 16;                          // tokens staged per block
constexpr int kTPT = kTB * kHead / kThreads;     // (token, channel) pairs each thread stages
static_assert(kTPT == 4, "staging: four tokens per thread");

struct __align__(16) V7Smem {
  float f[5][kTB][kHead];  // per key row: a, b, exp(w), k, r
  float v[kTB][kHead];     // per value column
  float y[kTB][kHead];     // outputs of the block
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum over the 8 lanes of an aligned group of 8 (every lane receives the same sum).
__device__ __forceinline__ float sum8(float x) {
  x += dpp<0x141>(x);  // row_half_mirror: lane i <-> 7 - i
  x += dpp<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  return x;
}

template <bool BF16>
__global__ void __launch_bounds__(kThreads) wkv7_scan_kernel(V7Params p) {
  __shared__ V7Smem sm;
  const int h = blockIdx.x;
  const int unit = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane & 7;                        // key rows 8g .. 8g+7
  const int col = 16 * wave + 2 * (lane >> 3);   // value columns col, col + 1
  const long C = (long)p.H * kHead;
  const long base = (long)unit * p.T * C + h * kHead;  // token 0, channel 0 of this (row, head)
  const int T = p.T;

  int row_in = -1;
  if (p.state_in) {
    row_in = p.state_map ? p.state_map[unit] : (p.n_state == 1 ? 0 : unit);
    if (row_in < 0 || row_in >= p.n_state) {
      if (tid == 0 && p.dev_status) atomicOr(p.dev_status, WKV_DEV_BAD_STATE_MAP);
      return;
    }
  }
  float hs[8][2];
  if (row_in >= 0) {
    const float *sp = p.state_in + ((long)row_in * p.H + h) * (kHead * kHead);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float2 s2 = *reinterpret_cast<const float2 *>(sp + (8 * g + i) * kHead + col);
      hs[i][0] = s2.x;
      hs[i][1] = s2.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) hs[i][0] = hs[i][1] = 0.f;
  }

  // staging role: channel `lane`, tokens 4 wave .. 4 wave + 3 of a block (rows past the end
  // reread the last token: staged but never used)
  float pa[kTPT], pb[kTPT], pw[kTPT], pk[kTPT], pr[kTPT], pv[kTPT];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int q = 0; q < kTPT; ++q) {
      const long e = base + (long)min(t0 + kTPT * wave + q, T - 1) * C + lane;
      pa[q] = load1<BF16>(p.a, e);
      pb[q] = load1<BF16>(p.b, e);
      pw[q] = load1<BF16>(p.w, e);
      pk[q] = load1<BF16>(p.k, e);
      pr[q] = load1<BF16>(p.r, e);
      pv[q] = load1<BF16>(p.v, e);
    }
  };
  if (T > 0) fetch(0);
  for (int t0 = 0; t0 < T; t0 += kTB) {
    const int nb = min(kTB, T - t0);
#pragma unroll
    for (int q = 0; q < kTPT; ++q) {
      const int tt = kTPT * wave + q;
      sm.f[0][tt][lane] = pa[q];
      sm.f[1][tt][lane] = pb[q];
      sm.f[2][tt][lane] = fast_exp(pw[q]);
      sm.f[3][tt][lane] = pk[q];
      sm.f[4][tt][lane] = pr[q];
      sm.v[tt][lane] = pv[q];
    }
    if (t0 + kTB < T) fetch(t0 + kTB);  // the next block, in flight during this one
    __syncthreads();

    for (int tt = 0; tt < nb; ++tt) {
      const float4 *f4p[5];
#pragma unroll
      for (int m = 0; m < 5; ++m) f4p[m] = reinterpret_cast<const float4 *>(&sm.f[m][tt][8 * g]);
      float fa[8], fb[8], fd[8], fk[8], fr[8];
      auto unpack = [&](float (&dst)[8], const float4 *src) {
        const float4 lo = src[0], hi = src[1];
        dst[0] = lo.x; dst[1] = lo.y; dst[2] = lo.z; dst[3] = lo.w;
        dst[4] = hi.x; dst[5] = hi.y; dst[6] = hi.z; dst[7] = hi.w;
      };
      unpack(fa, f4p[0]);
      const float2 vv = *reinterpret_cast<const float2 *>(&sm.v[tt][col]);
      // sa over this lane's 8 key rows, then over the column's 8 lanes
      float s0 = fa[0] * hs[0][0], s1 = fa[0] * hs[0][1];
#pragma unroll
      for (int i = 1; i < 8; ++i) {
        s0 = fmaf(fa[i], hs[i][0], s0);
        s1 = fmaf(fa[i], hs[i][1], s1);
      }
      s0 = sum8(s0);
      s1 = sum8(s1);
      unpack(fb, f4p[1]);
      unpack(fd, f4p[2]);
      unpack(fk, f4p[3]);
      unpack(fr, f4p[4]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        hs[i][0] = fmaf(fk[i], vv.x, fmaf(fb[i], s0, fd[i] * hs[i][0]));
        hs[i][1] = fmaf(fk[i], vv.y, fmaf(fb[i], s1, fd[i] * hs[i][1]));
      }
      float y0 = fr[0] * hs[0][0], y1 = fr[0] * hs[0][1];
#pragma unroll
      for (int i = 1; i < 8; ++i) {
        y0 = fmaf(fr[i], hs[i][0], y0);
        y1 = fmaf(fr[i], hs[i][1], y1);
      }
      y0 = sum8(y0);
      y1 = sum8(y1);
      if (g == 0) *reinterpret_cast<float2 *>(&sm.y[tt][col]) = make_float2(y0, y1);
    }
    __syncthreads();
    // store the block's outputs: thread -> (token 4 wave + q, channel lane), coalesced rows
#pragma unroll
    for (int q = 0; q < kTPT; ++q) {
      const int tt = kTPT * wave + q;
      if (tt < nb) {
        const long e = base + (long)(t0 + tt) * C + lane;
        const float yv = sm.y[tt][lane];
        if (p.y_bf16) static_cast<uint16_t *>(p.y)[e] = bf16_bits(yv);
        else static_cast<float *>(p.y)[e] = yv;
      }
    }
    // the next staging rewrites the token arrays and outputs after this block's reads
    __syncthreads();
  }

  if (p.state_out) {
    float *sp = p.state_out + ((long)unit * p.H + h) * (kHead * kHead);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<float2 *>(sp + (8 * g + i) * kHead + col) = make_float2(hs[i][0], hs[i][1]);
  }
}

}  // namespace

hipError_t launch_wkv7_scan(const V7Params &p, bool bf16, hipStream_t s) {
  dim3 grid(p.H, p.B);
  if (bf16) hipLaunchKernelGGL((wkv7_scan_kernel<true>), grid, dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL((wkv7_scan_kernel<false>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace wkv
