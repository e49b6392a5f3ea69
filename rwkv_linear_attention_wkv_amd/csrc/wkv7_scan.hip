// WKV v7 (the generalized delta rule of the rwkv_ops page's generalized_delta_rule
// operator: r, w, k, v, a, b of shape [B, T, H, K], state [.., K, V]).  Per (batch
// row, head), with the state h[key i][value j] and d_t = exp(-exp(w_t)):
//   sa[j]    = sum_i a_t[i] h[i][j]
//   h[i][j] <- d_t[i] h[i][j] + b_t[i] sa[j] + k_t[i] v_t[j]
//   y_t[j]   = sum_i r_t[i] h[i][j]        (with the updated state)
// (the standard RWKV-7 recurrence; the page gives the interface only, and its padding
// note, w += (1 - mask) * -1e9, needs the rwkv6op decay exp(-exp(w))).
//
// Value columns j evolve independently, so one 512-thread workgroup per (row, head)
// gives each wave 8 columns, and each lane 8 key rows of one column (8 state values in
// registers): lane 8m + g of wave w holds rows 8g .. 8g+7 of column 8w + m.  The two
// sums over key rows are sums over the 8 lanes of a column, formed on DPP (half-row
// mirror, then two quad permutes), so the token loop needs no barrier; two waves per
// SIMD hide each other's dependency chains.  After a token's update the lane forms
// r^T h (that token's output) and the next token's a^T h from the same state values, as
// two interleaved sums.  Tokens are staged through LDS in blocks of 64 (8 consecutive
// tokens per wave) as one record per token, so that a token's reads are one running base
// address plus immediate offsets; they are read back as 16-byte broadcasts two tokens
// ahead of their use (three register sets), and the next block's tokens are loaded from
// HBM while one is computed.
//
// Rescaled frame.  Inside a block let G_t[i] = d_0[i] ... d_t[i] (from the block start,
// G_{-1} = 1) and carry g[i][j] = h[i][j] / G_t[i] instead of h.  The recurrence becomes
//   sa[j]    = sum_i (a_t[i] G_{t-1}[i]) g[i][j]
//   g[i][j] <- g[i][j] + (b_t[i] / G_t[i]) sa[j] + (k_t[i] / G_t[i]) v_t[j]
//   y_t[j]   = sum_i (r_t[i] G_t[i]) g[i][j]
// (two FMAs per state value for the update instead of a multiply and two FMAs), and
// h = G_last g at the block end.  The staging pass forms the scaled factors (1 / G from
// the hardware reciprocal, within an ulp: a rounding-level change of the increments):
// each wave posts the running product of its 8 decays per key row through LDS one
// barrier ahead, and every wave chains the 8 posted products in the same order.  A
// block where some G falls below 2^-64 (so that 1/G would leave the safe range) is
// staged and run in the direct form instead; the test is on values every wave holds
// bitwise alike, so all waves take the same branch.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "wkv.h"

namespace wkv {
namespace {

constexpr int kThreads = 512;
constexpr int kTB = 64;                          // tokens staged per block
constexpr int kTPT = kTB * kHead / kThreads;     // (token, channel) pairs each thread stages
constexpr int kWaves = kThreads / 64;
static_assert(kWaves * kTPT == kTB, "staging shape: consecutive tokens per wave");
constexpr float kMinFrame = 0x1p-64f;            // smallest block decay product of the frame form

constexpr int kSP = kHead + 2;  // padded row of the LDS state tile (8-byte aligned rows)

struct __align__(16) V7Smem {
  float y[kTB][kHead];      // outputs of the block
  // Per token of the block, one 1.5 KiB record: per key row a, b, d, k, r (direct form) or
  // a G_{t-1}, b / G_t, G_t, k / G_t, r G_t (frame form), then v per value column.  The two
  // records past the block are read ahead at the last tokens and never used.
  float tok[kTB + 2][6][kHead];
  float dp[kWaves][kHead];  // per key row: the product of each wave's decays
  float st[kHead][kSP];     // the state on its way in from and out to HBM
};

template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  // x + x[lane permuted by CTRL]; full row and bank masks, so every source lane is valid
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
// Sum over the 8 lanes of an aligned group of 8 (every lane receives the same sum).
__device__ __forceinline__ float sum8(float x) {
  x = dpp_add<0x141>(x);  // row_half_mirror: lane i <-> 7 - i
  x = dpp_add<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x = dpp_add<0x4E>(x);   // quad_perm [2, 3, 0, 1]
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
  const int col = 8 * wave + (lane >> 3);        // value column
  const long C = p.tok_stride;                                     // elements between tokens
  const long base = unit * p.row_stride + h * p.head_stride;       // token 0, channel 0 of (row, head)
  const int T = p.T;

  int row_in = -1;
  if (p.state_in) {
    row_in = p.state_map ? p.state_map[unit] : (p.n_state == 1 ? 0 : unit);
    if (row_in < 0 || row_in >= p.n_state) {
      if (tid == 0 && p.dev_status) atomicOr(p.dev_status, WKV_DEV_BAD_STATE_MAP);
      return;
    }
  }
  // The state tile moves between HBM and the lanes through LDS: HBM sees whole 1 KiB runs
  // (thread t handles the 16-byte pieces t, t + 256, ...), the lanes their 8 x 2 blocks.
  float hs[8];
  if (row_in >= 0) {
    const float4 *sp = reinterpret_cast<const float4 *>(p.state_in + ((long)row_in * p.H + h) * (kHead * kHead));
#pragma unroll
    for (int q = 0; q < kHead * kHead / 4 / kThreads; ++q) {
      const int e = tid + kThreads * q;  // 16-byte piece: row e / 16, columns 4 (e % 16) ..
      const float4 x = sp[e];
      float *d = &sm.st[e >> 4][4 * (e & 15)];
      *reinterpret_cast<float2 *>(d) = make_float2(x.x, x.y);
      *reinterpret_cast<float2 *>(d + 2) = make_float2(x.z, x.w);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) hs[i] = sm.st[8 * g + i][col];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) hs[i] = 0.f;
  }

  // staging role: channel `lane`, tokens kTPT wave .. kTPT wave + kTPT - 1 of a block (rows
  // past the end reread the last token: staged but never used)
  float pa[kTPT], pb[kTPT], pw[kTPT], pk[kTPT], pr[kTPT], pv[kTPT], pd[kTPT];
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
  // The fetched block's decays (1 for rows past the end, so that they neither shrink the
  // block's product nor change the verdict below) and this wave's running product of them.
  auto decays = [&](int t0) {
    float c = 1.f;
#pragma unroll
    for (int q = 0; q < kTPT; ++q) {
      pd[q] = t0 + kTPT * wave + q < T ? decay_of(pw[q]) : 1.f;
      c = q ? c * pd[q] : pd[q];
    }
    sm.dp[wave][lane] = c;
  };
  if (T > 0) {
    fetch(0);
    decays(0);
  }
  __syncthreads();  // the first block's decay products
  for (int t0 = 0; t0 < T; t0 += kTB) {
    const int nb = min(kTB, T - t0);
    // Decay products in one fixed order in every wave: `ex` is G before this wave's first
    // token, `all` the block's product (its smallest G).  A wave's own G continue ex by the
    // running product of its decays, the value it posted, so a run of decays equal to 1
    // leaves G bitwise as it was.
    float ex = 1.f, all = 1.f;
#pragma unroll
    for (int u = 0; u < kWaves; ++u) {
      if (u == wave) ex = all;
      all *= sm.dp[u][lane];
    }
    const bool frame = __ballot(all < kMinFrame) == 0;  // same verdict in every wave
    const int t2 = kTPT * wave;
    if (frame) {
      float c = 1.f, gprev = ex;
#pragma unroll
      for (int q = 0; q < kTPT; ++q) {
        c = q ? c * pd[q] : pd[q];
        const float gq = ex * c;
        const float iq = __builtin_amdgcn_rcpf(gq);
        sm.tok[t2 + q][0][lane] = pa[q] * gprev;
        sm.tok[t2 + q][1][lane] = pb[q] * iq;
        sm.tok[t2 + q][2][lane] = gq;
        sm.tok[t2 + q][3][lane] = pk[q] * iq;
        sm.tok[t2 + q][4][lane] = pr[q] * gq;
        sm.tok[t2 + q][5][lane] = pv[q];
        gprev = gq;
      }
    } else {
#pragma unroll
      for (int q = 0; q < kTPT; ++q) {
        sm.tok[t2 + q][0][lane] = pa[q];
        sm.tok[t2 + q][1][lane] = pb[q];
        sm.tok[t2 + q][2][lane] = pd[q];
        sm.tok[t2 + q][3][lane] = pk[q];
        sm.tok[t2 + q][4][lane] = pr[q];
        sm.tok[t2 + q][5][lane] = pv[q];
      }
    }
    if (t0 + kTB < T) fetch(t0 + kTB);  // the next block, in flight during this one
    __syncthreads();

    // One token step from its staged factors.  The factors of the token after next are
    // read into a third register set before this token's arithmetic, so the LDS latency
    // overlaps two tokens' work.
    struct Fac {
      float4 f[5][2];  // the lane's 8 key rows of the five planes (the frame form skips the decay)
      float v;         // v of the lane's column
    };
    auto read_fac = [&](Fac &F, int tt, auto is_frame) {
#pragma unroll
      for (int m = 0; m < 5; ++m) {
        if (decltype(is_frame)::value && m == 2) continue;
        const float4 *src = reinterpret_cast<const float4 *>(&sm.tok[tt][m][8 * g]);
        F.f[m][0] = src[0];
        F.f[m][1] = src[1];
      }
      F.v = sm.tok[tt][5][col];
    };
    auto unpack = [](float (&dst)[8], const float4 (&src)[2]) {
      dst[0] = src[0].x; dst[1] = src[0].y; dst[2] = src[0].z; dst[3] = src[0].w;
      dst[4] = src[1].x; dst[5] = src[1].y; dst[6] = src[1].z; dst[7] = src[1].w;
    };
    // sum over the column's 64 key rows of x[i] * hs[i] (two chains of four per lane)
    auto dot8 = [&](const float (&x)[8]) {
      float s0 = x[0] * hs[0], s1 = x[4] * hs[4];
#pragma unroll
      for (int i = 1; i < 4; ++i) {
        s0 = fmaf(x[i], hs[i], s0);
        s1 = fmaf(x[i + 4], hs[i + 4], s1);
      }
      return sum8(s0 + s1);
    };
    // One token: the update from sa (a^T h before it), then r^T h for this token's output
    // and the next token's a^T h from the updated state, as two interleaved sums.
    auto step = [&](const Fac &F, const Fac &Fn, int tt, float sa, auto is_frame) {
      float fb[8], fk[8], fr[8], fan[8];
      unpack(fb, F.f[1]);
      unpack(fk, F.f[3]);
      unpack(fr, F.f[4]);
      if constexpr (decltype(is_frame)::value) {
#pragma unroll
        for (int i = 0; i < 8; ++i) hs[i] = fmaf(fk[i], F.v, fmaf(fb[i], sa, hs[i]));
      } else {
        float fd[8];
        unpack(fd, F.f[2]);
#pragma unroll
        for (int i = 0; i < 8; ++i) hs[i] = fmaf(fk[i], F.v, fmaf(fb[i], sa, fd[i] * hs[i]));
      }
      unpack(fan, Fn.f[0]);
      const float y = dot8(fr);
      const float san = dot8(fan);
      if (g == 0) sm.y[tt][col] = y;
      return san;
    };
    auto run_block = [&](auto is_frame) {
      Fac F0, F1, F2;
      read_fac(F0, 0, is_frame);
      read_fac(F1, 1, is_frame);
      float fa0[8];
      unpack(fa0, F0.f[0]);
      float sa = dot8(fa0);
      for (int tt = 0; tt < nb; tt += 3) {
        read_fac(F2, tt + 2, is_frame);  // past the block's last token: read, never used
        sa = step(F0, F1, tt, sa, is_frame);
        if (tt + 1 < nb) {
          read_fac(F0, tt + 3, is_frame);
          sa = step(F1, F2, tt + 1, sa, is_frame);
          if (tt + 2 < nb) {
            read_fac(F1, tt + 4, is_frame);
            sa = step(F2, F0, tt + 2, sa, is_frame);
          }
        }
      }
    };
    if (frame) {
      run_block(std::true_type{});
      // back from the frame: h = G_last g
      const float4 *gl = reinterpret_cast<const float4 *>(&sm.tok[nb - 1][2][8 * g]);
      float gv[8];
      const float4 gsrc[2] = {gl[0], gl[1]};
      unpack(gv, gsrc);
#pragma unroll
      for (int i = 0; i < 8; ++i) hs[i] *= gv[i];
    } else {
      run_block(std::false_type{});
    }
    __syncthreads();
    // store the block's outputs: thread -> (token kTPT wave + q, channel lane), coalesced rows
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
    // every wave has read this block's decay products (before the barrier above): the next
    // block's may be written
    if (t0 + kTB < T) decays(t0 + kTB);
    // the next staging rewrites the token arrays and outputs after this block's reads
    __syncthreads();
  }

  if (p.state_out) {
#pragma unroll
    for (int i = 0; i < 8; ++i) sm.st[8 * g + i][col] = hs[i];
    __syncthreads();
    float4 *sp = reinterpret_cast<float4 *>(p.state_out + ((long)unit * p.H + h) * (kHead * kHead));
#pragma unroll
    for (int q = 0; q < kHead * kHead / 4 / kThreads; ++q) {
      const int e = tid + kThreads * q;
      const float *d = &sm.st[e >> 4][4 * (e & 15)];
      const float2 lo = *reinterpret_cast<const float2 *>(d), hi = *reinterpret_cast<const float2 *>(d + 2);
      sp[e] = make_float4(lo.x, lo.y, hi.x, hi.y);
    }
  }
}

// Calls of at most kShortMax tokens per row (T = 1 decode steps): two waves per (row,
// head), wave c holding value columns 32c .. 32c+31.  Lane l of a wave holds key rows
// 32 (l / 32) .. +31 of column 32c + l % 32 (32 registers), so each sum over key rows is
// a sum inside the lane plus one exchange with the lane 32 away, and the state moves
// as 128-byte row pieces.  Against one wave per (row, head) with whole columns in the
// lanes, this halves each wave's dependent work and doubles the waves in flight, which
// shortens the tail after the state stream.  The key-row factors of a token reach the
// lanes through LDS (the two halves read rows 32 apart: different banks); v is read
// per lane.
constexpr int kCW = 32;               // value columns per wave
constexpr int kLG = 64 / kCW;         // lanes per column (key-row groups)
constexpr int kRL = kHead / kLG;      // key rows per lane
template <bool BF16>
__global__ void __launch_bounds__(64 * kLG) wkv7_short_kernel(V7Params p) {
  __shared__ __align__(16) float sf[5][kHead];  // a, b, d = exp(-exp(w)), k, r of the token
  const int h = blockIdx.x;
  const int unit = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int col = kCW * (tid >> 6) + lane % kCW;  // value column j
  const int r0 = kRL * (lane / kCW);              // first key row of the lane
  const long C = p.tok_stride;
  const long base = unit * p.row_stride + h * p.head_stride;

  int row_in = -1;
  if (p.state_in) {
    row_in = p.state_map ? p.state_map[unit] : (p.n_state == 1 ? 0 : unit);
    if (row_in < 0 || row_in >= p.n_state) {
      if (tid == 0 && p.dev_status) atomicOr(p.dev_status, WKV_DEV_BAD_STATE_MAP);
      return;
    }
  }
  float hc[kRL];
  if (row_in >= 0) {
    const float *sp = p.state_in + ((long)row_in * p.H + h) * (kHead * kHead) + r0 * kHead + col;
#pragma unroll
    for (int i = 0; i < kRL; ++i) hc[i] = sp[i * kHead];
  } else {
#pragma unroll
    for (int i = 0; i < kRL; ++i) hc[i] = 0.f;
  }
  // sum over the column's 64 key rows of x[i] h[i] (four chains in the lane, then the other half)
  auto colsum = [&](int m) {
    float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i4 = 0; i4 < kRL / 4; ++i4) {
      const float4 x = *reinterpret_cast<const float4 *>(&sf[m][r0 + 4 * i4]);
      s4[0] = fmaf(x.x, hc[4 * i4], s4[0]);
      s4[1] = fmaf(x.y, hc[4 * i4 + 1], s4[1]);
      s4[2] = fmaf(x.z, hc[4 * i4 + 2], s4[2]);
      s4[3] = fmaf(x.w, hc[4 * i4 + 3], s4[3]);
    }
    float part = (s4[0] + s4[1]) + (s4[2] + s4[3]);
#pragma unroll
    for (int m = kCW; m < 64; m <<= 1) part += __shfl_xor(part, m);  // same sum in every group
    return part;
  };
  for (int t = 0; t < p.T; ++t) {
    const long e = base + (long)t * C;
    if (tid < kHead) {
      sf[0][tid] = load1<BF16>(p.a, e + tid);
      sf[1][tid] = load1<BF16>(p.b, e + tid);
      sf[2][tid] = decay_of(load1<BF16>(p.w, e + tid));
      sf[3][tid] = load1<BF16>(p.k, e + tid);
      sf[4][tid] = load1<BF16>(p.r, e + tid);
    }
    const float vj = load1<BF16>(p.v, e + col);
    __syncthreads();  // the factors' stores before the reads
    const float sa = colsum(0);
#pragma unroll
    for (int i4 = 0; i4 < kRL / 4; ++i4) {
      const float4 b4 = *reinterpret_cast<const float4 *>(&sf[1][r0 + 4 * i4]);
      const float4 d4 = *reinterpret_cast<const float4 *>(&sf[2][r0 + 4 * i4]);
      const float4 k4 = *reinterpret_cast<const float4 *>(&sf[3][r0 + 4 * i4]);
      const float bb[4] = {b4.x, b4.y, b4.z, b4.w}, dd[4] = {d4.x, d4.y, d4.z, d4.w};
      const float kk[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float &x = hc[4 * i4 + q];
        x = fmaf(kk[q], vj, fmaf(bb[q], sa, dd[q] * x));
      }
    }
    const float y = colsum(4);
    if (lane < kCW) {
      if (p.y_bf16) static_cast<uint16_t *>(p.y)[e + col] = bf16_bits(y);
      else static_cast<float *>(p.y)[e + col] = y;
    }
    __syncthreads();  // the reads finish before the next token's factors are stored
  }
  if (p.state_out) {
    float *sp = p.state_out + ((long)unit * p.H + h) * (kHead * kHead) + r0 * kHead + col;
#pragma unroll
    for (int i = 0; i < kRL; ++i) sp[i * kHead] = hc[i];
  }
}

}  // namespace

hipError_t launch_wkv7_scan(const V7Params &p, bool bf16, hipStream_t s) {
  dim3 grid(p.H, p.B);
  if (p.T <= kShortMax) {
    if (bf16) hipLaunchKernelGGL((wkv7_short_kernel<true>), grid, dim3(64 * kLG), 0, s, p);
    else hipLaunchKernelGGL((wkv7_short_kernel<false>), grid, dim3(64 * kLG), 0, s, p);
  } else {
    if (bf16) hipLaunchKernelGGL((wkv7_scan_kernel<true>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((wkv7_scan_kernel<false>), grid, dim3(kThreads), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace wkv
