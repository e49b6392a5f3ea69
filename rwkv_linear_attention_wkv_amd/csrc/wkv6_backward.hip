// Backward of the WKV v6 recurrence (gradients for training), as three
// token-sequential sweeps on the vector ALUs.
//
// Forward (the rwkv_ops page's RWKV6_OP call; the standard RWKV-6 recurrence),
// per (batch row, head), S indexed [key i][value j]:
//   y_t[j] = sum_i r_t[i] (S_{t-1}[i][j] + u[i] k_t[i] v_t[j])
//   S_t[i][j] = d_t[i] S_{t-1}[i][j] + k_t[i] v_t[j],   d_t = exp(-exp(x_t))
// With upstream gradients dy (of y) and dS_T (of the final state), and
// G_t = dL/dS_t (G_{T-1} = dS_T, G_{t-1} = d_t G_t + r_t dy_t^T):
//   dr_t[i] = sum_j S_{t-1}[i][j] dy_t[j] + u[i] k_t[i] (dy_t . v_t)
//   dk_t[i] = sum_j G_t[i][j] v_t[j]      + u[i] r_t[i] (dy_t . v_t)
//   dv_t[j] = sum_i G_t[i][j] k_t[i]      + (sum_i r_t[i] u[i] k_t[i]) dy_t[j]
//   du[i]   = sum_t r_t[i] k_t[i] (dy_t . v_t)
//   dS_0    = G_{-1}
// and, for the log decay lam = -exp(x), with the tilde parts (no u term),
//   dlam_t[i] = sum_{tau > t} r_tau[i] dr~_tau[i] + sum_j dS_T[i][j] S_T[i][j]
//               - sum_{s >= t} k_s[i] dk~_s[i],       dx_t[i] = -exp(x_t[i]) dlam_t[i]
// (every pair (s, tau) whose decay path crosses token t, counted once).
//
// Each sweep is one state recurrence of the same shape: a 64 x 64 fp32 state
// X in registers (wave w owns rows 8w..8w+7, lane c column c), tokens walked
// in order (or in reverse), per token
//   out[c] = sum_row P[row] X[row][c],   then   X[row][c] <- a X[row][c] + Q[row] R[c]
// with the decay a on the rows or on the columns:
//   TFWD (time forward, X = S^T, rows j, columns i, column decay):
//       P = dy, Q = v, R = k, a = d[i]  -> dr (and du per batch row)
//   BWD  (time reversed, X = G, rows i, columns j, row decay):
//       P = k, Q = r, R = dy, a = d[i]  -> dv, and dS_0 at the end
//   TBWD (time reversed, X = G^T, rows j, columns i, column decay):
//       P = v, Q = dy, R = r, a = d[i]  -> dk, and dx from dr (TFWD's output)
// Tokens are staged through LDS as fp32 in blocks (wave w stages a run of
// consecutive tokens of the block, lane = channel), per-wave partial outputs
// are summed through LDS in a fixed order (deterministic), and the
// per-channel sums over time (du, the dlam running sums) are walked by wave
// 0, one token after the other.  TFWD and BWD do not depend on each other:
// they run as one launch (blockIdx.z picks the sweep) with 16-token blocks, so
// that two workgroups (64 KiB of LDS each) share a CU and each SIMD holds four
// waves; TBWD reads TFWD's dr and runs after it with 32-token blocks.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "wkv.h"

namespace wkv {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kRows = kHead / kWaves;  // state rows per wave

enum Sweep { TFWD = 0, BWD = 1, TBWD = 2 };

template <int KTB>
struct Smem {
  float p[KTB][kHead], q[KTB][kHead];  // row factors
  float al[KTB][kHead];                // decay d per (token, channel)
  float r[KTB][kHead];                 // column factor R
  float e0[KTB][kHead], e1[KTB][kHead], e2[KTB][kHead];  // per-sweep extras
  float w[KTB][kHead];                 // per (token, channel) terms of the time sums
  float y[KTB][kWaves][kHead];         // per-wave partial outputs
  float bon[KTB];
};

template <int MODE, bool BF16, int KTB>
__device__ __forceinline__ void sweep(const BwdParams &p, Smem<KTB> &sm, int h, int b) {
  constexpr bool REV = MODE != TFWD;      // tokens walked from the last one
  constexpr bool COLDECAY = MODE != BWD;  // decay on the state's columns (transposed state)
  constexpr int TPW = KTB / kWaves;       // tokens each wave stages per block
  constexpr int CPT = kHead * KTB / kThreads;  // channels per thread in the reduction
  static_assert(TPW * kWaves == KTB && CPT * kThreads == kHead * KTB && (CPT == 2 || CPT == 4), "block shape");
  auto &s_p = sm.p; auto &s_q = sm.q; auto &s_al = sm.al; auto &s_r = sm.r;
  auto &s_e0 = sm.e0; auto &s_e1 = sm.e1; auto &s_e2 = sm.e2; auto &s_w = sm.w; auto &s_y = sm.y;
  auto &s_bon = sm.bon;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long C = (long)p.H * kHead;
  const int T = p.T;
  const long row0 = (long)b * T;  // first token row of this batch row

  // ---- initial state
  float X[kRows];
#pragma unroll
  for (int a = 0; a < kRows; ++a) X[a] = 0.f;
  const long head_off = (long)h * kHead * kHead;
  if (MODE == TFWD) {
    if (p.state_in) {
      const int row_in = p.state_map ? p.state_map[b] : (p.n_state == 1 ? 0 : b);
      if (row_in < 0 || row_in >= p.n_state) {
        if (tid == 0 && p.dev_status) atomicOr(p.dev_status, WKV_DEV_BAD_STATE_MAP);
        return;
      }
      const float *s0 = p.state_in + (long)row_in * p.H * kHead * kHead + head_off;
#pragma unroll
      for (int a = 0; a < kRows; ++a) X[a] = s0[lane * kHead + kRows * wave + a];  // X[j][i] = S0[i][j]
    }
  } else if (p.d_state_out) {
    const float *g = p.d_state_out + (long)b * p.H * kHead * kHead + head_off;
#pragma unroll
    for (int a = 0; a < kRows; ++a)
      X[a] = COLDECAY ? g[lane * kHead + kRows * wave + a] : g[(kRows * wave + a) * kHead + lane];
  }
  // TBWD: the decay gradient of channel `lane` as one running difference (walked by wave 0).
  // The two sums over the sequence grow with its length while their difference does not, so
  // the difference itself is carried, with a compensation term (Kahan): rounding stays
  // relative to the difference and the per-token terms, not to the sums.
  float dsum = 0.f, dcomp = 0.f, dusum = 0.f;
  auto dadd = [&](float x) {
    const float yk = x - dcomp;
    const float t = dsum + yk;
    dcomp = (t - dsum) - yk;
    dsum = t;
  };
  if (MODE == TBWD && wave == 0 && p.d_state_out && p.state_final) {
    const float *g = p.d_state_out + (long)b * p.H * kHead * kHead + head_off + lane * kHead;
    const float *sf = p.state_final + (long)b * p.H * kHead * kHead + head_off + lane * kHead;
    for (int j = 0; j < kHead; ++j) dadd(g[j] * sf[j]);
  }
  const float uc = p.u[h * kHead + lane];

  // token of processing step q (0 .. T-1)
  auto tok = [&](int q) -> long { return row0 + (REV ? (T - 1 - q) : q); };
  // the next block's inputs, loaded one block ahead (steps past the end reread the last one)
  float pr[TPW], pk[TPW], pv[TPW], px[TPW], pdy[TPW], pdr[TPW];
  auto fetch = [&](int q0) {
#pragma unroll
    for (int t4 = 0; t4 < TPW; ++t4) {
      const long e = tok(min(q0 + TPW * wave + t4, T - 1)) * C + h * kHead + lane;
      pr[t4] = load1<BF16>(p.r, e);
      pk[t4] = load1<BF16>(p.k, e);
      pv[t4] = load1<BF16>(p.v, e);
      px[t4] = load1<BF16>(p.w, e);
      pdy[t4] = p.dy[e];
      pdr[t4] = MODE == TBWD ? p.dr[e] : 0.f;
    }
  };
  if (T > 0) fetch(0);
  for (int q0 = 0; q0 < T; q0 += KTB) {
    const int nb = min(KTB, T - q0);
    // ---- stage this block (token of step q0 + tt at row tt)
    float bon[TPW];
#pragma unroll
    for (int t4 = 0; t4 < TPW; ++t4) {
      const int tt = TPW * wave + t4;
      const float ex = fast_exp(px[t4]);
      s_al[tt][lane] = fast_exp(-ex);
      if (MODE == TFWD) {
        s_p[tt][lane] = pdy[t4];
        s_q[tt][lane] = pv[t4];
        s_r[tt][lane] = pk[t4];
        s_e0[tt][lane] = pr[t4];
        bon[t4] = pdy[t4] * pv[t4];
      } else if (MODE == BWD) {
        s_p[tt][lane] = pk[t4];
        s_q[tt][lane] = pr[t4];
        s_r[tt][lane] = pdy[t4];
        bon[t4] = pk[t4] * uc * pr[t4];
      } else {
        s_p[tt][lane] = pv[t4];
        s_q[tt][lane] = pdy[t4];
        s_r[tt][lane] = pr[t4];
        s_e0[tt][lane] = pk[t4];
        s_e1[tt][lane] = pdr[t4];
        s_e2[tt][lane] = -ex;
        bon[t4] = pv[t4] * pdy[t4];
      }
    }
    fetch(q0 + KTB);  // in flight during this block
#pragma unroll
    for (int t4 = 0; t4 < TPW; ++t4) {  // bonus scalar: sum over the 64 channels of the token
      float x = bon[t4];
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
      bon[t4] = x;
    }
    if (lane == 0) {
#pragma unroll
      for (int t4 = 0; t4 < TPW; ++t4) s_bon[TPW * wave + t4] = bon[t4];
    }
    __syncthreads();

    // ---- the recurrence over the block's tokens
    for (int tt = 0; tt < nb; ++tt) {
      const float rc = s_r[tt][lane];
      float y0 = 0.f, y1 = 0.f;
      if (COLDECAY) {
        const float ac = s_al[tt][lane];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const float4 p4 = *reinterpret_cast<const float4 *>(&s_p[tt][kRows * wave + 4 * g]);
          const float4 q4 = *reinterpret_cast<const float4 *>(&s_q[tt][kRows * wave + 4 * g]);
          y0 = fmaf(p4.x, X[4 * g], y0); X[4 * g] = fmaf(ac, X[4 * g], q4.x * rc);
          y1 = fmaf(p4.y, X[4 * g + 1], y1); X[4 * g + 1] = fmaf(ac, X[4 * g + 1], q4.y * rc);
          y0 = fmaf(p4.z, X[4 * g + 2], y0); X[4 * g + 2] = fmaf(ac, X[4 * g + 2], q4.z * rc);
          y1 = fmaf(p4.w, X[4 * g + 3], y1); X[4 * g + 3] = fmaf(ac, X[4 * g + 3], q4.w * rc);
        }
      } else {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const float4 p4 = *reinterpret_cast<const float4 *>(&s_p[tt][kRows * wave + 4 * g]);
          const float4 q4 = *reinterpret_cast<const float4 *>(&s_q[tt][kRows * wave + 4 * g]);
          const float4 a4 = *reinterpret_cast<const float4 *>(&s_al[tt][kRows * wave + 4 * g]);
          y0 = fmaf(p4.x, X[4 * g], y0); X[4 * g] = fmaf(a4.x, X[4 * g], q4.x * rc);
          y1 = fmaf(p4.y, X[4 * g + 1], y1); X[4 * g + 1] = fmaf(a4.y, X[4 * g + 1], q4.y * rc);
          y0 = fmaf(p4.z, X[4 * g + 2], y0); X[4 * g + 2] = fmaf(a4.z, X[4 * g + 2], q4.z * rc);
          y1 = fmaf(p4.w, X[4 * g + 3], y1); X[4 * g + 3] = fmaf(a4.w, X[4 * g + 3], q4.w * rc);
        }
      }
      s_y[tt][wave][lane] = y0 + y1;
    }
    __syncthreads();

    // ---- sum the wave partials in a fixed order, add the u terms, store
    {
      const int tt = tid / (kHead / CPT), c = CPT * (tid % (kHead / CPT));
      if (tt < nb) {
        float o[CPT];
#pragma unroll
        for (int m = 0; m < CPT; ++m) o[m] = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
#pragma unroll
          for (int m = 0; m < CPT; ++m) o[m] += s_y[tt][w][c + m];
        const float bt = s_bon[tt];
        float res[CPT], wt[CPT];
#pragma unroll
        for (int m = 0; m < CPT; ++m) {
          const float um = p.u[h * kHead + c + m], rm = s_r[tt][c + m];
          if (MODE == TFWD) {  // dr; time-sum term of du: r k (dy . v)
            res[m] = fmaf(um * rm, bt, o[m]);
            wt[m] = s_e0[tt][c + m] * rm * bt;
          } else if (MODE == BWD) {  // dv
            res[m] = fmaf(bt, rm, o[m]);
            wt[m] = 0.f;
          } else {  // dk; decay-gradient term r dr~ (next steps) and k dk~ (this step)
            const float kk = s_e0[tt][c + m];
            res[m] = fmaf(um * rm, bt, o[m]);
            const float drt = s_e1[tt][c + m] - um * kk * bt;  // dr without its u term
            s_e1[tt][c + m] = rm * drt;
            wt[m] = kk * o[m];
          }
        }
        float *out = (MODE == TFWD ? p.dr : (MODE == BWD ? p.dv : p.dk)) + tok(q0 + tt) * C + h * kHead + c;
        if constexpr (CPT == 4) {
          *reinterpret_cast<float4 *>(out) = make_float4(res[0], res[1], res[2], res[3]);
          if (MODE != BWD) *reinterpret_cast<float4 *>(&s_w[tt][c]) = make_float4(wt[0], wt[1], wt[2], wt[3]);
        } else {
          *reinterpret_cast<float2 *>(out) = make_float2(res[0], res[1]);
          if (MODE != BWD) *reinterpret_cast<float2 *>(&s_w[tt][c]) = make_float2(wt[0], wt[1]);
        }
      }
    }
    __syncthreads();
    // ---- sums over time, one channel per lane of wave 0, in processing order
    if (MODE != BWD && wave == 0) {
      if (MODE == TFWD) {
        for (int tt = 0; tt < nb; ++tt) dusum += s_w[tt][lane];
      } else {
        for (int tt = 0; tt < nb; ++tt) {
          dadd(-s_w[tt][lane]);  // - k_t dk~_t: counted from this step on
          p.dw[tok(q0 + tt) * C + h * kHead + lane] = s_e2[tt][lane] * dsum;
          dadd(s_e1[tt][lane]);  // + r_t dr~_t: counted for the steps before t
        }
      }
    }
    // The next staging writes the token arrays after this block's reads (ordered by this
    // barrier); s_y is written again only after the next staging barrier.
    __syncthreads();
  }

  if (MODE == TFWD && wave == 0 && p.du_rows) p.du_rows[(long)b * C + h * kHead + lane] = dusum;
  if (MODE == BWD && p.d_state_in) {
    float *g = p.d_state_in + (long)b * p.H * kHead * kHead + head_off;
#pragma unroll
    for (int a = 0; a < kRows; ++a) g[(kRows * wave + a) * kHead + lane] = X[a];
  }
}

template <bool BF16>
__global__ void __launch_bounds__(kThreads, 2) wkv6_bwd_pair_kernel(BwdParams p) {
  __shared__ __align__(16) Smem<16> sm;
  if (blockIdx.z == 0) sweep<TFWD, BF16, 16>(p, sm, blockIdx.x, blockIdx.y);
  else sweep<BWD, BF16, 16>(p, sm, blockIdx.x, blockIdx.y);
}

template <bool BF16>
__global__ void __launch_bounds__(kThreads) wkv6_bwd_tbwd_kernel(BwdParams p) {
  __shared__ __align__(16) Smem<32> sm;
  sweep<TBWD, BF16, 32>(p, sm, blockIdx.x, blockIdx.y);
}

// du[c] = sum over batch rows of du_rows[b][c], in row order.
__global__ void __launch_bounds__(256) wkv6_du_sum_kernel(const float *du_rows, float *du, int B, int C) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  float s = 0.f;
  for (int b = 0; b < B; ++b) s += du_rows[(long)b * C + c];
  du[c] = s;
}

}  // namespace

hipError_t launch_wkv6_backward(const BwdParams &p, bool bf16, hipStream_t s) {
  // TFWD and BWD together, then TBWD (it reads TFWD's dr)
  if (bf16) hipLaunchKernelGGL(wkv6_bwd_pair_kernel<true>, dim3(p.H, p.B, 2), dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL(wkv6_bwd_pair_kernel<false>, dim3(p.H, p.B, 2), dim3(kThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (bf16) hipLaunchKernelGGL(wkv6_bwd_tbwd_kernel<true>, dim3(p.H, p.B), dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL(wkv6_bwd_tbwd_kernel<false>, dim3(p.H, p.B), dim3(kThreads), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int C = p.H * kHead;
  hipLaunchKernelGGL(wkv6_du_sum_kernel, dim3((C + 255) / 256), dim3(256), 0, s, p.du_rows, p.du, p.B, C);
  return hipGetLastError();
}

}  // namespace wkv
