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
// With E_t[i] = sum_j G_t[i][j] S_t[i][j] this is dlam_t = E_t - k_t dk~_t, and
// E_{t-1} = E_t - k_t dk~_t + r_t dr~_t, E_{T-1} = sum_j dS_T S_T: the running
// difference walked backwards.  Its rounding accumulates with the number of
// steps walked, so the walk restarts from E_t itself every kSpan tokens, with
// S_t kept by the forward sweep.
//
// Each sweep is one state recurrence of the same shape: a 64 x 64 fp32 state
// X in registers (wave w owns rows 8w..8w+7; lanes 2m and 2m+1 hold the two
// halves of those rows for columns 2m and 2m+1), tokens walked in order (or in
// reverse), per token
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
// are summed through LDS in a fixed order (deterministic).  Of the
// per-channel sums over time, du is walked by wave 0 one token after the
// other, and the dlam running sums are a prefix over the block (in-wave sums
// plus the earlier waves' totals) on a compensated carry, reset to E at the
// span ends (the forward sweep leaves S_t in the dw rows that the dk/dw sweep
// writes last, so no workspace is needed).  Inside a block
// the state is carried in a frame rescaled by the block's running decay
// product, which makes each step two FMAs per state element instead of three
// (blocks whose decay product underflows the frame take the direct form).
// The row factors reach every lane as LDS broadcast reads, whose bytes bound
// a step: the 4 x 2 tile per lane needs 8 of them per step for 8 elements.
// TFWD and BWD do not depend on each other: they run as one launch
// (blockIdx.z picks the sweep) with 16-token blocks, so that two workgroups
// (70 KiB of LDS each) share a CU and each SIMD holds four waves; TBWD reads
// TFWD's dr and runs after it with 32-token blocks.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "wkv.h"

namespace wkv {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kRows = kHead / kWaves;  // state rows per wave
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kFrameLog2 = 80.f;  // largest log2 decay of one block the rescaled frame takes
// Every kSpan tokens the forward sweep leaves the state S in the dw rows of the span's last
// kHead tokens (of its own head), and the dk/dw sweep restarts its decay-gradient sum there
// from the exact identity (see the time sums below).  A multiple of both block lengths.
constexpr int kSpan = 256;

enum Sweep { TFWD = 0, BWD = 1, TBWD = 2 };

// The value of lane l ^ 1 (quad permute on DPP).
__device__ __forceinline__ float xor_lane1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}

template <int KTB>
struct Smem {
  float p[KTB][kHead], q[KTB][kHead];  // row factors (rescaled in the frame, row decay)
  float al[KTB][kHead];                // direct form: decay d; frame, column decay: output factor
  float r[KTB][kHead];                 // column factor R
  float rt[KTB][kHead];                // frame, column decay: R rescaled
  float e0[KTB][kHead], e1[KTB][kHead], e2[KTB][kHead];  // per-sweep extras
  float w[KTB][kHead];                 // per (token, channel) terms of the time sums
  float y[KTB][kWaves][kHead];         // per-wave partial outputs
  float tot[kWaves][kHead];            // log2 decay of each staging wave's tokens
  float dend[kHead];                   // decay product of the block per channel
  float bon[KTB];
  float ek[kWaves][kHead];             // per-wave parts of sum_j G[i][j] S[i][j] at a span end
};

template <int MODE, bool BF16, int KTB>
__device__ __forceinline__ void sweep(const BwdParams &p, Smem<KTB> &sm, int h, int b) {
  constexpr bool REV = MODE != TFWD;      // tokens walked from the last one
  constexpr bool COLDECAY = MODE != BWD;  // decay on the state's columns (transposed state)
  constexpr int TPW = KTB / kWaves;       // tokens each wave stages per block
  constexpr int CPT = kHead * KTB / kThreads;  // channels per thread in the reduction
  static_assert(TPW * kWaves == KTB && CPT * kThreads == kHead * KTB && (CPT == 2 || CPT == 4), "block shape");
  auto &s_p = sm.p; auto &s_q = sm.q; auto &s_al = sm.al; auto &s_r = sm.r; auto &s_rt = sm.rt;
  auto &s_e0 = sm.e0; auto &s_e1 = sm.e1; auto &s_e2 = sm.e2; auto &s_w = sm.w; auto &s_y = sm.y;
  auto &s_bon = sm.bon;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long C = (long)p.H * kHead;
  const int T = p.T;
  const long row0 = (long)b * T;  // first token row of this batch row

  // ---- initial state
  // The state tile of this thread: rows xr0 .. xr0+3 and columns xc0, xc0+1 (lanes 2m and 2m+1
  // hold the two row halves of wave w's eight rows for the same two columns), so that per step
  // a lane reads four row factors of each kind and two column factors.
  const int half = lane & 1;
  const int xr0 = kRows * wave + 4 * half;
  const int xc0 = 2 * (lane >> 1);
  float X[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a) X[a][0] = X[a][1] = 0.f;
  const long head_off = (long)h * kHead * kHead;
  // After the chunked passes: only the units they marked (the mark sits in this unit's dw
  // element of the last token, which no sweep writes before the dk/dw sweep reads it here).
  if (p.marked_only && T > 0 &&
      __float_as_uint(p.dw[(row0 + T - 1) * C + (long)h * kHead]) != kBwdFallbackMark)
    return;
  // A batch row whose state_map entry is out of range is skipped by all three sweeps
  // alike (its token and state gradients are not written), and its share of du is
  // zero, so du still sums the other rows.
  if (p.state_in) {
    const int row_in = p.state_map ? p.state_map[b] : (p.n_state == 1 ? 0 : b);
    if (row_in < 0 || row_in >= p.n_state) {
      if (MODE == TFWD) {
        if (tid == 0 && p.dev_status) atomicOr(p.dev_status, WKV_DEV_BAD_STATE_MAP);
        if (wave == 0 && p.du_rows) p.du_rows[(long)b * C + h * kHead + lane] = 0.f;
      }
      return;
    }
  }
  if (MODE == TFWD) {
    if (p.state_in) {
      const int row_in = p.state_map ? p.state_map[b] : (p.n_state == 1 ? 0 : b);
      const float *s0 = p.state_in + (long)row_in * p.H * kHead * kHead + head_off;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c) X[a][c] = s0[(xc0 + c) * kHead + xr0 + a];  // X[j][i] = S0[i][j]
    }
  } else if (p.d_state_out) {
    const float *g = p.d_state_out + (long)b * p.H * kHead * kHead + head_off;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        X[a][c] = COLDECAY ? g[(xc0 + c) * kHead + xr0 + a] : g[(xr0 + a) * kHead + xc0 + c];
  }
  // TBWD: the decay gradient of channel `lane` as one running difference (every wave holds the
  // same copy).  The two sums over the sequence grow with its length while their difference
  // does not, so the difference itself is carried, with a compensation term (Kahan) across
  // blocks: rounding stays relative to the difference and the per-block terms, not to the sums.
  float dsum = 0.f, dcomp = 0.f, dusum = 0.f;
  auto dadd = [&](float x) {
    const float yk = x - dcomp;
    const float t = dsum + yk;
    dcomp = (t - dsum) - yk;
    dsum = t;
  };
  if (MODE == TBWD && p.d_state_out && p.state_final) {
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
  // Blocks in processing order.  The dk/dw sweep takes the ragged block first, so that its later
  // blocks start on tokens kSpan * c - 1 (the forward sweep's span ends); the others take it last.
  const int nb0 = (MODE == TBWD && T % KTB != 0) ? T % KTB : KTB;
  // dk/dw sweep: the kept state of the next span end, loaded one block ahead (this thread's tile)
  float ck[4][2];
  auto fetch_kept = [&](int q1) {
    if (MODE == TBWD && q1 > 0 && q1 < T && (T - q1) % kSpan == 0) {
      const long t0 = row0 + (T - q1) - kHead;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const float *sv = &p.dw[(t0 + xr0 + a) * C + h * kHead + xc0];  // dw is only 4-byte aligned
        ck[a][0] = sv[0];
        ck[a][1] = sv[1];
      }
    }
  };
  if (T > 0) fetch(0);
  fetch_kept(nb0);
  for (int q0 = 0, nbn = nb0; q0 < T; q0 += nbn, nbn = KTB) {
    const int nb = min(nbn, T - q0);
    if (MODE == TBWD && q0 > 0 && (T - q0) % kSpan == 0) {
      // ck: the state S after token T-1-q0, left by the forward sweep in this head's dw rows of
      // the kHead tokens up to that one (row j holds S[.][j]), in the same tile layout as X = G^T.
      // E[i] = sum_j G[i][j] S[i][j] is the exact value of the running difference here.
      float e0 = 0.f, e1 = 0.f;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        e0 = fmaf(X[a][0], ck[a][0], e0);
        e1 = fmaf(X[a][1], ck[a][1], e1);
      }
      e0 += xor_lane1(e0);
      e1 += xor_lane1(e1);
      sm.ek[wave][xc0 + half] = half ? e1 : e0;  // read after the staging barrier below
    }
    // ---- stage this block (token of step q0 + tt at row tt).  Part 1: the factors that do
    // not depend on the frame, the bonus scalars, and the log2 decays (lam2 = log2 d) with
    // this thread's running sums in processing order (exclusive cex, inclusive cin).
    float bon[TPW], lam2[TPW], cex[TPW], cin[TPW], fp[TPW], fq[TPW];
    float run = 0.f;
#pragma unroll
    for (int t4 = 0; t4 < TPW; ++t4) {
      const int tt = TPW * wave + t4;
      const float ex = fast_exp(px[t4]);
      lam2[t4] = -ex * kLog2e;
      cex[t4] = run;
      run += lam2[t4];
      cin[t4] = run;
      if (MODE == TFWD) {
        fp[t4] = pdy[t4];
        fq[t4] = pv[t4];
        s_r[tt][lane] = pk[t4];
        s_e0[tt][lane] = pr[t4];
        bon[t4] = pdy[t4] * pv[t4];
      } else if (MODE == BWD) {
        fp[t4] = pk[t4];
        fq[t4] = pr[t4];
        s_r[tt][lane] = pdy[t4];
        bon[t4] = pk[t4] * uc * pr[t4];
      } else {
        fp[t4] = pv[t4];
        fq[t4] = pdy[t4];
        s_r[tt][lane] = pr[t4];
        s_e0[tt][lane] = pk[t4];
        s_e1[tt][lane] = pdr[t4];
        s_e2[tt][lane] = -ex;
        bon[t4] = pv[t4] * pdy[t4];
      }
    }
    sm.tot[wave][lane] = run;
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
    // Part 2.  With D_t the decay product from the block start through step t (per channel,
    // processing order), the registers carry X / D in the rescaled frame, so each step is two
    // FMAs per state element: out += P' X', X' += Q' R', and X = D_last X' at the block end.
    //   row decay (BWD):     P' = P D_{t-1},  Q' = Q / D_t,  R' = R
    //   column decay:        P' = P,  Q' = Q,  R' = R / D_t, and out is scaled by D_{t-1}
    // A block whose decay product falls below 2^-kFrameLog2 in some channel takes the direct
    // form X <- d X + Q R (the same decision in every wave: each sums all waves' totals).
    float before = 0.f, total = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float t = sm.tot[w][lane];
      before += w < wave ? t : 0.f;
      total += t;
    }
    const bool direct = __any(!(total >= -kFrameLog2));
    if (MODE == TBWD && q0 > 0 && (T - q0) % kSpan == 0) {  // restart the carry (fixed order)
      float e = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) e += sm.ek[w][lane];
      dsum = e;
      dcomp = 0.f;
    }
#pragma unroll
    for (int t4 = 0; t4 < TPW; ++t4) {
      const int tt = TPW * wave + t4;
      const float ce = before + cex[t4], ci = before + cin[t4];
      if (direct) {
        s_p[tt][lane] = fp[t4];
        s_q[tt][lane] = fq[t4];
        s_al[tt][lane] = __builtin_amdgcn_exp2f(lam2[t4]);
      } else if (!COLDECAY) {
        s_p[tt][lane] = fp[t4] * __builtin_amdgcn_exp2f(ce);
        s_q[tt][lane] = fq[t4] * __builtin_amdgcn_exp2f(-ci);
      } else {
        s_p[tt][lane] = fp[t4];
        s_q[tt][lane] = fq[t4];
        s_rt[tt][lane] = s_r[tt][lane] * __builtin_amdgcn_exp2f(-ci);
        s_al[tt][lane] = __builtin_amdgcn_exp2f(ce);
      }
      if (tt == nb - 1) sm.dend[lane] = __builtin_amdgcn_exp2f(ci);
    }
    fetch(q0 + nb);  // in flight during this block
    fetch_kept(q0 + nb);
    __syncthreads();

    // ---- the recurrence over the block's tokens.  ya, yb: this lane's partial outputs of
    // columns xc0 and xc0 + 1 over its four rows; the two row halves are added across the lane
    // pair, and lane 2m + half stores column xc0 + half of the wave's partial.
    auto store_out = [&](int tt, float ya, float yb) {
      const float send = half ? ya : yb;
      const float mine = half ? yb : ya;
      s_y[tt][wave][xc0 + half] = mine + xor_lane1(send);
    };
    if (!direct) {
      auto frame_step = [&](int tt) {
        const float2 rc = *reinterpret_cast<const float2 *>(COLDECAY ? &s_rt[tt][xc0] : &s_r[tt][xc0]);
        const float4 p4 = *reinterpret_cast<const float4 *>(&s_p[tt][xr0]);
        const float4 q4 = *reinterpret_cast<const float4 *>(&s_q[tt][xr0]);
        const float pp[4] = {p4.x, p4.y, p4.z, p4.w}, qq[4] = {q4.x, q4.y, q4.z, q4.w};
        float ya = pp[0] * X[0][0], yb = pp[0] * X[0][1];
        X[0][0] = fmaf(qq[0], rc.x, X[0][0]);
        X[0][1] = fmaf(qq[0], rc.y, X[0][1]);
#pragma unroll
        for (int a = 1; a < 4; ++a) {
          ya = fmaf(pp[a], X[a][0], ya);
          yb = fmaf(pp[a], X[a][1], yb);
          X[a][0] = fmaf(qq[a], rc.x, X[a][0]);
          X[a][1] = fmaf(qq[a], rc.y, X[a][1]);
        }
        store_out(tt, ya, yb);
      };
      // four steps per iteration, so that the LDS offsets of the steps are constants
      int tt = 0;
      for (; tt + 4 <= nb; tt += 4) {
        frame_step(tt);
        frame_step(tt + 1);
        frame_step(tt + 2);
        frame_step(tt + 3);
      }
      for (; tt < nb; ++tt) frame_step(tt);
      if (COLDECAY) {
        const float2 dd = *reinterpret_cast<const float2 *>(&sm.dend[xc0]);
#pragma unroll
        for (int a = 0; a < 4; ++a) { X[a][0] *= dd.x; X[a][1] *= dd.y; }
      } else {
        const float4 d4 = *reinterpret_cast<const float4 *>(&sm.dend[xr0]);
        const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int a = 0; a < 4; ++a) { X[a][0] *= dd[a]; X[a][1] *= dd[a]; }
      }
    } else {
      for (int tt = 0; tt < nb; ++tt) {
        const float2 rc = *reinterpret_cast<const float2 *>(&s_r[tt][xc0]);
        const float4 p4 = *reinterpret_cast<const float4 *>(&s_p[tt][xr0]);
        const float4 q4 = *reinterpret_cast<const float4 *>(&s_q[tt][xr0]);
        const float pp[4] = {p4.x, p4.y, p4.z, p4.w}, qq[4] = {q4.x, q4.y, q4.z, q4.w};
        float ya = 0.f, yb = 0.f;
        if (COLDECAY) {
          const float2 ac = *reinterpret_cast<const float2 *>(&s_al[tt][xc0]);
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            ya = fmaf(pp[a], X[a][0], ya);
            yb = fmaf(pp[a], X[a][1], yb);
            X[a][0] = fmaf(ac.x, X[a][0], qq[a] * rc.x);
            X[a][1] = fmaf(ac.y, X[a][1], qq[a] * rc.y);
          }
        } else {
          const float4 a4 = *reinterpret_cast<const float4 *>(&s_al[tt][xr0]);
          const float aa[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            ya = fmaf(pp[a], X[a][0], ya);
            yb = fmaf(pp[a], X[a][1], yb);
            X[a][0] = fmaf(aa[a], X[a][0], qq[a] * rc.x);
            X[a][1] = fmaf(aa[a], X[a][1], qq[a] * rc.y);
          }
        }
        store_out(tt, ya, yb);
      }
    }
    __syncthreads();

    if (MODE == TFWD && (q0 + nb) % kSpan == 0 && q0 + nb < T) {
      // S after token q0+nb-1 (X = S^T, in plain form at the block end) into this head's dw rows
      // of the kHead tokens up to that one; the dk/dw sweep reads it before it writes them.
      const long t0 = row0 + q0 + nb - kHead;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float *sv = &p.dw[(t0 + xr0 + a) * C + h * kHead + xc0];
        sv[0] = X[a][0];
        sv[1] = X[a][1];
      }
    }
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
        if (COLDECAY && !direct) {  // the frame's output factor D_{t-1} of column c + m
#pragma unroll
          for (int m = 0; m < CPT; ++m) o[m] *= s_al[tt][c + m];
        }
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
    // ---- sums over time, one channel per lane, in processing order
    if (MODE == TFWD && wave == 0) {
      for (int tt = 0; tt < nb; ++tt) dusum += s_w[tt][lane];
    }
    if (MODE == TBWD) {
      // dlam at step t = carry + sum over the block's earlier steps m of (r_m dr~_m - k_m dk~_m)
      // - k_t dk~_t.  Every wave takes TPW consecutive steps: in-wave running sums, the totals of
      // the earlier waves through LDS, and the block total added to the carry (each wave keeps
      // the same carry: it adds the same totals in the same order).
      float ex[TPW], run2 = 0.f;
#pragma unroll
      for (int t4 = 0; t4 < TPW; ++t4) {
        const int tt = TPW * wave + t4;
        ex[t4] = run2;
        run2 += tt < nb ? s_e1[tt][lane] - s_w[tt][lane] : 0.f;
      }
      sm.tot[wave][lane] = run2;
      __syncthreads();
      float before = 0.f, total = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float t = sm.tot[w][lane];
        before += w < wave ? t : 0.f;
        total += t;
      }
      const float carry = dsum + before;
#pragma unroll
      for (int t4 = 0; t4 < TPW; ++t4) {
        const int tt = TPW * wave + t4;
        if (tt < nb) p.dw[tok(q0 + tt) * C + h * kHead + lane] = s_e2[tt][lane] * ((carry + ex[t4]) - s_w[tt][lane]);
      }
      dadd(total);
    }
    // The next staging writes the token arrays after this block's reads (ordered by this
    // barrier); s_y is written again only after the next staging barrier.
    __syncthreads();
  }

  if (MODE == TFWD && wave == 0 && p.du_rows) p.du_rows[(long)b * C + h * kHead + lane] = dusum;
  if (MODE == BWD && p.d_state_in) {
    float *g = p.d_state_in + (long)b * p.H * kHead * kHead + head_off;
#pragma unroll
    for (int a = 0; a < 4; ++a) {  // d_state_in is only 4-byte aligned: two 4-byte stores
      g[(xr0 + a) * kHead + xc0] = X[a][0];
      g[(xr0 + a) * kHead + xc0 + 1] = X[a][1];
    }
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
