// WKV v4: channel-wise exponential-decay weighted average with a bonus on the
// current token (the RWKV-v4 walk-through page, RWKV_TimeMix.forward: the WKV
// of (time_decay, time_first, k, v), gated by sigmoid(r)).
//
// Per channel c with lambda = -exp(time_decay[c]) and u = time_first[c], the
// state (a, b, p) stands for numerator A = a e^p and denominator B = b e^p:
//   out:    q = max(p, u + k_t)
//           wkv_t = (e^(p-q) a + e^(u+k_t-q) v_t) / (e^(p-q) b + e^(u+k_t-q))
//   update: q' = max(p + lambda, k_t)
//           a <- e^(p+lambda-q') a + e^(k_t-q') v_t ; b likewise with v = 1 ; p <- q'
// Keeping p as the running maximum exponent makes every exponential <= 1, so
// nothing overflows however large k or the sequence gets.  One of the two
// exponentials of each pair is exactly 1 (its argument is 0), so only one is
// evaluated.
//
// Time is split into G segments so that B*C channels alone need not fill the
// chip.  A workgroup owns 64 channels of one batch row and G waves, wave g
// owning tokens [g*L, g*L + L).  The recurrence is affine in (A, B), so a
// segment acts on the state entering it as
//   A_out = e^(L lambda) A_in + A_seg,   B_out = e^(L lambda) B_in + B_seg,
// with (A_seg, B_seg) the segment's state from a zero start.  Pass 1: every
// wave but the last computes its segment's (a, b, p) from zero.  Pass 2: wave g
// folds the initial state and segments 0..g-1 (through LDS) into its entry
// state.  Pass 3: every wave rescans its segment from that state, writing y;
// the last wave writes the final state.  k and v are read twice; the second
// read follows the first within the same workgroup.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace wkv {
namespace {

constexpr int kLanes = 64;   // channels per workgroup (one per lane)
constexpr int kMaxSeg = 16;  // waves (time segments) per workgroup
constexpr int kBlk = 8;      // tokens loaded per batch of loads

// (a, b, p) <- the state after absorbing one token (k, v) with per-step log decay lam.
__device__ __forceinline__ void absorb(float &a, float &b, float &p, float lam, float k, float v) {
  const float wd = p + lam;
  const float ex = fast_exp(-fabsf(wd - k));
  const bool dbig = wd >= k;
  const float f1 = dbig ? 1.f : ex;
  const float f2 = dbig ? ex : 1.f;
  a = f1 * a + f2 * v;
  b = f1 * b + f2;
  p = dbig ? wd : k;
}

template <bool BF16, bool HAS_R>
__global__ void __launch_bounds__(kLanes * kMaxSeg) wkv4_scan_kernel(V4Params p, int seg_len) {
  __shared__ float agg[kMaxSeg][3][kLanes];
  const int lane = threadIdx.x & (kLanes - 1);
  const int g = threadIdx.x / kLanes;
  const int G = blockDim.x / kLanes;
  const int c = blockIdx.x * kLanes + lane;
  const int b = blockIdx.y;
  const bool live = c < p.C;
  const long C = p.C;
  const int t0 = min(g * seg_len, p.T);
  const int t1 = min(t0 + seg_len, p.T);
  const float lam = live ? -fast_exp(p.tau[c]) : 0.f;
  const float u = live ? p.u[c] : 0.f;
  const long base = (long)b * p.T * C + c;

  // pass 1: segment aggregate from a zero state (the last segment's is never needed)
  if (g + 1 < G) {
    float a = 0.f, bb = 0.f, pp = -1e38f;
    if (live) {
      for (int t = t0; t < t1; t += kBlk) {
        float kk[kBlk], vv[kBlk];
#pragma unroll
        for (int j = 0; j < kBlk; ++j) {
          const int tt = min(t + j, t1 - 1);
          kk[j] = load1<BF16>(p.k, base + (long)tt * C);
          vv[j] = load1<BF16>(p.v, base + (long)tt * C);
        }
#pragma unroll
        for (int j = 0; j < kBlk; ++j)
          if (t + j < t1) absorb(a, bb, pp, lam, kk[j], vv[j]);
      }
    }
    agg[g][0][lane] = a;
    agg[g][1][lane] = bb;
    agg[g][2][lane] = pp;
  }
  __syncthreads();
  if (!live) return;

  // pass 2: entry state of this segment
  float a = 0.f, bb = 0.f, pp = -1e38f;
  if (p.state_in) {
    a = p.state_in[(3L * b + 0) * C + c];
    bb = p.state_in[(3L * b + 1) * C + c];
    pp = p.state_in[(3L * b + 2) * C + c];
  }
  const float lam_seg = lam * (float)seg_len;
  for (int j = 0; j < g; ++j) {
    const float sa = agg[j][0][lane], sb = agg[j][1][lane], sp = agg[j][2][lane];
    const float wd = pp + lam_seg;
    const float ex = fast_exp(-fabsf(wd - sp));
    const bool dbig = wd >= sp;
    const float f1 = dbig ? 1.f : ex;
    const float f2 = dbig ? ex : 1.f;
    a = f1 * a + f2 * sa;
    bb = f1 * bb + f2 * sb;
    pp = dbig ? wd : sp;
  }

  // pass 3: outputs of this segment
  for (int t = t0; t < t1; t += kBlk) {
    float kk[kBlk], vv[kBlk], rr[kBlk];
#pragma unroll
    for (int j = 0; j < kBlk; ++j) {
      const int tt = min(t + j, t1 - 1);
      kk[j] = load1<BF16>(p.k, base + (long)tt * C);
      vv[j] = load1<BF16>(p.v, base + (long)tt * C);
      rr[j] = HAS_R ? load1<BF16>(p.r, base + (long)tt * C) : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kBlk; ++j) {
      if (t + j >= t1) break;
      const float kt = kk[j], vt = vv[j];
      const float ww = u + kt;
      const float ex = fast_exp(-fabsf(pp - ww));  // e^(min - max)
      const bool pbig = pp >= ww;
      const float e1 = pbig ? 1.f : ex;
      const float e2 = pbig ? ex : 1.f;
      float out = (e1 * a + e2 * vt) * fast_rcp(e1 * bb + e2);
      if (HAS_R) out *= fast_rcp(1.f + fast_exp(-rr[j]));
      p.y[base + (long)(t + j) * C] = out;
      absorb(a, bb, pp, lam, kt, vt);
    }
  }
  if (g + 1 == G && p.state_out) {
    p.state_out[(3L * b + 0) * C + c] = a;
    p.state_out[(3L * b + 1) * C + c] = bb;
    p.state_out[(3L * b + 2) * C + c] = pp;
  }
}

template <bool BF16, bool HAS_R>
hipError_t launch(const V4Params &p, hipStream_t s) {
  const int cblocks = (p.C + kLanes - 1) / kLanes;
  // Enough waves to cover the chip (about 16 per CU on 256 CUs) without segments shorter than 16 tokens.
  const long want = (4096L + (long)cblocks * p.B - 1) / ((long)cblocks * p.B);
  int G = (int)std::min<long>(kMaxSeg, std::max<long>(1, want));
  G = std::max(1, std::min(G, (p.T + 15) / 16));
  const int seg_len = p.T > 0 ? (p.T + G - 1) / G : 0;
  if (p.T > 0) G = (p.T + seg_len - 1) / seg_len;  // every segment non-empty
  dim3 grid(cblocks, p.B);
  hipLaunchKernelGGL((wkv4_scan_kernel<BF16, HAS_R>), grid, dim3(kLanes * G), 0, s, p, seg_len);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_wkv4(const V4Params &p, bool bf16, hipStream_t s) {
  const bool r = p.r != nullptr;
  if (bf16) return r ? launch<true, true>(p, s) : launch<true, false>(p, s);
  return r ? launch<false, true>(p, s) : launch<false, false>(p, s);
}

}  // namespace wkv
