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
// Time is split into segments so that B*C channels alone need not fill the
// chip.  A workgroup owns 64 channels of one batch row and G waves; the
// sequence is walked in rounds of G*16 tokens, wave g owning tokens
// [16g, 16g + 16) of the round.  The recurrence is affine in (A, B), so a
// segment of n tokens acts on the state entering it as
//   A_out = e^(n lambda) A_in + A_seg,   B_out = e^(n lambda) B_in + B_seg,
// with (A_seg, B_seg) the segment's state from a zero start.  Each round:
// every wave loads its 16 tokens into registers, forms its segment's
// (a, b, p) from zero and posts it to LDS;
// after a barrier it folds the round's entry state and the segments before
// its own into its entry state and rescans its tokens, writing y; the wave
// holding the round's last token posts the state it ends with, which every
// wave picks up after the second barrier as the next round's entry state.
// k, v and r are read once.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace wkv {
namespace {

constexpr int kLanes = 64;   // channels per workgroup (one per lane)
constexpr int kMaxSeg = 16;  // waves (time segments) per workgroup
constexpr int kSeg = 16;     // tokens per wave and round, held in registers

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

// (a, b, p) <- a segment with aggregate (sa, sb, sp) applied after decaying by lam_seg.
__device__ __forceinline__ void fold(float &a, float &b, float &p, float lam_seg, float sa, float sb, float sp) {
  const float wd = p + lam_seg;
  const float ex = fast_exp(-fabsf(wd - sp));
  const bool dbig = wd >= sp;
  const float f1 = dbig ? 1.f : ex;
  const float f2 = dbig ? ex : 1.f;
  a = f1 * a + f2 * sa;
  b = f1 * b + f2 * sb;
  p = dbig ? wd : sp;
}

template <bool BF16, bool HAS_R>
__global__ void __launch_bounds__(kLanes * kMaxSeg) wkv4_scan_kernel(V4Params p) {
  __shared__ float agg[kMaxSeg][3][kLanes];
  __shared__ float rstate[3][kLanes];
  const int lane = threadIdx.x & (kLanes - 1);
  const int g = threadIdx.x / kLanes;
  const int G = blockDim.x / kLanes;
  const int c = blockIdx.x * kLanes + lane;
  const int b = blockIdx.y;
  const bool live = c < p.C;
  const long C = p.C;
  const float lam = live ? -fast_exp(p.tau[c]) : 0.f;
  const float u = live ? p.u[c] : 0.f;
  const long base = (long)b * p.T * C + c;

  // entry state of the current round (the same in every wave)
  float ra = 0.f, rb = 0.f, rp = -1e38f;
  if (live && p.state_in) {
    ra = p.state_in[(3L * b + 0) * C + c];
    rb = p.state_in[(3L * b + 1) * C + c];
    rp = p.state_in[(3L * b + 2) * C + c];
  }
  const int per_round = G * kSeg;
  for (int r0 = 0; r0 < p.T; r0 += per_round) {
    const int t0 = r0 + g * kSeg;
    const int n = max(0, min(kSeg, p.T - t0));
    float kk[kSeg], vv[kSeg], rr[kSeg];
#pragma unroll
    for (int j = 0; j < kSeg; ++j) {
      const long e = base + (long)min(t0 + j, p.T - 1) * C;  // rows past the end: reread the last, unused
      kk[j] = live ? load1<BF16>(p.k, e) : 0.f;
      vv[j] = live ? load1<BF16>(p.v, e) : 0.f;
      rr[j] = (HAS_R && live) ? load1<BF16>(p.r, e) : 0.f;
    }
    // segment aggregate from a zero state
    float a = 0.f, bb = 0.f, pp = -1e38f;
#pragma unroll
    for (int j = 0; j < kSeg; ++j)
      if (j < n) absorb(a, bb, pp, lam, kk[j], vv[j]);
    agg[g][0][lane] = a;
    agg[g][1][lane] = bb;
    agg[g][2][lane] = pp;
    __syncthreads();
    if (n > 0) {
      // entry state: the round's, then the (full) segments before this one
      a = ra; bb = rb; pp = rp;
      const float lam_seg = lam * (float)kSeg;
      for (int w = 0; w < g; ++w) fold(a, bb, pp, lam_seg, agg[w][0][lane], agg[w][1][lane], agg[w][2][lane]);
#pragma unroll
      for (int j = 0; j < kSeg; ++j) {
        if (j >= n) break;
        const float kt = kk[j], vt = vv[j];
        const float ww = u + kt;
        const float ex = fast_exp(-fabsf(pp - ww));  // e^(min - max)
        const bool pbig = pp >= ww;
        const float e1 = pbig ? 1.f : ex;
        const float e2 = pbig ? ex : 1.f;
        float out = (e1 * a + e2 * vt) * fast_rcp(e1 * bb + e2);
        if (HAS_R) out *= fast_rcp(1.f + fast_exp(-rr[j]));
        if (live) p.y[base + (long)(t0 + j) * C] = out;
        absorb(a, bb, pp, lam, kt, vt);
      }
      if (t0 + n == min(p.T, r0 + per_round)) {  // this wave holds the round's last token
        rstate[0][lane] = a;
        rstate[1][lane] = bb;
        rstate[2][lane] = pp;
      }
    }
    __syncthreads();
    ra = rstate[0][lane];
    rb = rstate[1][lane];
    rp = rstate[2][lane];
    // the next round's first barrier orders these reads before rstate is written again
  }
  if (g == 0 && live && p.state_out) {
    p.state_out[(3L * b + 0) * C + c] = ra;
    p.state_out[(3L * b + 1) * C + c] = rb;
    p.state_out[(3L * b + 2) * C + c] = rp;
  }
}

template <bool BF16, bool HAS_R>
hipError_t launch(const V4Params &p, hipStream_t s) {
  const int cblocks = (p.C + kLanes - 1) / kLanes;
  // Enough waves to cover the chip (about 16 per CU on 256 CUs), but no more segments than tokens need.
  const long want = (4096L + (long)cblocks * p.B - 1) / ((long)cblocks * p.B);
  int G = (int)std::min<long>(kMaxSeg, std::max<long>(1, want));
  G = std::max(1, std::min(G, (p.T + kSeg - 1) / kSeg));
  dim3 grid(cblocks, p.B);
  hipLaunchKernelGGL((wkv4_scan_kernel<BF16, HAS_R>), grid, dim3(kLanes * G), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_wkv4(const V4Params &p, bool bf16, hipStream_t s) {
  const bool r = p.r != nullptr;
  if (bf16) return r ? launch<true, true>(p, s) : launch<true, false>(p, s);
  return r ? launch<false, true>(p, s) : launch<false, false>(p, s);
}

}  // namespace wkv
