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
//
// Rounds whose tokens all exist (and 64 | C) take a straight-line path: the
// tokens are read with buffer loads whose per-token offsets are scalar; the
// next round's k and v are requested right after the first barrier, into a
// second register set, so their latency hides behind the fold and the
// rescan, and a round's r (needed only by the rescan) is requested as the
// round starts.  The last, partial round takes the guarded path.
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

// y for one token from the state before it: the weighted average with the
// bonus u on the current token, times sigmoid(r) (one reciprocal for both).
template <bool HAS_R>
__device__ __forceinline__ float wkv_out(float a, float b, float p, float u, float k, float v, float r) {
  const float ww = u + k;
  const float ex = fast_exp(-fabsf(p - ww));  // e^(min - max)
  const bool pbig = p >= ww;
  const float e1 = pbig ? 1.f : ex;
  const float e2 = pbig ? ex : 1.f;
  float den = e1 * b + e2;
  if (HAS_R) den *= 1.f + fast_exp(-r);
  return (e1 * a + e2 * v) * fast_rcp(den);
}

template <bool BF16>
__device__ __forceinline__ float buf_load(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
  if constexpr (BF16) return bf16_lo(__builtin_amdgcn_raw_buffer_load_b16(rs, voff, soff, 0));
  else return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0));
}

template <bool BF16, bool HAS_R, bool OUTB>
__global__ void __launch_bounds__(kLanes * kMaxSeg) wkv4_scan_kernel(V4Params p) {
  __shared__ float agg[kMaxSeg][3][kLanes];
  __shared__ float rstate[3][kLanes];
  const int lane = threadIdx.x & (kLanes - 1);
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);  // wave-uniform
  const int G = blockDim.x / kLanes;
  const int c = blockIdx.x * kLanes + lane;
  const int b = blockIdx.y;
  const bool live = c < p.C;
  const long C = p.C;
  const float lam = live ? -fast_exp(p.tau[c]) : 0.f;
  const float u = live ? p.u[c] : 0.f;
  const long base = (long)b * p.T * C + c;
  const long base_ld = (long)b * p.T * C + (live ? c : p.C - 1);

  // entry state of the current round (the same in every wave)
  float ra = 0.f, rb = 0.f, rp = -1e38f;
  if (live && p.state_in) {
    ra = p.state_in[(3L * b + 0) * C + c];
    rb = p.state_in[(3L * b + 1) * C + c];
    rp = p.state_in[(3L * b + 2) * C + c];
  }
  const int per_round = G * kSeg;
  int r_begin = 0;  // first token the guarded path handles
  if (p.C % kLanes == 0 && (long)per_round * C * 4 <= 0x7fffffffL) {
    constexpr int kElt = BF16 ? 2 : 4;
    const int full_rounds = p.T / per_round;
    const int voff = c * kElt;                         // this lane's channel
    const int soff_g = g * kSeg * (int)C * kElt;       // this wave's first token in a round
    const int tstride = (int)C * kElt;                 // one token row
    // resources covering one round of one batch row
    auto rsrc = [&](const void *base, int r0) {
      const char *q = static_cast<const char *>(base) + ((long)b * p.T + r0) * C * kElt;
      return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(q), 0, per_round * (int)C * kElt, 0x00020000);
    };
    float ka[kSeg], va[kSeg], kb[kSeg], vb[kSeg];
    auto load_kv = [&](int r0, float (&kk)[kSeg], float (&vv)[kSeg]) {
      const auto rk = rsrc(p.k, r0), rv = rsrc(p.v, r0);
#pragma unroll
      for (int j = 0; j < kSeg; ++j) {
        kk[j] = buf_load<BF16>(rk, voff, soff_g + j * tstride);
        vv[j] = buf_load<BF16>(rv, voff, soff_g + j * tstride);
      }
    };
    // one full round from the registers (kk, vv); requests the next round's k, v into (nk, nv)
    auto full_round = [&](int r0, float (&kk)[kSeg], float (&vv)[kSeg], float (&nk)[kSeg], float (&nv)[kSeg],
                          bool more) {
      float rr[kSeg];
      if (HAS_R) {
        const auto rr_ = rsrc(p.r, r0);
#pragma unroll
        for (int j = 0; j < kSeg; ++j) rr[j] = buf_load<BF16>(rr_, voff, soff_g + j * tstride);
      }
      __builtin_amdgcn_sched_barrier(0);  // issue the r loads now, ahead of the segment aggregate
      float a = vv[0], bb = 1.f, pp = kk[0];  // the first token absorbed into a zero state
#pragma unroll
      for (int j = 1; j < kSeg; ++j) absorb(a, bb, pp, lam, kk[j], vv[j]);
      agg[g][0][lane] = a;
      agg[g][1][lane] = bb;
      agg[g][2][lane] = pp;
      __syncthreads();
      if (more) load_kv(r0 + per_round, nk, nv);
      a = ra; bb = rb; pp = rp;
      const float lam_seg = lam * (float)kSeg;
      for (int w = 0; w < g; ++w) fold(a, bb, pp, lam_seg, agg[w][0][lane], agg[w][1][lane], agg[w][2][lane]);
      constexpr int kOut = OUTB ? 2 : 4;
      const auto ry = __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<char *>(p.y) + ((long)b * p.T + r0) * C * kOut, 0, per_round * (int)C * kOut, 0x00020000);
      const int soff_y = g * kSeg * (int)C * kOut;
#pragma unroll
      for (int j = 0; j < kSeg; ++j) {
        const float out = wkv_out<HAS_R>(a, bb, pp, u, kk[j], vv[j], HAS_R ? rr[j] : 0.f);
        if constexpr (OUTB)
          __builtin_amdgcn_raw_buffer_store_b16(bf16_bits(out), ry, c * 2, soff_y + j * (int)C * 2, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(out), ry, c * 4, soff_y + j * (int)C * 4, 0);
        absorb(a, bb, pp, lam, kk[j], vv[j]);
      }
      if (g == G - 1) {  // this wave holds the round's last token
        rstate[0][lane] = a;
        rstate[1][lane] = bb;
        rstate[2][lane] = pp;
      }
      __syncthreads();
      ra = rstate[0][lane];
      rb = rstate[1][lane];
      rp = rstate[2][lane];
    };
    if (full_rounds > 0) load_kv(0, ka, va);
    int r = 0;
    for (; r + 2 <= full_rounds; r += 2) {
      full_round(r * per_round, ka, va, kb, vb, true);
      full_round((r + 1) * per_round, kb, vb, ka, va, r + 2 < full_rounds);
    }
    if (r < full_rounds) full_round(r * per_round, ka, va, kb, vb, false);
    r_begin = full_rounds * per_round;
  }
  for (int r0 = r_begin; r0 < p.T; r0 += per_round) {
    const int t0 = r0 + g * kSeg;
    const int n = max(0, min(kSeg, p.T - t0));
    float kk[kSeg], vv[kSeg], rr[kSeg];
#pragma unroll
    for (int j = 0; j < kSeg; ++j) {
      // rows past the end reread the last one and lanes past C read channel C - 1: unused,
      // and the loads need no branch
      const long e = base_ld + (long)min(t0 + j, p.T - 1) * C;
      kk[j] = load1<BF16>(p.k, e);
      vv[j] = load1<BF16>(p.v, e);
      rr[j] = HAS_R ? load1<BF16>(p.r, e) : 0.f;
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
        if (j < n) {  // n is wave-uniform
          const float out = wkv_out<HAS_R>(a, bb, pp, u, kk[j], vv[j], rr[j]);
          if (live) {
            if constexpr (OUTB) static_cast<uint16_t *>(p.y)[base + (long)(t0 + j) * C] = bf16_bits(out);
            else static_cast<float *>(p.y)[base + (long)(t0 + j) * C] = out;
          }
          absorb(a, bb, pp, lam, kk[j], vv[j]);
        }
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

template <bool BF16, bool HAS_R, bool OUTB>
hipError_t launch(const V4Params &p, hipStream_t s) {
  const int cblocks = (p.C + kLanes - 1) / kLanes;
  // Enough waves to cover the chip (about 16 per CU on 256 CUs), but no more segments than tokens need.
  const long want = (4096L + (long)cblocks * p.B - 1) / ((long)cblocks * p.B);
  int G = (int)std::min<long>(kMaxSeg, std::max<long>(1, want));
  G = std::max(1, std::min(G, (p.T + kSeg - 1) / kSeg));
  dim3 grid(cblocks, p.B);
  hipLaunchKernelGGL((wkv4_scan_kernel<BF16, HAS_R, OUTB>), grid, dim3(kLanes * G), 0, s, p);
  return hipGetLastError();
}

template <bool OUTB>
hipError_t launch_out(const V4Params &p, bool bf16, hipStream_t s) {
  const bool r = p.r != nullptr;
  if (bf16) return r ? launch<true, true, OUTB>(p, s) : launch<true, false, OUTB>(p, s);
  return r ? launch<false, true, OUTB>(p, s) : launch<false, false, OUTB>(p, s);
}

}  // namespace

hipError_t launch_wkv4(const V4Params &p, bool bf16, hipStream_t s) {
  return p.y_bf16 ? launch_out<true>(p, bf16, s) : launch_out<false>(p, bf16, s);
}

}  // namespace wkv
