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
#include "common.hpp"
#include "kernels.hpp"

namespace wkv {
namespace {

constexpr int kThreads = 64;

template <bool BF16, bool HAS_R>
__global__ void __launch_bounds__(kThreads) wkv4_scan_kernel(V4Params p) {
  const int c = blockIdx.x * kThreads + threadIdx.x;
  const int b = blockIdx.y;
  if (c >= p.C) return;
  const long C = p.C;
  const float lam = -fast_exp(p.tau[c]);
  const float u = p.u[c];
  float a = 0.f, bb = 0.f, pp = -1e38f;
  if (p.state_in) {
    a = p.state_in[(3L * b + 0) * C + c];
    bb = p.state_in[(3L * b + 1) * C + c];
    pp = p.state_in[(3L * b + 2) * C + c];
  }
  const long base = (long)b * p.T * C + c;
  float kn = 0.f, vn = 0.f, rn = 0.f;
  if (p.T > 0) {
    kn = load1<BF16>(p.k, base);
    vn = load1<BF16>(p.v, base);
    if (HAS_R) rn = load1<BF16>(p.r, base);
  }
  for (int t = 0; t < p.T; ++t) {
    const long e = base + (long)t * C;
    const float kt = kn, vt = vn, rt = rn;
    if (t + 1 < p.T) {  // prefetch the next token
      kn = load1<BF16>(p.k, e + C);
      vn = load1<BF16>(p.v, e + C);
      if (HAS_R) rn = load1<BF16>(p.r, e + C);
    }
    // output with the bonus on the current token
    const float ww = u + kt;
    const float ex = fast_exp(-fabsf(pp - ww));  // e^(min - max)
    const bool pbig = pp >= ww;
    const float e1 = pbig ? 1.f : ex;
    const float e2 = pbig ? ex : 1.f;
    float out = (e1 * a + e2 * vt) * fast_rcp(e1 * bb + e2);
    if (HAS_R) out *= fast_rcp(1.f + fast_exp(-rt));
    p.y[e] = out;
    // decay the state and absorb this token
    const float wd = pp + lam;
    const float ex2 = fast_exp(-fabsf(wd - kt));
    const bool dbig = wd >= kt;
    const float f1 = dbig ? 1.f : ex2;
    const float f2 = dbig ? ex2 : 1.f;
    a = f1 * a + f2 * vt;
    bb = f1 * bb + f2;
    pp = dbig ? wd : kt;
  }
  if (p.state_out) {
    p.state_out[(3L * b + 0) * C + c] = a;
    p.state_out[(3L * b + 1) * C + c] = bb;
    p.state_out[(3L * b + 2) * C + c] = pp;
  }
}

template <bool BF16, bool HAS_R>
hipError_t launch(const V4Params &p, hipStream_t s) {
  dim3 grid((p.C + kThreads - 1) / kThreads, p.B);
  hipLaunchKernelGGL((wkv4_scan_kernel<BF16, HAS_R>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_wkv4(const V4Params &p, bool bf16, hipStream_t s) {
  const bool r = p.r != nullptr;
  if (bf16) return r ? launch<true, true>(p, s) : launch<true, false>(p, s);
  return r ? launch<false, true>(p, s) : launch<false, false>(p, s);
}

}  // namespace wkv
