// 64-token chunked WKV v5 / v6 with the contractions on MFMA (gfx950).
//
// Same recurrence as the token-sequential scan (the rwkv_ops page's RWKV6_OP:
// r, k, v, w, u, init_state, state_map -> y, y_state; S indexed [key i][value j]):
//   y_t[j] = sum_i r_t[i] (S[i][j] + u[i] k_t[i] v_t[j]),  S[i][j] <- d_t[i] S[i][j] + k_t[i] v_t[j]
// rewritten exactly, chunk by chunk.  Inside a chunk of L = 64 tokens let
// Lam_t[i] = sum_{m<=t} log d_m[i] (inclusive, from the chunk start).  Then
//   rbar_t = r_t * exp(Lam_{t-1}),  ktil_s = k_s * exp(-Lam_s),  khat_s = k_s * exp(Lam_{L-1} - Lam_s)
//   A[t][s] = rbar_t . ktil_s  (s < t),  A[t][t] = sum_i r_t[i] u[i] k_t[i],  A[t][s] = 0 (s > t)
//   Y = A V + rbar S0                  (S0 = state at the chunk start)
//   S1 = diag(exp(Lam_{L-1})) S0 + khat^T V
// which equals the token recurrence in exact arithmetic.
//
// Precision.  Every MFMA runs on bf16 operands with fp32 accumulation.  V is
// the exact bf16 input; every other operand (rbar, ktil, khat, A, S) is split
// into hi = bf16(x) and lo = bf16(x - hi), and each product is formed as
// hi*hi + hi*lo + lo*hi (v only needs hi*v + lo*v), which keeps about 16
// significant bits per term.  All products that survive the mask are bounded
// by |r k| because exp(Lam_{t-1} - Lam_s) <= 1 for s < t.
//
// Range.  ktil carries exp(-Lam_s) >= 1.  A chunk whose accumulated log2
// decay in some channel is below -kMaxLog2 sets WKV_DEV_DECAY_RANGE (its
// outputs are not trustworthy; the token-sequential scan has no such limit).
// Per-step decays exp(-exp(x)) with x <= 0 stay far inside this range.
//
// Work decomposition.  One 512-thread workgroup (8 waves) per (batch row,
// head) walks the chunks in order with the fp32 state in MFMA accumulators.
//   precompute: thread (channel i, token group g of 8) loads its 8 tokens,
//     forms the log-decay prefix (group totals exchanged through LDS) and
//     writes rbar, ktil (row-major [token][channel]), khat and V transposed
//     ([channel][token]) as bf16 to LDS, plus the bonus diagonal.
//   MFMA: wave (jb, part) owns value columns 16jb..16jb+15; part 0 computes
//     output token blocks {0, 3}, part 1 blocks {1, 2} (equal MFMA counts),
//     and key-row blocks {0,1} / {2,3} of the state update.  Each wave forms
//     the A^T tiles it needs (v_mfma_f32_16x16x32_bf16), keeps them in
//     registers and feeds them straight back as the A operand of A V (the K
//     order of an accumulator tile is a permutation that the V operand
//     reads in the same order).  The state is exchanged between waves as
//     bf16 hi/lo S^T in a ping-pong LDS buffer.
#include "common.hpp"
#include "kernels.hpp"
#include "wkv.h"

namespace wkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int L = 64;          // tokens per chunk
constexpr int kThreads = 512;  // 8 waves
constexpr int RS = 72;         // LDS row stride in bf16 elements (144 bytes: conflict-free 16-lane b128 reads)
constexpr int BS = kHead + 4;  // row stride of the fp32 bonus partials
constexpr float kMaxLog2 = 100.f;

struct Smem {
  uint16_t rb_hi[L][RS], rb_lo[L][RS];            // rbar   [token][channel]
  uint16_t kt_hi[L][RS], kt_lo[L][RS];            // ktil   [token][channel]
  uint16_t kh_hi[kHead][RS], kh_lo[kHead][RS];    // khat^T [channel][token]
  uint16_t vt[kHead][RS];                         // V^T    [value col][token]
  uint16_t st_hi[2][kHead][RS], st_lo[2][kHead][RS];  // S^T [value col][key row], ping-pong
  float bp[L][BS];                                // bonus partials r*u*k [token][channel]
  float tot[8][kHead];                            // log2-decay total of each 8-token group
  float bonus[L];
  float pl[kHead];                                // exp(Lam_{L-1}) per key row
  int range_bad;
};

__device__ __forceinline__ uint16_t bf16_bits_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// hi = bf16(f), lo = bf16(f - hi), both round-to-nearest-even.
__device__ __forceinline__ void split(float f, uint16_t &hi, uint16_t &lo) {
  hi = bf16_bits_rne(f);
  lo = bf16_bits_rne(f - bf16_bits_to_f32(hi));
}

__device__ __forceinline__ bf16x8 ld8(const uint16_t *p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(p));
}
// two runs of 4 consecutive bf16 (8-byte aligned) as one operand
__device__ __forceinline__ bf16x8 ld4x2(const uint16_t *p0, const uint16_t *p1) {
  const uint2 a = *reinterpret_cast<const uint2 *>(p0);
  const uint2 b = *reinterpret_cast<const uint2 *>(p1);
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <bool V6>
__global__ void __launch_bounds__(kThreads) wkv56_chunked_kernel(ScanParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem &sm = *reinterpret_cast<Smem *>(smem_raw);

  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const long C = (long)p.H * kHead;
  const int T = p.T;
  const long tok0 = (long)b * T;

  int row_in = -1;
  if (p.state_in) {
    row_in = p.state_map ? p.state_map[b] : (p.n_state == 1 ? 0 : b);
    if (row_in < 0 || row_in >= p.n_state) {
      if (tid == 0 && p.dev_status) atomicOr(p.dev_status, WKV_DEV_BAD_STATE_MAP);
      return;
    }
  }

  // ---- MFMA-phase roles
  const int jb = wave & 3;    // value columns 16jb .. 16jb+15
  const int part = wave >> 2;  // token blocks {0,3} / {1,2}; key-row blocks {0,1} / {2,3}
  const int g = lane >> 4;    // operand k-group / accumulator row group
  const int l16 = lane & 15;
  const int jcol = 16 * jb + l16;

  // state tiles owned: key rows 16*ib + 4g + e, ib = 2*part + q; column jcol
  f32x4 Sacc[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int ib = 2 * part + q;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * ib + 4 * g + e;
      Sacc[q][e] = row_in >= 0 ? p.state_in[(((long)row_in * p.H + h) * kHead + i) * kHead + jcol] : 0.f;
    }
  }
  auto publish_state = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int ib = 2 * part + q;
      uint16_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) split(Sacc[q][e], hi[e], lo[e]);
      *reinterpret_cast<uint2 *>(&sm.st_hi[buf][jcol][16 * ib + 4 * g]) =
          make_uint2(hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16));
      *reinterpret_cast<uint2 *>(&sm.st_lo[buf][jcol][16 * ib + 4 * g]) =
          make_uint2(lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16));
    }
  };
  publish_state(0);
  if (tid == 0) sm.range_bad = 0;

  // ---- precompute roles: channel ci, tokens 8*cg .. 8*cg+7 of the chunk
  const int ci = tid & 63;
  const int cg = tid >> 6;
  const float u_ci = p.u[h * kHead + ci];
  const float xs_ci = V6 ? 0.f : static_cast<const float *>(p.w)[h * kHead + ci];
  const uint16_t *R = static_cast<const uint16_t *>(p.r);
  const uint16_t *K = static_cast<const uint16_t *>(p.k);
  const uint16_t *Vv = static_cast<const uint16_t *>(p.v);
  const uint16_t *W = static_cast<const uint16_t *>(p.w);

  uint16_t nr[8], nk[8], nv[8], nx[8];
  auto prefetch = [&](int c) {
    const int t0 = c * L;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int tau = 8 * cg + t;
      if (t0 + tau < T) {
        const long e = (tok0 + t0 + tau) * C + h * kHead + ci;
        nr[t] = R[e];
        nk[t] = K[e];
        nv[t] = Vv[e];
        if (V6) nx[t] = W[e];
      } else {
        nr[t] = 0; nk[t] = 0; nv[t] = 0; nx[t] = 0;
      }
    }
  };

  const int nchunks = (T + L - 1) / L;
  prefetch(0);
  for (int c = 0; c < nchunks; ++c) {
    const int t0 = c * L;
    const int nvalid = min(L, T - t0);
    const int buf = c & 1;

    // ================= precompute (vector ALU)
    float rr[8], kk[8], cum[8];
    float run = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int tau = 8 * cg + t;
      const bool valid = tau < nvalid;
      rr[t] = bf16_bits_to_f32(nr[t]);
      kk[t] = bf16_bits_to_f32(nk[t]);
      const float x = V6 ? bf16_bits_to_f32(nx[t]) : xs_ci;
      // log2 of the decay exp(-exp(x)) is -exp(x) * log2(e)
      const float l2 = valid ? -fast_exp(x) * 1.4426950408889634f : 0.f;
      run += l2;
      cum[t] = run;
      sm.bp[tau][ci] = rr[t] * u_ci * kk[t];
    }
    *reinterpret_cast<uint4 *>(&sm.vt[ci][8 * cg]) =
        make_uint4(nv[0] | ((uint32_t)nv[1] << 16), nv[2] | ((uint32_t)nv[3] << 16),
                   nv[4] | ((uint32_t)nv[5] << 16), nv[6] | ((uint32_t)nv[7] << 16));
    sm.tot[cg][ci] = run;
    __syncthreads();

    float prefix = 0.f, total = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float tq = sm.tot[q][ci];
      if (q < cg) prefix += tq;
      total += tq;
    }
    const float pl = __builtin_amdgcn_exp2f(total);
    if (cg == 0) sm.pl[ci] = pl;
    if (total < -kMaxLog2) sm.range_bad = 1;
    uint16_t khh[8], khl[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int tau = 8 * cg + t;
      const float lam = prefix + cum[t];
      const float lam_prev = t ? prefix + cum[t - 1] : prefix;
      const float rb = rr[t] * __builtin_amdgcn_exp2f(lam_prev);
      const float kt = kk[t] * __builtin_amdgcn_exp2f(-lam);
      const float kh = kt * pl;
      uint16_t hi, lo;
      split(rb, hi, lo);
      sm.rb_hi[tau][ci] = hi;
      sm.rb_lo[tau][ci] = lo;
      split(kt, hi, lo);
      sm.kt_hi[tau][ci] = hi;
      sm.kt_lo[tau][ci] = lo;
      split(kh, khh[t], khl[t]);
    }
    *reinterpret_cast<uint4 *>(&sm.kh_hi[ci][8 * cg]) =
        make_uint4(khh[0] | ((uint32_t)khh[1] << 16), khh[2] | ((uint32_t)khh[3] << 16),
                   khh[4] | ((uint32_t)khh[5] << 16), khh[6] | ((uint32_t)khh[7] << 16));
    *reinterpret_cast<uint4 *>(&sm.kh_lo[ci][8 * cg]) =
        make_uint4(khl[0] | ((uint32_t)khl[1] << 16), khl[2] | ((uint32_t)khl[3] << 16),
                   khl[4] | ((uint32_t)khl[5] << 16), khl[6] | ((uint32_t)khl[7] << 16));
    __syncthreads();
    {  // bonus diagonal: b[tau] = sum_i r u k, 8 lanes per token
      const int tau = tid >> 3, q = tid & 7;
      const float4 a0 = *reinterpret_cast<const float4 *>(&sm.bp[tau][8 * q]);
      const float4 a1 = *reinterpret_cast<const float4 *>(&sm.bp[tau][8 * q + 4]);
      float s = ((a0.x + a0.y) + (a0.z + a0.w)) + ((a1.x + a1.y) + (a1.z + a1.w));
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s += __shfl_xor(s, 4);
      if (q == 0) sm.bonus[tau] = s;
    }
    if (c + 1 < nchunks) prefetch(c + 1);
    __syncthreads();

    // ================= MFMA phase
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int tb = part == 0 ? (pass == 0 ? 0 : 3) : (pass == 0 ? 1 : 2);
      // A^T tiles (sb, tb), sb <= tb: rows = key token s, cols = query token t
      f32x4 At[4];
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) {
        At[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (sb > tb) continue;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8 ah = ld8(&sm.kt_hi[16 * sb + l16][32 * s + 8 * g]);
          const bf16x8 al = ld8(&sm.kt_lo[16 * sb + l16][32 * s + 8 * g]);
          const bf16x8 bh = ld8(&sm.rb_hi[16 * tb + l16][32 * s + 8 * g]);
          const bf16x8 bl = ld8(&sm.rb_lo[16 * tb + l16][32 * s + 8 * g]);
          At[sb] = mfma(ah, bh, At[sb]);
          At[sb] = mfma(ah, bl, At[sb]);
          At[sb] = mfma(al, bh, At[sb]);
        }
        if (sb == tb) {  // causal mask and bonus diagonal
          const int t = 16 * tb + l16;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int s = 16 * sb + 4 * g + e;
            At[sb][e] = s < t ? At[sb][e] : (s == t ? sm.bonus[t] : 0.f);
          }
        }
      }
      f32x4 Y = {0.f, 0.f, 0.f, 0.f};
      // inter-chunk: Y += rbar S0  (K = key row i)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 ah = ld8(&sm.rb_hi[16 * tb + l16][32 * s + 8 * g]);
        const bf16x8 al = ld8(&sm.rb_lo[16 * tb + l16][32 * s + 8 * g]);
        const bf16x8 bh = ld8(&sm.st_hi[buf][jcol][32 * s + 8 * g]);
        const bf16x8 bl = ld8(&sm.st_lo[buf][jcol][32 * s + 8 * g]);
        Y = mfma(ah, bh, Y);
        Y = mfma(ah, bl, Y);
        Y = mfma(al, bh, Y);
      }
      // intra-chunk: Y += A V  (K = key token s; operand slot e of group g holds
      // s = 32sp + 4g + e for e < 4 and 32sp + 16 + 4g + (e-4) for e >= 4)
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        if (2 * sp > tb) continue;
        uint16_t ahi[8], alo[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          split(At[2 * sp][e], ahi[e], alo[e]);
          split(At[2 * sp + 1][e], ahi[4 + e], alo[4 + e]);
        }
        bf16x8 ah, al;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ah[e] = __builtin_bit_cast(__bf16, ahi[e]);
          al[e] = __builtin_bit_cast(__bf16, alo[e]);
        }
        const bf16x8 bv = ld4x2(&sm.vt[jcol][32 * sp + 4 * g], &sm.vt[jcol][32 * sp + 16 + 4 * g]);
        Y = mfma(ah, bv, Y);
        Y = mfma(al, bv, Y);
      }
      // store outputs: rows t = 16tb + 4g + e, column jcol
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * tb + 4 * g + e;
        if (t < nvalid) p.y[(tok0 + t0 + t) * C + h * kHead + jcol] = Y[e];
      }
    }

    // state update: S <- diag(pl) S + khat^T V  (K = key token s)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int ib = 2 * part + q;
#pragma unroll
      for (int e = 0; e < 4; ++e) Sacc[q][e] *= sm.pl[16 * ib + 4 * g + e];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 ah = ld8(&sm.kh_hi[16 * ib + l16][32 * s + 8 * g]);
        const bf16x8 al = ld8(&sm.kh_lo[16 * ib + l16][32 * s + 8 * g]);
        const bf16x8 bv = ld8(&sm.vt[jcol][32 * s + 8 * g]);
        Sacc[q] = mfma(ah, bv, Sacc[q]);
        Sacc[q] = mfma(al, bv, Sacc[q]);
      }
    }
    publish_state(buf ^ 1);
    __syncthreads();
  }

  if (tid == 0 && sm.range_bad && p.dev_status) atomicOr(p.dev_status, WKV_DEV_DECAY_RANGE);
  if (p.state_out) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int ib = 2 * part + q;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * ib + 4 * g + e;
        p.state_out[(((long)b * p.H + h) * kHead + i) * kHead + jcol] = Sacc[q][e];
      }
    }
  }
}

template <bool V6>
hipError_t launch(const ScanParams &p, hipStream_t s) {
  const size_t lds = sizeof(Smem);
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&wkv56_chunked_kernel<V6>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    configured = true;
  }
  dim3 grid(p.H, p.units);
  hipLaunchKernelGGL((wkv56_chunked_kernel<V6>), grid, dim3(kThreads), lds, s, p);
  return hipGetLastError();
}

}  // namespace

size_t wkv56_chunked_lds_bytes() { return sizeof(Smem); }

hipError_t launch_wkv56_chunked(const ScanParams &p, bool v6, bool bf16, hipStream_t s) {
  if (!bf16) return hipErrorInvalidValue;  // the ABI layer routes fp32 inputs to the scan
  return v6 ? launch<true>(p, s) : launch<false>(p, s);
}

}  // namespace wkv
