// 64-token chunked WKV v5 / v6 with the contractions on MFMA (gfx950).
//
// Same recurrence as the token-sequential scan (the rwkv_ops page's RWKV6_OP:
// r, k, v, w, u, init_state, state_map -> y, y_state; S indexed [key i][value j]):
//   y_t[j] = sum_i r_t[i] (S[i][j] + u[i] k_t[i] v_t[j]),  S[i][j] <- d_t[i] S[i][j] + k_t[i] v_t[j]
// rewritten exactly, chunk by chunk.  Inside a chunk of L = 64 tokens let
// Lam_t[i] = sum_{m<=t} log d_m[i] (inclusive, from the chunk start) and
//   rbar_t = r_t * exp(Lam_{t-1}),  ktil_s = k_s * exp(-Lam_s).
// Then, with S0 the state at the chunk start,
//   A[t][s] = rbar_t . ktil_s (s < t),  A[t][t] = sum_i r_t[i] u[i] k_t[i],  A[t][s] = 0 (s > t)
//   Y  = A V + rbar S0
//   S1 = diag(exp(Lam_{L-1})) (S0 + ktil^T V)
// which equals the token recurrence in exact arithmetic.  The last line adds
// the chunk's keys in the frame of the chunk start and rescales once; fp32
// rounding of that sum is relative to its larger term, so the rescale keeps
// the usual relative accuracy.
//
// Precision.  Every MFMA runs on bf16 operands with fp32 accumulation.  V is
// the exact bf16 input; every other operand (rbar, ktil, A, S) is split into
// hi = bf16(x) and lo = bf16(x - hi) (both round-to-nearest-even) and each
// product is formed as hi*hi + hi*lo + lo*hi (v only needs hi*v + lo*v),
// about 16 significant bits per term.  Every product that survives the causal
// mask is bounded by |r k|, since exp(Lam_{t-1} - Lam_s) <= 1 for s < t.
//
// Range.  ktil carries exp(-Lam_s) >= 1.  A chunk whose accumulated log2
// decay in some channel is below -kMaxLog2 sets WKV_DEV_DECAY_RANGE (its
// outputs are then not trustworthy; the token-sequential scan has no such
// limit).  Per-step decays exp(-exp(x)) with x <= 0 stay far inside it.
//
// Work decomposition: one 1024-thread workgroup (16 waves) per (batch row,
// head) walks the chunks in order as a two-stage pipeline, so that the
// vector-ALU work of one chunk overlaps the matrix-core work of the previous
// one.  Every operand the producers write is double-buffered in LDS.
//   producers (waves 0-7), chunk c+1: thread (channel pair cp, token group tg
//     of 4) consumes its inputs (4-byte loads issued one chunk ahead), forms
//     the log2-decay prefix (wave totals exchanged through LDS), and writes
//     rbar, ktil row-major and V transposed as bf16 hi / lo; the bonus
//     diagonal is reduced across the lanes of a half-wave.
//   consumers (waves 8-15), chunk c:
//     M1: the ten causal 16x16 tiles of A^T (v_mfma_f32_16x16x32_bf16),
//       masked and stored to LDS as A hi / lo;
//     M2: four waves own the 32x32 output tiles (v_mfma_f32_32x32x16_bf16:
//       rbar S0 + A V); four waves own the 32x32 state tiles in fp32
//       accumulators.  They transpose ktil on the matrix core (a product with
//       the identity is exact for bf16 values) and reuse the accumulator
//       layout as the A operand of ktil^T V by reading V in the matching
//       permuted token order.  The state goes to the output waves as bf16
//       hi / lo S^T in a ping-pong buffer.
#include <atomic>

#include "common.hpp"
#include "kernels.hpp"
#include "wkv.h"

namespace wkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int L = 64;           // tokens per chunk
constexpr int kThreads = 1024;  // 16 waves: 8 producers, 8 consumers
constexpr int RS = 72;          // LDS row stride in bf16 elements (144 bytes)
constexpr float kMaxLog2 = 100.f;

struct Ops {                      // one chunk's operands, written by the producers
  uint16_t rb_hi[L][RS], rb_lo[L][RS];  // rbar [token][key row]
  uint16_t kt_hi[L][RS], kt_lo[L][RS];  // ktil [token][key row]
  uint16_t vt[kHead][RS];               // V^T  [value col][token]
  float bonus[L];
  float pl[kHead];                      // exp(Lam_{L-1}) per key row
};

struct Smem {
  Ops ops[2];
  uint16_t a_hi[L][RS], a_lo[L][RS];                  // A   [query token][key token]
  uint16_t st_hi[2][kHead][RS], st_lo[2][kHead][RS];  // S^T [value col][key row], ping-pong
  float2 wtot[8][32];                                 // log2-decay total of each producer wave, per channel pair
  int range_bad;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Two floats -> packed bf16 pair (round to nearest even): low half = a.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = static_cast<__bf16>(a);
  v[1] = static_cast<__bf16>(b);
  return __builtin_bit_cast(uint32_t, v);
}
// Split two floats into packed hi and lo bf16 pairs.
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
  hi = pack_bf16(a, b);
  lo = pack_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

__device__ __forceinline__ bf16x8 ld8(const uint16_t *p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(p));
}
__device__ __forceinline__ bf16x8 ld4x2(const uint16_t *p0, const uint16_t *p1) {
  const uint2 a = *reinterpret_cast<const uint2 *>(p0);
  const uint2 b = *reinterpret_cast<const uint2 *>(p1);
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}
__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(bf16x8, make_uint4(a, b, c, d));
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Cross-lane helpers without address arithmetic: quad permutes on DPP, other
// xor distances inside 32-lane groups on the LDS swizzle crossbar.
__device__ __forceinline__ float xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}
template <int M>
__device__ __forceinline__ float xor_swz(float x) {  // M in {4, 8, 16}
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1F | (M << 10)));
}

// A wave-uniform 64-bit value the compiler cannot rewrite into per-lane
// induction variables (keeps per-chunk bases in scalar registers).
__device__ __forceinline__ long uniform64(long x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((unsigned long)x >> 32));
  return (long)(((unsigned long)hi << 32) | lo);
}

// Keeps the compiler from moving work on a prefetched register above this
// point, so the wait for the load lands here.
__device__ __forceinline__ void pin(uint32_t &x) { asm volatile("" : "+v"(x)); }

template <bool V6>
__global__ void __launch_bounds__(kThreads) wkv56_chunked_kernel(ScanParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem &sm = *reinterpret_cast<Smem *>(smem_raw);

  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int hh = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform role selector
  const bool producer = wave_u < 8;
  const long C = (long)p.H * kHead;
  const int T = p.T;
  const long tok0 = (long)b * T;
  const int nchunks = (T + L - 1) / L;

  int row_in = -1;
  if (p.state_in) {
    row_in = p.state_map ? p.state_map[b] : (p.n_state == 1 ? 0 : b);
    if (row_in < 0 || row_in >= p.n_state) {
      if (tid == 0 && p.dev_status) atomicOr(p.dev_status, WKV_DEV_BAD_STATE_MAP);
      return;
    }
  }

  // ---------------- producer roles: channels 2cp, 2cp+1; tokens 4tg .. 4tg+3 of a chunk
  const int cp = tid & 31;
  const int tg = (tid >> 5) & 15;
  const int pwave = wave_u & 7;
  // ---------------- consumer roles
  const int cw = wave_u & 7;             // consumer wave 0..7
  const bool y_wave = cw < 4;            // M2: output tile / state tile
  const int tile_r = (cw & 3) >> 1;      // token block (output) / key-row block (state)
  const int tile_c = cw & 1;             // value-column block
  const int l32 = lane & 31;
  const int jcol = 32 * tile_c + l32;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  f32x16 S = {};  // state waves: rows 32*tile_r + 8*(e/4) + 4*hh + e%4, column jcol
  auto publish_state = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t h0, l0, h1, l1;
      split2(S[4 * q], S[4 * q + 1], h0, l0);
      split2(S[4 * q + 2], S[4 * q + 3], h1, l1);
      const int i0 = 32 * tile_r + 8 * q + 4 * hh;
      *reinterpret_cast<uint2 *>(&sm.st_hi[buf][jcol][i0]) = make_uint2(h0, h1);
      *reinterpret_cast<uint2 *>(&sm.st_lo[buf][jcol][i0]) = make_uint2(l0, l1);
    }
  };

  if (!producer) {
    if (!y_wave && row_in >= 0) {
      const float *sp = p.state_in + ((long)row_in * p.H + h) * (kHead * kHead);
#pragma unroll
      for (int e = 0; e < 16; ++e) S[e] = sp[(32 * tile_r + 8 * (e >> 2) + 4 * hh + (e & 3)) * kHead + jcol];
    }
    if (!y_wave) publish_state(0);
    // A tiles that the causal mask zeroes but the 32-wide K steps of A V read
    // (rows 0-15 x cols 16-31 and rows 32-47 x cols 48-63): zero them once.
    const int ct = tid - 512;
    if (ct < 128) {
      const int region = ct >> 6, rem = ct & 63;
      const int row = 32 * region + (rem >> 2), col = 16 + 32 * region + 4 * (rem & 3);
      *reinterpret_cast<uint2 *>(&sm.a_hi[row][col]) = make_uint2(0u, 0u);
      *reinterpret_cast<uint2 *>(&sm.a_lo[row][col]) = make_uint2(0u, 0u);
    }
  } else if (tid == 0) {
    sm.range_bad = 0;
  }

  // ---------------- producer state carried between its two phases
  float2 u2 = make_float2(0.f, 0.f), xs = make_float2(0.f, 0.f);
  if (producer) {
    u2 = *reinterpret_cast<const float2 *>(p.u + h * kHead + 2 * cp);
    if (!V6) xs = *reinterpret_cast<const float2 *>(static_cast<const float *>(p.w) + h * kHead + 2 * cp);
  }
  // byte offsets of this thread's four rows inside a chunk (the chunk base is wave-uniform)
  uint32_t roff[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) roff[t] = (uint32_t)(((4 * tg + t) * C + h * kHead + 2 * cp) * 2);
  uint32_t nr[4], nk[4], nv[4], nx[4];
  auto prefetch = [&](int c) {
    const long base = uniform64((tok0 + (long)c * L) * C * 2);  // bytes
    const char *pr = static_cast<const char *>(p.r) + base, *pk = static_cast<const char *>(p.k) + base;
    const char *pv = static_cast<const char *>(p.v) + base, *pw = static_cast<const char *>(p.w) + base;
    const int rows = T - c * L;  // rows past the end: read the chunk's last row, zeroed on use
    uint32_t o[4];
    if (rows >= L) {
#pragma unroll
      for (int t = 0; t < 4; ++t) o[t] = roff[t];
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) o[t] = (uint32_t)((min(4 * tg + t, rows - 1) * C + h * kHead + 2 * cp) * 2);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      nr[t] = *reinterpret_cast<const uint32_t *>(pr + o[t]);
      nk[t] = *reinterpret_cast<const uint32_t *>(pk + o[t]);
      nv[t] = *reinterpret_cast<const uint32_t *>(pv + o[t]);
      if (V6) nx[t] = *reinterpret_cast<const uint32_t *>(pw + o[t]);
    }
  };
  uint32_t rkeep[4], kkeep[4];  // this chunk's r and k words, carried to phase 2
  float cum0[4], cum1[4], lower0 = 0.f, lower1 = 0.f;

  // producer phase 1 of chunk c: decay, in-thread prefix, bonus, V^T, wave totals
  const int lane_x32 = (lane ^ 32) << 2;  // ds_bpermute address of the other half-wave
  auto produce1 = [&](int c) {
    Ops &o = sm.ops[c & 1];
    const int nvalid = min(L, T - c * L);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      pin(nr[t]); pin(nk[t]); pin(nv[t]);
      if (V6) pin(nx[t]);
    }
    if (nvalid < L) {  // partial last chunk: tokens past the end contribute nothing
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bool valid = 4 * tg + t < nvalid;
        nr[t] = valid ? nr[t] : 0u;
        nk[t] = valid ? nk[t] : 0u;
        nv[t] = valid ? nv[t] : 0u;
        if (V6) nx[t] = valid ? nx[t] : 0xff80ff80u;  // x = -inf: decay exactly 1
      }
    }
    // V^T: tokens 4tg..4tg+3 of channels 2cp (low halves) and 2cp+1 (high halves)
    *reinterpret_cast<uint2 *>(&o.vt[2 * cp][4 * tg]) =
        make_uint2(__builtin_amdgcn_perm(nv[1], nv[0], 0x05040100u), __builtin_amdgcn_perm(nv[3], nv[2], 0x05040100u));
    *reinterpret_cast<uint2 *>(&o.vt[2 * cp + 1][4 * tg]) =
        make_uint2(__builtin_amdgcn_perm(nv[1], nv[0], 0x07060302u), __builtin_amdgcn_perm(nv[3], nv[2], 0x07060302u));
    float bon[4];
    float run0 = 0.f, run1 = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t rw = nr[t], kw = nk[t];
      rkeep[t] = rw;
      kkeep[t] = kw;
      const float r0 = bf16_bits_to_f32(rw & 0xffffu), r1 = __uint_as_float(rw & 0xffff0000u);
      const float k0 = bf16_bits_to_f32(kw & 0xffffu), k1 = __uint_as_float(kw & 0xffff0000u);
      float x0 = xs.x, x1 = xs.y;
      if (V6) {
        x0 = bf16_bits_to_f32(nx[t] & 0xffffu);
        x1 = __uint_as_float(nx[t] & 0xffff0000u);
      }
      // log2 of the decay exp(-exp(x)) is -exp(x) * log2(e)
      run0 -= fast_exp(x0) * 1.4426950408889634f;
      run1 -= fast_exp(x1) * 1.4426950408889634f;
      cum0[t] = run0;
      cum1[t] = run1;
      bon[t] = fmaf(r1 * u2.y, k1, r0 * u2.x * k0);
    }
    if (!V6 && nvalid < L) {  // static decay: tokens past the end must not decay the prefix
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (4 * tg + t >= nvalid) {
          cum0[t] = t ? cum0[t - 1] : 0.f;
          cum1[t] = t ? cum1[t - 1] : 0.f;
        }
      }
      run0 = cum0[3];
      run1 = cum1[3];
    }
    if (c + 1 < nchunks) prefetch(c + 1);
    {  // bonus diagonal: sum over the 32 channel pairs of this token group (one half-wave)
      const bool up16 = lane & 16;
      float keep0 = up16 ? bon[2] : bon[0], keep1 = up16 ? bon[3] : bon[1];
      keep0 += xor_swz<16>(up16 ? bon[0] : bon[2]);
      keep1 += xor_swz<16>(up16 ? bon[1] : bon[3]);
      const bool up8 = lane & 8;
      float kk = up8 ? keep1 : keep0;
      kk += xor_swz<8>(up8 ? keep0 : keep1);
      kk += xor_swz<4>(kk);
      kk += xor2(kk);
      kk += xor1(kk);
      if ((lane & 7) == 0) o.bonus[4 * tg + (up16 ? 2 : 0) + (up8 ? 1 : 0)] = kk;
    }
    // wave totals: the upper half-wave (odd token group) adds the lower one's total
    lower0 = __int_as_float(__builtin_amdgcn_ds_bpermute(lane_x32, __float_as_int(run0)));
    lower1 = __int_as_float(__builtin_amdgcn_ds_bpermute(lane_x32, __float_as_int(run1)));
    if (hh) sm.wtot[pwave][cp] = make_float2(run0 + lower0, run1 + lower1);
  };

  // producer phase 2 of chunk c: prefix, scaled operands, bf16 hi / lo
  auto produce2 = [&](int c) {
    Ops &o = sm.ops[c & 1];
    float2 wt[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) wt[w] = sm.wtot[w][cp];
    float pre0 = hh ? lower0 : 0.f, pre1 = hh ? lower1 : 0.f, tot0 = 0.f, tot1 = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      if (w == pwave) { pre0 += tot0; pre1 += tot1; }  // pwave is wave-uniform: a scalar branch
      tot0 += wt[w].x;
      tot1 += wt[w].y;
    }
    if (tg == 0) *reinterpret_cast<float2 *>(&o.pl[2 * cp]) =
        make_float2(__builtin_amdgcn_exp2f(tot0), __builtin_amdgcn_exp2f(tot1));
    if (tot0 < -kMaxLog2 || tot1 < -kMaxLog2) sm.range_bad = 1;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int tau = 4 * tg + t;
      const float lp0 = t ? pre0 + cum0[t - 1] : pre0, lp1 = t ? pre1 + cum1[t - 1] : pre1;
      const float la0 = pre0 + cum0[t], la1 = pre1 + cum1[t];
      const float r0 = bf16_bits_to_f32(rkeep[t] & 0xffffu), r1 = __uint_as_float(rkeep[t] & 0xffff0000u);
      const float k0 = bf16_bits_to_f32(kkeep[t] & 0xffffu), k1 = __uint_as_float(kkeep[t] & 0xffff0000u);
      uint32_t hi, lo;
      split2(r0 * __builtin_amdgcn_exp2f(lp0), r1 * __builtin_amdgcn_exp2f(lp1), hi, lo);
      *reinterpret_cast<uint32_t *>(&o.rb_hi[tau][2 * cp]) = hi;
      *reinterpret_cast<uint32_t *>(&o.rb_lo[tau][2 * cp]) = lo;
      split2(k0 * __builtin_amdgcn_exp2f(-la0), k1 * __builtin_amdgcn_exp2f(-la1), hi, lo);
      *reinterpret_cast<uint32_t *>(&o.kt_hi[tau][2 * cp]) = hi;
      *reinterpret_cast<uint32_t *>(&o.kt_lo[tau][2 * cp]) = lo;
    }
  };

  // consumer M1 of chunk c: causal A^T tiles, masked, stored as A hi / lo
  constexpr unsigned long long kM1Sb = 0x3210210100ull, kM1Tb = 0x3333222110ull;  // tile ti: (sb, tb) nibbles
  auto m1_tile = [&](const Ops &o, int ti) {
    const int sb = (int)((kM1Sb >> (4 * ti)) & 15), tb = (int)((kM1Tb >> (4 * ti)) & 15);
    const int t = 16 * tb + l16;
    bf16x8 ah[2], al[2], bh[2], bl[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      ah[s] = ld8(&o.kt_hi[16 * sb + l16][32 * s + 8 * g4]);
      al[s] = ld8(&o.kt_lo[16 * sb + l16][32 * s + 8 * g4]);
      bh[s] = ld8(&o.rb_hi[t][32 * s + 8 * g4]);
      bl[s] = ld8(&o.rb_lo[t][32 * s + 8 * g4]);
    }
    const float bon = o.bonus[t];
    f32x4 At = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      At = mfma16(ah[s], bh[s], At);
      At = mfma16(ah[s], bl[s], At);
      At = mfma16(al[s], bh[s], At);
    }
    // lane holds A^T[s = 16sb + 4g4 + e][t]; keep s < t, put the bonus on s == t
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int sidx = 16 * sb + 4 * g4 + e;
      At[e] = sidx < t ? At[e] : (sidx == t ? bon : 0.f);
    }
    uint32_t h0, l0, h1, l1;
    split2(At[0], At[1], h0, l0);
    split2(At[2], At[3], h1, l1);
    *reinterpret_cast<uint2 *>(&sm.a_hi[t][16 * sb + 4 * g4]) = make_uint2(h0, h1);
    *reinterpret_cast<uint2 *>(&sm.a_lo[t][16 * sb + 4 * g4]) = make_uint2(l0, l1);
  };
  auto consume1 = [&](int c) {
    const Ops &o = sm.ops[c & 1];
    m1_tile(o, cw);
    if (cw < 2) m1_tile(o, cw + 8);
  };

  // consumer M2 of chunk c
  auto consume2 = [&](int c) {
    const Ops &o = sm.ops[c & 1];
    const int buf = c & 1;
    const int nvalid = min(L, T - c * L);
    if (y_wave) {
      const int trow = 32 * tile_r + l32;
      f32x16 Y = {};
#pragma unroll
      for (int s2 = 0; s2 < 4; s2 += 2) {  // rbar S0, K = key row, two K steps per batch of loads
        bf16x8 ah[2], al[2], bh[2], bl[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int col = 16 * (s2 + q) + 8 * hh;
          ah[q] = ld8(&o.rb_hi[trow][col]);
          al[q] = ld8(&o.rb_lo[trow][col]);
          bh[q] = ld8(&sm.st_hi[buf][jcol][col]);
          bl[q] = ld8(&sm.st_lo[buf][jcol][col]);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          Y = mfma32(ah[q], bh[q], Y);
          Y = mfma32(ah[q], bl[q], Y);
          Y = mfma32(al[q], bh[q], Y);
        }
      }
      // A V, K = key token (causal: up to the tile's last token)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        if (half > tile_r) break;
        bf16x8 xh[2], xl[2], bv[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int col = 32 * half + 16 * s + 8 * hh;
          xh[s] = ld8(&sm.a_hi[trow][col]);
          xl[s] = ld8(&sm.a_lo[trow][col]);
          bv[s] = ld8(&o.vt[jcol][col]);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          Y = mfma32(xh[s], bv[s], Y);
          Y = mfma32(xl[s], bv[s], Y);
        }
      }
      char *yb = reinterpret_cast<char *>(p.y) + uniform64(((tok0 + (long)c * L) * C + h * kHead) * 4);
      const uint32_t lane_off = (uint32_t)((jcol + (32 * tile_r + 4 * hh) * C) * 4);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = 32 * tile_r + 8 * (e >> 2) + 4 * hh + (e & 3);
        if (nvalid == L || t < nvalid)
          *reinterpret_cast<float *>(yb + lane_off + (uint32_t)((8 * (e >> 2) + (e & 3)) * C * 4)) = Y[e];
      }
    } else {
      // S += ktil^T V, K = key token, in two 32-token blocks.  The transpose
      // T[s][i] = sum_i' ktil[s][i'] I[i'][i] leaves lane (i, hh) holding tokens
      // 32sb + 8q + 4hh + (0..3); K step ks of the update uses q = 2ks, 2ks+1, so
      // operand slot e maps to token 32sb + 16ks + 8(e/4) + 4hh + e%4, and V is
      // read in that same order.
      const int irow = 32 * tile_r + l32;
      bf16x8 id[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int kbase = 32 * tile_r + 16 * ks + 8 * hh;  // channels i' of this K step
#pragma unroll
        for (int e = 0; e < 8; ++e) id[ks][e] = (kbase + e == irow) ? (__bf16)1.0f : (__bf16)0.0f;
      }
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        bf16x8 src[2][2];  // [hi / lo][K step]
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int kbase = 32 * tile_r + 16 * ks + 8 * hh;
          src[0][ks] = ld8(&o.kt_hi[32 * sb + l32][kbase]);
          src[1][ks] = ld8(&o.kt_lo[32 * sb + l32][kbase]);
        }
        f32x16 Th = {}, Tl = {};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          Th = mfma32(src[0][ks], id[ks], Th);
          Tl = mfma32(src[1][ks], id[ks], Tl);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 ah = as_bf16x8(pack_bf16(Th[8 * ks + 0], Th[8 * ks + 1]), pack_bf16(Th[8 * ks + 2], Th[8 * ks + 3]),
                                      pack_bf16(Th[8 * ks + 4], Th[8 * ks + 5]), pack_bf16(Th[8 * ks + 6], Th[8 * ks + 7]));
          const bf16x8 al = as_bf16x8(pack_bf16(Tl[8 * ks + 0], Tl[8 * ks + 1]), pack_bf16(Tl[8 * ks + 2], Tl[8 * ks + 3]),
                                      pack_bf16(Tl[8 * ks + 4], Tl[8 * ks + 5]), pack_bf16(Tl[8 * ks + 6], Tl[8 * ks + 7]));
          const int s0 = 32 * sb + 16 * ks + 4 * hh;
          const bf16x8 bv = ld4x2(&o.vt[jcol][s0], &o.vt[jcol][s0 + 8]);
          S = mfma32(ah, bv, S);
          S = mfma32(al, bv, S);
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 pl4 = *reinterpret_cast<const float4 *>(&o.pl[32 * tile_r + 8 * q + 4 * hh]);
        S[4 * q] *= pl4.x;
        S[4 * q + 1] *= pl4.y;
        S[4 * q + 2] *= pl4.z;
        S[4 * q + 3] *= pl4.w;
      }
      publish_state(buf ^ 1);
    }
  };

  // Iteration c: producers prepare chunk c + 1 while consumers process chunk c.
  // The two roles run separate loops (so each keeps only its own registers
  // live) that execute the same number of workgroup barriers.
  if (producer) {
    prefetch(0);
    for (int c = -1; c < nchunks; ++c) {
      if (c + 1 < nchunks) produce1(c + 1);
      __syncthreads();
      if (c + 1 < nchunks) produce2(c + 1);
      __syncthreads();
    }
  } else {
    for (int c = -1; c < nchunks; ++c) {
      if (c >= 0) consume1(c);
      __syncthreads();
      if (c >= 0) consume2(c);
      __syncthreads();
    }
  }

  if (tid == 0 && sm.range_bad && p.dev_status) atomicOr(p.dev_status, WKV_DEV_DECAY_RANGE);
  if (!producer && !y_wave && p.state_out) {
    float *sp = p.state_out + ((long)b * p.H + h) * (kHead * kHead);
#pragma unroll
    for (int e = 0; e < 16; ++e) sp[(32 * tile_r + 8 * (e >> 2) + 4 * hh + (e & 3)) * kHead + jcol] = S[e];
  }
}

template <bool V6>
hipError_t launch(const ScanParams &p, hipStream_t s) {
  // The dynamic-LDS limit is a per-device function attribute: set it once per device.
  static std::atomic<unsigned long long> configured{0};
  const size_t lds = sizeof(Smem);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = 1ull << (dev & 63);
  if (!(configured.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&wkv56_chunked_kernel<V6>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    configured.fetch_or(bit, std::memory_order_acq_rel);
  }
  dim3 grid(p.H, p.units);
  hipLaunchKernelGGL((wkv56_chunked_kernel<V6>), grid, dim3(kThreads), lds, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_wkv56_chunked(const ScanParams &p, bool v6, bool bf16, hipStream_t s) {
  if (!bf16) return hipErrorInvalidValue;  // the ABI layer routes fp32 inputs to the scan
  return v6 ? launch<true>(p, s) : launch<false>(p, s);
}

}  // namespace wkv
