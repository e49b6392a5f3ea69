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
// decay in some channel is below -kMaxLog2 (or -inf: a decay of exactly 0)
// would overflow that factor, so it is not run in this form: the consumer
// waves walk its 64 tokens one at a time with the direct recurrence
//   y_t[j] = sum_i r_t[i] S[i][j] + bonus_t v_t[j],  S[i][j] <- d_t[i] S[i][j] + k_t[i] v_t[j]
// in fp32, where every factor is at most 1, and the next chunk continues on
// the matrix cores from the state this leaves.  Per-step decays exp(-exp(x))
// with x <= 0 never need it (at most 92 log2 units per chunk).
//
// Work decomposition: one 1024-thread workgroup (16 waves) per (batch row,
// head) walks the chunks in order as a pipeline with one workgroup barrier
// per step, so that the vector-ALU work of later chunks overlaps the
// matrix-core work of the current one.  At step i:
//   producers (waves 0-7) finish chunk i+1 and start chunk i+2.  Thread
//     (channel pair cp, token group tg of 4) consumes its inputs (4-byte
//     loads issued one step ahead), forms its part of the log2-decay prefix
//     and the bonus diagonal (reduced across the lanes of a half-wave) and
//     posts its wave's decay total; one step later it adds the totals of the
//     waves before it and writes rbar, ktil row-major and V transposed as
//     bf16 hi / lo into the chunk's operand buffer.
//   consumers (waves 8-15) process chunk i (v_mfma_f32_32x32x16_bf16):
//     two output waves own the 32-token blocks with all 64 value columns.
//     Each forms the causal 32x32 blocks of A^T that its token block needs in
//     accumulators (the rbar registers serve both A^T = ktil rbar^T and
//     rbar S0), masks them, splits them into bf16 hi / lo in registers and
//     adds A V, reading V in the token order the accumulator layout gives.  Four state waves own the
//     32x32 fp32 state tiles: they read ktil^T with the LDS transpose load,
//     add ktil^T V, rescale, and publish the state as bf16 hi / lo S^T in a
//     ping-pong buffer for the next chunk's outputs.  The two remaining waves do
//     no math (they read chunk i+3's rows early in the step; see their loop).
// Operand buffers and the decay totals are double-buffered in LDS.
#pragma once

#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma_ops.hpp"
#include "wkv.h"

namespace wkv {
namespace {

constexpr int L = 64;           // tokens per chunk
constexpr int kThreads = 1024;  // 16 waves: 8 producers, 8 consumers
constexpr int RS = 72;          // LDS row stride in bf16 elements (144 bytes)
constexpr float kMaxLog2 = 100.f;
constexpr int kWarmAhead = 3;   // chunk distance of the early reads of the idle consumer waves

// A chunk that runs directly keeps the same arrays with other contents:
// rb_hi = r and rb_lo = k as loaded (bf16), kt_hi / kt_lo = upper / lower 16
// bits of the fp32 decay d_t[i], all [token][key row].
struct alignas(16) Ops {          // one chunk's operands, written by the producers
  uint16_t rb_hi[L][RS], rb_lo[L][RS];  // rbar [token][key row]
  uint16_t kt_hi[L][RS], kt_lo[L][RS];  // ktil [token][key row]
  uint16_t vt[kHead][RS];               // V^T  [value col][token]
  float bonus[L];
  float pl[kHead];                      // exp(Lam_{L-1}) per key row
  int direct;                           // 1: this chunk takes the direct recurrence
};

constexpr int SFS = 68;  // row stride (floats) of the fp32 state while a chunk runs directly

struct Smem {
  Ops ops[2];
  // S^T [value col][key row] as bf16 hi / lo, ping-pong by chunk parity.  While a
  // chunk runs directly, the buffer of its own parity holds the fp32 state
  // [key row][SFS] instead (the output waves then do not read it).
  uint16_t st[2][2][kHead][RS];
  float2 wtot[2][8][32];                              // log2-decay total of each producer wave, per channel pair
};
static_assert(sizeof(float) * kHead * SFS <= sizeof(uint16_t) * 2 * kHead * RS, "fp32 state fits one S^T buffer");

template <bool V6, bool OUTB, bool SAVE>
__global__ void __launch_bounds__(kThreads) wkv56_chunked_kernel(ScanParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem &sm = *reinterpret_cast<Smem *>(smem_raw);

  // Consecutive workgroups go to different XCDs (round robin over the 8), so
  // batch row = id % B puts all heads of a row on one XCD (when B divides
  // into the XCD count): they stream the same token rows at about the same
  // time, which keeps HBM page and L2 locality.
  const int wg = blockIdx.x;
  const int b = wg % p.units;
  const int h = wg / p.units;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int hh = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform role selector
  const bool producer = wave_u < 8;
  const int T = p.T;
  const long ts = p.tok_stride;                                // elements between tokens
  const long base = b * p.row_stride + h * p.head_stride;      // (row b, head h), token 0, channel 0
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

  f32x16 S = {};  // state waves: rows 32*tile_r + 8*(e/4) + 4*hh + e%4, column jcol
  auto publish_state = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t h0, l0, h1, l1;
      split2(S[4 * q], S[4 * q + 1], h0, l0);
      split2(S[4 * q + 2], S[4 * q + 3], h1, l1);
      const int i0 = 32 * tile_r + 8 * q + 4 * hh;
      *reinterpret_cast<uint2 *>(&sm.st[buf][0][jcol][i0]) = make_uint2(h0, h1);
      *reinterpret_cast<uint2 *>(&sm.st[buf][1][jcol][i0]) = make_uint2(l0, l1);
    }
  };

  if (!producer) {
    if (!y_wave && row_in >= 0) {
      const float *sp = p.state_in + ((long)row_in * p.H + h) * (kHead * kHead);
#pragma unroll
      for (int e = 0; e < 16; ++e) S[e] = sp[(32 * tile_r + 8 * (e >> 2) + 4 * hh + (e & 3)) * kHead + jcol];
    }
    if (!y_wave) publish_state(0);
  }

  // ---------------- producer state carried between its two phases
  float2 u2 = make_float2(0.f, 0.f), xs = make_float2(0.f, 0.f);
  if (producer) {
    u2 = *reinterpret_cast<const float2 *>(p.u + h * kHead + 2 * cp);
    if (!V6) xs = *reinterpret_cast<const float2 *>(static_cast<const float *>(p.w) + h * kHead + 2 * cp);
  }
  // Token rows are read with buffer loads: one resource per input array and
  // chunk (wave-uniform, in scalar registers) whose record count ends at the
  // head's last channel of the row's last token, so tokens past it read as
  // zero (r = k = v = 0 adds nothing); per-thread offsets are fixed.  Loaded words of chunk c live in register set c & 1 from the load
  // (issued one step ahead) until phase 2 of chunk c, one step after phase 1.
  uint32_t roff[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) roff[t] = (uint32_t)(((4 * tg + t) * ts + 2 * cp) * 2);
  const unsigned long long row_end = (unsigned long long)(base + (long)(T - 1) * ts + kHead) * 2;  // end of this head's row
  auto rsrc_at = [&](const void *base, unsigned long long off) {
    const unsigned long long rem = off < row_end ? row_end - off : 0ull;
    const int n = (int)(rem > 0x7fffffffull ? 0x7fffffffull : rem);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(static_cast<const char *>(base) + off), 0, n,
                                             0x00020000);
  };
  uint32_t ld[2][3][4];  // [set][r, k, v][token of the thread's group]
  uint32_t ldx[4];       // x words: consumed in phase 1, before the next chunk's load reuses them
  auto prefetch = [&](int c, auto set_c) {
    constexpr int S = decltype(set_c)::value;
    const unsigned long long off = (unsigned long long)uniform64((base + (long)c * L * ts) * 2);
    const auto rr = rsrc_at(p.r, off), rk = rsrc_at(p.k, off), rv = rsrc_at(p.v, off);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      ld[S][0][t] = __builtin_amdgcn_raw_buffer_load_b32(rr, (int)roff[t], 0, 0);
      ld[S][1][t] = __builtin_amdgcn_raw_buffer_load_b32(rk, (int)roff[t], 0, 0);
      ld[S][2][t] = __builtin_amdgcn_raw_buffer_load_b32(rv, (int)roff[t], 0, 0);
    }
    if (V6) {
      const auto rw = rsrc_at(p.w, off);
#pragma unroll
      for (int t = 0; t < 4; ++t) ldx[t] = __builtin_amdgcn_raw_buffer_load_b32(rw, (int)roff[t], 0, 0);
    }
  };
  // carried from phase 1 to phase 2 of a chunk (one pipeline step apart): the
  // per-token log2 decays of the thread's two channels and the lower half-wave's total
  float lam0[4], lam1[4], lower0 = 0.f, lower1 = 0.f;

  // producer phase 1 of chunk c: decay, in-thread prefix, wave totals; loads chunk c + 1.
  // The tail masks are applied to every chunk: with a single code path the words loaded
  // for the next chunk land in their final registers and are not copied (a copy would
  // wait for the load right after issuing it).
  const int lane_x32 = (lane ^ 32) << 2;  // ds_bpermute address of the other half-wave
  auto produce1 = [&](int c, auto set_c) {
    constexpr int S = decltype(set_c)::value;
    const int nvalid = min(L, T - c * L);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      pin(ld[S][0][t]); pin(ld[S][1][t]); pin(ld[S][2][t]);
      if (V6) pin(ldx[t]);
    }
    uint32_t nx[4] = {0u, 0u, 0u, 0u};
    if (V6) {
#pragma unroll
      for (int t = 0; t < 4; ++t) nx[t] = ldx[t];
    }
    if (V6) {  // tokens past the end do not decay (x = -inf)
#pragma unroll
      for (int t = 0; t < 4; ++t) nx[t] = 4 * tg + t < nvalid ? nx[t] : 0xff80ff80u;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float x0 = xs.x, x1 = xs.y;
      if (V6) {
        x0 = bf16_bits_to_f32(nx[t] & 0xffffu);
        x1 = __uint_as_float(nx[t] & 0xffff0000u);
      }
      // log2 of the decay exp(-exp(x)) is -exp(x) * log2(e)
      lam0[t] = -(fast_exp(x0) * 1.4426950408889634f);
      lam1[t] = -(fast_exp(x1) * 1.4426950408889634f);
    }
    if (!V6) {  // static decay: tokens past the end do not decay
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bool past = 4 * tg + t >= nvalid;
        lam0[t] = past ? 0.f : lam0[t];
        lam1[t] = past ? 0.f : lam1[t];
      }
    }
    const float run0 = ((lam0[0] + lam0[1]) + lam0[2]) + lam0[3];
    const float run1 = ((lam1[0] + lam1[1]) + lam1[2]) + lam1[3];
    // next chunk (rows past the end read as zero or belong to the next batch row; masked on use)
    prefetch(c + 1, std::integral_constant<int, S ^ 1>{});
    // wave totals: the upper half-wave (odd token group) adds the lower one's total
    lower0 = __int_as_float(__builtin_amdgcn_ds_bpermute(lane_x32, __float_as_int(run0)));
    lower1 = __int_as_float(__builtin_amdgcn_ds_bpermute(lane_x32, __float_as_int(run1)));
    if (hh) sm.wtot[c & 1][pwave][cp] = make_float2(run0 + lower0, run1 + lower1);
  };

  // producer phase 2 of chunk c: prefix, scaled operands as bf16 hi / lo, V^T, bonus
  auto produce2 = [&](int c, auto set_c) {
    constexpr int S = decltype(set_c)::value;
    Ops &o = sm.ops[c & 1];
    const uint32_t *rw = ld[S][0], *kw = ld[S][1], *vw = ld[S][2];  // zero past the last token
    // decay prefix of the waves before this one (pwave is wave-uniform) and the
    // chunk totals, from the eight wave totals read four at a time
    float pre0 = hh ? lower0 : 0.f, pre1 = hh ? lower1 : 0.f, tot0 = 0.f, tot1 = 0.f;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float2 wt[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) wt[q] = sm.wtot[c & 1][4 * half + q][cp];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float m = 4 * half + q < pwave ? 1.f : 0.f;
        pre0 = fmaf(m, wt[q].x, pre0);
        pre1 = fmaf(m, wt[q].y, pre1);
        tot0 += wt[q].x;
        tot1 += wt[q].y;
      }
    }
    // The chunk leaves the exponent range when some channel's total is below
    // -kMaxLog2 (or is -inf).  Every producer wave sees all 64 channels and the
    // same totals, so the ballot gives every wave the same answer.
    const bool direct = __builtin_amdgcn_ballot_w64(!(tot0 >= -kMaxLog2 && tot1 >= -kMaxLog2)) != 0;
    if (pwave == 0 && lane == 0) o.direct = direct ? 1 : 0;
    if (!direct) {
      if (pwave == 0 && !hh)  // exp(Lam_{L-1}) per key row
        *reinterpret_cast<float2 *>(&o.pl[2 * cp]) =
            make_float2(__builtin_amdgcn_exp2f(tot0), __builtin_amdgcn_exp2f(tot1));
      float c0 = 0.f, c1 = 0.f;  // in-thread inclusive prefix of the log2 decays
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int tau = 4 * tg + t;
        const float lp0 = t ? pre0 + c0 : pre0, lp1 = t ? pre1 + c1 : pre1;
        c0 = t ? c0 + lam0[t] : lam0[t];
        c1 = t ? c1 + lam1[t] : lam1[t];
        const float la0 = pre0 + c0, la1 = pre1 + c1;
        const float r0 = bf16_bits_to_f32(rw[t] & 0xffffu), r1 = __uint_as_float(rw[t] & 0xffff0000u);
        const float k0 = bf16_bits_to_f32(kw[t] & 0xffffu), k1 = __uint_as_float(kw[t] & 0xffff0000u);
        uint32_t hi, lo;
        split2(r0 * __builtin_amdgcn_exp2f(lp0), r1 * __builtin_amdgcn_exp2f(lp1), hi, lo);
        *reinterpret_cast<uint32_t *>(&o.rb_hi[tau][2 * cp]) = hi;
        *reinterpret_cast<uint32_t *>(&o.rb_lo[tau][2 * cp]) = lo;
        split2(k0 * __builtin_amdgcn_exp2f(-la0), k1 * __builtin_amdgcn_exp2f(-la1), hi, lo);
        *reinterpret_cast<uint32_t *>(&o.kt_hi[tau][2 * cp]) = hi;
        *reinterpret_cast<uint32_t *>(&o.kt_lo[tau][2 * cp]) = lo;
      }
    } else {
      // direct recurrence: r and k as loaded, the per-token decays d = 2^lam split
      // into their upper and lower 16 bits (the same addresses as the MFMA form)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int tau = 4 * tg + t;
        const uint32_t d0 = __float_as_uint(__builtin_amdgcn_exp2f(lam0[t]));
        const uint32_t d1 = __float_as_uint(__builtin_amdgcn_exp2f(lam1[t]));
        *reinterpret_cast<uint32_t *>(&o.rb_hi[tau][2 * cp]) = rw[t];
        *reinterpret_cast<uint32_t *>(&o.rb_lo[tau][2 * cp]) = kw[t];
        *reinterpret_cast<uint32_t *>(&o.kt_hi[tau][2 * cp]) = __builtin_amdgcn_perm(d1, d0, 0x07060302u);
        *reinterpret_cast<uint32_t *>(&o.kt_lo[tau][2 * cp]) = __builtin_amdgcn_perm(d1, d0, 0x05040100u);
      }
    }
    // bonus diagonal: the sum over the 32 channel pairs of a token group (one half-wave)
    float bon[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float r0 = bf16_bits_to_f32(rw[t] & 0xffffu), r1 = __uint_as_float(rw[t] & 0xffff0000u);
      const float k0 = bf16_bits_to_f32(kw[t] & 0xffffu), k1 = __uint_as_float(kw[t] & 0xffff0000u);
      bon[t] = fmaf(r1 * u2.y, k1, r0 * u2.x * k0);
    }
    float bsum;
    {
      const bool up16 = lane & 16;
      float keep0 = up16 ? bon[2] : bon[0], keep1 = up16 ? bon[3] : bon[1];
      keep0 += xor_swz<16>(up16 ? bon[0] : bon[2]);
      keep1 += xor_swz<16>(up16 ? bon[1] : bon[3]);
      const bool up8 = lane & 8;
      bsum = up8 ? keep1 : keep0;
      bsum += xor_swz<8>(up8 ? keep0 : keep1);
      bsum += xor_swz<4>(bsum);
      bsum += xor2(bsum);
      bsum += xor1(bsum);
    }
    // V^T: tokens 4tg..4tg+3 of channels 2cp (low halves) and 2cp+1 (high halves)
    *reinterpret_cast<uint2 *>(&o.vt[2 * cp][4 * tg]) = make_uint2(
        __builtin_amdgcn_perm(vw[1], vw[0], 0x05040100u), __builtin_amdgcn_perm(vw[3], vw[2], 0x05040100u));
    *reinterpret_cast<uint2 *>(&o.vt[2 * cp + 1][4 * tg]) = make_uint2(
        __builtin_amdgcn_perm(vw[1], vw[0], 0x07060302u), __builtin_amdgcn_perm(vw[3], vw[2], 0x07060302u));
    if ((lane & 7) == 0) o.bonus[4 * tg + ((lane & 16) ? 2 : 0) + ((lane & 8) ? 1 : 0)] = bsum;
  };

  // consumer work on chunk c
  auto consume = [&](int c) {
    const Ops &o = sm.ops[c & 1];
    const int buf = c & 1;
    const int nvalid = min(L, T - c * L);
    if (y_wave) {
      // Output tile: tokens 32 TB + (0..31) x all 64 value columns (two 32x32
      // accumulators), accumulated transposed (Y^T) so that each lane ends up
      // with one token's columns.  Per K step q (key rows 16q + 8hh + 0..7) the lane's rbar row
      // is the B operand of both
      //   Y^T += S0^T rbar^T     (S^T rows from LDS as the A operand)
      //   AT  += ktil rbar^T     (ktil rows of each causal s-block as the A operand)
      // AT then holds A^T[s = 32 sb + 8(e/4) + 4hh + e%4][t] in lane (t, hh).
      auto out_tile = [&](auto tb_c) {
        constexpr int TB = decltype(tb_c)::value;
        const int trow = 32 * TB + l32;
        f32x16 Y[2] = {f32x16{}, f32x16{}}, AT[TB + 1];
#pragma unroll
        for (int sb = 0; sb <= TB; ++sb) AT[sb] = f32x16{};
        // Operands of K step q.  Each group of the next step's operands is
        // loaded as soon as the products of this step that read the same group
        // have been issued, so the loads overlap the remaining products while
        // only the rbar pair needs a second set of registers.  With two A^T
        // blocks (TB = 1) the r̄ S0 and A^T products take separate passes over
        // K (rbar read twice) to stay within the register budget.
        auto col_of = [&](int q) { return 16 * q + 8 * hh; };
        auto k_pass = [&](auto do_y_c, auto do_at_c) {
          constexpr bool DY = decltype(do_y_c)::value, DA = decltype(do_at_c)::value;
          bf16x8 rh = ld8(&o.rb_hi[trow][col_of(0)]), rl = ld8(&o.rb_lo[trow][col_of(0)]);
          bf16x8 sh[2], sl[2], kh[TB + 1], kl[TB + 1];
          if (DY) {
#pragma unroll
            for (int tc = 0; tc < 2; ++tc) {
              sh[tc] = ld8(&sm.st[buf][0][32 * tc + l32][col_of(0)]);
              sl[tc] = ld8(&sm.st[buf][1][32 * tc + l32][col_of(0)]);
            }
          }
          if (DA) {
#pragma unroll
            for (int sb = 0; sb <= TB; ++sb) {
              kh[sb] = ld8(&o.kt_hi[32 * sb + l32][col_of(0)]);
              kl[sb] = ld8(&o.kt_lo[32 * sb + l32][col_of(0)]);
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int nc = col_of(q + 1);
            if (DY) {
#pragma unroll
              for (int tc = 0; tc < 2; ++tc) {
                Y[tc] = mfma32(sh[tc], rh, Y[tc]);
                Y[tc] = mfma32(sl[tc], rh, Y[tc]);
                Y[tc] = mfma32(sh[tc], rl, Y[tc]);
                __builtin_amdgcn_sched_barrier(0);
                if (q < 3) {
                  sh[tc] = ld8(&sm.st[buf][0][32 * tc + l32][nc]);
                  sl[tc] = ld8(&sm.st[buf][1][32 * tc + l32][nc]);
                }
                __builtin_amdgcn_sched_barrier(0);
              }
            }
            if (DA) {
#pragma unroll
              for (int sb = 0; sb <= TB; ++sb) {
                AT[sb] = mfma32(kh[sb], rh, AT[sb]);
                AT[sb] = mfma32(kh[sb], rl, AT[sb]);
                AT[sb] = mfma32(kl[sb], rh, AT[sb]);
                __builtin_amdgcn_sched_barrier(0);
                if (q < 3) {
                  kh[sb] = ld8(&o.kt_hi[32 * sb + l32][nc]);
                  kl[sb] = ld8(&o.kt_lo[32 * sb + l32][nc]);
                }
                __builtin_amdgcn_sched_barrier(0);
              }
            }
            if (q < 3) {
              rh = ld8(&o.rb_hi[trow][nc]);
              rl = ld8(&o.rb_lo[trow][nc]);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        };
        if (TB == 0) {
          k_pass(std::true_type{}, std::true_type{});
        } else {
          k_pass(std::true_type{}, std::false_type{});
          k_pass(std::false_type{}, std::true_type{});
        }
        {  // diagonal block: keep s < t, the bonus on s == t, zero above
          const float bon = o.bonus[trow];
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int sl = 8 * (e >> 2) + 4 * hh + (e & 3);
            AT[TB][e] = sl < l32 ? AT[TB][e] : (sl == l32 ? bon : 0.f);
          }
        }
        // Y^T += V^T A^T.  K step (sb, ks) uses AT[sb][8ks .. 8ks+7] as the B operand:
        // slot 8hh + e' is token s = 32 sb + 16 ks + 8(e'/4) + 4hh + e'%4, and V^T is
        // read in that order.
#pragma unroll
        for (int sb = 0; sb <= TB; ++sb) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const int s0 = 32 * sb + 16 * ks + 4 * hh;
            bf16x8 bv[2];
#pragma unroll
            for (int tc = 0; tc < 2; ++tc) bv[tc] = ld4x2(&o.vt[32 * tc + l32][s0], &o.vt[32 * tc + l32][s0 + 8]);
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) split2(AT[sb][8 * ks + 2 * m], AT[sb][8 * ks + 2 * m + 1], hw[m], lw[m]);
            const bf16x8 ah = as_bf16x8(hw[0], hw[1], hw[2], hw[3]), al = as_bf16x8(lw[0], lw[1], lw[2], lw[3]);
#pragma unroll
            for (int tc = 0; tc < 2; ++tc) {
              Y[tc] = mfma32(bv[tc], ah, Y[tc]);
              Y[tc] = mfma32(bv[tc], al, Y[tc]);
            }
          }
        }
        // Y^T accumulators: lane (token trow, hh) holds y[trow][32 tc + 8m + 4hh + 0..3] in
        // Y[tc][4m .. 4m+3], four 16-byte (fp32) or 8-byte (bf16) stores per lane and column block
        constexpr int ESZ = OUTB ? 2 : 4;
        char *yb = reinterpret_cast<char *>(p.y) + uniform64((base + (long)c * L * ts) * ESZ);
        char *yrow = yb + (uint32_t)((trow * ts + 4 * hh) * ESZ);
        if (nvalid == L || trow < nvalid) {
#pragma unroll
          for (int tc = 0; tc < 2; ++tc)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              if constexpr (OUTB)
                reinterpret_cast<uint2 *>(yrow)[8 * tc + 2 * m] =
                    make_uint2(pack_bf16(Y[tc][4 * m], Y[tc][4 * m + 1]), pack_bf16(Y[tc][4 * m + 2], Y[tc][4 * m + 3]));
              else
                reinterpret_cast<float4 *>(yrow)[8 * tc + 2 * m] =
                    make_float4(Y[tc][4 * m], Y[tc][4 * m + 1], Y[tc][4 * m + 2], Y[tc][4 * m + 3]);
            }
        }
      };
      // output waves 0 and 1 own token blocks 0 and 1 with all 64 value columns, so each A^T
      // block is formed once; consumer waves 2 and 3 have no output work
      if (cw == 1) out_tile(std::integral_constant<int, 1>{});
      else if (cw == 0) out_tile(std::integral_constant<int, 0>{});
    } else {
      // S += ktil^T V over the chunk's 64 tokens in four K steps of 16.  The
      // A operand (row = key i = 32 tile_r + lane % 32, slots 8hh + e = tokens
      // 16 ks + 8hh + e) is read transposed from the row-major ktil: lane group
      // g = lane / 16 covers keys 32 tile_r + 16 (g & 1) + (0..15), and its
      // source lane 4a + b points at ktil[token 16 ks + 8hh + a (+4)][key + 4b].
      const int g = lane >> 4;
      const int kcol = 32 * tile_r + 16 * (g & 1) + 4 * (lane & 3);
      const int trow0 = 8 * (g >> 1) + ((lane >> 2) & 3);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int tr = 16 * ks + trow0;
        const uint2 h0 = ld_tr(&o.kt_hi[tr][kcol]), h1 = ld_tr(&o.kt_hi[tr + 4][kcol]);
        const uint2 l0 = ld_tr(&o.kt_lo[tr][kcol]), l1 = ld_tr(&o.kt_lo[tr + 4][kcol]);
        const bf16x8 bv = ld8(&o.vt[jcol][16 * ks + 8 * hh]);
        S = mfma32(as_bf16x8(h0.x, h0.y, h1.x, h1.y), bv, S);
        S = mfma32(as_bf16x8(l0.x, l0.y, l1.x, l1.y), bv, S);
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

  // Direct recurrence over chunk c, for chunks outside the exponent range.  The
  // eight consumer waves share it by value columns: wave cw owns columns
  // 8cw .. 8cw + 7, and lane 8m + q holds rows 8q .. 8q + 7 of column 8cw + m, so
  // a token's output is a sum inside the lane and over the column's eight lanes
  // (three DPP adds), and the state update needs no exchange at all.  The state
  // moves from the state waves' tile layout to this one and back through the fp32
  // buffer in st[c & 1], with one extra workgroup barrier each way (every wave of
  // the workgroup takes them).  Lane q keeps the output of the q-th token of each
  // group of eight, so a store covers eight tokens.
  auto direct_chunk = [&](int c) {
    const Ops &o = sm.ops[c & 1];
    float *sf = reinterpret_cast<float *>(&sm.st[c & 1][0][0][0]);  // [key row][SFS]
    const int nvalid = min(L, T - c * L);
    // Addresses of this rare path are built from an opaque copy of the lane
    // index, so the compiler does not hoist them out of the chunk loop (where
    // they would hold registers across the matrix-core path).
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int tile_off = (32 * tile_r + 4 * (ln >> 5)) * SFS + 32 * tile_c + (ln & 31);
    if (!y_wave) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sf[tile_off + (8 * (e >> 2) + (e & 3)) * SFS] = S[e];
    }
    __syncthreads();
    const int q = ln & 7, col = 8 * cw + (ln >> 3);
    float s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = sf[(8 * q + e) * SFS + col];
    constexpr int ESZ = OUTB ? 2 : 4;
    char *yb = reinterpret_cast<char *>(p.y) + (base + (long)c * L * ts + col) * ESZ;
    for (int t0 = 0; t0 < L; t0 += 8) {
      const uint4 v8 = *reinterpret_cast<const uint4 *>(&o.vt[col][t0]);
      const float4 b0 = *reinterpret_cast<const float4 *>(&o.bonus[t0]);
      const float4 b1 = *reinterpret_cast<const float4 *>(&o.bonus[t0 + 4]);
      const float vv[8] = {bf16_lo(v8.x), bf16_hi(v8.x), bf16_lo(v8.y), bf16_hi(v8.y),
                           bf16_lo(v8.z), bf16_hi(v8.z), bf16_lo(v8.w), bf16_hi(v8.w)};
      const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      float ykeep = 0.f;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const int t = t0 + tt;
        const uint4 rr = *reinterpret_cast<const uint4 *>(&o.rb_hi[t][8 * q]);
        const uint4 kk = *reinterpret_cast<const uint4 *>(&o.rb_lo[t][8 * q]);
        const uint4 dh = *reinterpret_cast<const uint4 *>(&o.kt_hi[t][8 * q]);
        const uint4 dl = *reinterpret_cast<const uint4 *>(&o.kt_lo[t][8 * q]);
        const float r[8] = {bf16_lo(rr.x), bf16_hi(rr.x), bf16_lo(rr.y), bf16_hi(rr.y),
                            bf16_lo(rr.z), bf16_hi(rr.z), bf16_lo(rr.w), bf16_hi(rr.w)};
        const float k[8] = {bf16_lo(kk.x), bf16_hi(kk.x), bf16_lo(kk.y), bf16_hi(kk.y),
                            bf16_lo(kk.z), bf16_hi(kk.z), bf16_lo(kk.w), bf16_hi(kk.w)};
        float d[8];
        {
          const uint32_t hw[4] = {dh.x, dh.y, dh.z, dh.w}, lw[4] = {dl.x, dl.y, dl.z, dl.w};
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            d[2 * m] = __uint_as_float(__builtin_amdgcn_perm(hw[m], lw[m], 0x05040100u));
            d[2 * m + 1] = __uint_as_float(__builtin_amdgcn_perm(hw[m], lw[m], 0x07060302u));
          }
        }
        float p0 = r[0] * s[0], p1 = r[1] * s[1];
#pragma unroll
        for (int e = 2; e < 8; e += 2) {
          p0 = fmaf(r[e], s[e], p0);
          p1 = fmaf(r[e + 1], s[e + 1], p1);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = fmaf(d[e], s[e], k[e] * vv[tt]);
        float part = p0 + p1;
        part += xor1(part);
        part += xor2(part);
        part += mirror8(part);
        const float yv = fmaf(bb[tt], vv[tt], part);
        ykeep = q == tt ? yv : ykeep;
      }
      if (t0 + q < nvalid) {
        char *yp = yb + (long)(t0 + q) * ts * ESZ;
        if constexpr (OUTB)
          *reinterpret_cast<uint16_t *>(yp) = bf16_bits(ykeep);
        else
          *reinterpret_cast<float *>(yp) = ykeep;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) sf[(8 * q + e) * SFS + col] = s[e];
    __syncthreads();
    if (!y_wave) {
#pragma unroll
      for (int e = 0; e < 16; ++e) S[e] = sf[tile_off + (8 * (e >> 2) + (e & 3)) * SFS];
      publish_state((c & 1) ^ 1);
    }
  };
  // wave-uniform: does chunk c take the direct recurrence?
  auto is_direct = [&](int c) { return __builtin_amdgcn_readfirstlane(sm.ops[c & 1].direct) != 0; };

  // Step i: producers finish chunk i + 1 and start chunk i + 2 while the
  // consumers process chunk i.  Producers, output waves and state waves run
  // separate loops (so each keeps only its own registers live) with one
  // workgroup barrier per step, plus two when chunk i runs directly.
  if (producer) {
    // step i works on chunks i + 1 (register set (i + 1) & 1) and i + 2 (set i & 1);
    // the loop is unrolled by two so that the sets are fixed in each copy
    auto step = [&](int i, auto par) {
      constexpr int P = decltype(par)::value;
      if (i >= -1 && i + 1 < nchunks) produce2(i + 1, std::integral_constant<int, P ^ 1>{});
      if (i + 2 < nchunks) produce1(i + 2, std::integral_constant<int, P>{});
    };
    prefetch(0, std::integral_constant<int, 0>{});
    // the producers' vector-ALU chain is the longest per step: let them issue first
    __builtin_amdgcn_s_setprio(2);
    auto direct_barriers = [&](int i) {
      if (i >= 0 && is_direct(i)) {
        __syncthreads();
        __syncthreads();
      }
    };
    for (int i = -2; i < nchunks; i += 2) {
      step(i, std::integral_constant<int, 0>{});
      direct_barriers(i);
      __syncthreads();
      if (i + 1 < nchunks) {
        step(i + 1, std::integral_constant<int, 1>{});
        direct_barriers(i + 1);
        __syncthreads();
      }
    }
  } else if (cw >= 2 && cw < 4) {
    // The two consumer waves without output work run their own copy of the chunk loop.  In
    // it they read one word of each 64-byte half of every token row of chunk i + kWarmAhead
    // (r, k on one wave, v and the v6 decays on the other) right after the barrier that opens
    // step i, ahead of the producers' own loads of that chunk late in the step, and fold the
    // words into a value that is never stored (T is never negative).  Measured sustained at
    // B=8 T=4096 H=32 and B=4 H=40: 191-193 / 187 us; with these waves in the output waves'
    // loop, 203 / 198 us; with their own loop but without this code, also 203 / 198 us; with
    // this code but a distance so large that no read is ever issued, 190 / 187 us.  So the
    // time this saves comes from how the kernel compiles with this branch in it (the hot
    // loops of the other roles are the same instructions), not from the reads; the reads cost
    // nothing in HBM bytes (measured traffic equals the algorithmic).
    const int w2 = cw - 2;
    const uint32_t wofs0 = (uint32_t)(((lane >> 1) * ts) * 2 + (lane & 1) * 64);
    const uint32_t wofs1 = wofs0 + (uint32_t)(32 * ts * 2);
    uint32_t wl[4] = {0u, 0u, 0u, 0u}, acc = 0u;
    for (int i = -2; i < nchunks; ++i) {
      if (i >= 0 && is_direct(i)) direct_chunk(i);
      acc ^= (wl[0] ^ wl[1]) ^ (wl[2] ^ wl[3]);
      const int cwarm = i + kWarmAhead;
      if (cwarm < nchunks) {
        const unsigned long long off = (unsigned long long)uniform64((base + (long)cwarm * L * ts) * 2);
        const auto ra = rsrc_at(w2 ? p.v : p.r, off);
        wl[0] = __builtin_amdgcn_raw_buffer_load_b32(ra, (int)wofs0, 0, 0);
        wl[1] = __builtin_amdgcn_raw_buffer_load_b32(ra, (int)wofs1, 0, 0);
        if (!w2 || V6) {
          const auto rb = rsrc_at(w2 ? p.w : p.k, off);
          wl[2] = __builtin_amdgcn_raw_buffer_load_b32(rb, (int)wofs0, 0, 0);
          wl[3] = __builtin_amdgcn_raw_buffer_load_b32(rb, (int)wofs1, 0, 0);
        }
      }
      __syncthreads();
    }
    acc ^= (wl[0] ^ wl[1]) ^ (wl[2] ^ wl[3]);
    if (T < 0) sm.wtot[0][0][0].x = __uint_as_float(acc);
  } else if (y_wave) {
    for (int i = -2; i < nchunks; ++i) {
      if (i >= 0) {
        if (is_direct(i)) direct_chunk(i);
        else consume(i);
      }
      __syncthreads();
    }
  } else {
    // SAVE: the state at the start of every later chunk, as the state waves hold it after
    // chunk i (fp32, before its bf16 split), into [row, head, chunk - 1] of chunk_states
    float *cs = nullptr;
    if constexpr (SAVE) cs = p.chunk_states + ((long)b * p.H + h) * (long)(nchunks - 1) * (kHead * kHead);
    for (int i = -2; i < nchunks; ++i) {
      if (i >= 0) {
        if (is_direct(i)) direct_chunk(i);
        else consume(i);
        if constexpr (SAVE) {
          if (i + 1 < nchunks) {
            float *sp = cs + (long)i * (kHead * kHead);
#pragma unroll
            for (int e = 0; e < 16; ++e) sp[(32 * tile_r + 8 * (e >> 2) + 4 * hh + (e & 3)) * kHead + jcol] = S[e];
          }
        }
      }
      __syncthreads();
    }
  }

  if (!producer && !y_wave && p.state_out) {
    float *sp = p.state_out + ((long)b * p.H + h) * (kHead * kHead);
#pragma unroll
    for (int e = 0; e < 16; ++e) sp[(32 * tile_r + 8 * (e >> 2) + 4 * hh + (e & 3)) * kHead + jcol] = S[e];
  }
}

template <bool V6, bool OUTB, bool SAVE>
hipError_t launch(const ScanParams &p, hipStream_t s) {
  // The dynamic-LDS limit is a per-device function attribute: set it once per device.
  static std::atomic<unsigned long long> configured{0};
  const size_t lds = sizeof(Smem);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = 1ull << (dev & 63);
  if (!(configured.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&wkv56_chunked_kernel<V6, OUTB, SAVE>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    configured.fetch_or(bit, std::memory_order_acq_rel);
  }
  dim3 grid(p.H * p.units);
  hipLaunchKernelGGL((wkv56_chunked_kernel<V6, OUTB, SAVE>), grid, dim3(kThreads), lds, s, p);
  return hipGetLastError();
}

}  // namespace
}  // namespace wkv
