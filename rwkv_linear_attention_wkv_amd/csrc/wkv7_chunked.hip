// 64-token chunked WKV v7 (the generalized delta rule of the rwkv_ops page's
// generalized_delta_rule operator) with the contractions on MFMA (gfx950).
//
// Recurrence, per (batch row, head), state h[key i][value j], d_t = exp(-exp(w_t)):
//   sa_t = a_t^T h_{t-1},  h_t = diag(d_t) h_{t-1} + b_t sa_t^T + k_t v_t^T,  y_t = h_t^T r_t
// (the standard RWKV-7 recurrence, as the token-sequential kernel).
//
// Chunked form.  Inside a chunk of L = 64 tokens that starts from the state H0, let
// P_t[i] be the inclusive log2-decay prefix (P_{-1} = 0), D_t = diag(2^P_t), and, as rows
// of L x 64 matrices,
//   Ab_t = D_{t-1} a_t,   Rb_t = D_t r_t,   Bt_s = D_s^{-1} b_s,   Kt_s = D_s^{-1} k_s.
// Unrolling the recurrence from H0 gives, with SA the rows sa_t and Y the rows y_t,
//   SA = Ab H0 + tril_{-1}(Ab Bt^T) SA + tril_{-1}(Ab Kt^T) V
//   Y  = Rb H0 + tril_0(Rb Bt^T) SA + tril_0(Rb Kt^T) V
//   H1 = D_{L-1} (H0 + Bt^T SA + Kt^T V)
// (every product that survives a mask carries 2^(P_{t'} - P_s) <= 1).  The first line
// is the unit lower-triangular system (I - M) SA = RHS, M = tril_{-1}(Ab Bt^T),
// RHS = Ab H0 + tril_{-1}(Ab Kt^T) V, solved by forward substitution in fp32; the
// transitions diag(d) + b a^T of the RWKV-7 time mix are contractions, so (I - M)^{-1}
// stays bounded.
//
// Precision.  Products run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation; every
// operand that is not an exact bf16 input is split into hi + lo bf16 and a product is
// hi*hi + hi*lo + lo*hi (two products against the exact V), as in the v6 chunked kernel.
//
// Range.  Kt and Bt carry 2^(-P_s) >= 1.  A chunk whose log2-decay total is below
// -kMaxLog2 (or -inf) in some channel runs the direct recurrence instead: every wave
// walks the chunk's tokens one at a time over 8 value columns (lane 8m + q holds rows
// 8q .. 8q+7 of one column), the two sums over key rows being DPP sums over a column's
// eight lanes.  Decays exp(-exp(w)) with w <= 0 never need it.
//
// Work decomposition: one 512-thread workgroup (8 waves) per (row, head) walks its
// chunks in order, four workgroup barriers per chunk:
//   stage   all waves: thread (channel pair cp, token group tg) turns its 4 tokens of the
//           (one chunk ahead) loaded words into log2 decays, posts its wave's totals,
//           [barrier] adds the earlier waves' totals and writes Ab, Rb, Bt, Kt as bf16
//           hi / lo [token][key], V^T [col][token] and the final decay; requests the next
//           chunk's words.  [barrier]
//   A       waves 0 .. 3 (token block, value-column block): RHS^T = H0^T Ab^T + V^T Gak^T to
//           LDS (fp32);
//           waves 4 .. 7 (one 32 x 32 tile of the fp32 state each): H += Kt^T V, and waves
//           4 .. 6 one 32 x 32 block of M each, to LDS (fp32).  [barrier]
//   solve   waves 4 .. 7: value columns 16 (w - 4) + 4g .. +3, sixteen lanes (one per
//           residue of the token index mod 16) hold their rows; each final row is broadcast
//           to them and added to the later rows; SA^T to LDS as bf16 hi / lo.
//           Meanwhile, on the matrix cores, waves 0, 1 (token block 0 / 1) form
//           Y^T = H0^T Rb^T + V^T Grk^T, with the causal
//           32 x 32 blocks Grk^T = Kt Rb^T formed in registers and used from there (the
//           accumulator layout is the operand layout, with the token order permuted
//           alike on the other side), and the blocks Grb^T = Bt Rb^T.  [barrier]
//   C       waves 0, 1: Y^T += SA^T Grb^T, then y;
//           waves 4 .. 7: H = D_{L-1} (H + Bt^T SA)
//           and H^T published as bf16 hi / lo for the next chunk; then every wave starts
//           the next chunk's stage.
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma_ops.hpp"
#include "wkv.h"

namespace wkv {
namespace {

constexpr int L = 64;           // tokens per chunk
constexpr int kThreads = 512;   // 8 waves
constexpr int RS = 72;          // LDS row stride in bf16 elements (144 bytes)
constexpr int SFS = 68;         // row stride (floats) of the fp32 state of a direct chunk
constexpr float kMaxLog2 = 100.f;

// Operand planes.  MFMA chunks: Ab, Rb, Bt, Kt as hi / lo pairs.  Direct chunks: a, r, b,
// k as loaded in the hi planes, the decay's upper / lower 16 bits in planes 1 / 3.
enum { AB = 0, RB = 2, BT = 4, KT = 6 };

struct alignas(16) Smem7 {
  uint16_t op[8][L][RS];       // [token][key]
  uint16_t vt[kHead][RS];      // V^T [col][token]
  uint16_t ht[2][kHead][RS];   // H0^T hi / lo [col][key]
  uint16_t sat[2][kHead][RS];  // SA^T hi / lo [col][token]
  // fp32 rows padded to 68 floats, so that 32 lanes writing 32 consecutive rows spread over
  // the banks
  float rhs[L][SFS];           // RHS [token][col]; with mp: the fp32 state of a direct chunk
  float mp[L][SFS];            // M[16u + p][s] at [s][4 p + u] (column s of M for the solve)
  uint16_t mlo[2][32][40];     // M[32 + t][s], s < 32, as bf16 hi / lo [t][s]
  float pl[kHead];             // 2^P_{L-1} per key row
  float2 wtot[8][32];          // log2-decay total of each wave, per channel pair
  int direct;
};
static_assert(sizeof(float) * kHead * SFS <= sizeof(float) * 2 * L * SFS, "direct state fits");
static_assert(sizeof(Smem7) <= 160 * 1024, "one workgroup's LDS");

// Lane (lane & ~3) | q to the four lanes of its quad (DPP quad permute); q must fold to a
// constant.
template <int Q>
__device__ __forceinline__ float bcast4_c(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x55 * Q, 0xF, 0xF, false));
}
__device__ __forceinline__ float bcast4(float x, int q) {
  switch (q) {
    case 0: return bcast4_c<0>(x);
    case 1: return bcast4_c<1>(x);
    case 2: return bcast4_c<2>(x);
    default: return bcast4_c<3>(x);
  }
}

// Lane Q of each row of 16 lanes to the whole row (DPP row_newbcast).
template <int Q>
__device__ __forceinline__ float bcast16_c(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x150 + Q, 0xF, 0xF, false));
}

// f(integral_constant<int, I>) for I = I0 .. N - 1, so that every step's indices are
// compile-time constants (a rolled loop would keep the register arrays it indexes in memory)
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

template <bool OUTB>
__global__ void __launch_bounds__(kThreads) wkv7_chunked_kernel(V7Params p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem7 &sm = *reinterpret_cast<Smem7 *>(smem_raw);

  // batch row = id % B: the heads of a row go to one XCD (see the v6 chunked kernel)
  const int b = blockIdx.x % p.B;
  const int h = blockIdx.x / p.B;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = p.T;
  const long ts = p.tok_stride;
  const long base = b * p.row_stride + h * p.head_stride;
  const int nchunks = (T + L - 1) / L;

  int row_in = -1;
  if (p.state_in) {
    row_in = p.state_map ? p.state_map[b] : (p.n_state == 1 ? 0 : b);
    if (row_in < 0 || row_in >= p.n_state) {
      if (tid == 0 && p.dev_status) atomicOr(p.dev_status, WKV_DEV_BAD_STATE_MAP);
      return;
    }
  }

  // ---------------- state waves 4 .. 7: a 32 x 32 tile of the fp32 state each
  const bool state_wave = wave >= 4;
  const int tile_r = ((wave - 4) & 3) >> 1;  // key-row block
  const int tile_c = (wave - 4) & 1;         // value-column block
  const int jcol = 32 * tile_c + l32;
  f32x16 H = {};  // rows 32 tile_r + 8 (e/4) + 4 hh + e%4, column jcol
  auto publish_state = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t h0, l0, h1, l1;
      split2(H[4 * q], H[4 * q + 1], h0, l0);
      split2(H[4 * q + 2], H[4 * q + 3], h1, l1);
      const int i0 = 32 * tile_r + 8 * q + 4 * hh;
      *reinterpret_cast<uint2 *>(&sm.ht[0][jcol][i0]) = make_uint2(h0, h1);
      *reinterpret_cast<uint2 *>(&sm.ht[1][jcol][i0]) = make_uint2(l0, l1);
    }
  };
  if (state_wave) {
    if (row_in >= 0) {
      const float *sp = p.state_in + ((long)row_in * p.H + h) * (kHead * kHead);
#pragma unroll
      for (int e = 0; e < 16; ++e) H[e] = sp[(32 * tile_r + 8 * (e >> 2) + 4 * hh + (e & 3)) * kHead + jcol];
    }
    publish_state();
  }

  // ---------------- staging: channels 2cp, 2cp+1 of tokens 4tg .. 4tg+3
  const int cp = tid & 31;
  const int tg = tid >> 5;
  uint32_t roff[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) roff[t] = (uint32_t)(((4 * tg + t) * ts + 2 * cp) * 2);
  const unsigned long long row_end = (unsigned long long)(base + (long)(T - 1) * ts + kHead) * 2;
  auto rsrc_at = [&](const void *ptr, unsigned long long off) __attribute__((always_inline)) {
    const unsigned long long rem = off < row_end ? row_end - off : 0ull;
    const int n = (int)(rem > 0x7fffffffull ? 0x7fffffffull : rem);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(static_cast<const char *>(ptr) + off), 0, n,
                                             0x00020000);
  };
  enum { LR = 0, LW, LK, LV, LA, LB };
  uint32_t ld[6][4];  // words of r, w, k, v, a, b; rows past the end read as zero
  // The next chunk's words of arrays n0 .. n1 - 1 (the chunk loop issues them where each role
  // can wait: see there).
  auto prefetch = [&](int c, int n0, int n1) __attribute__((always_inline)) {
    const unsigned long long off = (unsigned long long)uniform64((base + (long)c * L * ts) * 2);
    const void *src[6] = {p.r, p.w, p.k, p.v, p.a, p.b};
#pragma unroll
    for (int n = n0; n < n1; ++n) {
      const auto rs = rsrc_at(src[n], off);
#pragma unroll
      for (int t = 0; t < 4; ++t) ld[n][t] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)roff[t], 0, 0);
    }
  };
  float lam0[4], lam1[4], lower0 = 0.f, lower1 = 0.f;
  const int lane_x32 = (lane ^ 32) << 2;
  // stage, first half: log2 decays and the wave totals (tokens past the end do not decay)
  auto stage1 = [&](int c) __attribute__((always_inline)) {
    const int nvalid = min(L, T - c * L);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t x = 4 * tg + t < nvalid ? ld[LW][t] : 0xff80ff80u;
      lam0[t] = -(fast_exp(bf16_bits_to_f32(x & 0xffffu)) * 1.4426950408889634f);
      lam1[t] = -(fast_exp(__uint_as_float(x & 0xffff0000u)) * 1.4426950408889634f);
    }
    const float run0 = ((lam0[0] + lam0[1]) + lam0[2]) + lam0[3];
    const float run1 = ((lam1[0] + lam1[1]) + lam1[2]) + lam1[3];
    lower0 = __int_as_float(__builtin_amdgcn_ds_bpermute(lane_x32, __float_as_int(run0)));
    lower1 = __int_as_float(__builtin_amdgcn_ds_bpermute(lane_x32, __float_as_int(run1)));
    if (hh) sm.wtot[wave][cp] = make_float2(run0 + lower0, run1 + lower1);
  };
  // stage, second half: prefix, operands, V^T
  auto stage2 = [&](int c) __attribute__((always_inline)) {
    float pre0 = hh ? lower0 : 0.f, pre1 = hh ? lower1 : 0.f, tot0 = 0.f, tot1 = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const float2 wt = sm.wtot[w][cp];
      const float m = w < wave ? 1.f : 0.f;
      pre0 = fmaf(m, wt.x, pre0);
      pre1 = fmaf(m, wt.y, pre1);
      tot0 += wt.x;
      tot1 += wt.y;
    }
    const bool direct = __builtin_amdgcn_ballot_w64(!(tot0 >= -kMaxLog2 && tot1 >= -kMaxLog2)) != 0;
    if (wave == 0 && lane == 0) sm.direct = direct ? 1 : 0;
    const uint32_t *rw = ld[LR], *kw = ld[LK], *vw = ld[LV], *aw = ld[LA], *bw = ld[LB];
    auto lo_of = [](uint32_t x) { return bf16_bits_to_f32(x & 0xffffu); };
    auto hi_of = [](uint32_t x) { return __uint_as_float(x & 0xffff0000u); };
    if (!direct) {
      if (wave == 0 && !hh)
        *reinterpret_cast<float2 *>(&sm.pl[2 * cp]) =
            make_float2(__builtin_amdgcn_exp2f(tot0), __builtin_amdgcn_exp2f(tot1));
      float c0 = pre0, c1 = pre1;  // running prefix
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int tau = 4 * tg + t;
        const float ex0 = __builtin_amdgcn_exp2f(c0), ex1 = __builtin_amdgcn_exp2f(c1);  // D_{t-1}
        c0 += lam0[t];
        c1 += lam1[t];
        const float in0 = __builtin_amdgcn_exp2f(c0), in1 = __builtin_amdgcn_exp2f(c1);      // D_t
        const float iv0 = __builtin_amdgcn_exp2f(-c0), iv1 = __builtin_amdgcn_exp2f(-c1);    // D_t^{-1}
        uint32_t hi, lo;
        split2(lo_of(aw[t]) * ex0, hi_of(aw[t]) * ex1, hi, lo);
        *reinterpret_cast<uint32_t *>(&sm.op[AB][tau][2 * cp]) = hi;
        *reinterpret_cast<uint32_t *>(&sm.op[AB + 1][tau][2 * cp]) = lo;
        split2(lo_of(rw[t]) * in0, hi_of(rw[t]) * in1, hi, lo);
        *reinterpret_cast<uint32_t *>(&sm.op[RB][tau][2 * cp]) = hi;
        *reinterpret_cast<uint32_t *>(&sm.op[RB + 1][tau][2 * cp]) = lo;
        split2(lo_of(bw[t]) * iv0, hi_of(bw[t]) * iv1, hi, lo);
        *reinterpret_cast<uint32_t *>(&sm.op[BT][tau][2 * cp]) = hi;
        *reinterpret_cast<uint32_t *>(&sm.op[BT + 1][tau][2 * cp]) = lo;
        split2(lo_of(kw[t]) * iv0, hi_of(kw[t]) * iv1, hi, lo);
        *reinterpret_cast<uint32_t *>(&sm.op[KT][tau][2 * cp]) = hi;
        *reinterpret_cast<uint32_t *>(&sm.op[KT + 1][tau][2 * cp]) = lo;
      }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int tau = 4 * tg + t;
        const uint32_t d0 = __float_as_uint(__builtin_amdgcn_exp2f(lam0[t]));
        const uint32_t d1 = __float_as_uint(__builtin_amdgcn_exp2f(lam1[t]));
        *reinterpret_cast<uint32_t *>(&sm.op[AB][tau][2 * cp]) = aw[t];
        *reinterpret_cast<uint32_t *>(&sm.op[RB][tau][2 * cp]) = rw[t];
        *reinterpret_cast<uint32_t *>(&sm.op[BT][tau][2 * cp]) = bw[t];
        *reinterpret_cast<uint32_t *>(&sm.op[KT][tau][2 * cp]) = kw[t];
        *reinterpret_cast<uint32_t *>(&sm.op[AB + 1][tau][2 * cp]) = __builtin_amdgcn_perm(d1, d0, 0x07060302u);
        *reinterpret_cast<uint32_t *>(&sm.op[RB + 1][tau][2 * cp]) = __builtin_amdgcn_perm(d1, d0, 0x05040100u);
      }
    }
    // V^T: tokens 4tg .. 4tg+3 of channels 2cp (low halves) and 2cp+1 (high halves)
    *reinterpret_cast<uint2 *>(&sm.vt[2 * cp][4 * tg]) = make_uint2(
        __builtin_amdgcn_perm(vw[1], vw[0], 0x05040100u), __builtin_amdgcn_perm(vw[3], vw[2], 0x05040100u));
    *reinterpret_cast<uint2 *>(&sm.vt[2 * cp + 1][4 * tg]) = make_uint2(
        __builtin_amdgcn_perm(vw[1], vw[0], 0x07060302u), __builtin_amdgcn_perm(vw[3], vw[2], 0x07060302u));
  };

  // ---------------- MFMA building blocks
  // acc += A B^T over the 64 keys: A, B rows (the lane's) as bf16 hi / lo, 3 products.
  // The next step's operands are requested while this step's products issue (one step of
  // lookahead, so the loads of a pass do not all hold registers at once).
  auto mm_keys = [&](f32x16 &acc, const uint16_t *ah, const uint16_t *al, const uint16_t *bh,
                     const uint16_t *bl) __attribute__((always_inline)) {
    bf16x8 a0 = ld8(ah + 8 * hh), a1 = ld8(al + 8 * hh), b0 = ld8(bh + 8 * hh), b1 = ld8(bl + 8 * hh);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x8 c0 = a0, c1 = a1, d0 = b0, d1 = b1;
      if (q < 3) {
        const int k = 16 * (q + 1) + 8 * hh;
        a0 = ld8(ah + k); a1 = ld8(al + k); b0 = ld8(bh + k); b1 = ld8(bl + k);
      }
      acc = mfma32(c0, d0, acc);
      acc = mfma32(c1, d0, acc);
      acc = mfma32(c0, d1, acc);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // acc += A G over the 32 tokens s of block sb, G (s x t) in the accumulator layout of g
  // (lane t, rows s): A's row is read in the matching token order (slot 8hh + j of K step
  // ks is token 32 sb + 16 ks + 4 hh + 8 (j / 4) + j % 4).  A exact (al == nullptr: two
  // products) or hi / lo (three).
  auto mm_g = [&](f32x16 &acc, const uint16_t *ah, const uint16_t *al, const f32x16 &g, int sb) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int s0 = 32 * sb + 16 * ks + 4 * hh;
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) split2(g[8 * ks + 2 * m], g[8 * ks + 2 * m + 1], hw[m], lw[m]);
      const bf16x8 gh = as_bf16x8(hw[0], hw[1], hw[2], hw[3]), gl = as_bf16x8(lw[0], lw[1], lw[2], lw[3]);
      const bf16x8 a0 = ld4x2(ah + s0, ah + s0 + 8);
      acc = mfma32(a0, gh, acc);
      acc = mfma32(a0, gl, acc);
      if (al) acc = mfma32(ld4x2(al + s0, al + s0 + 8), gh, acc);
    }
  };
  // G^T block (sb, tb): rows s = 32 sb + .. of plane pair `zs`, columns t = 32 tb + lane of
  // plane pair `xt`, masked to s < t (strict) or s <= t.
  auto gram_t = [&](int zs, int xt, int sb, int tb, bool strict) __attribute__((always_inline)) {
    f32x16 g = {};
    mm_keys(g, &sm.op[zs][32 * sb + l32][0], &sm.op[zs + 1][32 * sb + l32][0], &sm.op[xt][32 * tb + l32][0],
            &sm.op[xt + 1][32 * tb + l32][0]);
    if (sb == tb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int s = 8 * (e >> 2) + 4 * hh + (e & 3);
        g[e] = (strict ? s < l32 : s <= l32) ? g[e] : 0.f;
      }
    }
    return g;
  };
  // the transposed key-side operand of the state update: A = Z^T (rows key, K = tokens)
  auto state_update = [&](int zs, const uint16_t (*bh)[RS], const uint16_t (*bl)[RS]) __attribute__((always_inline)) {
    const int g = lane >> 4;
    const int kcol = 32 * tile_r + 16 * (g & 1) + 4 * (lane & 3);
    const int trow0 = 8 * (g >> 1) + ((lane >> 2) & 3);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int tr = 16 * ks + trow0;
      const uint2 h0 = ld_tr(&sm.op[zs][tr][kcol]), h1 = ld_tr(&sm.op[zs][tr + 4][kcol]);
      const uint2 l0 = ld_tr(&sm.op[zs + 1][tr][kcol]), l1 = ld_tr(&sm.op[zs + 1][tr + 4][kcol]);
      const bf16x8 zh = as_bf16x8(h0.x, h0.y, h1.x, h1.y), zl = as_bf16x8(l0.x, l0.y, l1.x, l1.y);
      const bf16x8 b0 = ld8(&bh[jcol][16 * ks + 8 * hh]);
      H = mfma32(zh, b0, H);
      H = mfma32(zl, b0, H);
      if (bl) H = mfma32(zh, ld8(&bl[jcol][16 * ks + 8 * hh]), H);
    }
  };

  f32x16 Yt[2], Gb[2];  // output waves: Y^T tiles of their token block, Grb^T blocks
  constexpr int ESZ = OUTB ? 2 : 4;

  // ---------------- one MFMA chunk, phases A .. C (each ends at a workgroup barrier)
  // output waves: token block TB (a compile-time constant, so Gb is indexed statically)
  auto out_a = [&](auto tb_c) __attribute__((always_inline)) {
    constexpr int TB = decltype(tb_c)::value;
    const int trow = 32 * TB + l32;
    Yt[0] = Yt[1] = f32x16{};
#pragma unroll
    for (int tc = 0; tc < 2; ++tc)
      mm_keys(Yt[tc], &sm.ht[0][32 * tc + l32][0], &sm.ht[1][32 * tc + l32][0], &sm.op[RB][trow][0],
              &sm.op[RB + 1][trow][0]);
#pragma unroll
    for (int sb = 0; sb <= TB; ++sb) {
      const f32x16 g = gram_t(KT, RB, sb, TB, false);
#pragma unroll
      for (int tc = 0; tc < 2; ++tc) mm_g(Yt[tc], &sm.vt[32 * tc + l32][0], nullptr, g, sb);
    }
  };
  auto out_b = [&](auto tb_c) __attribute__((always_inline)) {  // while the state waves solve: the Grb^T blocks
    constexpr int TB = decltype(tb_c)::value;
#pragma unroll
    for (int sb = 0; sb <= TB; ++sb) Gb[sb] = gram_t(BT, RB, sb, TB, false);
  };
  auto out_c = [&](auto tb_c, int c) __attribute__((always_inline)) {
    constexpr int TB = decltype(tb_c)::value;
    const int trow = 32 * TB + l32;
#pragma unroll
    for (int sb = 0; sb <= TB; ++sb)
#pragma unroll
      for (int tc = 0; tc < 2; ++tc) mm_g(Yt[tc], &sm.sat[0][32 * tc + l32][0], &sm.sat[1][32 * tc + l32][0], Gb[sb], sb);
    const int nvalid = min(L, T - c * L);
    if (trow < nvalid) {
      char *yrow = reinterpret_cast<char *>(p.y) + (base + (long)(c * L + trow) * ts + 4 * hh) * ESZ;
#pragma unroll
      for (int tc = 0; tc < 2; ++tc)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if constexpr (OUTB)
            reinterpret_cast<uint2 *>(yrow)[8 * tc + 2 * m] = make_uint2(
                pack_bf16(Yt[tc][4 * m], Yt[tc][4 * m + 1]), pack_bf16(Yt[tc][4 * m + 2], Yt[tc][4 * m + 3]));
          else
            reinterpret_cast<float4 *>(yrow)[8 * tc + 2 * m] =
                make_float4(Yt[tc][4 * m], Yt[tc][4 * m + 1], Yt[tc][4 * m + 2], Yt[tc][4 * m + 3]);
        }
    }
  };

  // RHS^T tile of token block tb = wave & 1, value-column block tc = 1 - (wave >> 1)
  // (waves 0 .. 3 share the four tiles; a block's Gak^T is formed by both of its waves)
  auto rhs_a = [&]() __attribute__((always_inline)) {
    const int tb = wave & 1, tc = 1 - (wave >> 1);
    const int trow = 32 * tb + l32;
    f32x16 R = {};
    mm_keys(R, &sm.ht[0][32 * tc + l32][0], &sm.ht[1][32 * tc + l32][0], &sm.op[AB][trow][0],
            &sm.op[AB + 1][trow][0]);
    for (int sb = 0; sb <= tb; ++sb) {
      const f32x16 g = gram_t(KT, AB, sb, tb, true);
      mm_g(R, &sm.vt[32 * tc + l32][0], nullptr, g, sb);
    }
    // lane (t, hh) holds RHS[t][32 tc + 8m + 4hh + 0..3] in R[4m .. 4m+3]
#pragma unroll
    for (int m = 0; m < 4; ++m)
      *reinterpret_cast<float4 *>(&sm.rhs[trow][32 * tc + 8 * m + 4 * hh]) =
          make_float4(R[4 * m], R[4 * m + 1], R[4 * m + 2], R[4 * m + 3]);
  };
  auto state_a = [&]() __attribute__((always_inline)) {
    {
      state_update(KT, sm.vt, nullptr);  // H += Kt^T V
      if (wave < 7) {
        // M block (tb, sb) in {(0,0), (1,0), (1,1)}: C = Ab Bt^T, lane s, rows t
        const int tb = wave == 4 ? 0 : 1, sb = wave == 6 ? 1 : 0;
        f32x16 mm = {};
        mm_keys(mm, &sm.op[AB][32 * tb + l32][0], &sm.op[AB + 1][32 * tb + l32][0], &sm.op[BT][32 * sb + l32][0],
                &sm.op[BT + 1][32 * sb + l32][0]);
        const int s = 32 * sb + l32;
        if (wave != 5) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int t = 32 * tb + 8 * (e >> 2) + 4 * hh + (e & 3);
            sm.mp[s][4 * (t & 15) + (t >> 4)] = s < t ? mm[e] : 0.f;
          }
        } else {  // block (1, 0) as bf16 hi / lo only: the solve adds it on the matrix cores
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int t = 8 * (e >> 2) + 4 * hh + (e & 3);
            const uint16_t hi = bf16_bits(mm[e]);
            sm.mlo[0][t][l32] = hi;
            sm.mlo[1][t][l32] = bf16_bits(mm[e] - __uint_as_float((uint32_t)hi << 16));
          }
        }
      }
    }
  };

  // forward substitution (I - M) SA = RHS on the four state waves, right-looking: lane
  // 16g + p of state wave sw owns value columns 16 sw + 4g .. +3 and the rows t = 16u + p
  // (u = 0..3), which start as RHS; once row s is final, its owner hands SA[s] to the
  // sixteen lanes of its DPP row in one broadcast per column, and each adds M[t][s] SA[s]
  // to its later rows.  The lanes of one row residue read the same column of M, four
  // values per step; column s is read kPF steps ahead.  In two halves: rows 0..31 first,
  // then rows 32..63 receive the sum over s < 32 as one product on the matrix cores
  // (M's block below the diagonal as bf16 hi / lo against SA^T), then rows 32..63.
  auto solve = [&]() __attribute__((always_inline)) {
    // Per-lane bases formed here from an opaque copy of the lane index: every access below
    // is one of them plus a constant offset.  (With the plain indices the compiler hoisted
    // the 63 column addresses of M, which lie past the 64 KiB reach of the offset field,
    // out of the chunk loop, and spilled.)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int sw = wave - 4;
    const int pq = ln & 15, cq = 16 * sw + 4 * (ln >> 4);
    const float *mcol = &sm.mp[0][0] + 4 * pq;          // + s * SFS: M[16u + p][s], u = 0..3
    float *rrow = &sm.rhs[0][0] + pq * SFS + cq;        // + 16u * SFS: RHS[16u + p][col .. col + 3]
    uint16_t *shi = &sm.sat[0][0][0] + cq * RS + pq, *slo = &sm.sat[1][0][0] + cq * RS + pq;
    float R[4][4];  // [u][c]: row 16u + p, column col + c
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4 r4 = *reinterpret_cast<const float4 *>(rrow + 16 * u * SFS);
      R[u][0] = r4.x; R[u][1] = r4.y; R[u][2] = r4.z; R[u][3] = r4.w;
    }
    constexpr int kPF = 2;
    float4 mq[kPF];
    auto steps = [&](auto s0_c, auto s1_c) __attribute__((always_inline)) {  // rows s0 .. s1 - 1 final
      constexpr int S0 = decltype(s0_c)::value, S1 = decltype(s1_c)::value, UE = (S1 + 15) / 16;
      static_for<S0, S0 + kPF>([&](auto s_c) __attribute__((always_inline)) {
        constexpr int s = decltype(s_c)::value;
        mq[s % kPF] = *reinterpret_cast<const float4 *>(mcol + s * SFS);
      });
      static_for<S0, S1>([&](auto s_c) __attribute__((always_inline)) {
        constexpr int s = decltype(s_c)::value, us = s >> 4, q = s & 15;
        float x[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) x[c] = bcast16_c<q>(R[us][c]);
        const float4 m4 = mq[s % kPF];
        const float mv[4] = {m4.x, m4.y, m4.z, m4.w};
        if constexpr (s + kPF < S1) mq[s % kPF] = *reinterpret_cast<const float4 *>(mcol + (s + kPF) * SFS);
#pragma unroll
        for (int u = us; u < UE; ++u)
#pragma unroll
          for (int c = 0; c < 4; ++c) R[u][c] = fmaf(mv[u], x[c], R[u][c]);
      });
    };
    auto store_rows = [&](int u0) __attribute__((always_inline)) {  // SA^T[col + c][16u + p], u = u0, u0 + 1
#pragma unroll
      for (int u = u0; u < u0 + 2; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint16_t hi = bf16_bits(R[u][c]);
          shi[c * RS + 16 * u] = hi;
          slo[c * RS + 16 * u] = bf16_bits(R[u][c] - __uint_as_float((uint32_t)hi << 16));
        }
    };
    steps(std::integral_constant<int, 0>{}, std::integral_constant<int, 32>{});
    store_rows(0);
    asm volatile("" ::: "memory");  // the product below reads those rows
    {
      // rows 32..63 += M[32.., 0..31] SA[0..31] for the 32 columns 32 (sw / 2) .. +31 (the
      // other wave's 16 of them are not final yet and are dropped); through this wave's own
      // columns of the RHS rows 32..63 back to the solve layout
      const int cb = 32 * (sw >> 1);
      f32x16 acc = {};
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) {
        const int k = 16 * kq + 8 * hh;
        const bf16x8 ah = ld8(&sm.mlo[0][l32][k]), al = ld8(&sm.mlo[1][l32][k]);
        const bf16x8 bh = ld8(&sm.sat[0][cb + l32][k]), bl = ld8(&sm.sat[1][cb + l32][k]);
        acc = mfma32(ah, bh, acc);
        acc = mfma32(al, bh, acc);
        acc = mfma32(ah, bl, acc);
      }
      if ((l32 >> 4) == (sw & 1)) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sm.rhs[32 + 8 * (e >> 2) + 4 * hh + (e & 3)][cb + l32] = acc[e];
      }
      asm volatile("" ::: "memory");  // one wave's LDS accesses complete in order
#pragma unroll
      for (int u = 2; u < 4; ++u) {
        const float4 r4 = *reinterpret_cast<const float4 *>(rrow + 16 * u * SFS);
        R[u][0] += r4.x; R[u][1] += r4.y; R[u][2] += r4.z; R[u][3] += r4.w;
      }
    }
    steps(std::integral_constant<int, 32>{}, std::integral_constant<int, L - 1>{});
    store_rows(2);
  };

  auto state_c = [&]() __attribute__((always_inline)) {
    {
      state_update(BT, sm.sat[0], sm.sat[1]);  // H += Bt^T SA
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 pl4 = *reinterpret_cast<const float4 *>(&sm.pl[32 * tile_r + 8 * q + 4 * hh]);
        H[4 * q] *= pl4.x;
        H[4 * q + 1] *= pl4.y;
        H[4 * q + 2] *= pl4.z;
        H[4 * q + 3] *= pl4.w;
      }
      publish_state();
    }
  };

  // ---------------- a chunk outside the exponent range: the recurrence token by token
  auto direct_chunk_a = [&]() __attribute__((always_inline)) {  // state waves: tile layout -> fp32 [key][SFS]
    if (state_wave) {
      float *sf = &sm.rhs[0][0];
#pragma unroll
      for (int e = 0; e < 16; ++e) sf[(32 * tile_r + 8 * (e >> 2) + 4 * hh + (e & 3)) * SFS + jcol] = H[e];
    }
  };
  auto direct_chunk_b = [&](int c) __attribute__((always_inline)) {
    float *sf = &sm.rhs[0][0];
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int q = ln & 7, col = 8 * wave + (ln >> 3);
    const int nvalid = min(L, T - c * L);
    float s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = sf[(8 * q + e) * SFS + col];
    char *yb = reinterpret_cast<char *>(p.y) + (base + (long)c * L * ts + col) * ESZ;
    auto row8 = [](const uint4 x, float *f) {
      f[0] = bf16_lo(x.x); f[1] = bf16_hi(x.x); f[2] = bf16_lo(x.y); f[3] = bf16_hi(x.y);
      f[4] = bf16_lo(x.z); f[5] = bf16_hi(x.z); f[6] = bf16_lo(x.w); f[7] = bf16_hi(x.w);
    };
    for (int t0 = 0; t0 < L; t0 += 8) {
      float vv[8];
      row8(*reinterpret_cast<const uint4 *>(&sm.vt[col][t0]), vv);
      float ykeep = 0.f;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const int t = t0 + tt;
        float a[8], r[8], bb[8], k[8], d[8];
        row8(*reinterpret_cast<const uint4 *>(&sm.op[AB][t][8 * q]), a);
        row8(*reinterpret_cast<const uint4 *>(&sm.op[RB][t][8 * q]), r);
        row8(*reinterpret_cast<const uint4 *>(&sm.op[BT][t][8 * q]), bb);
        row8(*reinterpret_cast<const uint4 *>(&sm.op[KT][t][8 * q]), k);
        {
          const uint4 dh = *reinterpret_cast<const uint4 *>(&sm.op[AB + 1][t][8 * q]);
          const uint4 dl = *reinterpret_cast<const uint4 *>(&sm.op[RB + 1][t][8 * q]);
          const uint32_t hw[4] = {dh.x, dh.y, dh.z, dh.w}, lw[4] = {dl.x, dl.y, dl.z, dl.w};
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            d[2 * m] = __uint_as_float(__builtin_amdgcn_perm(hw[m], lw[m], 0x05040100u));
            d[2 * m + 1] = __uint_as_float(__builtin_amdgcn_perm(hw[m], lw[m], 0x07060302u));
          }
        }
        float s0 = a[0] * s[0], s1 = a[1] * s[1];
#pragma unroll
        for (int e = 2; e < 8; e += 2) {
          s0 = fmaf(a[e], s[e], s0);
          s1 = fmaf(a[e + 1], s[e + 1], s1);
        }
        float sa = s0 + s1;
        sa += xor1(sa);
        sa += xor2(sa);
        sa += mirror8(sa);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = fmaf(bb[e], sa, fmaf(k[e], vv[tt], d[e] * s[e]));
        float y0 = r[0] * s[0], y1 = r[1] * s[1];
#pragma unroll
        for (int e = 2; e < 8; e += 2) {
          y0 = fmaf(r[e], s[e], y0);
          y1 = fmaf(r[e + 1], s[e + 1], y1);
        }
        float yv = y0 + y1;
        yv += xor1(yv);
        yv += xor2(yv);
        yv += mirror8(yv);
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
  };
  auto direct_chunk_c = [&]() __attribute__((always_inline)) {  // state waves: back to the tile layout, publish
    if (state_wave) {
      const float *sf = &sm.rhs[0][0];
#pragma unroll
      for (int e = 0; e < 16; ++e) H[e] = sf[(32 * tile_r + 8 * (e >> 2) + 4 * hh + (e & 3)) * SFS + jcol];
      publish_state();
    }
  };

  // ---------------- chunk loop.  Each role runs its own copy of the loop (the same
  // barriers in the same order), so each keeps only its own registers live.
  // ROLE 0 / 1: output waves of token block 0 / 1; 2: RHS waves; 3: state waves.
  auto run_chunks = [&](auto role_c) __attribute__((always_inline)) {
    constexpr int ROLE = decltype(role_c)::value;
    prefetch(0, 0, 6);
    stage1(0);
    for (int c = 0; c < nchunks; ++c) {
      __syncthreads();  // wave totals posted; the previous chunk's readers are done
      stage2(c);
      // The next chunk's 24 words per thread.  Issuing loads blocks a wave for as long as the
      // requests queue (about 1,300 cycles per chunk with every wave issuing all of them here),
      // so each role issues them where it has time: the output and RHS waves after the third
      // barrier, where the state waves solve and they wait; the state waves, busy in every
      // phase, half here and half at the end of their next phase.
      const bool more = c + 1 < nchunks;
      if constexpr (ROLE == 3) {
        if (more) prefetch(c + 1, 0, 3);
      }
      __syncthreads();  // operands of chunk c in place
      const bool direct = __builtin_amdgcn_readfirstlane(sm.direct) != 0;
      if (!direct) {
        if constexpr (ROLE < 3) rhs_a();
        else state_a();
        if constexpr (ROLE == 3) {
          if (more) prefetch(c + 1, 3, 6);
        }
        __syncthreads();
        if constexpr (ROLE < 3) {
          if (more) prefetch(c + 1, 0, 6);
        }
        if constexpr (ROLE < 2) {
          out_a(std::integral_constant<int, ROLE>{});
          out_b(std::integral_constant<int, ROLE>{});
        } else if constexpr (ROLE == 3) {
          solve();
        }
        __syncthreads();
        if constexpr (ROLE < 2) out_c(std::integral_constant<int, ROLE>{}, c);
        else if constexpr (ROLE == 3) state_c();
      } else {
        if constexpr (ROLE < 3) {
          if (more) prefetch(c + 1, 0, 6);
        } else {
          if (more) prefetch(c + 1, 3, 6);
        }
        if constexpr (ROLE == 3) direct_chunk_a();
        __syncthreads();
        direct_chunk_b(c);
        __syncthreads();
        if constexpr (ROLE == 3) direct_chunk_c();
      }
      if (more) stage1(c + 1);
    }
    if constexpr (ROLE == 3) {
      if (p.state_out) {
        float *sp = p.state_out + ((long)b * p.H + h) * (kHead * kHead);
#pragma unroll
        for (int e = 0; e < 16; ++e) sp[(32 * tile_r + 8 * (e >> 2) + 4 * hh + (e & 3)) * kHead + jcol] = H[e];
      }
    }
  };
  if (wave == 0) run_chunks(std::integral_constant<int, 0>{});
  else if (wave == 1) run_chunks(std::integral_constant<int, 1>{});
  else if (wave < 4) run_chunks(std::integral_constant<int, 2>{});
  else run_chunks(std::integral_constant<int, 3>{});
}

template <bool OUTB>
hipError_t launch(const V7Params &p, hipStream_t s) {
  static std::atomic<unsigned long long> configured{0};
  const size_t lds = sizeof(Smem7);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = 1ull << (dev & 63);
  if (!(configured.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&wkv7_chunked_kernel<OUTB>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    configured.fetch_or(bit, std::memory_order_acq_rel);
  }
  hipLaunchKernelGGL((wkv7_chunked_kernel<OUTB>), dim3(p.H * p.B), dim3(kThreads), lds, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_wkv7_chunked(const V7Params &p, bool bf16, hipStream_t s) {
  if (!bf16) return hipErrorInvalidValue;  // the ABI layer routes fp32 inputs to the scan
  return p.y_bf16 ? launch<true>(p, s) : launch<false>(p, s);
}

}  // namespace wkv
