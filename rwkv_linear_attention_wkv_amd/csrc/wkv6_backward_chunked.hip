// Backward of the WKV v6 recurrence in 64-token chunks, with the contractions on MFMA (gfx950).
//
// Forward (the rwkv_ops page's RWKV6_OP call; the standard RWKV-6 recurrence), per (batch
// row, head), S indexed [key i][value j], d_t = exp(lam_t), lam_t = -exp(x_t):
//   y_t[j] = sum_i r_t[i] (S_{t-1}[i][j] + u[i] k_t[i] v_t[j]),  S_t = diag(d_t) S_{t-1} + k_t v_t^T.
// Inside a chunk of L = 64 tokens that starts from S_c, with Lam_t the inclusive in-chunk sum of
// lam and, as rows, rb_t = r_t exp(Lam_{t-1}), kt_s = k_s exp(-Lam_s), A = tril_{-1}(rb kt^T),
// b_t = r_t . (u * k_t):
//   Y = A V + diag(b) V + rb S_c,   S_{c+1} = diag(exp(Lam_{L-1})) (S_c + kt^T V).
// With G = dL/dS_{c+1} carried backwards over the chunks and Gh = diag(exp(Lam_{L-1})) G:
//   dV  = A^T dY + diag(b) dY + kt Gh          dA = tril_{-1}(dY V^T)
//   drb = dY S_c^T + dA kt                     dkt = dA^T rb + V Gh^T
//   G_c = rb^T dY + Gh                          (the gradient at the chunk start)
//   dr_t = exp(Lam_{t-1}) drb_t + u k_t db_t,   dk_s = exp(-Lam_s) dkt_s + u r_s db_s,
//   du = sum_t r_t k_t db_t,   db_t = dy_t . v_t,
//   dlam_m = sum_{t >= m} (rb_{t+1} drb_{t+1} [t+1 < L] - kt_t dkt_t) + E_{c+1},
//   E_{c+1}[i] = sum_j S_{c+1}[i][j] G[i][j],   dx = -exp(x) dlam,
// which equals the reverse-mode derivative of the token recurrence in exact arithmetic (every
// pair (s, t) whose decay path crosses token m counted once; the chunk's last term is the
// derivative through exp(Lam_{L-1}), and E is exact at every chunk boundary, so the decay
// gradient's running difference spans at most one chunk).
//
// Two launches.  Pass 1 walks each (row, head) forward and leaves the chunk start states
// S_1 .. S_{n-1} in that head's dr rows of the chunk before (64 token rows x 64 channels,
// exactly one state), which pass 2 reads before it writes those rows; no workspace.  Pass 2
// walks the chunks in reverse with one 512-thread workgroup per (row, head).  When the caller
// hands over the states the chunked forward saved (wkv6_forward_train), pass 1 is skipped and
// pass 2 reads them there.
//
// Range.  kt carries exp(-Lam_s) >= 1.  Pass 1 checks every chunk's log2-decay total (the
// same arithmetic as pass 2); a (row, head) with a chunk below -kMaxLog2 in some channel (or
// an out-of-range state_map entry) is marked, by a NaN with a payload no arithmetic or bf16
// input produces, in its dw element of the last token and channel 0, and left to the
// token-sequential sweeps, which are launched next and skip every unit that is not marked.
// Without pass 1, pass 2 makes the same checks as it reaches each chunk and, at the first that
// fails, stores the mark (after the real dw value it may have stored there) and stops; the
// sweeps then redo the whole unit.
//
// Precision.  Operands that are not exact bf16 inputs are split into bf16 hi + lo and each
// product is hi*hi + hi*lo + lo*hi (two products against the exact v), fp32 accumulation;
// E_c is formed in fp32 from the state as stored.
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma_ops.hpp"
#include "wkv.h"

namespace wkv {
namespace {

constexpr int L = 64;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// Cache policy of the gradient stores: non-temporal (streamed past the caches; 3-4% faster than
// default stores on B=8 T=4096 H=32, which compete with the next chunk's loads).
constexpr int kStoreNT = 2;
constexpr int kThreads = 512;
constexpr int RS = 72;   // bf16 row stride of the operand planes
constexpr int PFS = 68;  // fp32 row stride
constexpr float kMaxLog2 = 100.f;
constexpr float kLog2e = 1.4426950408889634f;

// Planes [token or key][key or value], bf16: rb, kt (hi / lo), v, dy (hi / lo), S_c (hi / lo),
// Gh (hi / lo), the raw x words, and (RK, two planes' room) the raw r and k of a (token,
// channel) packed in one 32-bit word (k in the upper half).
enum Plane { RBH, RBL, KTH, KTL, VV, DYH, DYL, SCH, SCL, GHH, GHL, XR, RK, RK_END = RK + 1, NPL };

struct alignas(16) Smem2 {
  uint16_t pl[NPL][L][RS];
  float P[L][PFS];       // inclusive log2-decay prefix [token][key]
  float bon[L], dbon[L]; // r . (u * k) and dy . v per token
  float E[2][kHead];     // sum_j S G at the chunk starts, by chunk parity
  float dl[kHead];       // 2^P_{L-1} per key row
  float2 wtot[8][32];    // log2-decay total of each wave's tokens, per channel pair
  float dlt[8][kHead];   // dlam: each wave's token-group total
};
// In phases 4 and 5 the dlam terms of a chunk reuse the S_c and Gh planes, and the staged dr,
// dk, dv the rb, kt and dy planes (free by then), each as one fp32 plane of stride PFS
static_assert(sizeof(float) * L * PFS <= 2 * sizeof(uint16_t) * L * RS, "fp32 plane fits two bf16 planes");

struct alignas(16) Smem1 {
  uint16_t pl[3][L][RS];  // kt hi / lo, v
  float dl[kHead];
  float2 wtot[8][32];
};

__device__ __forceinline__ float *fplane(Smem2 &sm, int first) { return reinterpret_cast<float *>(&sm.pl[first][0][0]); }
// The packed raw r / k words, [token][channel] with a row stride of RS 32-bit words.
__device__ __forceinline__ uint32_t *rkplane(Smem2 &sm) { return reinterpret_cast<uint32_t *>(&sm.pl[RK][0][0]); }

// ---------------- MFMA helpers (v_mfma_f32_32x32x16_bf16; lane l: row / column l % 32, K
// slots 8 (l / 32) .. +7 of each 16-wide K step; accumulator element e of lane l holds row
// 8 (e / 4) + 4 (l / 32) + e % 4, column l % 32).
// Transposed operand read: lane l gets M[r0 + 8 (l / 32) + 0..7][c0 + l % 32] of a row-major M.
__device__ __forceinline__ bf16x8 ldT(const uint16_t (*M)[RS], int r0, int c0, int lane) {
  const int r = r0 + 8 * (lane >> 5) + ((lane >> 2) & 3);
  const int c = c0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const uint2 a = ld_tr(&M[r][c]), b = ld_tr(&M[r + 4][c]);
  return as_bf16x8(a.x, a.y, b.x, b.y);
}
// The same in the K order of an accumulator used as the other operand: lane l gets rows
// r0 + 4 (l / 32) + 0..3 and r0 + 8 + 4 (l / 32) + 0..3.
__device__ __forceinline__ bf16x8 ldTp(const uint16_t (*M)[RS], int r0, int c0, int lane) {
  const int r = r0 + 4 * (lane >> 5) + ((lane >> 2) & 3);
  const int c = c0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const uint2 a = ld_tr(&M[r][c]), b = ld_tr(&M[r + 8][c]);
  return as_bf16x8(a.x, a.y, b.x, b.y);
}
__device__ __forceinline__ bf16x8 ldN(const uint16_t (*M)[RS], int r0, int k0, int lane) {
  return ld8(&M[r0 + (lane & 31)][k0 + 8 * (lane >> 5)]);
}

// The products below issue one K step at a time: the next step's operands are read while this
// step's products issue, and a scheduling barrier keeps the compiler from hoisting further reads
// (each would hold registers across the whole pass).
// acc[m][n] += sum_k X[m0 + m][k] Y[n0 + n][k] over the 64 k (both row-major, [*][k]).
// xl / yl == nullptr: that operand is exact (two products).
__device__ __forceinline__ void mm_nn(f32x16 &acc, const uint16_t (*xh)[RS], const uint16_t (*xl)[RS],
                                      const uint16_t (*yh)[RS], const uint16_t (*yl)[RS], int m0, int n0,
                                      int lane) {
  bf16x8 a = ldN(xh, m0, 0, lane), b = ldN(yh, n0, 0, lane), a2 = a, b2 = b;
  if (xl) a2 = ldN(xl, m0, 0, lane);
  if (yl) b2 = ldN(yl, n0, 0, lane);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bf16x8 ca = a, cb = b, ca2 = a2, cb2 = b2;
    if (q < 3) {
      a = ldN(xh, m0, 16 * (q + 1), lane);
      b = ldN(yh, n0, 16 * (q + 1), lane);
      if (xl) a2 = ldN(xl, m0, 16 * (q + 1), lane);
      if (yl) b2 = ldN(yl, n0, 16 * (q + 1), lane);
    }
    acc = mfma32(ca, cb, acc);
    if (xl) acc = mfma32(ca2, cb, acc);
    if (yl) acc = mfma32(ca, cb2, acc);
    __builtin_amdgcn_sched_barrier(0);
  }
}
// acc[m][n] += sum_k X[m0 + m][k] Y[k][n0 + n] (Y row-major [k][n]), both hi / lo.
__device__ __forceinline__ void mm_nt(f32x16 &acc, const uint16_t (*xh)[RS], const uint16_t (*xl)[RS],
                                      const uint16_t (*yh)[RS], const uint16_t (*yl)[RS], int m0, int n0,
                                      int lane) {
  bf16x8 a = ldN(xh, m0, 0, lane), a2 = ldN(xl, m0, 0, lane), b = ldT(yh, 0, n0, lane), b2 = ldT(yl, 0, n0, lane);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bf16x8 ca = a, cb = b, ca2 = a2, cb2 = b2;
    if (q < 3) {
      a = ldN(xh, m0, 16 * (q + 1), lane);
      a2 = ldN(xl, m0, 16 * (q + 1), lane);
      b = ldT(yh, 16 * (q + 1), n0, lane);
      b2 = ldT(yl, 16 * (q + 1), n0, lane);
    }
    acc = mfma32(ca, cb, acc);
    acc = mfma32(ca2, cb, acc);
    acc = mfma32(ca, cb2, acc);
    __builtin_amdgcn_sched_barrier(0);
  }
}
// acc[m][n] += sum_k X[k][m0 + m] Y[k][n0 + n] (both row-major [k][*]), both hi / lo.
__device__ __forceinline__ void mm_tt(f32x16 &acc, const uint16_t (*xh)[RS], const uint16_t (*xl)[RS],
                                      const uint16_t (*yh)[RS], const uint16_t (*yl)[RS], int m0, int n0,
                                      int lane) {
  bf16x8 a = ldT(xh, 0, m0, lane), a2 = ldT(xl, 0, m0, lane), b = ldT(yh, 0, n0, lane), b2 = ldT(yl, 0, n0, lane);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bf16x8 ca = a, cb = b, ca2 = a2, cb2 = b2;
    if (q < 3) {
      a = ldT(xh, 16 * (q + 1), m0, lane);
      a2 = ldT(xl, 16 * (q + 1), m0, lane);
      b = ldT(yh, 16 * (q + 1), n0, lane);
      b2 = ldT(yl, 16 * (q + 1), n0, lane);
    }
    acc = mfma32(ca, cb, acc);
    acc = mfma32(ca2, cb, acc);
    acc = mfma32(ca, cb2, acc);
    __builtin_amdgcn_sched_barrier(0);
  }
}
// acc[m][n] += sum_k Z[k][m] Y[k0 + k][n0 + n] over the 32 rows k of the accumulator block Z
// (lane l holds its column m = l % 32), split into bf16 hi / lo on the fly; Y row-major [k][n].
__device__ __forceinline__ void mm_za(f32x16 &acc, const f32x16 &z, const uint16_t (*yh)[RS],
                                      const uint16_t (*yl)[RS], int k0, int n0, int lane) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const bf16x8 bh = ldTp(yh, k0 + 16 * ks, n0, lane), bl = ldTp(yl, k0 + 16 * ks, n0, lane);
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) split2(z[8 * ks + 2 * m], z[8 * ks + 2 * m + 1], hw[m], lw[m]);
    const bf16x8 ah = as_bf16x8(hw[0], hw[1], hw[2], hw[3]), al = as_bf16x8(lw[0], lw[1], lw[2], lw[3]);
    acc = mfma32(ah, bh, acc);
    acc = mfma32(al, bh, acc);
    acc = mfma32(ah, bl, acc);
    __builtin_amdgcn_sched_barrier(0);
  }
}
// Keep z[e] where the block's row (8 (e / 4) + 4 (l / 32) + e % 4) and the lane's column
// satisfy row > col (keep_row_gt) or row < col, zero elsewhere.
template <bool ROW_GT>
__device__ __forceinline__ void mask_diag(f32x16 &z, int lane) {
  // Element e holds row - 4h = 8 (e / 4) + e % 4 (an immediate) against dd = col - 4h.  dd comes
  // from an opaque copy of the lane index, so the 16 conditions are formed here, in every chunk,
  // instead of being held across the chunk loop in scalar register pairs.
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const int dd = (ln & 31) - 4 * (ln >> 5);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int ce = 8 * (e >> 2) + (e & 3);
    const bool keep = ROW_GT ? ce > dd : ce < dd;
    z[e] = keep ? z[e] : 0.f;
  }
}

// ---------------- token staging shared by both passes.  Thread (cp = tid % 32, tg = tid / 32)
// holds channels 2cp, 2cp+1 of tokens 4tg .. 4tg+3 (wave w: tokens 8w .. 8w+7).
struct Stage {
  float lam0[4], lam1[4];   // log2 decays of the thread's tokens
  float lower0, lower1;     // the lower half-wave's total (upper half adds it)
};

// log2 decays from the x words (tokens past nvalid do not decay), in-thread totals, and the
// wave totals posted to wtot (the upper half-wave adds the lower one's).
__device__ __forceinline__ void stage_decay(Stage &st, const uint32_t (&xw)[4], int tg, int nvalid, int lane,
                                            float2 (*wtot)[32], int wave, int cp) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const bool past = 4 * tg + t >= nvalid;
    st.lam0[t] = past ? 0.f : -(fast_exp(bf16_lo(xw[t])) * kLog2e);
    st.lam1[t] = past ? 0.f : -(fast_exp(bf16_hi(xw[t])) * kLog2e);
  }
  const float run0 = ((st.lam0[0] + st.lam0[1]) + st.lam0[2]) + st.lam0[3];
  const float run1 = ((st.lam1[0] + st.lam1[1]) + st.lam1[2]) + st.lam1[3];
  const int x32 = (lane ^ 32) << 2;
  st.lower0 = __int_as_float(__builtin_amdgcn_ds_bpermute(x32, __float_as_int(run0)));
  st.lower1 = __int_as_float(__builtin_amdgcn_ds_bpermute(x32, __float_as_int(run1)));
  if (lane & 32) wtot[wave][cp] = make_float2(run0 + st.lower0, run1 + st.lower1);
}
// After the barrier: the prefix of the earlier waves and the chunk totals; true when the chunk
// leaves the exponent range in some channel (every wave sees every channel: a uniform answer).
__device__ __forceinline__ bool stage_prefix(const Stage &st, const float2 (*wtot)[32], int wave, int cp, int lane,
                                             float &pre0, float &pre1, float &tot0, float &tot1) {
  pre0 = (lane & 32) ? st.lower0 : 0.f;
  pre1 = (lane & 32) ? st.lower1 : 0.f;
  tot0 = 0.f;
  tot1 = 0.f;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const float2 t = wtot[w][cp];
    const float m = w < wave ? 1.f : 0.f;
    pre0 = fmaf(m, t.x, pre0);
    pre1 = fmaf(m, t.y, pre1);
    tot0 += t.x;
    tot1 += t.y;
  }
  return __builtin_amdgcn_ballot_w64(!(tot0 >= -kMaxLog2 && tot1 >= -kMaxLog2)) != 0;
}

// Buffer resource over one head's token row segment [base, row_end) bytes of an array; reads
// past the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_at(const void *p, unsigned long long off,
                                                          unsigned long long row_end) {
  const unsigned long long rem = off < row_end ? row_end - off : 0ull;
  const int n = (int)(rem > 0x7fffffffull ? 0x7fffffffull : rem);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(static_cast<const char *>(p) + off), 0, n, 0x00020000);
}

__device__ __forceinline__ float *mark_of(const BwdParams &p, int b, int h) {
  const long C = (long)p.H * kHead;
  return p.dw + ((long)b * p.T + (p.T - 1)) * C + (long)h * kHead;
}

// ================================ pass 1: chunk start states
__global__ void __launch_bounds__(kThreads) wkv6_bwdc_state_kernel(BwdParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem1 &sm = *reinterpret_cast<Smem1 *>(smem_raw);
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cp = tid & 31, tg = tid >> 5, hh = lane >> 5, l32 = lane & 31;
  const int T = p.T, nch = (T + L - 1) / L;
  const long C = (long)p.H * kHead;
  float *mark = mark_of(p, b, h);

  int row_in = -1;
  if (p.state_in) {
    row_in = p.state_map ? p.state_map[b] : (p.n_state == 1 ? 0 : b);
    if (row_in < 0 || row_in >= p.n_state) {  // the sweeps report it and skip the row
      if (tid == 0) *reinterpret_cast<uint32_t *>(mark) = kBwdFallbackMark;
      return;
    }
  }
  // state waves 0 .. 3: 32 x 32 tile (key block wave / 2, value block wave % 2)
  const bool state_wave = wave < 4;
  const int tile_r = (wave >> 1) & 1, tile_c = wave & 1;
  const int jcol = 32 * tile_c + l32;
  f32x16 S = {};
  if (state_wave && row_in >= 0) {
    const float *s0 = p.state_in + ((long)row_in * p.H + h) * (kHead * kHead);
#pragma unroll
    for (int e = 0; e < 16; ++e) S[e] = s0[(32 * tile_r + 8 * (e >> 2) + 4 * hh + (e & 3)) * kHead + jcol];
  }

  const long base = ((long)b * T) * C + (long)h * kHead;  // elements: token 0, channel 0 of the head
  const unsigned long long row_end = (unsigned long long)(base + (long)(T - 1) * C + kHead) * 2;
  uint32_t roff[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) roff[t] = (uint32_t)(((4 * tg + t) * C + 2 * cp) * 2);
  uint32_t xw[4], kw[4], vw[4];
  auto prefetch = [&](int c) {
    const unsigned long long off = (unsigned long long)uniform64((base + (long)c * L * C) * 2);
    const auto rx = rsrc_at(p.w, off, row_end), rk = rsrc_at(p.k, off, row_end), rv = rsrc_at(p.v, off, row_end);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      xw[t] = __builtin_amdgcn_raw_buffer_load_b32(rx, (int)roff[t], 0, 0);
      kw[t] = __builtin_amdgcn_raw_buffer_load_b32(rk, (int)roff[t], 0, 0);
      vw[t] = __builtin_amdgcn_raw_buffer_load_b32(rv, (int)roff[t], 0, 0);
    }
  };
  prefetch(0);
  Stage st;
  for (int c = 0; c < nch; ++c) {
    const int nvalid = min(L, T - c * L);
    stage_decay(st, xw, tg, nvalid, lane, sm.wtot, wave, cp);
    __syncthreads();  // wave totals posted; the previous chunk's products are done
    float pre0, pre1, tot0, tot1;
    if (stage_prefix(st, sm.wtot, wave, cp, lane, pre0, pre1, tot0, tot1)) {
      if (tid == 0) *reinterpret_cast<uint32_t *>(mark) = kBwdFallbackMark;
      return;  // every wave takes this branch at the same chunk
    }
    if (c + 1 == nch) break;  // the last chunk's end state is not needed
    if (wave == 0 && !hh)
      *reinterpret_cast<float2 *>(&sm.dl[2 * cp]) = make_float2(__builtin_amdgcn_exp2f(tot0), __builtin_amdgcn_exp2f(tot1));
    float c0 = pre0, c1 = pre1;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int tau = 4 * tg + t;
      c0 += st.lam0[t];
      c1 += st.lam1[t];
      uint32_t hi, lo;
      split2(bf16_lo(kw[t]) * __builtin_amdgcn_exp2f(-c0), bf16_hi(kw[t]) * __builtin_amdgcn_exp2f(-c1), hi, lo);
      *reinterpret_cast<uint32_t *>(&sm.pl[0][tau][2 * cp]) = hi;
      *reinterpret_cast<uint32_t *>(&sm.pl[1][tau][2 * cp]) = lo;
      *reinterpret_cast<uint32_t *>(&sm.pl[2][tau][2 * cp]) = vw[t];
    }
    prefetch(c + 1);  // c + 1 < nch here
    __syncthreads();  // planes of chunk c in place
    if (state_wave) {
      // S += kt^T V over the chunk's tokens; then S_{c+1} = diag(2^P_{L-1}) S
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x8 a = ldT(sm.pl[0], 16 * q, 32 * tile_r, lane), al = ldT(sm.pl[1], 16 * q, 32 * tile_r, lane);
        const bf16x8 bv = ldT(sm.pl[2], 16 * q, 32 * tile_c, lane);
        S = mfma32(a, bv, S);
        S = mfma32(al, bv, S);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = 32 * tile_r + 8 * (e >> 2) + 4 * hh + (e & 3);
        S[e] *= sm.dl[row];
        // S_{c+1} into this head's dr rows of chunk c (a full chunk: c + 1 < nch)
        p.dr[(base + ((long)c * L + row) * C) + jcol] = S[e];
      }
    }
  }
  if (tid == 0) *mark = 0.f;  // not marked (pass 2 writes the real value)
}

// ================================ pass 2: the gradients, chunks in reverse
// Roles (wave): 0, 1: dV of token block s = 0 / 1 (with A blocks of that s block);
// 2, 3: dkt of s block 0 / 1 (with dA blocks); 4, 5: drb of t block 0 / 1 (with dA^T blocks);
// 6, 7: G tiles of key block 0 / 1.
__global__ void __launch_bounds__(kThreads) wkv6_bwdc_kernel(BwdParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem2 &sm = *reinterpret_cast<Smem2 *>(smem_raw);
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cp = tid & 31, tg = tid >> 5, hh = lane >> 5, l32 = lane & 31;
  const int T = p.T, nch = (T + L - 1) / L;
  const long C = (long)p.H * kHead;
  // With the forward's saved states there is no state pass: this pass itself leaves a unit to
  // the sweeps (a rejected state_map row, a chunk out of the exponent range), by storing the
  // mark from the thread that stores that dw element in the chunk loop (its store came first).
  const bool saved = p.chunk_states != nullptr;
  if (!saved && __float_as_uint(*mark_of(p, b, h)) == kBwdFallbackMark) return;  // the sweeps take this unit
  const int tlast = (T - 1) - (nch - 1) * L;  // the last token's place in its chunk
  auto leave_to_sweeps = [&]() {
    if (wave == (tlast >> 3) && lane == 0) {
      __threadfence();
      *reinterpret_cast<uint32_t *>(mark_of(p, b, h)) = kBwdFallbackMark;
    }
  };
  const int row_in = p.state_in ? (p.state_map ? p.state_map[b] : (p.n_state == 1 ? 0 : b)) : -1;
  if (saved && p.state_in && (row_in < 0 || row_in >= p.n_state)) {
    leave_to_sweeps();
    return;
  }
  const long base = ((long)b * T) * C + (long)h * kHead;
  // S_c (c >= 1): the saved states, or the dr rows of chunk c - 1 where the state pass left them
  const float *sbase = saved ? p.chunk_states + ((long)b * p.H + h) * (long)(nch - 1) * (kHead * kHead) : p.dr + base;
  const long schunk = saved ? (long)(kHead * kHead) : (long)L * C, srow = saved ? (long)kHead : C;
  const long head_off = ((long)b * p.H + h) * (kHead * kHead);
  const unsigned long long row_end2 = (unsigned long long)(base + (long)(T - 1) * C + kHead) * 2;
  const unsigned long long row_end4 = row_end2 * 2;
  uint32_t roff2[4], roff4[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    roff2[t] = (uint32_t)(((4 * tg + t) * C + 2 * cp) * 2);
    roff4[t] = roff2[t] * 2;
  }
  const float u0 = p.u[h * kHead + 2 * cp], u1 = p.u[h * kHead + 2 * cp + 1];
  const float ul = p.u[h * kHead + l32], uh2 = p.u[h * kHead + 32 + l32];  // lane's columns of the outputs

  // ---- prefetched inputs of the next chunk (in processing order)
  uint32_t xw[4], rw[4], kw[4], vw[4];
  float dy0[4], dy1[4];
  float sc[8];  // S_c: row tid / 8, columns 8 (tid % 8) .. +7
  const int sci = tid >> 3, scj = 8 * (tid & 7);
  auto prefetch = [&](int c) {
    const unsigned long long off = (unsigned long long)uniform64((base + (long)c * L * C) * 2);
    const auto rx = rsrc_at(p.w, off, row_end2), rr = rsrc_at(p.r, off, row_end2);
    const auto rk = rsrc_at(p.k, off, row_end2), rv = rsrc_at(p.v, off, row_end2);
    const auto rd = rsrc_at(p.dy, off * 2, row_end4);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      xw[t] = __builtin_amdgcn_raw_buffer_load_b32(rx, (int)roff2[t], 0, 0);
      rw[t] = __builtin_amdgcn_raw_buffer_load_b32(rr, (int)roff2[t], 0, 0);
      kw[t] = __builtin_amdgcn_raw_buffer_load_b32(rk, (int)roff2[t], 0, 0);
      vw[t] = __builtin_amdgcn_raw_buffer_load_b32(rv, (int)roff2[t], 0, 0);
      dy0[t] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rd, (int)roff4[t], 0, 0));  // dy: 4-byte aligned
      dy1[t] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rd, (int)roff4[t] + 4, 0, 0));
    }
    if (c >= 1) {
      const float *s = sbase + (long)(c - 1) * schunk + sci * srow + scj;
      const float4 a = *reinterpret_cast<const float4 *>(s), q = *reinterpret_cast<const float4 *>(s + 4);
      sc[0] = a.x; sc[1] = a.y; sc[2] = a.z; sc[3] = a.w; sc[4] = q.x; sc[5] = q.y; sc[6] = q.z; sc[7] = q.w;
    } else if (row_in >= 0) {
      const float *s = p.state_in + ((long)row_in * p.H + h) * (kHead * kHead) + sci * kHead + scj;
#pragma unroll
      for (int m = 0; m < 8; ++m) sc[m] = s[m];
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) sc[m] = 0.f;
    }
  };

  const int gi = wave & 1;  // G waves: key block of the state-gradient tiles
  // E at the sequence end: sum_j S_T dS_T (row sci, 8 columns per thread, 8 threads per row)
  {
    float e = 0.f;
    if (p.d_state_out && p.state_final) {
      const float *g = p.d_state_out + head_off + sci * kHead + scj, *s = p.state_final + head_off + sci * kHead + scj;
#pragma unroll
      for (int m = 0; m < 8; ++m) e = fmaf(g[m], s[m], e);
    }
    e += xor1(e);
    e += xor2(e);
    e += xor_swz<4>(e);
    if ((tid & 7) == 0) sm.E[nch & 1][sci] = e;
  }
  float du0 = 0.f, du1 = 0.f;

  // Each role runs its own copy of the chunk loop (the same barriers in the same order), so
  // that only its own registers stay live.  ROLE 0: dV waves, 1: dkt waves, 2: drb waves, 3: G.
  auto run_chunks = [&](auto role_c) __attribute__((always_inline)) -> bool {
  constexpr int ROLE = decltype(role_c)::value;
  // G waves: the gradient of the state at the current chunk end, tiles (key block gi, value
  // blocks 0 / 1)
  f32x16 G[2] = {f32x16{}, f32x16{}};
  if constexpr (ROLE == 3) {
    if (p.d_state_out) {
      const float *g = p.d_state_out + head_off;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          G[jb][e] = g[(32 * gi + 8 * (e >> 2) + 4 * hh + (e & 3)) * kHead + 32 * jb + l32];
    }
  }
  prefetch(nch - 1);
  // Wait for the first chunk's words here, once: otherwise this path into the loop (the
  // prefetch the newest memory operation) makes the compiler's merged waits at the top of the
  // loop wait for everything in flight, the previous chunk's stores included, in every chunk.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  Stage st;
  for (int c = nch - 1; c >= 0; --c) {
    const int nvalid = min(L, T - c * L);
    // ---------- stage A: decays, raw planes, dy hi / lo, S_c hi / lo, bonus and dy . v
    stage_decay(st, xw, tg, nvalid, lane, sm.wtot, wave, cp);
    float bn[4], db[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int tau = 4 * tg + t;
      *reinterpret_cast<uint2 *>(&rkplane(sm)[tau * RS + 2 * cp]) =
          make_uint2(__builtin_amdgcn_perm(kw[t], rw[t], 0x05040100u), __builtin_amdgcn_perm(kw[t], rw[t], 0x07060302u));
      *reinterpret_cast<uint32_t *>(&sm.pl[XR][tau][2 * cp]) = xw[t];
      *reinterpret_cast<uint32_t *>(&sm.pl[VV][tau][2 * cp]) = vw[t];
      uint32_t hi, lo;
      split2(dy0[t], dy1[t], hi, lo);
      *reinterpret_cast<uint32_t *>(&sm.pl[DYH][tau][2 * cp]) = hi;
      *reinterpret_cast<uint32_t *>(&sm.pl[DYL][tau][2 * cp]) = lo;
      const float r0 = bf16_lo(rw[t]), r1 = bf16_hi(rw[t]), k0 = bf16_lo(kw[t]), k1 = bf16_hi(kw[t]);
      bn[t] = fmaf(r1 * u1, k1, r0 * u0 * k0);
      db[t] = fmaf(dy1[t], bf16_hi(vw[t]), dy0[t] * bf16_lo(vw[t]));
    }
    {  // Sums over the 32 channel pairs of the half-wave, of all eight values at once: each of
       // three exchange steps keeps half of the lane's values and adds the other lane's matching
       // half, so lane group g = (lane / 4) % 8 ends with value g (the bonus of token g for g < 4,
       // dy . v of token g - 4 above), and two DPP steps finish the sums.
      // (lane bits from an opaque copy: formed here, not held across the loop as masks)
      int ln = lane;
      asm volatile("" : "+v"(ln));
      float w4[4], w2[2];
      const bool b4 = ln & 16, b3 = ln & 8, b2 = ln & 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) w4[j] = (b4 ? db[j] : bn[j]) + xor_swz<16>(b4 ? bn[j] : db[j]);
#pragma unroll
      for (int j = 0; j < 2; ++j) w2[j] = (b3 ? w4[2 + j] : w4[j]) + xor_swz<8>(b3 ? w4[j] : w4[2 + j]);
      float w1 = (b2 ? w2[1] : w2[0]) + xor_swz<4>(b2 ? w2[0] : w2[1]);
      w1 += xor2(w1);
      w1 += xor1(w1);
      if ((ln & 3) == 0) {
        const int g = (ln >> 2) & 7;
        (g < 4 ? sm.bon : sm.dbon)[4 * tg + (g & 3)] = w1;
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      uint32_t hi, lo;
      split2(sc[2 * m], sc[2 * m + 1], hi, lo);
      *reinterpret_cast<uint32_t *>(&sm.pl[SCH][sci][scj + 2 * m]) = hi;
      *reinterpret_cast<uint32_t *>(&sm.pl[SCL][sci][scj + 2 * m]) = lo;
    }
    __syncthreads();  // B1
    // ---------- stage B: prefix, rb and kt hi / lo, P, the chunk decay
    {
      float pre0, pre1, tot0, tot1;
      // in range when the state pass ran (it checked every chunk); else checked here
      if (stage_prefix(st, sm.wtot, wave, cp, lane, pre0, pre1, tot0, tot1) && saved) {
        leave_to_sweeps();
        return true;
      }
      if (wave == 0 && !hh)
        *reinterpret_cast<float2 *>(&sm.dl[2 * cp]) = make_float2(__builtin_amdgcn_exp2f(tot0), __builtin_amdgcn_exp2f(tot1));
      {  // du += r k (dy . v) over the thread's tokens, the dy . v sums as stage A left them
        const float4 d4 = *reinterpret_cast<const float4 *>(&sm.dbon[4 * tg]);
        const float dbt[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          du0 = fmaf(bf16_lo(rw[t]) * bf16_lo(kw[t]), dbt[t], du0);
          du1 = fmaf(bf16_hi(rw[t]) * bf16_hi(kw[t]), dbt[t], du1);
        }
      }
      float c0 = pre0, c1 = pre1;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int tau = 4 * tg + t;
        const float e0 = __builtin_amdgcn_exp2f(c0), e1 = __builtin_amdgcn_exp2f(c1);  // 2^P_{t-1}
        c0 += st.lam0[t];
        c1 += st.lam1[t];
        *reinterpret_cast<float2 *>(&sm.P[tau][2 * cp]) = make_float2(c0, c1);
        uint32_t hi, lo;
        split2(bf16_lo(rw[t]) * e0, bf16_hi(rw[t]) * e1, hi, lo);
        *reinterpret_cast<uint32_t *>(&sm.pl[RBH][tau][2 * cp]) = hi;
        *reinterpret_cast<uint32_t *>(&sm.pl[RBL][tau][2 * cp]) = lo;
        split2(bf16_lo(kw[t]) * __builtin_amdgcn_exp2f(-c0), bf16_hi(kw[t]) * __builtin_amdgcn_exp2f(-c1), hi, lo);
        *reinterpret_cast<uint32_t *>(&sm.pl[KTH][tau][2 * cp]) = hi;
        *reinterpret_cast<uint32_t *>(&sm.pl[KTL][tau][2 * cp]) = lo;
      }
    }
    __syncthreads();  // B2
    // ---------- phase 3a: products that do not need Gh; the G waves form Gh
    f32x16 acc[2] = {f32x16{}, f32x16{}};  // the wave's output blocks (value or key blocks 0 / 1)
    float sv[2][16];  // G waves: S_c at their G tile elements, in fp32, for E_c
    if constexpr (ROLE == 0) {
      const int sb = wave;
      // A[t][s] = rb_t . kt_s (s < t), blocks tb >= sb; dV += A^T dY
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        if (tb < sb) continue;
        f32x16 Z = {};
        mm_nn(Z, sm.pl[RBH], sm.pl[RBL], sm.pl[KTH], sm.pl[KTL], 32 * tb, 32 * sb, lane);
        if (tb == sb) {  // keep s < t; the bonus r_t . (u * k_t) on s == t gives dV its b_s dy_s
          // (the conditions as in mask_diag; on the diagonal row == col, one bonus read per lane)
          int ln = lane;
          asm volatile("" : "+v"(ln));
          const int col = ln & 31, dd = col - 4 * (ln >> 5);
          const float bonc = sm.bon[32 * tb + col];
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int ce = 8 * (e >> 2) + (e & 3);
            Z[e] = ce > dd ? Z[e] : (ce == dd ? bonc : 0.f);
          }
        }
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) mm_za(acc[jb], Z, sm.pl[DYH], sm.pl[DYL], 32 * tb, 32 * jb, lane);
      }
    } else if constexpr (ROLE == 1) {
      const int sb = wave - 2;
      // dA[t][s] = dy_t . v_s (s < t), blocks tb >= sb; dkt += dA^T rb
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        if (tb < sb) continue;
        f32x16 Z = {};
        mm_nn(Z, sm.pl[DYH], sm.pl[DYL], sm.pl[VV], nullptr, 32 * tb, 32 * sb, lane);
        if (tb == sb) mask_diag<true>(Z, lane);
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) mm_za(acc[ib], Z, sm.pl[RBH], sm.pl[RBL], 32 * tb, 32 * ib, lane);
      }
    } else if constexpr (ROLE == 2) {
      const int tb = wave - 4;
      // dA^T[s][t] blocks sb <= tb; drb += dA kt; drb += dY S_c^T
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        if (sb > tb) continue;
        f32x16 Z = {};
        mm_nn(Z, sm.pl[VV], nullptr, sm.pl[DYH], sm.pl[DYL], 32 * sb, 32 * tb, lane);
        if (sb == tb) mask_diag<false>(Z, lane);
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) mm_za(acc[ib], Z, sm.pl[KTH], sm.pl[KTL], 32 * sb, 32 * ib, lane);
      }
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) mm_nn(acc[ib], sm.pl[DYH], sm.pl[DYL], sm.pl[SCH], sm.pl[SCL], 32 * tb, 32 * ib, lane);
    } else {
      // Gh = diag(2^P_{L-1}) G, kept in registers and published as bf16 hi / lo
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int l32 = ln & 31, hh = ln >> 5;
      // S_c at the G tile's elements for E_c in phase 3b, loaded in fp32 from where the
      // prefetch took it (the saved states, the dr rows of the chunk before, or state_in) while
      // this role has little else to do: two-byte reads of its hi / lo planes in 3b cost more
      {
        const float *sp = p.dr;  // no state (c == 0 without state_in): a resource with no records
        long sr = 0;
        int nrec = 0;
        if (c >= 1) {
          sp = sbase + (long)(c - 1) * schunk;
          sr = srow;
          nrec = 0x7fffffff;
        } else if (row_in >= 0) {
          sp = p.state_in + ((long)row_in * p.H + h) * (kHead * kHead);
          sr = kHead;
          nrec = 0x7fffffff;
        }
        // One buffer resource at the state (reads past no records return zero), the lane's row
        // and column as the vector offset, each element's row step as a scalar offset: no
        // per-element 64-bit address arithmetic.  Offsets stay below 64 rows of the state.
        const auto rs = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<char *>(uniform64(reinterpret_cast<long>(sp))), 0,
                                                          nrec, 0x00020000);
        const int vo = (int)(((32 * gi + 4 * hh) * sr + l32) * 4);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int so = __builtin_amdgcn_readfirstlane((int)((8 * (e >> 2) + (e & 3)) * sr * 4));
            sv[jb][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, vo + 128 * jb, so, 0));
          }
      }
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row0 = 32 * gi + 8 * q + 4 * hh;
          const float4 d = *reinterpret_cast<const float4 *>(&sm.dl[row0]);
          G[jb][4 * q] *= d.x; G[jb][4 * q + 1] *= d.y; G[jb][4 * q + 2] *= d.z; G[jb][4 * q + 3] *= d.w;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const uint16_t hb = bf16_bits(G[jb][4 * q + m]);
            sm.pl[GHH][row0 + m][32 * jb + l32] = hb;
            sm.pl[GHL][row0 + m][32 * jb + l32] = bf16_bits(G[jb][4 * q + m] - bf16_lo(hb));
          }
        }
    }
    __syncthreads();  // B3
    // The next chunk's rows.  Issuing a wave's 28 loads blocks it for a few thousand cycles while
    // the requests queue (all eight waves issuing them at the end of stage B took about 3,500
    // cycles of every chunk), so each role issues them where it would otherwise wait: the dkt
    // and drb waves here (the drb waves have no work in 3b), the dV and G waves after B4.  They
    // arrive during phases 4 and 5, and the registers they land in are free in 3a.
    if constexpr (ROLE == 1 || ROLE == 2) {
      if (c > 0) prefetch(c - 1);
    }
    // ---------- phase 3b: the products with Gh; G_c and E_c
    if constexpr (ROLE == 0) {
      const int sb = wave;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) mm_nt(acc[jb], sm.pl[KTH], sm.pl[KTL], sm.pl[GHH], sm.pl[GHL], 32 * sb, 32 * jb, lane);
    } else if constexpr (ROLE == 1) {
      const int sb = wave - 2;
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) mm_nn(acc[ib], sm.pl[VV], nullptr, sm.pl[GHH], sm.pl[GHL], 32 * sb, 32 * ib, lane);
    } else if constexpr (ROLE == 3) {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int l32 = ln & 31, hh = ln >> 5;
      float ep[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) ep[e] = 0.f;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        mm_tt(G[jb], sm.pl[RBH], sm.pl[RBL], sm.pl[DYH], sm.pl[DYL], 32 * gi, 32 * jb, lane);  // G_c = rb^T dY + Gh
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = 32 * gi + 8 * (e >> 2) + 4 * hh + (e & 3), col = 32 * jb + l32;
          const float s = sv[jb][e];
          ep[e] = fmaf(s, G[jb][e], ep[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {  // sum over the 32 columns of the half-wave
        float x = ep[e];
        x += xor1(x);
        x += xor2(x);
        x += xor_swz<4>(x);
        x += xor_swz<8>(x);
        x += xor_swz<16>(x);
        ep[e] = x;
      }
      if (l32 == 0) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sm.E[c & 1][32 * gi + 8 * (e >> 2) + 4 * hh + (e & 3)] = ep[e];
      }
    }
    __syncthreads();  // B4
    if constexpr (ROLE == 0 || ROLE == 3) {
      if (c > 0) prefetch(c - 1);
    }
    // ---------- phase 4: outputs and the dlam terms (T1 = rb drb in the Gh planes, T2 = kt dkt in
    // the S_c planes, both fp32 [token][key])
    float *T1 = fplane(sm, GHH), *T2 = fplane(sm, SCH);
    const long tok0 = base + (long)c * L * C;
    // Stores go through a buffer resource at the chunk's first row (scalar registers) and lane
    // and scalar offsets, so no per-element 64-bit address is kept.
    const uint32_t C4 = (uint32_t)(C * 4);
    if constexpr (ROLE < 3) {
      // Per-element LDS offsets from an opaque copy of the lane index: they are the same in
      // every chunk, and hoisted out of the chunk loop they would hold a register each.
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int l32 = ln & 31, hh = ln >> 5;
      const int blk = wave & 1;  // the wave's token block
      // dv, dk, dr go to the planes of dy, kt, rb (free until the next chunk's staging) and
      // from there to HBM as whole rows in phase 5
      float *stg = fplane(sm, ROLE == 0 ? DYH : (ROLE == 1 ? KTH : RBH));
#pragma unroll
      for (int ob = 0; ob < 2; ++ob) {
        const int col = 32 * ob + l32;
        const float uc = ob ? uh2 : ul;
        const uint32_t *rk = rkplane(sm);
        // All of the column block's operands are read before any result is written: the
        // compiler cannot tell the planes written below from the planes read, so reads
        // interleaved with the writes would each wait for the LDS round trip in turn.
        uint32_t wv[16];
        float pv[16], dbv[16];
        if constexpr (ROLE != 0) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row0 = 32 * blk + 8 * q + 4 * hh;  // rows row0 .. row0 + 3 of elements 4q .. 4q+3
            const float4 db4 = *reinterpret_cast<const float4 *>(&sm.dbon[row0]);
            dbv[4 * q] = db4.x;
            dbv[4 * q + 1] = db4.y;
            dbv[4 * q + 2] = db4.z;
            dbv[4 * q + 3] = db4.w;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              const int row = row0 + m;
              wv[4 * q + m] = rk[row * RS + col];
              // dk needs P_s, dr needs P_{t-1} (0 before the chunk's first token)
              pv[4 * q + m] = ROLE == 1 ? sm.P[row][col] : sm.P[row ? row - 1 : 0][col];
            }
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row0 = 32 * blk + 8 * q + 4 * hh;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const int e = 4 * q + m, row = row0 + m;
            float val;
            if constexpr (ROLE == 0) {  // dv (the bonus b_s dy_s is on A's diagonal)
              val = acc[ob][e];
            } else if constexpr (ROLE == 1) {  // dk = 2^-P_s dkt + u r_s db_s
              const float dkt = acc[ob][e] * __builtin_amdgcn_exp2f(-pv[e]);
              val = fmaf(uc * bf16_lo(wv[e]), dbv[e], dkt);
              T2[row * PFS + col] = bf16_hi(wv[e]) * dkt;
            } else {  // dr = 2^P_{t-1} drb + u k_t db_t
              const float drb = acc[ob][e] * __builtin_amdgcn_exp2f(row ? pv[e] : 0.f);
              val = fmaf(uc * bf16_hi(wv[e]), dbv[e], drb);
              T1[row * PFS + col] = bf16_lo(wv[e]) * drb;
            }
            stg[row * PFS + col] = val;
          }
        }
      }
    }
    __syncthreads();  // B5
    // ---------- phase 5: dlam by a suffix sum over the chunk's tokens, lane = key channel
    {
      int i = lane;
      asm volatile("" : "+v"(i));
      // the token rows from an opaque vector copy of the wave index: one base address plus
      // immediate offsets, where uniform per-token row addresses would each hold a scalar
      // register (more than there are) across the chunk loop
      int wv = wave;
      asm volatile("" : "+v"(wv));
      const float Eend = sm.E[(c + 1) & 1][i];
      float s[8], xv[8];
      float run = 0.f;
#pragma unroll
      for (int q = 7; q >= 0; --q) {
        const int t = 8 * wv + q;
        // row t + 1 = 64 (read for the last token, then not used) is still inside the two
        // bf16 planes that hold T1
        const float t1n = T1[(t + 1) * PFS + i];
        const float t1 = t < L - 1 ? t1n : Eend;
        run += t1 - T2[t * PFS + i];
        s[q] = run;
        xv[q] = bf16_lo(sm.pl[XR][t][i]);
      }
      {  // the staged dr, dk, dv: 16-byte non-temporal row stores, six per thread (before B6,
         // after which the next chunk's staging may overwrite those planes)
#pragma unroll
        for (int k6 = 0; k6 < 6; ++k6) {
          const int pk = k6 >> 1;
          const float *stg = fplane(sm, pk == 0 ? RBH : (pk == 1 ? KTH : DYH));
          float *outp = pk == 0 ? p.dr : (pk == 1 ? p.dk : p.dv);
          const int row = 32 * (k6 & 1) + (tid >> 4), c4 = tid & 15;
          const float4 v = *reinterpret_cast<const float4 *>(&stg[row * PFS + 4 * c4]);
          // (rows past the chunk's last valid token lie past the resource's records: dropped)
          const auto ro = __builtin_amdgcn_make_buffer_rsrc(outp + uniform64(tok0), 0,
                                                            (int)((uint32_t)(nvalid - 1) * C4 + 4u * kHead), 0x00020000);
          const u32x4 w4 = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
          __builtin_amdgcn_raw_buffer_store_b128(w4, ro, (int)((uint32_t)row * C4 + 16u * (uint32_t)c4), 0, kStoreNT);
        }
      }
      sm.dlt[wave][i] = run;
      __syncthreads();  // B6
      float carry = 0.f;
#pragma unroll
      for (int w = 7; w > 0; --w) carry += w > wave ? sm.dlt[w][i] : 0.f;
      // The resource ends at the chunk's last valid token row, so the stores of rows past it are
      // dropped and every path issues the same eight stores: with a branch per token, the
      // compiler's count of memory operations in flight would make the next chunk's first waits
      // for its prefetched words wait for these stores as well.
      const auto rw2 = __builtin_amdgcn_make_buffer_rsrc(p.dw + uniform64(tok0), 0,
                                                         (int)((uint32_t)(nvalid - 1) * C4 + 4u * kHead), 0x00020000);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int t = 8 * wave + q;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(-fast_exp(xv[q]) * (s[q] + carry)), rw2, i * 4,
                                              (int)((uint32_t)t * C4), kStoreNT);
      }
    }
  }
    if constexpr (ROLE == 3) {  // the initial-state gradient
      if (p.d_state_in) {
        float *g = p.d_state_in + head_off;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            g[(32 * gi + 8 * (e >> 2) + 4 * hh + (e & 3)) * kHead + 32 * jb + l32] = G[jb][e];
      }
    }
    return false;
  };
  bool left;  // the same in every wave (a workgroup-uniform decision at the same point)
  if (wave < 2) left = run_chunks(std::integral_constant<int, 0>{});
  else if (wave < 4) left = run_chunks(std::integral_constant<int, 1>{});
  else if (wave < 6) left = run_chunks(std::integral_constant<int, 2>{});
  else left = run_chunks(std::integral_constant<int, 3>{});
  if (left) return;

  __syncthreads();  // the P plane is free: reduce du over the 16 token groups
  *reinterpret_cast<float2 *>(&sm.P[tg][2 * cp]) = make_float2(du0, du1);
  __syncthreads();
  if (tid < kHead && p.du_rows) {
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < 16; ++g) s += sm.P[g][tid];
    p.du_rows[(long)b * C + h * kHead + tid] = s;
  }
}

}  // namespace

hipError_t launch_wkv6_backward_chunked(const BwdParams &p, hipStream_t s) {
  static std::atomic<unsigned long long> configured{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = 1ull << (dev & 63);
  if (!(configured.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&wkv6_bwdc_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(Smem2));
    if (e != hipSuccess) return e;
    configured.fetch_or(bit, std::memory_order_acq_rel);
  }
  if (!p.chunk_states) {
    hipLaunchKernelGGL(wkv6_bwdc_state_kernel, dim3(p.H, p.B), dim3(kThreads), sizeof(Smem1), s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(wkv6_bwdc_kernel, dim3(p.H, p.B), dim3(kThreads), sizeof(Smem2), s, p);
  return hipGetLastError();
}

}  // namespace wkv
