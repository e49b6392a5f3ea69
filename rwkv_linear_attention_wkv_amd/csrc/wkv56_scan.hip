// Token-sequential WKV v5 / v6 scan on the vector ALUs (dense rows, varlen
// slots and T = 1 decode share this kernel).
//
// Recurrence per (row or slot, head), with S indexed [key i][value j]:
//   y_t[j] = sum_i r_t[i] (S[i][j] + u[i] k_t[i] v_t[j])
//   S[i][j] <- d_t[i] S[i][j] + k_t[i] v_t[j],   d_t[i] = exp(-exp(w_t[i]))
// (the rwkv_ops page's RWKV6_OP call: r, k, v, w, u, init_state, state_map ->
// y, y_state; the standard RWKV-5/6 recurrence).
//
// Varlen calls: workgroups take the slots longest first (up to 256 slots), and a slot
// that consumes at most kShortMax tokens runs the few-token form on one wave.
//
// Work decomposition: one 512-thread workgroup per (head, unit).  Wave w owns
// key rows 8w..8w+7 of the fp32 state and lane j owns value column j, so the
// state is read and written as coalesced 256-byte rows and stays in
// registers for the whole call (8 values per lane).  Tokens are staged 32 at
// a time through LDS as fp32 with each token's bonus r . (u * k); the next
// block's tokens are loaded while the current one is computed.  Per token a
// lane updates its 8 state values and forms its wave's partial output over
// the wave's rows, reading the row factors as LDS broadcasts; the eight
// partials and the bonus term are then summed through LDS in a fixed order,
// so results are deterministic.
//
// Rescaled frame.  Inside a block let D_t[i] be the decay product from the
// block start through token t.  The registers carry St = S / D, for which
//   y_t[j] = sum_i (r_t[i] D_{t-1}[i]) St[i][j] + bonus,
//   St[i][j] += (k_t[i] / D_t[i]) v_t[j],
// two FMAs per state element and token instead of three; S = D St at the
// block end.  The row factors are formed once per (token, channel) while
// staging, from a log2-decay prefix over the block.  Rounding stays relative
// to the terms of the true state, since every term is scaled by a power of
// the decay and scaled back.  A block whose decay product in some channel
// falls below 2^-80 (where 1 / D would leave the fp32 range) takes the direct
// form S <- d S + k v instead.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "varlen_short.hpp"
#include "wkv.h"

namespace wkv {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kRows = kHead / kWaves;  // key rows per wave
constexpr int kTB = 32;                 // tokens staged per block
static_assert(4 * kWaves == kTB && 16 * kTB == kThreads, "staging: four tokens per wave; reduce: one (token, quad) per thread");
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kFrameLog2 = 80.f;  // largest log2 decay of one block the rescaled frame takes
constexpr int kOrderMax = 256;      // varlen calls with at most this many slots run longest first

struct __align__(16) ScanSmem {
  float rk[2][kTB][kHead];       // rescaled frame operands: [0] = rh, [1] = kh
  float v[kTB][kHead];
  float y[kWaves][kTB][kHead];   // per-wave partial outputs
  float r[kTB][kHead], k[kTB][kHead], d[kTB][kHead];  // direct form
  float dend[kHead];             // decay product of the block per key row
  float tot[kWaves][kHead];      // log2 decay of each staging wave's tokens
  float bon[kTB];                // r . (u * k) per token
  unsigned long long off_sum;  // varlen: 64-bit sum of the earlier slots' lengths
  int meta[3];
  int frame;                     // 1: the current block takes the direct form
  int order_unit;                // varlen: the slot this workgroup takes (longest first)
  int lens[kOrderMax];           // varlen: the slots' lengths, for the order
};

template <bool V6, bool BF16, bool VARLEN>
__global__ void __launch_bounds__(kThreads) wkv56_scan_kernel(ScanParams p) {
  const int h = blockIdx.x;
  int unit = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;  // value column j
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // key rows kRows*wave ..

  // One LDS object, the arrays of the token loop first: their offsets stay below 64 KiB, so the
  // loop's reads and writes are a per-thread base register plus an instruction offset.
  __shared__ ScanSmem sm;
  auto &s_rk = sm.rk;
  auto &s_v = sm.v;
  auto &s_y = sm.y;
  auto &s_r = sm.r, &s_k = sm.k, &s_d = sm.d;
  auto &s_dend = sm.dend;
  auto &s_tot = sm.tot;
  auto &s_bon = sm.bon;
  auto &s_meta = sm.meta;
  auto &s_frame = sm.frame;

  long tok0;  // varlen: packed row of the slot's first token
  int ntok;
  int row_in = -1;
  int row_out;

  if constexpr (VARLEN) {
    // Longest first: workgroup row blockIdx.y takes the slot of rank blockIdx.y in the order
    // of decreasing length (ties by slot index), so that the longest slots start first and
    // the short ones fill in behind them instead of leaving a long tail.
    if (p.units <= kOrderMax) {
      for (int i = tid; i < p.units; i += kThreads) sm.lens[i] = p.lengths[i];
      __syncthreads();
      for (int i = tid; i < p.units; i += kThreads) {
        const int li = sm.lens[i];
        int rank = 0;
        for (int j = 0; j < p.units; ++j) {
          const int lj = sm.lens[j];
          rank += (lj > li) | ((lj == li) & (j < i));
        }
        if (rank == (int)blockIdx.y) sm.order_unit = i;
      }
      __syncthreads();
      unit = sm.order_unit;
    }
    // Offset of this slot = sum of earlier lengths; validate the slot.
    // The sum is 64-bit (65535 slots of up to 2^31 - 1 tokens cannot wrap it), and
    // one invalid length anywhere makes every slot's offset meaningless, so every
    // slot is then rejected.
    if (tid == 0) { sm.off_sum = 0ull; s_meta[1] = 0; s_meta[2] = 0; }
    __syncthreads();
    const int my_row = p.state_map ? p.state_map[unit] : unit;
    long sum = 0;
    int bad = 0, dup = 0;
    for (int i = tid; i < p.units; i += kThreads) {
      const int L = p.lengths[i];
      if (i < unit) sum += L;
      bad |= (L < 0) | (L > p.max_len);
      if (p.state_map && i != unit && p.state_map[i] == my_row) dup = 1;
    }
    if (sum) atomicAdd(&sm.off_sum, (unsigned long long)sum);
    if (bad) atomicOr(&s_meta[1], 1);
    if (dup) atomicOr(&s_meta[2], 1);
    __syncthreads();
    const long off = (long)sm.off_sum;
    const int my_len = p.lengths[unit];
    int status = 0;
    if (my_len < 0 || my_len > p.max_len || s_meta[1]) status |= WKV_DEV_BAD_LENGTH;
    if (my_row < 0 || my_row >= p.n_state) status |= WKV_DEV_BAD_STATE_MAP;
    if (s_meta[2]) status |= WKV_DEV_DUPLICATE_ROW;
    if (!(status & WKV_DEV_BAD_LENGTH) && off + my_len > (long)p.total_tokens)
      status |= WKV_DEV_TOKEN_OVERFLOW;
    if (status) {
      if (tid == 0 && p.dev_status) atomicOr(p.dev_status, status);
      return;
    }
    tok0 = off;
    ntok = my_len;
    row_in = my_row;
    row_out = my_row;
    // A slot of at most kShortMax tokens takes the few-token form on one wave (the state
    // column in the lane); the other waves leave.
    if (ntok <= kShortMax) {
      if (wave != 0) return;
      float sc[kHead];
      const float *sp = p.state_in + ((long)my_row * p.H + h) * (kHead * kHead) + lane;
#pragma unroll
      for (int i = 0; i < kHead; ++i) sc[i] = sp[i * kHead];
      static_assert(sizeof(sm.r) >= sizeof(float) * kShortLdsFloats, "few-token staging fits");
      short_slot_wave<BF16>(p, h, lane, off, ntok, my_row, sc, &sm.r[0][0]);
      return;
    }
  } else {
    tok0 = 0;
    ntok = p.T;
    row_out = unit;
    if (p.state_in) {
      row_in = p.state_map ? p.state_map[unit] : (p.n_state == 1 ? 0 : unit);
      if (row_in < 0 || row_in >= p.n_state) {
        if (tid == 0 && p.dev_status) atomicOr(p.dev_status, WKV_DEV_BAD_STATE_MAP);
        return;
      }
    }
  }

  // element offset of this unit's token 0 in this head; tokens are tok_stride apart
  const long ts = p.tok_stride;
  const long base = VARLEN ? tok0 * ts + h * p.head_stride : unit * p.row_stride + h * p.head_stride;

  // ---- this lane's column of the wave's key rows, in registers
  float s[kRows];
  if (row_in >= 0 && p.state_in) {
    const float *sp = p.state_in + ((long)row_in * p.H + h) * (kHead * kHead) + lane;
#pragma unroll
    for (int a = 0; a < kRows; ++a) s[a] = sp[(kRows * wave + a) * kHead];
  } else {
#pragma unroll
    for (int a = 0; a < kRows; ++a) s[a] = 0.f;
  }
  // Staging role: wave sw stages tokens 4 sw .. 4 sw + 3 of a block and lane
  // j channel j.  Decays are kept as log2 (lam = log2 d); cum is this thread's
  // running sum over its four tokens.
  const float uc = p.u[h * kHead + lane];
  float lam_static = 0.f;
  if constexpr (!V6) lam_static = -fast_exp(static_cast<const float *>(p.w)[h * kHead + lane]) * kLog2e;
  // the next block's tokens, loaded one block ahead (rows past the end reread the last row)
  float pr[4], pk[4], pv[4], px[4];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      const long e = base + min(t0 + 4 * wave + t4, ntok - 1) * ts + lane;
      pr[t4] = load1<BF16>(p.r, e);
      pk[t4] = load1<BF16>(p.k, e);
      pv[t4] = load1<BF16>(p.v, e);
      px[t4] = V6 ? load1<BF16>(p.w, e) : 0.f;
    }
  };
  if (ntok > 0) fetch(0);
  for (int t0 = 0; t0 < ntok; t0 += kTB) {
    const int nb = min(kTB, ntok - t0);
    // -- stage r, k, v, d and the bonus; in-thread log-decay prefix
    float rr[4], kk[4], cum[4], bon[4];
    float run = 0.f;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      const int tt = 4 * wave + t4;
      const bool valid = tt < nb;
      const float lam = valid ? (V6 ? -fast_exp(px[t4]) * kLog2e : lam_static) : 0.f;  // no decay past the end
      run += lam;
      cum[t4] = run;
      rr[t4] = pr[t4];
      kk[t4] = pk[t4];
      s_r[tt][lane] = pr[t4];
      s_k[tt][lane] = pk[t4];
      s_d[tt][lane] = __builtin_amdgcn_exp2f(lam);
      s_v[tt][lane] = pv[t4];
      bon[t4] = pr[t4] * uc * pk[t4];
    }
    s_tot[wave][lane] = run;
    if (tid == 0) s_frame = 0;
    fetch(t0 + kTB);  // the next block, in flight during this one
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {  // bonus: sum over the 64 channels of the token
      float x = bon[t4];
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
      bon[t4] = x;
    }
    if (lane == 0) {
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) s_bon[4 * wave + t4] = bon[t4];
    }
    __syncthreads();
    // -- rescaled frame operands: with Lam_t the log2 decay from the block start
    //    through token t, rh_t = r_t 2^Lam_{t-1} and kh_t = k_t 2^-Lam_t.
    {
      float pre = 0.f;
      for (int w = 0; w < wave; ++w) pre += s_tot[w][lane];
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const int tt = 4 * wave + t4;
        const float lprev = pre + (t4 ? cum[t4 - 1] : 0.f), lcur = pre + cum[t4];
        s_rk[0][tt][lane] = rr[t4] * __builtin_amdgcn_exp2f(lprev);
        s_rk[1][tt][lane] = kk[t4] * __builtin_amdgcn_exp2f(-lcur);
      }
      if (wave == kWaves - 1) {
        const float lend = pre + cum[3];
        s_dend[lane] = __builtin_amdgcn_exp2f(lend);
        if (lend < -kFrameLog2) s_frame = 1;  // too much decay in one block for the frame
      }
    }
    __syncthreads();

    if (s_frame == 0) {
      // Rescaled frame: the registers hold St = S / D (D = decay product from the block
      // start), so per token y += rh . St and St += kh v: two FMAs per state element.
      // Per-thread LDS pointers, formed once in vector registers: every read and write of the
      // loop is then one of them plus a constant offset (no per-token address arithmetic).
      int w2 = 2 * wave;  // the wave's rows in float4 units
      asm volatile("" : "+v"(w2));
      const float4 *rk4 = reinterpret_cast<const float4 *>(&s_rk[0][0][0]) + w2;
      const float *vp = &s_v[0][lane];
      float *yp = &s_y[wave][0][lane];
      constexpr int kRow4 = kHead / 4, kKh4 = kTB * kHead / 4;  // float4 strides: token, rh -> kh
#pragma unroll 4
      for (int tt = 0; tt < nb; ++tt) {
        const float vj = vp[tt * kHead];
        const float4 r0 = rk4[tt * kRow4], r1 = rk4[tt * kRow4 + 1];
        const float4 k0 = rk4[kKh4 + tt * kRow4], k1 = rk4[kKh4 + tt * kRow4 + 1];
        float y0 = r0.x * s[0];
        s[0] = fmaf(k0.x, vj, s[0]);
        float y1 = r0.y * s[1];
        s[1] = fmaf(k0.y, vj, s[1]);
        y0 = fmaf(r0.z, s[2], y0); s[2] = fmaf(k0.z, vj, s[2]);
        y1 = fmaf(r0.w, s[3], y1); s[3] = fmaf(k0.w, vj, s[3]);
        y0 = fmaf(r1.x, s[4], y0); s[4] = fmaf(k1.x, vj, s[4]);
        y1 = fmaf(r1.y, s[5], y1); s[5] = fmaf(k1.y, vj, s[5]);
        y0 = fmaf(r1.z, s[6], y0); s[6] = fmaf(k1.z, vj, s[6]);
        y1 = fmaf(r1.w, s[7], y1); s[7] = fmaf(k1.w, vj, s[7]);
        yp[tt * kHead] = y0 + y1;
      }
      // back to S at the block end
      const float4 d0 = *reinterpret_cast<const float4 *>(&s_dend[kRows * wave]);
      const float4 d1 = *reinterpret_cast<const float4 *>(&s_dend[kRows * wave + 4]);
      s[0] *= d0.x; s[1] *= d0.y; s[2] *= d0.z; s[3] *= d0.w;
      s[4] *= d1.x; s[5] *= d1.y; s[6] *= d1.z; s[7] *= d1.w;
    } else {
      // direct form: S <- d S + k v
      for (int tt = 0; tt < nb; ++tt) {
        const float vj = s_v[tt][lane];
        float y0 = 0.f, y1 = 0.f;
#pragma unroll
        for (int g = 0; g < 2; ++g) {  // (the rare path: not tuned)
          const float4 r4 = *reinterpret_cast<const float4 *>(&s_r[tt][kRows * wave + 4 * g]);
          const float4 k4 = *reinterpret_cast<const float4 *>(&s_k[tt][kRows * wave + 4 * g]);
          const float4 d4 = *reinterpret_cast<const float4 *>(&s_d[tt][kRows * wave + 4 * g]);
          y0 = fmaf(r4.x, s[4 * g], y0); s[4 * g] = fmaf(d4.x, s[4 * g], k4.x * vj);
          y1 = fmaf(r4.y, s[4 * g + 1], y1); s[4 * g + 1] = fmaf(d4.y, s[4 * g + 1], k4.y * vj);
          y0 = fmaf(r4.z, s[4 * g + 2], y0); s[4 * g + 2] = fmaf(d4.z, s[4 * g + 2], k4.z * vj);
          y1 = fmaf(r4.w, s[4 * g + 3], y1); s[4 * g + 3] = fmaf(d4.w, s[4 * g + 3], k4.w * vj);
        }
        s_y[wave][tt][lane] = y0 + y1;
      }
    }
    __syncthreads();
    {  // sum the wave partials in a fixed order, add the bonus term, store fp32 outputs
      const int tt = tid >> 4, j = 4 * (tid & 15);
      if (tt < nb) {
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float4 a = *reinterpret_cast<const float4 *>(&s_y[w][tt][j]);
          o.x += a.x; o.y += a.y; o.z += a.z; o.w += a.w;
        }
        const float b = s_bon[tt];
        const float4 v4 = *reinterpret_cast<const float4 *>(&s_v[tt][j]);
        o = f4(fmaf(b, v4.x, o.x), fmaf(b, v4.y, o.y), fmaf(b, v4.z, o.z), fmaf(b, v4.w, o.w));
        const long ye = base + (t0 + tt) * ts + j;
        if (p.y_bf16)
          *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.y) + ye) = make_uint2(pack_bf16(o.x, o.y), pack_bf16(o.z, o.w));
        else
          *reinterpret_cast<float4 *>(static_cast<float *>(p.y) + ye) = o;
      }
    }
    // The next staging writes the token arrays after this block's reads (ordered by this
    // barrier); s_y is written again only after the next staging barrier.
    __syncthreads();
  }

  if (p.state_out) {
    if (VARLEN && ntok == 0 && p.state_out == p.state_in) return;  // empty slot: untouched
    float *sp = p.state_out + ((long)row_out * p.H + h) * (kHead * kHead) + lane;
#pragma unroll
    for (int a = 0; a < kRows; ++a) sp[(kRows * wave + a) * kHead] = s[a];
  }
}

template <bool V6, bool BF16, bool VARLEN>
hipError_t launch(const ScanParams &p, hipStream_t s) {
  dim3 grid(p.H, p.units);
  hipLaunchKernelGGL((wkv56_scan_kernel<V6, BF16, VARLEN>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_wkv56_scan(const ScanParams &p, bool v6, bool bf16, bool varlen, hipStream_t s) {
  if (varlen)  // varlen always carries a per-token decay
    return bf16 ? launch<true, true, true>(p, s) : launch<true, false, true>(p, s);
  if (v6) return bf16 ? launch<true, true, false>(p, s) : launch<true, false, false>(p, s);
  return bf16 ? launch<false, true, false>(p, s) : launch<false, false, false>(p, s);
}

}  // namespace wkv
