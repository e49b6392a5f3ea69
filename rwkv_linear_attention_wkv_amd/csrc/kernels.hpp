// Host-side launchers of the WKV kernels (internal to libwkv.so).
// Arguments have been validated by the C ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv {

constexpr int kHeadSize = 64;  // the only head size the kernels are built for

// v5 / v6 token-sequential scan.  Dense form: unit = batch row (tokens
// [b*T, b*T+T)); varlen form: unit = slot (tokens at the slot's packed offset).
struct ScanParams {
  int units;        // B (dense) or num_slots (varlen)
  int T;            // tokens per row (dense)
  int H;
  const void *r, *k, *v, *w;  // w: [H*N] fp32 (v5) or token array (v6)
  const float *u;
  void *y;          // fp32, or bf16 when y_bf16
  bool y_bf16;      // y rounded to bf16 (nearest even) instead of fp32
  // Dense layout: element (row b, token t, head h, channel i) of r, k, v, w
  // (v6) and y sits at b * row_stride + t * tok_stride + h * head_stride + i.
  // [B,T,H,N]: (T*H*N, H*N, N); head-first [B,H,T,N]: (H*T*N, N, T*N).
  // Varlen rows are packed [total_tokens, H*N]: tok_stride H*N, head_stride N.
  long row_stride, tok_stride, head_stride;
  const float *state_in;
  const int32_t *state_map;
  int n_state;
  float *state_out;
  int32_t *dev_status;
  // varlen only
  const int32_t *lengths;
  int max_len;
  int total_tokens;
  // chunked v6 with saved states only: [units, H, ceil(T/64) - 1, 64, 64], the state at the
  // start of chunks 1 .. ceil(T/64) - 1 (after tokens 64c - 1), [key][value]
  float *chunk_states;
};

hipError_t launch_wkv56_scan(const ScanParams &p, bool v6, bool bf16, bool varlen, hipStream_t s);

// v6 varlen calls whose slots consume at most kShortMax tokens (decode steps):
// one wave per (slot, head), state column per lane.
constexpr int kShortMax = 8;
hipError_t launch_wkv6_varlen_short(const ScanParams &p, bool bf16, hipStream_t s);

// v5 / v6 64-token chunked form with MFMA contractions (dense rows only).
hipError_t launch_wkv56_chunked(const ScanParams &p, bool v6, bool bf16, hipStream_t s);
// The v6 chunked form that also writes p.chunk_states (bf16 inputs, [B, T, H*64] rows).
hipError_t launch_wkv6_chunked_save(const ScanParams &p, hipStream_t s);

// v6 backward: three token-sequential sweeps (dr and du, dk and dw, dv and the
// initial-state gradient) and the sum of du over the batch.
struct BwdParams {
  int B, T, H;
  const void *r, *k, *v, *w;  // [B, T, H*64] inputs of the forward call
  const float *u, *dy;
  const float *state_in;
  const int32_t *state_map;
  int n_state;
  const float *state_final, *d_state_out;  // [B, H, 64, 64]
  float *dr, *dk, *dv, *dw, *du, *du_rows, *d_state_in;
  int32_t *dev_status;
  int marked_only;  // sweeps: only the (row, head) units the chunked passes left to them
  // chunked: the chunk start states saved by the forward ([B, H, ceil(T/64) - 1, 64, 64]);
  // NULL: the state pass computes them into dr
  const float *chunk_states;
};

// The chunked backward's mark on a (row, head) it leaves to the sweeps: a NaN bit pattern in
// that unit's dw element of the last token and channel 0 (no arithmetic result or widened bf16
// input has this payload).
constexpr uint32_t kBwdFallbackMark = 0x7fc0dea1u;

hipError_t launch_wkv6_backward(const BwdParams &p, bool bf16, hipStream_t s);
// The chunked passes (bf16 inputs; the state pass only without p.chunk_states);
// launch_wkv6_backward with marked_only follows them.
hipError_t launch_wkv6_backward_chunked(const BwdParams &p, hipStream_t s);

// v7 generalized delta rule, token-sequential (dense rows, [B, T, H*64] token arrays).
struct V7Params {
  int B, T, H;
  const void *r, *w, *k, *v, *a, *b;  // w: decay parameter, decay exp(-exp(w))
  void *y;                            // fp32, or bf16 when y_bf16
  bool y_bf16;
  long row_stride, tok_stride, head_stride;  // token-array layout, as in ScanParams
  const float *state_in;              // [n_state, H, 64, 64] h[key][value], or NULL
  const int32_t *state_map;
  int n_state;
  float *state_out;                   // [B, H, 64, 64] or NULL
  int32_t *dev_status;
};

// Calls with T <= kShortMax run a one-wave-per-(row, head) kernel, longer ones the
// 256-thread token-block kernel.
hipError_t launch_wkv7_scan(const V7Params &p, bool bf16, hipStream_t s);

// v7 64-token chunked form with the contractions on MFMA (bf16 inputs, dense rows).
hipError_t launch_wkv7_chunked(const V7Params &p, bool bf16, hipStream_t s);

// v4 channel-wise scan.
struct V4Params {
  int B, T, C;
  const float *tau, *u;
  const void *k, *v, *r;
  void *y;       // fp32, or bf16 when y_bf16
  bool y_bf16;   // y rounded to bf16 (nearest even) instead of fp32
  const float *state_in;
  float *state_out;
};

hipError_t launch_wkv4(const V4Params &p, bool bf16, hipStream_t s);

}  // namespace wkv
