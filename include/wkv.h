/*
 * wkv.h — C ABI of the MI355X (gfx950) WKV time-mixing library (libwkv.so).
 *
 * The library computes the RWKV WKV recurrence in three forms:
 *
 *   v4  channel-wise exponential-decay weighted average with a bonus on the
 *       current token, carried as a numerically stable running-max state
 *       (a, b, p) per channel.  The call shape follows the RWKV-v4
 *       walk-through page ("代码连连看——RWKV", RWKV_TimeMix.forward, the
 *       RUN_CUDA(B, T, C, time_decay, time_first, k, v) call, whose result is
 *       gated by sigmoid(r)).
 *   v5  multi-head form with an N x N fp32 state per head and a static decay
 *       per head-channel.
 *   v6  the same with a per-token, per-channel decay.  Arguments follow the
 *       rwkv_ops page ("rwkv6op 使用方法": r, k, v, w of shape
 *       (batch, seq, hidden); u of shape (heads, head_size) or (hidden,);
 *       init_state (n_state, heads, head_size, head_size); state_map int32
 *       (batch,); y_state (batch, heads, head_size, head_size)).
 *
 * and a varlen entry point for batched serving where each slot consumes its
 * own number of tokens per call and keeps its state on the device between
 * calls (the web-rwkv page, batched inference section: slots of a model
 * state, a per-call token budget `token_chunk_size`, empty slots skipped).
 *
 * Definitions (no page prints them; these are the standard RWKV-4/5/6
 * recurrences).  Channel c = h*N + i; key index i (row of S), value index j
 * (column of S).
 *
 *   v4:   lambda_c = -exp(time_decay[c]); with A = a*e^p, B = b*e^p
 *         wkv_t = (A + e^(u_c + k_t) v_t) / (B + e^(u_c + k_t))
 *         y_t   = sigmoid(r_t) * wkv_t  (r given)  or  wkv_t  (r == NULL)
 *         A <- e^lambda_c A + e^(k_t) v_t ;  B <- e^lambda_c B + e^(k_t)
 *   v5/v6: d_t[i] = exp(-exp(w_t[i]))   (w constant over t for v5)
 *         y_t[j] = sum_i r_t[i] (S[i][j] + u[i] k_t[i] v_t[j])
 *         S[i][j] <- d_t[i] S[i][j] + k_t[i] v_t[j]
 *
 * Conventions shared by every entry point
 *   - Every array argument is a DEVICE pointer owned by the caller, row-major
 *     and contiguous, aligned to at least 16 bytes.  The library never
 *     allocates, frees or copies caller memory between host and device.
 *   - Token arrays are [B, T, C] (C = H*N) and y is fp32, except in the _ex
 *     entry points, which also take head-first [B, H, T, N] arrays and a bf16
 *     y.
 *   - Calls enqueue work on `stream` (a hipStream_t; NULL = default stream)
 *     and return before it completes.  Results are valid once the stream has
 *     been synchronised.
 *   - Errors are status codes; the library never aborts.  Host-checkable
 *     problems return before anything is enqueued.  Data problems that only
 *     the device can see set bits in *dev_status (if given) and skip the
 *     affected unit of work.
 *   - Functions are stateless and reentrant; identical inputs give bitwise
 *     identical outputs (no floating-point atomics).
 */
#ifndef WKV_H
#define WKV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WKV_ABI_VERSION 1

#if defined(__GNUC__)
#define WKV_API __attribute__((visibility("default")))
#else
#define WKV_API
#endif

typedef int32_t wkv_status;
#define WKV_OK               0  /* success (work enqueued)                        */
#define WKV_ERR_INVALID_ARG  1  /* bad dimension, NULL or misaligned pointer, ... */
#define WKV_ERR_UNSUPPORTED  2  /* head size other than 64, unknown dtype / algo  */
#define WKV_ERR_DEVICE       3  /* a HIP launch failed; see wkv_last_error()      */

typedef int32_t wkv_dtype;
#define WKV_F32   0             /* 32-bit IEEE float inputs                       */
#define WKV_BF16  1             /* bfloat16 inputs (upper half of an fp32)        */

typedef int32_t wkv_layout;
#define WKV_LAYOUT_BTHN 0       /* [B,T,H,N]: token rows hold every head          */
#define WKV_LAYOUT_BHTN 1       /* [B,H,T,N]: head-first, a head's tokens adjacent */

typedef int32_t wkv_algo;
#define WKV_ALGO_AUTO     0     /* library picks                                  */
#define WKV_ALGO_SCAN     1     /* token-sequential scan on the vector ALUs       */
#define WKV_ALGO_CHUNKED  2     /* 64-token chunks, contractions on MFMA          */

/* Bits OR-ed into *dev_status by the device (never cleared by the library). */
#define WKV_DEV_BAD_STATE_MAP  1  /* state_map entry outside [0, n_state)         */
#define WKV_DEV_BAD_LENGTH     2  /* varlen length < 0 or > max_len               */
#define WKV_DEV_TOKEN_OVERFLOW 4  /* varlen: sum of lengths exceeds total_tokens  */
#define WKV_DEV_DUPLICATE_ROW  8  /* varlen: two slots map to the same state row  */
/* Bit 16 is reserved.  Both algorithms take any decay parameter: the chunked
 * form runs a chunk whose accumulated decay would leave its exponent range
 * with the direct token recurrence instead, so no decay is a data error. */

/*
 * v4 forward (prefill over T tokens, or T = 1 decode).
 *   time_decay [C] fp32   raw parameter; per-step decay exp(-exp(time_decay))
 *   time_first [C] fp32   bonus u of the current token
 *   k, v       [B,T,C]    in_dtype
 *   r          [B,T,C]    in_dtype, optional: output gated by sigmoid(r)
 *   y          [B,T,C]    fp32 output
 *   state_in   [B,3,C]    fp32 planes (a, b, p), NULL = fresh sequence
 *                         (a = b = 0, p = -1e38)
 *   state_out  [B,3,C]    fp32 final state, NULL = not returned; may equal
 *                         state_in (in place)
 * T = 0 is a valid no-op (state_out, if given, receives state_in).
 */
WKV_API wkv_status wkv4_forward(int B, int T, int C,
                        const float *time_decay, const float *time_first,
                        const void *k, const void *v, const void *r,
                        wkv_dtype in_dtype, float *y,
                        const float *state_in, float *state_out,
                        void *stream);

/*
 * v4 forward with a choice of output dtype: as wkv4_forward, with
 *   y          [B,T,C]    out_dtype: WKV_F32, or WKV_BF16 (the fp32 result
 *                         rounded to nearest even; the rwkv_ops page's
 *                         single-step operator returns its output in the
 *                         input dtype)
 */
WKV_API wkv_status wkv4_forward_ex(int B, int T, int C,
                           const float *time_decay, const float *time_first,
                           const void *k, const void *v, const void *r,
                           wkv_dtype in_dtype, void *y, wkv_dtype out_dtype,
                           const float *state_in, float *state_out,
                           void *stream);

/*
 * v5 forward (static decay).
 *   r, k, v    [B,T,H*N]  in_dtype
 *   w          [H*N] fp32 raw decay parameter; decay exp(-exp(w))
 *   u          [H*N] fp32 bonus
 *   y          [B,T,H*N]  fp32 output
 *   state_in   [n_state,H,N,N] fp32 or NULL (zero initial state)
 *   state_map  [B] int32 or NULL: batch row b starts from
 *              state_in[state_map[b]]; with NULL, n_state must be 1 (shared)
 *              or B (one per row)
 *   state_out  [B,H,N,N] fp32 or NULL; may equal state_in only when
 *              state_map is NULL and n_state == B
 *   dev_status int32 device word or NULL (WKV_DEV_* bits)
 * N must be 64.
 */
WKV_API wkv_status wkv5_forward(int B, int T, int H, int N,
                        const void *r, const void *k, const void *v,
                        wkv_dtype in_dtype,
                        const float *w, const float *u, float *y,
                        const float *state_in, const int32_t *state_map, int n_state,
                        float *state_out, wkv_algo algo, int32_t *dev_status,
                        void *stream);

/*
 * v6 forward (per-token decay).  As wkv5_forward, except
 *   w          [B,T,H*N]  in_dtype raw decay parameter per token and channel
 */
WKV_API wkv_status wkv6_forward(int B, int T, int H, int N,
                        const void *r, const void *k, const void *v, const void *w,
                        wkv_dtype in_dtype, const float *u, float *y,
                        const float *state_in, const int32_t *state_map, int n_state,
                        float *state_out, wkv_algo algo, int32_t *dev_status,
                        void *stream);

/*
 * v5 / v6 forward with a choice of token layout and output dtype (the
 * rwkv_ops page's generalized_delta_rule interface takes both layouts through
 * its head_first flag, and its single-step operator returns the input dtype):
 *   layout     WKV_LAYOUT_BTHN: r, k, v, w (v6) and y are [B,T,H,N];
 *              WKV_LAYOUT_BHTN: they are [B,H,T,N]
 *   y          out_dtype: WKV_F32, or WKV_BF16 (the fp32 result rounded to
 *              nearest even)
 * Everything else as wkv5_forward / wkv6_forward (states are [.., H, N, N]
 * in both layouts; v5's w and u are [H*N]).  Both layouts give bitwise the
 * same values, and the bf16 output is bitwise the fp32 output rounded.
 */
WKV_API wkv_status wkv5_forward_ex(int B, int T, int H, int N,
                           const void *r, const void *k, const void *v,
                           wkv_dtype in_dtype, wkv_layout layout,
                           const float *w, const float *u, void *y, wkv_dtype out_dtype,
                           const float *state_in, const int32_t *state_map, int n_state,
                           float *state_out, wkv_algo algo, int32_t *dev_status,
                           void *stream);
WKV_API wkv_status wkv6_forward_ex(int B, int T, int H, int N,
                           const void *r, const void *k, const void *v, const void *w,
                           wkv_dtype in_dtype, wkv_layout layout,
                           const float *u, void *y, wkv_dtype out_dtype,
                           const float *state_in, const int32_t *state_map, int n_state,
                           float *state_out, wkv_algo algo, int32_t *dev_status,
                           void *stream);

/*
 * v6 forward for training: the chunked form (bf16 inputs, [B,T,H*N] rows), which
 * also saves the state at every chunk boundary for wkv6_backward_ex.  (The
 * rwkv_ops page's RWKV6_OP is the gradient-capable operator of this recurrence;
 * handing the forward's chunk-start states to the backward is this library's
 * own arrangement, so that the backward need not recompute them.)
 *   chunk_states [B,H,ceil(T/64)-1,N,N] fp32 DEVICE, 16-byte aligned (may be
 *                NULL when T <= 64): entry c-1 is the state after token 64c-1
 *                ([key][value], c = 1 .. ceil(T/64)-1), in fp32 as the kernel
 *                carries it; rows of a rejected state_map entry are not written
 * Every other argument, result and error as wkv6_forward_ex with layout
 * WKV_LAYOUT_BTHN and WKV_ALGO_CHUNKED: y and state_out are bitwise those of
 * that call.  Costs one extra write of the states (16 KiB per chunk and head).
 */
WKV_API wkv_status wkv6_forward_train(int B, int T, int H, int N,
                           const void *r, const void *k, const void *v, const void *w,
                           wkv_dtype in_dtype, const float *u, void *y, wkv_dtype out_dtype,
                           const float *state_in, const int32_t *state_map, int n_state,
                           float *state_out, float *chunk_states, int32_t *dev_status,
                           void *stream);

/*
 * v6 varlen forward for batched serving.
 *   lengths      [num_slots] int32 DEVICE: tokens slot s consumes this call
 *                (0 = empty slot: no work, its state row is untouched, or
 *                copied when state_out != state_in)
 *   max_len      host upper bound on every length (a length above it is a
 *                data error)
 *   total_tokens number of packed token rows in r, k, v, w, y
 *   r, k, v, w   [total_tokens, H*N] in_dtype; slot s owns rows
 *                [off_s, off_s + lengths[s]), off = exclusive prefix sum
 *   u            [H*N] fp32
 *   y            [total_tokens, H*N] fp32 (rows past sum(lengths) untouched)
 *   state_in     [n_state,H,N,N] fp32: slot s reads row state_map[s]
 *   state_out    [n_state,H,N,N] fp32: slot s writes row state_map[s];
 *                may equal state_in (the usual in-place serving loop)
 *   state_map    [num_slots] int32 DEVICE or NULL (identity; then
 *                n_state >= num_slots).  Entries must be distinct.
 * A length below 0 or above max_len in any slot sets WKV_DEV_BAD_LENGTH and
 * rejects every slot of the call (the offsets of the slots after it are
 * meaningless); offsets are summed in 64 bits, so lengths whose sum passes
 * total_tokens set WKV_DEV_TOKEN_OVERFLOW for the slots they push past it.
 * A rejected slot writes neither y nor its state row.
 * N must be 64.
 */
WKV_API wkv_status wkv6_forward_varlen(int num_slots, int H, int N,
                               const int32_t *lengths, int max_len, int total_tokens,
                               const void *r, const void *k, const void *v, const void *w,
                               wkv_dtype in_dtype, const float *u, float *y,
                               const float *state_in, float *state_out,
                               const int32_t *state_map, int n_state,
                               int32_t *dev_status, void *stream);

/* wkv6_forward_varlen with y [total_tokens, H*N] in out_dtype (WKV_F32 or
 * WKV_BF16, the fp32 result rounded to nearest even). */
WKV_API wkv_status wkv6_forward_varlen_ex(int num_slots, int H, int N,
                                  const int32_t *lengths, int max_len, int total_tokens,
                                  const void *r, const void *k, const void *v, const void *w,
                                  wkv_dtype in_dtype, const float *u, void *y, wkv_dtype out_dtype,
                                  const float *state_in, float *state_out,
                                  const int32_t *state_map, int n_state,
                                  int32_t *dev_status, void *stream);

/*
 * v6 backward: gradients for training (the RWKV-6 recurrence of wkv6_forward,
 * the rwkv_ops page's RWKV6_OP call, differentiated in reverse mode).
 * With the loss L = sum(dy * y) + sum(d_state_out * S_final) of a forward
 * call with the same r, k, v, w, u, state_in, state_map, n_state:
 *   dy           [B,T,H*N] fp32 gradient of y
 *   state_final  [B,H,N,N] fp32 the forward call's final state (its
 *                state_out); required when d_state_out is given, else unused
 *   d_state_out  [B,H,N,N] fp32 gradient of the final state, or NULL (zero)
 *   dr, dk, dv   [B,T,H*N] fp32 gradients of r, k, v
 *   dw           [B,T,H*N] fp32 gradient of the raw decay parameter w
 *   du           [H*N] fp32 gradient of u (summed over the batch)
 *   du_rows      [B,H*N] fp32 each batch row's share of du (also the staging
 *                for du; the caller provides it)
 *   d_state_in   [B,H,N,N] fp32 or NULL: gradient with respect to the initial
 *                state row b started from (rows that share a state_in row are
 *                not summed: the caller adds them)
 * A batch row whose state_map entry is outside [0, n_state) sets
 * WKV_DEV_BAD_STATE_MAP; its rows of dr, dk, dv, dw and d_state_in hold no
 * gradients (not written, apart from the staging described below), its du_rows
 * row is zero, and du sums the other rows.
 * All pointers are device pointers owned by the caller; the library
 * allocates nothing.  Outputs are written, not accumulated.  The
 * algorithm is WKV_ALGO_AUTO (see wkv6_backward_ex).  dr and dw also serve as
 * staging between the launches (chunk start states in dr, the forward state of
 * every 256th token and a per-unit mark in dw, each head in its own columns), so
 * neither may alias another argument.
 * N must be 64.  Deterministic (no atomics on data).
 */
WKV_API wkv_status wkv6_backward(int B, int T, int H, int N,
                         const void *r, const void *k, const void *v, const void *w,
                         wkv_dtype in_dtype, const float *u, const float *dy,
                         const float *state_in, const int32_t *state_map, int n_state,
                         const float *state_final, const float *d_state_out,
                         float *dr, float *dk, float *dv, float *dw,
                         float *du, float *du_rows, float *d_state_in,
                         int32_t *dev_status, void *stream);

/* wkv6_backward with a choice of algorithm:
 *   WKV_ALGO_SCAN     three token-sequential sweeps over the sequence (vector ALUs);
 *   WKV_ALGO_CHUNKED  64-token chunks on MFMA (bf16 inputs only, else
 *                     WKV_ERR_UNSUPPORTED): a pass that leaves each chunk's start
 *                     state in dr, then a reverse pass over the chunks that forms
 *                     every gradient from matrix products; a (row, head) with a
 *                     chunk whose decays leave the chunked form's exponent range
 *                     (a log2-decay total below -100 in some channel, e.g.
 *                     strong or zero decays) and a rejected state_map row are
 *                     left to the sweeps, so every input is covered;
 *   WKV_ALGO_AUTO     CHUNKED for bf16 inputs with T >= 64, else SCAN.
 *   chunk_states  NULL, or the states wkv6_forward_train saved in the forward
 *                 call of these inputs ([B,H,ceil(T/64)-1,N,N], 16-byte
 *                 aligned): the chunked algorithm then reads them instead of
 *                 computing them (one pass over k, v and w fewer; no state
 *                 staging in dr).  Ignored by the sweeps.
 * Precision: the sweeps compute in fp32 (dr, dk, dv, du, d_state_in about 1e-6
 * relative to the largest value, dw about 5e-5, coarser for decays near zero);
 * the chunked products take every operand that is not an exact bf16 input as
 * bf16 hi + lo (about 16 bits): about 1e-4 for dr .. d_state_in and 1e-3 for
 * dw, whose in-chunk running difference does not cancel those roundings.
 * Every other argument, result and error as wkv6_backward. */
WKV_API wkv_status wkv6_backward_ex(int B, int T, int H, int N,
                            const void *r, const void *k, const void *v, const void *w,
                            wkv_dtype in_dtype, const float *u, const float *dy,
                            const float *state_in, const int32_t *state_map, int n_state,
                            const float *state_final, const float *d_state_out,
                            float *dr, float *dk, float *dv, float *dw,
                            float *du, float *du_rows, float *d_state_in,
                            const float *chunk_states, wkv_algo algo,
                            int32_t *dev_status, void *stream);

/*
 * v6 backward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving or training loops, harnesses that forbid
 * hipMalloc): wkv6_backward without the du_rows workspace.  The per-row du
 * staging lives in a static device array of the library, 1,048,576 floats
 * (4 MiB) per GPU, held until the process ends, so B*H*N must be at most
 * 1,048,576 (larger calls return WKV_ERR_INVALID_ARG before anything is
 * enqueued).  The array's device address is looked up on the first call on
 * each device (the calling thread's current device must be the stream's).
 * Nothing is allocated or freed, by the library or any routine it calls.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (other streams, other threads) race and give wrong du.  Every other
 * argument, result and error as wkv6_backward; the results are bitwise those
 * of wkv6_backward.
 */
WKV_API wkv_status wkv6_backward_noalloc(int B, int T, int H, int N,
                                 const void *r, const void *k, const void *v, const void *w,
                                 wkv_dtype in_dtype, const float *u, const float *dy,
                                 const float *state_in, const int32_t *state_map, int n_state,
                                 const float *state_final, const float *d_state_out,
                                 float *dr, float *dk, float *dv, float *dw,
                                 float *du, float *d_state_in,
                                 int32_t *dev_status, void *stream);

/*
 * v7 forward: the generalized delta rule of the rwkv_ops page's
 * generalized_delta_rule operator (r, w, k, v, a, b of shape [B, T, H, K],
 * initial_state [N, H, K, V]; its single-step rwkv7_op_rnn call is this with
 * T = 1).  The page gives no formula; this is the standard RWKV-7
 * recurrence, with the decay exp(-exp(w)) of rwkv6op (the page's padding
 * note, w += (1 - mask) * -1e9 for padded tokens, needs their decay to be
 * exactly 1).  Per (batch row, head), state h[key i][value j]:
 *   sa[j] = sum_i a_t[i] h[i][j]
 *   h[i][j] <- d_t[i] h[i][j] + b_t[i] sa[j] + k_t[i] v_t[j],  d_t = exp(-exp(w_t))
 *   y_t[j] = sum_i r_t[i] h[i][j]              (the updated state)
 *   r, w, k, v, a, b [B,T,H*N] in_dtype, or [B,H,T,N] with layout
 *              WKV_LAYOUT_BHTN (the operators' head_first flag)
 *   y          the same layout, out_dtype (WKV_F32, or WKV_BF16: the fp32
 *              result rounded to nearest even)
 *   state_in, state_map, n_state, state_out, dev_status: as wkv6_forward
 *              (states [.., H, N, N] indexed [key][value])
 * N must be 64.  The algorithm is WKV_ALGO_AUTO: the 64-token chunked form on
 * MFMA for bf16 inputs with T >= 64 (the chunkwise operator the page names
 * next to the recurrent one), else the token-sequential kernel (prefill and
 * T = 1 decode).  Both are exact for any decay parameter.
 */
WKV_API wkv_status wkv7_forward(int B, int T, int H, int N,
                        const void *r, const void *w, const void *k, const void *v,
                        const void *a, const void *b, wkv_dtype in_dtype, wkv_layout layout,
                        void *y, wkv_dtype out_dtype,
                        const float *state_in, const int32_t *state_map, int n_state,
                        float *state_out, int32_t *dev_status, void *stream);

/* wkv7_forward with a choice of algorithm: WKV_ALGO_SCAN (token-sequential),
 * WKV_ALGO_CHUNKED (64-token chunks on MFMA; bf16 inputs only, else
 * WKV_ERR_UNSUPPORTED) or WKV_ALGO_AUTO. */
WKV_API wkv_status wkv7_forward_ex(int B, int T, int H, int N,
                           const void *r, const void *w, const void *k, const void *v,
                           const void *a, const void *b, wkv_dtype in_dtype, wkv_layout layout,
                           void *y, wkv_dtype out_dtype,
                           const float *state_in, const int32_t *state_map, int n_state,
                           float *state_out, wkv_algo algo, int32_t *dev_status, void *stream);

/*
 * Host-side token-budget split for the varlen serving loop (HOST arrays).
 * Hands one token at a time to every slot with tokens left, in slot order,
 * until `budget` tokens are given out or no slot has tokens left.
 *   remaining [num_slots] int32 >= 0   tokens each slot still has to consume
 *   take      [num_slots] int32 output tokens each slot consumes this call
 *   *total    receives sum(take)
 */
WKV_API wkv_status wkv_schedule_round_robin(int num_slots, const int32_t *remaining,
                                    int budget, int32_t *take, int32_t *total);

/* Algorithm a v5, v6 or v7 call (version 5, 6 or 7) of this shape and input
 * dtype runs when it requests `requested` (WKV_ALGO_AUTO: chunked for bf16
 * inputs with T >= 64, else the scan; the chunked form needs bf16 inputs).
 * Pure host function. */
WKV_API wkv_algo wkv_resolve_algo(int version, int B, int T, int H, int N, wkv_dtype in_dtype,
                                  wkv_algo requested);

WKV_API const char *wkv_status_string(wkv_status s);
/* Detail of the last non-OK return on the calling thread ("" if none). */
WKV_API const char *wkv_last_error(void);
WKV_API int wkv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WKV_H */
