// C ABI of libwkv.so: argument validation, algorithm choice and launch.
// Every host-checkable problem is reported before any HIP call, so the
// validation paths run (and are tested) on machines without a GPU.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "kernels.hpp"
#include "wkv.h"

namespace {

thread_local char g_last_error[512] = "";

wkv_status fail(wkv_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

wkv_status ok() {
  g_last_error[0] = '\0';
  return WKV_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool dtype_ok(wkv_dtype d) { return d == WKV_F32 || d == WKV_BF16; }

wkv_status launched(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(WKV_ERR_DEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

constexpr int kMaxGridY = 65535;
constexpr int kChunk = 64;
// The chunked kernel addresses a chunk's token rows with 32-bit offsets.
constexpr int kChunkedMaxRow = 1 << 23;

#define REQUIRE(cond, ...)                                        \
  do {                                                            \
    if (!(cond)) return fail(WKV_ERR_INVALID_ARG, __VA_ARGS__);   \
  } while (0)

// Shared validation of the dense v5 / v6 calls.
wkv_status check_dense56(const char *fn, int B, int T, int H, int N, const void *r, const void *k,
                         const void *v, const void *w, wkv_dtype in_dtype, const float *u,
                         const void *y, const float *state_in, const int32_t *state_map,
                         int n_state, const float *state_out, wkv_algo algo) {
  REQUIRE(B >= 1 && T >= 0 && H >= 1, "%s: need B >= 1, T >= 0, H >= 1 (got B=%d T=%d H=%d)", fn, B, T, H);
  if (N != wkv::kHeadSize) return fail(WKV_ERR_UNSUPPORTED, "%s: head size N=%d is not supported (only 64)", fn, N);
  if (!dtype_ok(in_dtype)) return fail(WKV_ERR_UNSUPPORTED, "%s: unknown input dtype %d", fn, in_dtype);
  if (algo != WKV_ALGO_AUTO && algo != WKV_ALGO_SCAN && algo != WKV_ALGO_CHUNKED)
    return fail(WKV_ERR_UNSUPPORTED, "%s: unknown algorithm %d", fn, algo);
  if (algo == WKV_ALGO_CHUNKED && in_dtype != WKV_BF16)
    return fail(WKV_ERR_UNSUPPORTED, "%s: the chunked algorithm needs bf16 inputs", fn);
  if (algo == WKV_ALGO_CHUNKED && (int64_t)H * N > kChunkedMaxRow)
    return fail(WKV_ERR_UNSUPPORTED, "%s: the chunked algorithm takes at most %d channels per token (H*N=%lld)",
                fn, kChunkedMaxRow, (long long)H * N);
  REQUIRE(B <= kMaxGridY, "%s: B=%d exceeds %d", fn, B, kMaxGridY);
  REQUIRE((int64_t)H * N <= (int64_t)1 << 30, "%s: H*N too large", fn);
  if (T > 0) {
    REQUIRE(r && k && v && w && u && y, "%s: r, k, v, w, u and y must be non-NULL", fn);
    REQUIRE(aligned(r, 16) && aligned(k, 16) && aligned(v, 16) && aligned(y, 16),
            "%s: r, k, v and y must be 16-byte aligned", fn);
    REQUIRE(aligned(w, 4) && aligned(u, 4), "%s: w and u must be 4-byte aligned", fn);
  }
  if (state_in) {
    REQUIRE(aligned(state_in, 16), "%s: state_in must be 16-byte aligned", fn);
    REQUIRE(n_state >= 1, "%s: n_state must be >= 1 when state_in is given (got %d)", fn, n_state);
    if (!state_map)
      REQUIRE(n_state == 1 || n_state == B, "%s: without state_map, n_state must be 1 or B (got %d, B=%d)", fn,
              n_state, B);
    else
      REQUIRE(aligned(state_map, 4), "%s: state_map must be 4-byte aligned", fn);
  } else {
    REQUIRE(!state_map, "%s: state_map given without state_in", fn);
  }
  if (state_out) {
    REQUIRE(aligned(state_out, 16), "%s: state_out must be 16-byte aligned", fn);
    if (state_out == state_in)
      REQUIRE(!state_map && n_state == B, "%s: in-place state needs state_map == NULL and n_state == B", fn);
  }
  return WKV_OK;
}

// Scratch of wkv6_backward_noalloc: each batch row's share of du, [B, H*N] fp32.
// Every GPU the library runs on holds its own copy until the process ends.
constexpr long kNoAllocScratchFloats = 1l << 20;  // 4 MiB: B * H * N <= 1,048,576
static __device__ __align__(256) float scratch[kNoAllocScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

// Device address of `scratch` on the current device, looked up once per device.  The
// array's name in host code is only a host-side stand-in, so kernels get this address.
wkv_status scratch_address(const char *fn, float **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(WKV_ERR_DEVICE, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(WKV_ERR_UNSUPPORTED, "%s: device %d is beyond the %d devices the scratch table holds", fn, dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(WKV_ERR_DEVICE, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", fn, dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<float *>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return WKV_OK;
}

// Validation and launch of the v6 backward, with du_rows from the caller or the scratch.
wkv_status backward6(const char *fn, int B, int T, int H, int N, const void *r, const void *k, const void *v,
                     const void *w, wkv_dtype in_dtype, const float *u, const float *dy, const float *state_in,
                     const int32_t *state_map, int n_state, const float *state_final, const float *d_state_out,
                     float *dr, float *dk, float *dv, float *dw, float *du, float *du_rows, bool use_scratch,
                     float *d_state_in, const float *chunk_states, wkv_algo algo, int32_t *dev_status,
                     void *stream) {
  wkv_status st = check_dense56(fn, B, T, H, N, r, k, v, w, in_dtype, u, dr, state_in, state_map, n_state,
                                nullptr, algo);
  if (st != WKV_OK) return st;
  if (T > 0) {
    REQUIRE(dy && dk && dv && dw, "%s: dy, dk, dv and dw must be non-NULL", fn);
    REQUIRE(aligned(dy, 4) && aligned(dk, 16) && aligned(dv, 16) && aligned(dw, 4),
            "%s: dk and dv must be 16-byte aligned, dy and dw 4-byte aligned", fn);
  }
  if (use_scratch) {
    REQUIRE(u && du, "%s: u and du must be non-NULL", fn);
    REQUIRE(aligned(du, 4), "%s: du must be 4-byte aligned", fn);
    REQUIRE((int64_t)B * H * N <= kNoAllocScratchFloats,
            "%s: B*H*N = %lld exceeds the library's scratch of %ld floats (use wkv6_backward with a du_rows "
            "workspace)", fn, (long long)B * H * N, kNoAllocScratchFloats);
  } else {
    REQUIRE(u && du && du_rows, "%s: u, du and du_rows must be non-NULL", fn);
    REQUIRE(aligned(du, 4) && aligned(du_rows, 4), "%s: du and du_rows must be 4-byte aligned", fn);
  }
  REQUIRE(!d_state_in || aligned(d_state_in, 4), "%s: d_state_in must be 4-byte aligned", fn);
  if (d_state_out) {
    REQUIRE(state_final, "%s: state_final (the forward call's final state) is needed with d_state_out", fn);
    REQUIRE(aligned(d_state_out, 4) && aligned(state_final, 4), "%s: d_state_out and state_final misaligned", fn);
  }
  REQUIRE(!dev_status || aligned(dev_status, 4), "%s: dev_status must be 4-byte aligned", fn);
  if (use_scratch) {
    st = scratch_address(fn, &du_rows);
    if (st != WKV_OK) return st;
  }
  wkv::BwdParams p{};
  p.B = B; p.T = T; p.H = H;
  p.r = r; p.k = k; p.v = v; p.w = w;
  p.u = u; p.dy = dy;
  p.state_in = state_in; p.state_map = state_map; p.n_state = n_state;
  p.state_final = state_final; p.d_state_out = d_state_out;
  p.dr = dr; p.dk = dk; p.dv = dv; p.dw = dw; p.du = du; p.du_rows = du_rows; p.d_state_in = d_state_in;
  p.dev_status = dev_status;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  // Chunked passes (AUTO: bf16 inputs, T >= 64), then the sweeps for the units they leave
  // (decays beyond the chunked form's exponent range, rejected state_map rows).
  const bool chunked = T > 0 && in_dtype == WKV_BF16 && (int64_t)H * N <= kChunkedMaxRow &&
                       (algo == WKV_ALGO_CHUNKED || (algo == WKV_ALGO_AUTO && T >= kChunk));
  if (chunked && T > kChunk && chunk_states) {
    REQUIRE(aligned(chunk_states, 16), "%s: chunk_states must be 16-byte aligned", fn);
    p.chunk_states = chunk_states;  // the forward's saved states: no state pass
  }
  if (chunked) {
    const hipError_t e = wkv::launch_wkv6_backward_chunked(p, hs);
    if (e != hipSuccess) return launched(e, fn);
    p.marked_only = 1;
  }
  return launched(wkv::launch_wkv6_backward(p, in_dtype == WKV_BF16, hs), fn);
}

}  // namespace

extern "C" {

int wkv_abi_version(void) { return WKV_ABI_VERSION; }

const char *wkv_last_error(void) { return g_last_error; }

const char *wkv_status_string(wkv_status s) {
  switch (s) {
    case WKV_OK: return "ok";
    case WKV_ERR_INVALID_ARG: return "invalid argument";
    case WKV_ERR_UNSUPPORTED: return "unsupported";
    case WKV_ERR_DEVICE: return "device error";
    default: return "unknown status";
  }
}

wkv_algo wkv_resolve_algo(int version, int B, int T, int H, int N, wkv_dtype in_dtype, wkv_algo requested) {
  (void)B; (void)H; (void)N;
  if (requested == WKV_ALGO_SCAN || requested == WKV_ALGO_CHUNKED) return requested;
  if ((version != 5 && version != 6 && version != 7) || in_dtype != WKV_BF16) return WKV_ALGO_SCAN;
  if ((int64_t)H * N > kChunkedMaxRow) return WKV_ALGO_SCAN;
  // Chunks only pay off once a row holds at least one full chunk.
  return T >= kChunk ? WKV_ALGO_CHUNKED : WKV_ALGO_SCAN;
}

wkv_status wkv4_forward_ex(int B, int T, int C, const float *time_decay, const float *time_first, const void *k,
                           const void *v, const void *r, wkv_dtype in_dtype, void *y, wkv_dtype out_dtype,
                           const float *state_in, float *state_out, void *stream) {
  const char *fn = "wkv4_forward";
  REQUIRE(B >= 1 && T >= 0 && C >= 1, "%s: need B >= 1, T >= 0, C >= 1 (got B=%d T=%d C=%d)", fn, B, T, C);
  if (!dtype_ok(in_dtype)) return fail(WKV_ERR_UNSUPPORTED, "%s: unknown input dtype %d", fn, in_dtype);
  if (!dtype_ok(out_dtype)) return fail(WKV_ERR_UNSUPPORTED, "%s: unknown output dtype %d", fn, out_dtype);
  REQUIRE(B <= kMaxGridY, "%s: B=%d exceeds %d", fn, B, kMaxGridY);
  REQUIRE(time_decay && time_first, "%s: time_decay and time_first must be non-NULL", fn);
  REQUIRE(aligned(time_decay, 4) && aligned(time_first, 4), "%s: time_decay/time_first misaligned", fn);
  if (T > 0) {
    REQUIRE(k && v && y, "%s: k, v and y must be non-NULL", fn);
    REQUIRE(aligned(k, 16) && aligned(v, 16) && aligned(y, 16) && (!r || aligned(r, 16)),
            "%s: k, v, r and y must be 16-byte aligned", fn);
  }
  REQUIRE(!state_in || aligned(state_in, 16), "%s: state_in must be 16-byte aligned", fn);
  REQUIRE(!state_out || aligned(state_out, 16), "%s: state_out must be 16-byte aligned", fn);
  if (T == 0 && (!state_out || state_out == state_in)) return ok();
  wkv::V4Params p{B, T, C, time_decay, time_first, k, v, r, y, out_dtype == WKV_BF16, state_in, state_out};
  return launched(wkv::launch_wkv4(p, in_dtype == WKV_BF16, static_cast<hipStream_t>(stream)), fn);
}

wkv_status wkv4_forward(int B, int T, int C, const float *time_decay, const float *time_first, const void *k,
                        const void *v, const void *r, wkv_dtype in_dtype, float *y, const float *state_in,
                        float *state_out, void *stream) {
  return wkv4_forward_ex(B, T, C, time_decay, time_first, k, v, r, in_dtype, y, WKV_F32, state_in, state_out,
                         stream);
}

static wkv_status dense56(int version, int B, int T, int H, int N, const void *r, const void *k, const void *v,
                          const void *w, wkv_dtype in_dtype, wkv_layout layout, const float *u, void *y,
                          wkv_dtype out_dtype, const float *state_in, const int32_t *state_map, int n_state,
                          float *state_out, wkv_algo algo, int32_t *dev_status, void *stream) {
  const char *fn = version == 5 ? "wkv5_forward" : "wkv6_forward";
  wkv_status st = check_dense56(fn, B, T, H, N, r, k, v, w, in_dtype, u, y, state_in, state_map, n_state,
                                state_out, algo);
  if (st != WKV_OK) return st;
  if (!dtype_ok(out_dtype)) return fail(WKV_ERR_UNSUPPORTED, "%s: unknown output dtype %d", fn, out_dtype);
  if (layout != WKV_LAYOUT_BTHN && layout != WKV_LAYOUT_BHTN)
    return fail(WKV_ERR_UNSUPPORTED, "%s: unknown layout %d", fn, layout);
  REQUIRE(!dev_status || aligned(dev_status, 4), "%s: dev_status must be 4-byte aligned", fn);
  if (T == 0 && !state_out) return ok();
  wkv::ScanParams p{};
  p.units = B;
  p.T = T;
  p.H = H;
  p.r = r; p.k = k; p.v = v; p.w = w;
  p.u = u;
  p.y = y;
  p.y_bf16 = out_dtype == WKV_BF16;
  const long C = (long)H * N;
  if (layout == WKV_LAYOUT_BTHN) {
    p.row_stride = (long)T * C; p.tok_stride = C; p.head_stride = N;
  } else {
    p.row_stride = (long)H * T * N; p.tok_stride = N; p.head_stride = (long)T * N;
  }
  p.state_in = state_in;
  p.state_map = state_map;
  p.n_state = n_state;
  p.state_out = state_out;
  p.dev_status = dev_status;
  const bool bf16 = in_dtype == WKV_BF16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const wkv_algo a = wkv_resolve_algo(version, B, T, H, N, in_dtype, algo);
  if (a == WKV_ALGO_CHUNKED && T > 0)
    return launched(wkv::launch_wkv56_chunked(p, version == 6, bf16, s), fn);
  return launched(wkv::launch_wkv56_scan(p, version == 6, bf16, false, s), fn);
}

wkv_status wkv5_forward_ex(int B, int T, int H, int N, const void *r, const void *k, const void *v,
                           wkv_dtype in_dtype, wkv_layout layout, const float *w, const float *u, void *y,
                           wkv_dtype out_dtype, const float *state_in, const int32_t *state_map, int n_state,
                           float *state_out, wkv_algo algo, int32_t *dev_status, void *stream) {
  return dense56(5, B, T, H, N, r, k, v, w, in_dtype, layout, u, y, out_dtype, state_in, state_map, n_state,
                 state_out, algo, dev_status, stream);
}

wkv_status wkv5_forward(int B, int T, int H, int N, const void *r, const void *k, const void *v, wkv_dtype in_dtype,
                        const float *w, const float *u, float *y, const float *state_in, const int32_t *state_map,
                        int n_state, float *state_out, wkv_algo algo, int32_t *dev_status, void *stream) {
  return dense56(5, B, T, H, N, r, k, v, w, in_dtype, WKV_LAYOUT_BTHN, u, y, WKV_F32, state_in, state_map,
                 n_state, state_out, algo, dev_status, stream);
}

wkv_status wkv6_forward_ex(int B, int T, int H, int N, const void *r, const void *k, const void *v, const void *w,
                           wkv_dtype in_dtype, wkv_layout layout, const float *u, void *y, wkv_dtype out_dtype,
                           const float *state_in, const int32_t *state_map, int n_state, float *state_out,
                           wkv_algo algo, int32_t *dev_status, void *stream) {
  return dense56(6, B, T, H, N, r, k, v, w, in_dtype, layout, u, y, out_dtype, state_in, state_map, n_state,
                 state_out, algo, dev_status, stream);
}

wkv_status wkv6_forward(int B, int T, int H, int N, const void *r, const void *k, const void *v, const void *w,
                        wkv_dtype in_dtype, const float *u, float *y, const float *state_in,
                        const int32_t *state_map, int n_state, float *state_out, wkv_algo algo,
                        int32_t *dev_status, void *stream) {
  return dense56(6, B, T, H, N, r, k, v, w, in_dtype, WKV_LAYOUT_BTHN, u, y, WKV_F32, state_in, state_map,
                 n_state, state_out, algo, dev_status, stream);
}

wkv_status wkv6_forward_train(int B, int T, int H, int N, const void *r, const void *k, const void *v,
                              const void *w, wkv_dtype in_dtype, const float *u, void *y, wkv_dtype out_dtype,
                              const float *state_in, const int32_t *state_map, int n_state, float *state_out,
                              float *chunk_states, int32_t *dev_status, void *stream) {
  const char *fn = "wkv6_forward_train";
  wkv_status st = check_dense56(fn, B, T, H, N, r, k, v, w, in_dtype, u, y, state_in, state_map, n_state,
                                state_out, WKV_ALGO_CHUNKED);
  if (st != WKV_OK) return st;
  if (!dtype_ok(out_dtype)) return fail(WKV_ERR_UNSUPPORTED, "%s: unknown output dtype %d", fn, out_dtype);
  REQUIRE(!dev_status || aligned(dev_status, 4), "%s: dev_status must be 4-byte aligned", fn);
  if (T > kChunk)
    REQUIRE(chunk_states && aligned(chunk_states, 16),
            "%s: chunk_states must be a non-NULL, 16-byte aligned device array (T > %d)", fn, kChunk);
  if (T == 0)  // no tokens, no chunk states: the plain forward (state_out from state_in)
    return dense56(6, B, T, H, N, r, k, v, w, in_dtype, WKV_LAYOUT_BTHN, u, y, out_dtype, state_in, state_map,
                   n_state, state_out, WKV_ALGO_AUTO, dev_status, stream);
  wkv::ScanParams p{};
  p.units = B;
  p.T = T;
  p.H = H;
  p.r = r; p.k = k; p.v = v; p.w = w;
  p.u = u;
  p.y = y;
  p.y_bf16 = out_dtype == WKV_BF16;
  const long C = (long)H * N;
  p.row_stride = (long)T * C; p.tok_stride = C; p.head_stride = N;
  p.state_in = state_in;
  p.state_map = state_map;
  p.n_state = n_state;
  p.state_out = state_out;
  p.dev_status = dev_status;
  p.chunk_states = chunk_states;
  return launched(wkv::launch_wkv6_chunked_save(p, static_cast<hipStream_t>(stream)), fn);
}

wkv_status wkv7_forward_ex(int B, int T, int H, int N, const void *r, const void *w, const void *k, const void *v,
                           const void *a, const void *b, wkv_dtype in_dtype, wkv_layout layout, void *y,
                           wkv_dtype out_dtype, const float *state_in, const int32_t *state_map, int n_state,
                           float *state_out, wkv_algo algo, int32_t *dev_status, void *stream) {
  const char *fn = "wkv7_forward";
  if (algo != WKV_ALGO_AUTO && algo != WKV_ALGO_SCAN && algo != WKV_ALGO_CHUNKED)
    return fail(WKV_ERR_UNSUPPORTED, "%s: unknown algorithm %d", fn, algo);
  if (algo == WKV_ALGO_CHUNKED && in_dtype != WKV_BF16)
    return fail(WKV_ERR_UNSUPPORTED, "%s: the chunked algorithm needs bf16 inputs", fn);
  if (algo == WKV_ALGO_CHUNKED && (int64_t)H * N > kChunkedMaxRow)
    return fail(WKV_ERR_UNSUPPORTED, "%s: the chunked algorithm takes at most %d channels per token (H*N=%lld)",
                fn, kChunkedMaxRow, (long long)H * N);
  REQUIRE(B >= 1 && T >= 0 && H >= 1, "%s: need B >= 1, T >= 0, H >= 1 (got B=%d T=%d H=%d)", fn, B, T, H);
  if (N != wkv::kHeadSize) return fail(WKV_ERR_UNSUPPORTED, "%s: head size N=%d is not supported (only 64)", fn, N);
  if (!dtype_ok(in_dtype)) return fail(WKV_ERR_UNSUPPORTED, "%s: unknown input dtype %d", fn, in_dtype);
  if (!dtype_ok(out_dtype)) return fail(WKV_ERR_UNSUPPORTED, "%s: unknown output dtype %d", fn, out_dtype);
  if (layout != WKV_LAYOUT_BTHN && layout != WKV_LAYOUT_BHTN)
    return fail(WKV_ERR_UNSUPPORTED, "%s: unknown layout %d", fn, layout);
  REQUIRE(B <= kMaxGridY, "%s: B=%d exceeds %d", fn, B, kMaxGridY);
  REQUIRE((int64_t)H * N <= (int64_t)1 << 30, "%s: H*N too large", fn);
  if (T > 0) {
    REQUIRE(r && w && k && v && a && b && y, "%s: r, w, k, v, a, b and y must be non-NULL", fn);
    REQUIRE(aligned(r, 16) && aligned(w, 16) && aligned(k, 16) && aligned(v, 16) && aligned(a, 16) &&
                aligned(b, 16) && aligned(y, 16),
            "%s: r, w, k, v, a, b and y must be 16-byte aligned", fn);
  }
  if (state_in) {
    REQUIRE(aligned(state_in, 16), "%s: state_in must be 16-byte aligned", fn);
    REQUIRE(n_state >= 1, "%s: n_state must be >= 1 when state_in is given (got %d)", fn, n_state);
    if (!state_map)
      REQUIRE(n_state == 1 || n_state == B, "%s: without state_map, n_state must be 1 or B (got %d, B=%d)", fn,
              n_state, B);
    else
      REQUIRE(aligned(state_map, 4), "%s: state_map must be 4-byte aligned", fn);
  } else {
    REQUIRE(!state_map, "%s: state_map given without state_in", fn);
  }
  if (state_out) {
    REQUIRE(aligned(state_out, 16), "%s: state_out must be 16-byte aligned", fn);
    if (state_out == state_in)
      REQUIRE(!state_map && n_state == B, "%s: in-place state needs state_map == NULL and n_state == B", fn);
  }
  REQUIRE(!dev_status || aligned(dev_status, 4), "%s: dev_status must be 4-byte aligned", fn);
  if (T == 0 && !state_out) return ok();
  wkv::V7Params p{};
  p.B = B; p.T = T; p.H = H;
  p.r = r; p.w = w; p.k = k; p.v = v; p.a = a; p.b = b;
  p.y = y;
  p.y_bf16 = out_dtype == WKV_BF16;
  if (layout == WKV_LAYOUT_BTHN) {
    p.row_stride = (long)T * H * N; p.tok_stride = (long)H * N; p.head_stride = N;
  } else {
    p.row_stride = (long)H * T * N; p.tok_stride = N; p.head_stride = (long)T * N;
  }
  p.state_in = state_in; p.state_map = state_map; p.n_state = n_state; p.state_out = state_out;
  p.dev_status = dev_status;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (T > 0 && wkv_resolve_algo(7, B, T, H, N, in_dtype, algo) == WKV_ALGO_CHUNKED)
    return launched(wkv::launch_wkv7_chunked(p, in_dtype == WKV_BF16, s), fn);
  return launched(wkv::launch_wkv7_scan(p, in_dtype == WKV_BF16, s), fn);
}

wkv_status wkv7_forward(int B, int T, int H, int N, const void *r, const void *w, const void *k, const void *v,
                        const void *a, const void *b, wkv_dtype in_dtype, wkv_layout layout, void *y,
                        wkv_dtype out_dtype, const float *state_in, const int32_t *state_map, int n_state,
                        float *state_out, int32_t *dev_status, void *stream) {
  return wkv7_forward_ex(B, T, H, N, r, w, k, v, a, b, in_dtype, layout, y, out_dtype, state_in, state_map,
                         n_state, state_out, WKV_ALGO_AUTO, dev_status, stream);
}

wkv_status wkv6_backward(int B, int T, int H, int N, const void *r, const void *k, const void *v, const void *w,
                         wkv_dtype in_dtype, const float *u, const float *dy, const float *state_in,
                         const int32_t *state_map, int n_state, const float *state_final,
                         const float *d_state_out, float *dr, float *dk, float *dv, float *dw, float *du,
                         float *du_rows, float *d_state_in, int32_t *dev_status, void *stream) {
  return backward6("wkv6_backward", B, T, H, N, r, k, v, w, in_dtype, u, dy, state_in, state_map, n_state,
                   state_final, d_state_out, dr, dk, dv, dw, du, du_rows, false, d_state_in, nullptr,
                   WKV_ALGO_AUTO, dev_status, stream);
}

wkv_status wkv6_backward_ex(int B, int T, int H, int N, const void *r, const void *k, const void *v,
                            const void *w, wkv_dtype in_dtype, const float *u, const float *dy,
                            const float *state_in, const int32_t *state_map, int n_state,
                            const float *state_final, const float *d_state_out, float *dr, float *dk, float *dv,
                            float *dw, float *du, float *du_rows, float *d_state_in,
                            const float *chunk_states, wkv_algo algo, int32_t *dev_status, void *stream) {
  return backward6("wkv6_backward_ex", B, T, H, N, r, k, v, w, in_dtype, u, dy, state_in, state_map, n_state,
                   state_final, d_state_out, dr, dk, dv, dw, du, du_rows, false, d_state_in, chunk_states, algo,
                   dev_status, stream);
}

wkv_status wkv6_backward_noalloc(int B, int T, int H, int N, const void *r, const void *k, const void *v,
                                 const void *w, wkv_dtype in_dtype, const float *u, const float *dy,
                                 const float *state_in, const int32_t *state_map, int n_state,
                                 const float *state_final, const float *d_state_out, float *dr, float *dk,
                                 float *dv, float *dw, float *du, float *d_state_in, int32_t *dev_status,
                                 void *stream) {
  return backward6("wkv6_backward_noalloc", B, T, H, N, r, k, v, w, in_dtype, u, dy, state_in, state_map,
                   n_state, state_final, d_state_out, dr, dk, dv, dw, du, nullptr, true, d_state_in, nullptr,
                   WKV_ALGO_AUTO, dev_status, stream);
}

wkv_status wkv6_forward_varlen_ex(int num_slots, int H, int N, const int32_t *lengths, int max_len,
                                  int total_tokens, const void *r, const void *k, const void *v, const void *w,
                                  wkv_dtype in_dtype, const float *u, void *y, wkv_dtype out_dtype,
                                  const float *state_in, float *state_out, const int32_t *state_map, int n_state,
                                  int32_t *dev_status, void *stream) {
  const char *fn = "wkv6_forward_varlen";
  REQUIRE(num_slots >= 0 && H >= 1 && max_len >= 0 && total_tokens >= 0,
          "%s: need num_slots >= 0, H >= 1, max_len >= 0, total_tokens >= 0", fn);
  if (N != wkv::kHeadSize) return fail(WKV_ERR_UNSUPPORTED, "%s: head size N=%d is not supported (only 64)", fn, N);
  if (!dtype_ok(in_dtype)) return fail(WKV_ERR_UNSUPPORTED, "%s: unknown input dtype %d", fn, in_dtype);
  if (!dtype_ok(out_dtype)) return fail(WKV_ERR_UNSUPPORTED, "%s: unknown output dtype %d", fn, out_dtype);
  REQUIRE(num_slots <= kMaxGridY, "%s: num_slots=%d exceeds %d", fn, num_slots, kMaxGridY);
  if (num_slots == 0) return ok();
  REQUIRE(lengths && aligned(lengths, 4), "%s: lengths must be a non-NULL, 4-byte aligned device array", fn);
  REQUIRE(u && aligned(u, 4), "%s: u must be non-NULL and 4-byte aligned", fn);
  REQUIRE(state_in && state_out, "%s: state_in and state_out must be non-NULL", fn);
  REQUIRE(aligned(state_in, 16) && aligned(state_out, 16), "%s: states must be 16-byte aligned", fn);
  REQUIRE(n_state >= 1, "%s: n_state must be >= 1", fn);
  if (!state_map)
    REQUIRE(n_state >= num_slots, "%s: without state_map, n_state (%d) must be >= num_slots (%d)", fn, n_state,
            num_slots);
  else
    REQUIRE(aligned(state_map, 4), "%s: state_map must be 4-byte aligned", fn);
  if (total_tokens > 0) {
    REQUIRE(r && k && v && w && y, "%s: r, k, v, w and y must be non-NULL", fn);
    REQUIRE(aligned(r, 16) && aligned(k, 16) && aligned(v, 16) && aligned(w, 16) && aligned(y, 16),
            "%s: r, k, v, w and y must be 16-byte aligned", fn);
  }
  REQUIRE(!dev_status || aligned(dev_status, 4), "%s: dev_status must be 4-byte aligned", fn);
  wkv::ScanParams p{};
  p.units = num_slots;
  p.H = H;
  p.r = r; p.k = k; p.v = v; p.w = w;
  p.u = u;
  p.y = y;
  p.y_bf16 = out_dtype == WKV_BF16;
  p.row_stride = 0; p.tok_stride = (long)H * N; p.head_stride = N;  // packed [total_tokens, H*N]
  p.state_in = state_in;
  p.state_map = state_map;
  p.n_state = n_state;
  p.state_out = state_out;
  p.dev_status = dev_status;
  p.lengths = lengths;
  p.max_len = max_len;
  p.total_tokens = total_tokens;
  const bool bf16 = in_dtype == WKV_BF16;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (max_len <= wkv::kShortMax) return launched(wkv::launch_wkv6_varlen_short(p, bf16, s), fn);
  return launched(wkv::launch_wkv56_scan(p, true, bf16, true, s), fn);
}

wkv_status wkv6_forward_varlen(int num_slots, int H, int N, const int32_t *lengths, int max_len, int total_tokens,
                               const void *r, const void *k, const void *v, const void *w, wkv_dtype in_dtype,
                               const float *u, float *y, const float *state_in, float *state_out,
                               const int32_t *state_map, int n_state, int32_t *dev_status, void *stream) {
  return wkv6_forward_varlen_ex(num_slots, H, N, lengths, max_len, total_tokens, r, k, v, w, in_dtype, u, y,
                                WKV_F32, state_in, state_out, state_map, n_state, dev_status, stream);
}

wkv_status wkv_schedule_round_robin(int num_slots, const int32_t *remaining, int budget, int32_t *take,
                                    int32_t *total) {
  const char *fn = "wkv_schedule_round_robin";
  REQUIRE(num_slots >= 0 && budget >= 0, "%s: need num_slots >= 0 and budget >= 0", fn);
  REQUIRE(num_slots == 0 || (remaining && take), "%s: remaining and take must be non-NULL", fn);
  for (int s = 0; s < num_slots; ++s) {
    REQUIRE(remaining[s] >= 0, "%s: remaining[%d] = %d is negative", fn, s, remaining[s]);
    take[s] = 0;
  }
  // Whole rounds first: every slot with tokens left gets one per round.
  int64_t left = budget;
  int64_t given = 0;
  while (left > 0) {
    int active = 0;
    int64_t min_rem = INT64_MAX;
    for (int s = 0; s < num_slots; ++s) {
      const int64_t rem = (int64_t)remaining[s] - take[s];
      if (rem > 0) {
        ++active;
        if (rem < min_rem) min_rem = rem;
      }
    }
    if (active == 0) break;
    const int64_t rounds = left / active < min_rem ? left / active : min_rem;
    if (rounds > 0) {
      for (int s = 0; s < num_slots; ++s)
        if ((int64_t)remaining[s] - take[s] > 0) take[s] += (int32_t)rounds;
      left -= rounds * active;
      given += rounds * active;
      continue;
    }
    // A partial round: the first `left` active slots in slot order get one more.
    for (int s = 0; s < num_slots && left > 0; ++s)
      if ((int64_t)remaining[s] - take[s] > 0) {
        ++take[s];
        --left;
        ++given;
      }
  }
  if (total) *total = (int32_t)given;
  return ok();
}

}  // extern "C"
