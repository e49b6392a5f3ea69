"""MI355X (gfx950) RWKV WKV time-mixing kernels (v4, v5, v6 and the v6 backward, v7) — thin PyTorch binding.

Every function here only checks and marshals arguments (shapes, dtypes,
device pointers, the current HIP stream) and calls the C ABI of libwkv.so
(include/wkv.h).  All arithmetic runs in the library's HIP kernels; there is
no CPU or PyTorch fallback, and importing the package fails if the library
has not been built.

Tensors are row-major and contiguous, token arrays [B, T, C] with C = H*N
(varlen: packed [total_tokens, C]), or head-first [B, H, T, N] for v5 / v6
with ``head_first=True``; inputs are torch.bfloat16 or torch.float32; y is
float32, or bfloat16 with ``out_dtype=torch.bfloat16`` (the fp32 result
rounded to nearest even); states are float32.  Calls are asynchronous on
torch's current stream.
"""
from __future__ import annotations

import ctypes

import torch

from . import _native
from ._native import (WKV_ALGO_AUTO, WKV_ALGO_CHUNKED, WKV_ALGO_SCAN, WKV_DEV_BAD_LENGTH,  # noqa: F401
                      WKV_DEV_BAD_STATE_MAP, WKV_DEV_DUPLICATE_ROW,
                      WKV_DEV_TOKEN_OVERFLOW, WkvError, check)

_lib = _native.load()

_ALGOS = {"auto": WKV_ALGO_AUTO, "scan": WKV_ALGO_SCAN, "chunked": WKV_ALGO_CHUNKED}

__all__ = ["wkv4_forward", "wkv5_forward", "wkv6_forward", "wkv6_forward_train", "wkv6_backward", "wkv6_forward_varlen", "varlen_plan", "VarlenPlan",
           "wkv7_forward", "wkv7_plan", "Wkv7Plan", "schedule_round_robin", "resolve_algo", "WkvError", "library"]


def library():
    """The loaded ctypes handle of libwkv.so."""
    return _lib


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return _native.WKV_BF16
    if t.dtype == torch.float32:
        return _native.WKV_F32
    raise TypeError(f"unsupported input dtype {t.dtype} (bfloat16 or float32)")


def _dev(t, name, dtype=None, shape=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(ref):
    return ctypes.c_void_p(torch.cuda.current_stream(ref.device).cuda_stream)


def _out_code(y, out_dtype):
    """Output dtype code: that of a given y, else out_dtype (float32 or bfloat16)."""
    dt = y.dtype if y is not None else out_dtype
    if dt == torch.float32:
        return _native.WKV_F32, dt
    if dt == torch.bfloat16:
        return _native.WKV_BF16, dt
    raise TypeError(f"unsupported output dtype {dt} (float32 or bfloat16)")


def _same_dtype(name_tensors):
    dts = {t.dtype for _, t in name_tensors if t is not None}
    if len(dts) != 1:
        raise TypeError("token inputs must share one dtype: " +
                        ", ".join(f"{n}={t.dtype}" for n, t in name_tensors if t is not None))


def wkv4_forward(time_decay, time_first, k, v, r=None, state=None, *, y=None, state_out=None,
                 return_state=True, out_dtype=torch.float32):
    """v4 WKV.  k, v, r: [B, T, C]; time_decay, time_first: [C] fp32; state: [B, 3, C] fp32 (a, b, p).

    Returns ``(y, state_out)`` (``state_out`` None unless ``return_state``); y is
    ``out_dtype`` (float32 or bfloat16) unless given.
    """
    B, T, C = k.shape
    _same_dtype([("k", k), ("v", v), ("r", r)])
    _dev(k, "k", shape=(B, T, C)); _dev(v, "v", shape=(B, T, C)); _dev(r, "r", shape=(B, T, C))
    _dev(time_decay, "time_decay", torch.float32, (C,)); _dev(time_first, "time_first", torch.float32, (C,))
    _dev(state, "state", torch.float32, (B, 3, C))
    oc, odt = _out_code(y, out_dtype)
    if y is None:
        y = torch.empty((B, T, C), dtype=odt, device=k.device)
    _dev(y, "y", odt, (B, T, C))
    if return_state and state_out is None:
        state_out = torch.empty((B, 3, C), dtype=torch.float32, device=k.device)
    _dev(state_out, "state_out", torch.float32, (B, 3, C))
    head = (B, T, C, _ptr(time_decay), _ptr(time_first), _ptr(k), _ptr(v), _ptr(r), _dtype_code(k), _ptr(y))
    tail = (_ptr(state), _ptr(state_out), _stream(k))
    if oc == _native.WKV_F32:
        check(_lib.wkv4_forward(*head, *tail))
    else:
        check(_lib.wkv4_forward_ex(*head, oc, *tail))
    return y, state_out


def _dense56(version, r, k, v, w, u, H, state, state_map, algo, y, state_out, return_state, dev_status,
             head_first=False, out_dtype=torch.float32):
    if head_first:
        if r.dim() != 4 or r.shape[1] != H:
            raise ValueError(f"head-first r must be [B, {H}, T, N], got {tuple(r.shape)}")
        B, _, T, N = r.shape
        C = H * N
        tok_shape = (B, H, T, N)
    else:
        B, T, C = r.shape
        if C % H:
            raise ValueError(f"C={C} is not a multiple of H={H}")
        N = C // H
        tok_shape = (B, T, C)
    _same_dtype([("r", r), ("k", k), ("v", v)] + ([("w", w)] if version == 6 else []))
    for name, t in (("r", r), ("k", k), ("v", v)):
        _dev(t, name, shape=tok_shape)
    if version == 6:
        _dev(w, "w", shape=tok_shape)
    else:
        _dev(w, "w", torch.float32, (C,))
    _dev(u.reshape(-1) if u.dim() == 2 else u, "u", torch.float32, (C,))
    n_state = 0
    if state is not None:
        _dev(state, "state", torch.float32)
        if state.dim() != 4 or tuple(state.shape[1:]) != (H, N, N):
            raise ValueError(f"state must be [n_state, {H}, {N}, {N}], got {tuple(state.shape)}")
        n_state = state.shape[0]
    _dev(state_map, "state_map", torch.int32, (B,))
    oc, odt = _out_code(y, out_dtype)
    if y is None:
        y = torch.empty(tok_shape, dtype=odt, device=r.device)
    _dev(y, "y", odt, tok_shape)
    if return_state and state_out is None:
        state_out = torch.empty((B, H, N, N), dtype=torch.float32, device=r.device)
    _dev(state_out, "state_out", torch.float32, (B, H, N, N))
    _dev(dev_status, "dev_status", torch.int32, (1,))
    a = _ALGOS[algo] if isinstance(algo, str) else int(algo)
    tail = (_ptr(state), _ptr(state_map), n_state, _ptr(state_out), a, _ptr(dev_status), _stream(r))
    toks = (_ptr(r), _ptr(k), _ptr(v)) if version == 5 else (_ptr(r), _ptr(k), _ptr(v), _ptr(w))
    if oc == _native.WKV_F32 and not head_first:
        if version == 5:
            check(_lib.wkv5_forward(B, T, H, N, *toks, _dtype_code(r), _ptr(w), _ptr(u), _ptr(y), *tail))
        else:
            check(_lib.wkv6_forward(B, T, H, N, *toks, _dtype_code(r), _ptr(u), _ptr(y), *tail))
    else:
        layout = _native.WKV_LAYOUT_BHTN if head_first else _native.WKV_LAYOUT_BTHN
        if version == 5:
            check(_lib.wkv5_forward_ex(B, T, H, N, *toks, _dtype_code(r), layout, _ptr(w), _ptr(u), _ptr(y), oc,
                                       *tail))
        else:
            check(_lib.wkv6_forward_ex(B, T, H, N, *toks, _dtype_code(r), layout, _ptr(u), _ptr(y), oc, *tail))
    return y, state_out


def wkv5_forward(r, k, v, w, u, H, state=None, state_map=None, *, algo="auto", y=None, state_out=None,
                 return_state=True, dev_status=None, head_first=False, out_dtype=torch.float32):
    """v5 WKV (static decay).  r, k, v: [B, T, H*N] ([B, H, T, N] with ``head_first``);
    w, u: [H*N] fp32 (w = raw decay parameter).

    ``state``: [n_state, H, N, N] fp32 initial states; ``state_map``: [B] int32.
    Returns ``(y, state_out [B, H, N, N] fp32 or None)``; y has the token layout
    of r and dtype ``out_dtype`` (float32 or bfloat16) unless given.
    """
    return _dense56(5, r, k, v, w, u, H, state, state_map, algo, y, state_out, return_state, dev_status,
                    head_first, out_dtype)


def wkv6_forward(r, k, v, w, u, H, state=None, state_map=None, *, algo="auto", y=None, state_out=None,
                 return_state=True, dev_status=None, head_first=False, out_dtype=torch.float32):
    """v6 WKV (per-token decay).  r, k, v, w: [B, T, H*N] ([B, H, T, N] with ``head_first``), one
    dtype; u: [H*N] or [H, N] fp32.

    Returns ``(y, state_out [B, H, N, N] fp32 or None)``; y has the token layout
    of r and dtype ``out_dtype`` (float32 or bfloat16) unless given.
    """
    return _dense56(6, r, k, v, w, u, H, state, state_map, algo, y, state_out, return_state, dev_status,
                    head_first, out_dtype)



def wkv6_forward_train(r, k, v, w, u, H, state=None, state_map=None, *, y=None, state_out=None,
                       return_state=True, dev_status=None, out_dtype=torch.float32, chunk_states=None):
    """:func:`wkv6_forward` in the chunked form (bf16 [B, T, H*N] inputs) that also saves the
    state at every 64-token chunk boundary for :func:`wkv6_backward`.

    Returns ``(y, state_out or None, chunk_states [B, H, ceil(T/64) - 1, N, N] fp32)``; y and
    state_out are bitwise those of ``wkv6_forward(..., algo="chunked")``.
    """
    B, T, C = r.shape
    if C % H:
        raise ValueError(f"C={C} is not a multiple of H={H}")
    N = C // H
    _same_dtype([("r", r), ("k", k), ("v", v), ("w", w)])
    for name, t in (("r", r), ("k", k), ("v", v), ("w", w)):
        _dev(t, name, shape=(B, T, C))
    _dev(u.reshape(-1) if u.dim() == 2 else u, "u", torch.float32, (C,))
    n_state = 0
    if state is not None:
        _dev(state, "state", torch.float32)
        if state.dim() != 4 or tuple(state.shape[1:]) != (H, N, N):
            raise ValueError(f"state must be [n_state, {H}, {N}, {N}], got {tuple(state.shape)}")
        n_state = state.shape[0]
    _dev(state_map, "state_map", torch.int32, (B,))
    oc, odt = _out_code(y, out_dtype)
    if y is None:
        y = torch.empty((B, T, C), dtype=odt, device=r.device)
    _dev(y, "y", odt, (B, T, C))
    if return_state and state_out is None:
        state_out = torch.empty((B, H, N, N), dtype=torch.float32, device=r.device)
    _dev(state_out, "state_out", torch.float32, (B, H, N, N))
    _dev(dev_status, "dev_status", torch.int32, (1,))
    nsave = max((T + 63) // 64 - 1, 0)
    if chunk_states is None:
        chunk_states = torch.empty((B, H, nsave, N, N), dtype=torch.float32, device=r.device)
    _dev(chunk_states, "chunk_states", torch.float32, (B, H, nsave, N, N))
    check(_lib.wkv6_forward_train(B, T, H, N, _ptr(r), _ptr(k), _ptr(v), _ptr(w), _dtype_code(r), _ptr(u),
                                  _ptr(y), oc, _ptr(state), _ptr(state_map), n_state, _ptr(state_out),
                                  _ptr(chunk_states) if nsave else None, _ptr(dev_status), _stream(r)))
    return y, state_out, chunk_states

def wkv6_backward(r, k, v, w, u, H, dy, state=None, state_map=None, *, state_final=None, d_state=None,
                  return_d_state=True, dev_status=None, library_scratch=False, algo="auto", chunk_states=None):
    """Gradients of :func:`wkv6_forward` (same r, k, v, w, u, H, state, state_map).

    ``dy`` [B, T, H*N] fp32 is the gradient of y; ``d_state`` [B, H, N, N] fp32
    (optional) the gradient of the final state, which then also needs
    ``state_final``, the forward call's final state.  Returns ``(dr, dk, dv,
    dw [B, T, H*N], du [H*N], d_state_in [B, H, N, N] or None)`` in fp32;
    ``d_state_in[b]`` is the gradient with respect to the initial state row b
    started from.  With ``library_scratch`` the call goes to
    ``wkv6_backward_noalloc``, whose du staging is the library's own device
    array (B*H*N <= 1,048,576; calls that overlap on one GPU race) instead of a
    workspace allocated here.  ``algo``: "auto" (chunked on MFMA for bf16 inputs with T >= 64),
    "scan" (three token-sequential sweeps) or "chunked" (bf16 only); the allocation-free call
    takes "auto" only.  ``chunk_states``: the states :func:`wkv6_forward_train` saved for these
    inputs; the chunked algorithm then skips its own pass over k, v and w (the sweeps ignore
    them).
    """
    B, T, C = r.shape
    if C % H:
        raise ValueError(f"C={C} is not a multiple of H={H}")
    N = C // H
    _same_dtype([("r", r), ("k", k), ("v", v), ("w", w)])
    for name, t in (("r", r), ("k", k), ("v", v), ("w", w)):
        _dev(t, name, shape=(B, T, C))
    _dev(u.reshape(-1) if u.dim() == 2 else u, "u", torch.float32, (C,))
    _dev(dy, "dy", torch.float32, (B, T, C))
    n_state = 0
    if state is not None:
        _dev(state, "state", torch.float32)
        if state.dim() != 4 or tuple(state.shape[1:]) != (H, N, N):
            raise ValueError(f"state must be [n_state, {H}, {N}, {N}], got {tuple(state.shape)}")
        n_state = state.shape[0]
    _dev(state_map, "state_map", torch.int32, (B,))
    _dev(d_state, "d_state", torch.float32, (B, H, N, N))
    _dev(state_final, "state_final", torch.float32, (B, H, N, N))
    _dev(dev_status, "dev_status", torch.int32, (1,))
    _dev(chunk_states, "chunk_states", torch.float32, (B, H, max((T + 63) // 64 - 1, 0), N, N))
    f32 = dict(dtype=torch.float32, device=r.device)
    dr, dk, dv, dw = (torch.empty((B, T, C), **f32) for _ in range(4))
    du = torch.empty((C,), **f32)
    d_state_in = torch.empty((B, H, N, N), **f32) if return_d_state else None
    head = (B, T, H, N, _ptr(r), _ptr(k), _ptr(v), _ptr(w), _dtype_code(r), _ptr(u), _ptr(dy),
            _ptr(state), _ptr(state_map), n_state, _ptr(state_final), _ptr(d_state),
            _ptr(dr), _ptr(dk), _ptr(dv), _ptr(dw), _ptr(du))
    a = _ALGOS[algo] if isinstance(algo, str) else int(algo)
    if library_scratch:
        if a != WKV_ALGO_AUTO or chunk_states is not None:
            raise ValueError("the allocation-free backward takes algo='auto' and no chunk_states only")
        check(_lib.wkv6_backward_noalloc(*head, _ptr(d_state_in), _ptr(dev_status), _stream(r)))
    else:
        du_rows = torch.empty((B, C), **f32)
        cs = _ptr(chunk_states) if chunk_states is not None and chunk_states.numel() else None
        check(_lib.wkv6_backward_ex(*head, _ptr(du_rows), _ptr(d_state_in), cs, a, _ptr(dev_status), _stream(r)))
    return dr, dk, dv, dw, du, d_state_in


class Wkv7Plan:
    """A validated, pre-marshalled ``wkv7_forward`` call.

    Calling the plan enqueues the kernel on the stream captured when the plan was made, with
    no per-call Python checks (for decode loops that repeat the same call on the same
    buffers), and returns ``(y, state_out)``.
    """

    def __init__(self, fn, args, y, state_out, tensors):
        self._fn = fn
        self._args = args
        self._tensors = tensors  # the plan holds raw pointers: keep their tensors alive
        self.y = y
        self.state_out = state_out

    def __call__(self):
        check(self._fn(*self._args))
        return self.y, self.state_out


def wkv7_plan(r, w, k, v, a, b, H, state=None, state_map=None, *, y=None, state_out=None, return_state=True,
              dev_status=None, out_dtype=torch.float32, head_first=False, algo="auto"):
    """Validate and marshal a v7 call once; see :func:`wkv7_forward` for the arguments."""
    if head_first:
        if r.dim() != 4 or r.shape[1] != H:
            raise ValueError(f"head-first r must be [B, {H}, T, N], got {tuple(r.shape)}")
        B, _, T, N = r.shape
        C = H * N
        tok_shape = (B, H, T, N)
    else:
        B, T, C = r.shape
        if C % H:
            raise ValueError(f"C={C} is not a multiple of H={H}")
        N = C // H
        tok_shape = (B, T, C)
    toks = [("r", r), ("w", w), ("k", k), ("v", v), ("a", a), ("b", b)]
    _same_dtype(toks)
    for name, t in toks:
        _dev(t, name, shape=tok_shape)
    n_state = 0
    if state is not None:
        _dev(state, "state", torch.float32)
        if state.dim() != 4 or tuple(state.shape[1:]) != (H, N, N):
            raise ValueError(f"state must be [n_state, {H}, {N}, {N}], got {tuple(state.shape)}")
        n_state = state.shape[0]
    _dev(state_map, "state_map", torch.int32, (B,))
    oc, odt = _out_code(y, out_dtype)
    if y is None:
        y = torch.empty(tok_shape, dtype=odt, device=r.device)
    _dev(y, "y", odt, tok_shape)
    if return_state and state_out is None:
        state_out = torch.empty((B, H, N, N), dtype=torch.float32, device=r.device)
    _dev(state_out, "state_out", torch.float32, (B, H, N, N))
    _dev(dev_status, "dev_status", torch.int32, (1,))
    layout = _native.WKV_LAYOUT_BHTN if head_first else _native.WKV_LAYOUT_BTHN
    args = (B, T, H, N, *(_ptr(t) for _, t in toks), _dtype_code(r), layout, _ptr(y), oc,
            _ptr(state), _ptr(state_map), n_state, _ptr(state_out), _ALGOS[algo], _ptr(dev_status), _stream(r))
    return Wkv7Plan(_lib.wkv7_forward_ex, args, y, state_out,
                    tuple(t for _, t in toks) + (y, state, state_map, state_out, dev_status))


def wkv7_forward(r, w, k, v, a, b, H, state=None, state_map=None, *, y=None, state_out=None, return_state=True,
                 dev_status=None, out_dtype=torch.float32, head_first=False, algo="auto"):
    """v7 generalized delta rule.  r, w, k, v, a, b: [B, T, H*N] ([B, H, T, N] with ``head_first``),
    one dtype; decay exp(-exp(w)).

    ``state``: [n_state, H, N, N] fp32 initial states h[key][value]; ``state_map``: [B] int32.
    ``algo``: "auto" (chunked for bf16 inputs with T >= 64), "scan" or "chunked".
    Returns ``(y, state_out [B, H, N, N] fp32 or None)``; y has the token layout of r and dtype
    ``out_dtype`` unless given.
    """
    return wkv7_plan(r, w, k, v, a, b, H, state, state_map, y=y, state_out=state_out, return_state=return_state,
                     dev_status=dev_status, out_dtype=out_dtype, head_first=head_first, algo=algo)()


class VarlenPlan:
    """A validated, pre-marshalled ``wkv6_forward_varlen`` call.

    Calling the plan enqueues the kernel on the stream captured when the plan
    was made, with no per-call Python checks (for serving loops that repeat
    the same call on the same buffers).  ``y`` is the output tensor.
    """

    def __init__(self, fn, args, y, tensors):
        self._fn = fn
        self._args = args
        self._tensors = tensors  # the plan holds raw pointers: keep their tensors alive
        self.y = y

    def __call__(self):
        check(self._fn(*self._args))
        return self.y


def varlen_plan(lengths, r, k, v, w, u, H, state, *, max_len, state_out=None, state_map=None, y=None,
                dev_status=None, out_dtype=torch.float32):
    """Validate and marshal a varlen call once; see :func:`wkv6_forward_varlen` for the arguments."""
    S = lengths.shape[0]
    total, C = r.shape
    if C % H:
        raise ValueError(f"C={C} is not a multiple of H={H}")
    N = C // H
    _dev(lengths, "lengths", torch.int32, (S,))
    _same_dtype([("r", r), ("k", k), ("v", v), ("w", w)])
    for name, t in (("r", r), ("k", k), ("v", v), ("w", w)):
        _dev(t, name, shape=(total, C))
    _dev(u.reshape(-1) if u.dim() == 2 else u, "u", torch.float32, (C,))
    _dev(state, "state", torch.float32)
    if state.dim() != 4 or tuple(state.shape[1:]) != (H, N, N):
        raise ValueError(f"state must be [n_state, {H}, {N}, {N}], got {tuple(state.shape)}")
    if state_out is None:
        state_out = state
    _dev(state_out, "state_out", torch.float32, tuple(state.shape))
    _dev(state_map, "state_map", torch.int32, (S,))
    oc, odt = _out_code(y, out_dtype)
    if y is None:
        y = torch.empty((total, C), dtype=odt, device=r.device)
    _dev(y, "y", odt, (total, C))
    _dev(dev_status, "dev_status", torch.int32, (1,))
    head = (S, H, N, _ptr(lengths), int(max_len), total, _ptr(r), _ptr(k), _ptr(v), _ptr(w), _dtype_code(r),
            _ptr(u), _ptr(y))
    tail = (_ptr(state), _ptr(state_out), _ptr(state_map), state.shape[0], _ptr(dev_status), _stream(r))
    if oc == _native.WKV_F32:
        fn, args = _lib.wkv6_forward_varlen, head + tail
    else:
        fn, args = _lib.wkv6_forward_varlen_ex, head + (oc,) + tail
    return VarlenPlan(fn, args, y, (lengths, r, k, v, w, u, y, state, state_out, state_map, dev_status))


def wkv6_forward_varlen(lengths, r, k, v, w, u, H, state, *, max_len, state_out=None, state_map=None,
                        y=None, dev_status=None, out_dtype=torch.float32):
    """Varlen v6 over packed token rows; updates ``state_out`` (default: ``state`` in place).

    ``lengths``: [S] int32 device tensor (tokens each slot consumes); ``r, k, v, w``:
    [total_tokens, H*N]; ``state``: [n_state, H, N, N] fp32; ``state_map``: [S] int32.
    Returns ``y`` [total_tokens, H*N] in ``out_dtype`` (float32 or bfloat16) unless given.
    """
    return varlen_plan(lengths, r, k, v, w, u, H, state, max_len=max_len, state_out=state_out,
                       state_map=state_map, y=y, dev_status=dev_status, out_dtype=out_dtype)()


def schedule_round_robin(remaining, budget):
    """Per-slot token counts for one serving call (host lists / arrays of int)."""
    import numpy as np
    rem = np.ascontiguousarray(remaining, dtype=np.int32)
    take = np.zeros_like(rem)
    total = ctypes.c_int32(0)
    i32p = ctypes.POINTER(ctypes.c_int32)
    check(_lib.wkv_schedule_round_robin(rem.size, rem.ctypes.data_as(i32p), int(budget),
                                        take.ctypes.data_as(i32p), ctypes.byref(total)))
    return take


def resolve_algo(version, B, T, H, N, algo="auto", dtype=torch.bfloat16):
    """Name of the algorithm the library runs for a v5, v6 or v7 call of this shape and input dtype."""
    a = _ALGOS[algo] if isinstance(algo, str) else int(algo)
    d = _native.WKV_BF16 if dtype == torch.bfloat16 else _native.WKV_F32
    code = _lib.wkv_resolve_algo(version, B, T, H, N, d, a)
    return {v: k for k, v in _ALGOS.items()}[code]
