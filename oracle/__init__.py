"""fp64 CPU oracle of the WKV recurrences (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg import this package.  The product library never links or calls it, and it
shares no code with the HIP kernels: the arithmetic lives in the plain C file
``wkv_oracle.c`` (double precision, one token at a time, compiled with
``-ffp-contract=off``); this module only converts arrays to float64, walks the
independent (batch row, head) / (slot, head) units and fans them out over host
threads.

Definitions (see the header of ``wkv_oracle.c`` for the passages they come
from):

* :func:`wkv4` — RWKV-v4 weighted average with decay ``exp(-exp(tau))``,
  bonus ``exp(u + k_t)`` on the current token, optional ``sigmoid(r)`` gate.
  The carried state is the pair (numerator A, denominator B).
* :func:`wkv56` — RWKV-5/6 multi-head recurrence with an N x N state per head,
  ``y_t = r_t (S + diag(u) k_t^T v_t)`` then ``S <- diag(d_t) S + k_t^T v_t``,
  ``d_t = exp(-exp(x_t))``.
* :func:`wkv6_varlen` — each slot runs :func:`wkv56` over its own packed token
  rows starting from ``state[state_map[s]]`` and writes that row back.
* :func:`wkv6_backward` — gradients of the v6 recurrence with respect to r,
  k, v, x, u and the initial state, by reverse-mode differentiation of the
  definition, one token at a time.
* :func:`wkv7` — the RWKV-7 generalized delta rule, ``h <- diag(d_t) h
  + b_t (a_t^T h) + k_t v_t^T`` then ``y_t = r_t^T h``, state [key][value],
  ``d_t = exp(-exp(w_t))``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wkv_oracle.c")
_LIB = os.path.join(_HERE, "build", "liboracle.so")
_lock = threading.Lock()
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


def build(out=_LIB, extra_flags=()):
    """Compile the C oracle with the host compiler (no HIP)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-std=c99", *extra_flags, _SRC, "-o", out + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(out + ".tmp", out)
    return out


def load(path=None):
    """Load (building first if needed) the oracle shared library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    lib.oracle_wkv4_row.restype = None
    lib.oracle_wkv4_row.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp]
    lib.oracle_wkv56_head.restype = None
    lib.oracle_wkv56_head.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_long,
                                      _dp, _dp, _dp, _dp, ctypes.c_long, _dp, _dp, _dp, _dp]
    lib.oracle_wkv6_head_bwd.restype = None
    lib.oracle_wkv6_head_bwd.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_long] + [_dp] * 14
    lib.oracle_wkv7_head.restype = None
    lib.oracle_wkv7_head.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_long] + [_dp] * 9
    return lib


def _f64(a):
    """Exact float64 copy of an input array (bf16 bit patterns are widened)."""
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.uint16:
        a = (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, offset=0):
    if a is None:
        return None
    return ctypes.cast(a.ctypes.data + 8 * int(offset), _dp)


def _threads(n):
    if n:
        return int(n)
    return max(1, min(16, os.cpu_count() or 1))


def wkv4(tau, u, k, v, r=None, A0=None, B0=None, threads=None, lib=None):
    """v4 recurrence in fp64.

    ``tau``, ``u``: [C]; ``k``, ``v``, ``r``: [B, T, C]; ``A0``, ``B0``:
    [B, C] carried numerator / denominator (None: zero state).
    Returns ``(y [B, T, C], A [B, C], B [B, C])``.
    """
    lib = lib or load()
    k = _f64(k)
    B, T, C = k.shape
    v, r = _f64(v), _f64(r)
    tau, u = _f64(tau), _f64(u)
    A0, B0 = _f64(A0), _f64(B0)
    y = np.zeros((B, T, C))
    Aout = np.zeros((B, C))
    Bout = np.zeros((B, C))
    step = max(1, -(-C // max(1, _threads(threads) // max(1, B))))
    units = [(b, c0, min(C, c0 + step)) for b in range(B) for c0 in range(0, C, step)]

    def run(unit):
        b, c0, c1 = unit
        base = b * T * C
        lib.oracle_wkv4_row(T, C, c0, c1, _ptr(tau), _ptr(u), _ptr(k, base), _ptr(v, base),
                            _ptr(r, base) if r is not None else None,
                            _ptr(A0, b * C) if A0 is not None else None,
                            _ptr(B0, b * C) if B0 is not None else None,
                            _ptr(y, base), _ptr(Aout, b * C), _ptr(Bout, b * C))

    _fan_out(run, units, threads)
    return y, Aout, Bout


def wkv56(r, k, v, x, u, H, N, state=None, state_map=None, units=None, threads=None, lib=None):
    """v5 (``x`` of shape [H*N]) or v6 (``x`` of shape [B, T, H*N]) recurrence in fp64.

    ``state``: [n_state, H, N, N] initial states (None: zero); row ``b`` starts
    from ``state[state_map[b]]`` (``state_map`` None: ``b`` if n_state == B,
    else 0).  ``units``: optional list of (b, h) pairs to evaluate (others are
    left zero).  Returns ``(y [B, T, H*N], S [B, H, N, N])``.
    """
    lib = lib or load()
    r, k, v, x, u = _f64(r), _f64(k), _f64(v), _f64(x), _f64(u)
    B, T, C = r.shape
    assert C == H * N
    static = x.ndim == 1
    st = _f64(state)
    if st is not None:
        n_state = st.shape[0]
        if state_map is None:
            state_map = np.arange(B) if n_state == B else np.zeros(B, dtype=np.int64)
    y = np.zeros((B, T, C))
    S = np.zeros((B, H, N, N))
    if units is None:
        units = [(b, h) for b in range(B) for h in range(H)]

    def run(unit):
        b, h = unit
        base = b * T * C + h * N
        xoff, xs = (h * N, 0) if static else (base, C)
        s0 = None
        if st is not None:
            s0 = _ptr(st, (int(state_map[b]) * H + h) * N * N)
        lib.oracle_wkv56_head(T, N, C, _ptr(r, base), _ptr(k, base), _ptr(v, base),
                              _ptr(x, xoff), xs, _ptr(u, h * N), s0,
                              _ptr(y, base), _ptr(S, (b * H + h) * N * N))

    _fan_out(run, units, threads)
    return y, S


def wkv6_varlen(lengths, r, k, v, x, u, H, N, state, state_map=None, threads=None, lib=None):
    """Varlen v6 in fp64 over packed token rows.

    ``lengths`` [S]; ``r, k, v, x``: [sum(lengths), H*N] with slot ``s`` at rows
    ``off[s]:off[s]+lengths[s]`` (``off`` = exclusive prefix sum);
    ``state`` [n_state, H, N, N]; slot ``s`` reads and writes row
    ``state_map[s]`` (None: identity).  Slots with zero length leave their row
    as it was.  Returns ``(y [sum(lengths), H*N], new_state)``.
    """
    lib = lib or load()
    lengths = np.asarray(lengths, dtype=np.int64)
    r, k, v, x, u = _f64(r), _f64(k), _f64(v), _f64(x), _f64(u)
    st = _f64(state)
    out_state = st.copy()
    S_slots = lengths.size
    if state_map is None:
        state_map = np.arange(S_slots)
    off = np.concatenate([[0], np.cumsum(lengths)[:-1]]) if S_slots else np.zeros(0, np.int64)
    C = H * N
    y = np.zeros((int(lengths.sum()), C))
    units = [(s, h) for s in range(S_slots) for h in range(H) if lengths[s] > 0]

    def run(unit):
        s, h = unit
        base = int(off[s]) * C + h * N
        row = int(state_map[s])
        lib.oracle_wkv56_head(int(lengths[s]), N, C, _ptr(r, base), _ptr(k, base), _ptr(v, base),
                              _ptr(x, base), C, _ptr(u, h * N),
                              _ptr(st, (row * H + h) * N * N),
                              _ptr(y, base), _ptr(out_state, (row * H + h) * N * N))

    _fan_out(run, units, threads)
    return y, out_state


def wkv6_backward(r, k, v, x, u, H, N, dy, state=None, state_map=None, d_state_out=None, units=None,
                  threads=None, lib=None):
    """Gradients of the v6 recurrence in fp64 (reverse mode through :func:`wkv56`).

    With ``L = sum(dy * y) + sum(d_state_out * S_final)`` for the outputs
    ``(y, S_final)`` of ``wkv56(r, k, v, x, u, H, N, state, state_map)``,
    returns ``(dr, dk, dv, dx [B, T, H*N], du [H*N], du_rows [B, H*N],
    d_state [B, H, N, N])``: ``d_state[b]`` is the gradient with respect to the
    initial state row ``b`` started from, ``du_rows[b]`` batch row ``b``'s
    share of ``du``.  ``units`` restricts the work to (b, h) pairs (others
    stay zero).
    """
    lib = lib or load()
    r, k, v, x, u = _f64(r), _f64(k), _f64(v), _f64(x), _f64(u)
    dy, dso = _f64(dy), _f64(d_state_out)
    B, T, C = r.shape
    assert C == H * N and x.shape == r.shape
    st = _f64(state)
    if st is not None and state_map is None:
        state_map = np.arange(B) if st.shape[0] == B else np.zeros(B, dtype=np.int64)
    dr, dk, dv, dx = (np.zeros((B, T, C)) for _ in range(4))
    du_rows = np.zeros((B, C))
    dS = np.zeros((B, H, N, N))
    if units is None:
        units = [(b, h) for b in range(B) for h in range(H)]

    def run(unit):
        b, h = unit
        base = b * T * C + h * N
        s0 = _ptr(st, (int(state_map[b]) * H + h) * N * N) if st is not None else None
        ds = _ptr(dso, (b * H + h) * N * N) if dso is not None else None
        lib.oracle_wkv6_head_bwd(T, N, C, _ptr(r, base), _ptr(k, base), _ptr(v, base), _ptr(x, base),
                                 _ptr(u, h * N), s0, _ptr(dy, base), ds,
                                 _ptr(dr, base), _ptr(dk, base), _ptr(dv, base), _ptr(dx, base),
                                 _ptr(du_rows, b * C + h * N), _ptr(dS, (b * H + h) * N * N))

    _fan_out(run, units, threads)
    return dr, dk, dv, dx, du_rows.sum(axis=0), du_rows, dS


def _fan_out(fn, units, threads):
    n = _threads(threads)
    if n == 1 or len(units) <= 1:
        for unit in units:
            fn(unit)
        return
    with ThreadPoolExecutor(max_workers=n) as ex:
        list(ex.map(fn, units))


def wkv7(r, w, k, v, a, b, H, N, state=None, state_map=None, units=None, threads=None, lib=None):
    """v7 generalized delta rule in fp64.

    ``r, w, k, v, a, b``: [B, T, H*N] (``w`` = raw decay parameter, decay
    ``exp(-exp(w))``); ``state``: [n_state,
    H, N, N] initial states h[key][value] (None: zero), row ``b`` starting from
    ``state[state_map[b]]`` (``state_map`` None: ``b`` if n_state == B, else 0).
    ``units``: optional list of (b, h) pairs to evaluate.  Returns
    ``(y [B, T, H*N], S [B, H, N, N])``.
    """
    lib = lib or load()
    r, w, k, v, a, b = (_f64(x) for x in (r, w, k, v, a, b))
    B, T, C = r.shape
    assert C == H * N
    st = _f64(state)
    if st is not None:
        n_state = st.shape[0]
        if state_map is None:
            state_map = np.arange(B) if n_state == B else np.zeros(B, dtype=np.int64)
    y = np.zeros((B, T, C))
    S = np.zeros((B, H, N, N))
    if units is None:
        units = [(bb, h) for bb in range(B) for h in range(H)]

    def run(unit):
        bb, h = unit
        base = bb * T * C + h * N
        s0 = None if st is None else _ptr(st, (int(state_map[bb]) * H + h) * N * N)
        lib.oracle_wkv7_head(T, N, C, _ptr(r, base), _ptr(w, base), _ptr(k, base), _ptr(v, base),
                             _ptr(a, base), _ptr(b, base), s0, _ptr(y, base), _ptr(S, (bb * H + h) * N * N))

    _fan_out(run, units, threads)
    return y, S
