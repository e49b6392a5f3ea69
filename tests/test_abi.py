"""C ABI of libwkv.so on the CPU: symbols, validation paths, host scheduler.

No test here launches a kernel: every call either fails host validation
(which happens before any HIP call) or is a pure host function.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from rwkv_linear_attention_wkv_amd import _native as nat

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wkv.h")

# fake, well-aligned device addresses; validation never dereferences them
P = 0x10000
MIS = 0x10002


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"WKV_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


@pytest.fixture(scope="module")
def lib():
    return nat.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 19, names
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(nat.SIGNATURES)
    assert lib.wkv_abi_version() == 1


def test_status_strings(lib):
    assert lib.wkv_status_string(0) == b"ok"
    assert lib.wkv_status_string(1) == b"invalid argument"
    assert lib.wkv_status_string(2) == b"unsupported"
    assert lib.wkv_status_string(3) == b"device error"
    assert lib.wkv_status_string(99) == b"unknown status"


def test_noalloc_backward_size_limit(lib):
    """The allocation-free backward rejects B*H*N beyond its 1,048,576-float scratch before any
    HIP call; the workspace variant takes the same shape."""
    E = nat.WKV_ERR_INVALID_ARG
    args = (1025, 8, 16, 64, P, P, P, P, 1, P, P, None, None, 0, None, None, P, P, P, P, P)
    assert lib.wkv6_backward_noalloc(*args, None, None, None) == E
    assert b"scratch" in lib.wkv_last_error()
    assert lib.wkv6_backward_noalloc(1, 8, 16, 64, P, P, P, P, 1, P, P, None, None, 0, None, None, P, P, P, P,
                                     None, None, None, None) == E  # du NULL
    assert lib.wkv6_backward(*args, None, None, None, None) == E  # du_rows NULL: the workspace is required


def v6(lib, B=2, T=8, H=2, N=64, r=P, k=P, v=P, w=P, dt=1, u=P, y=P, si=None, sm=None, ns=0, so=None,
       algo=0, ds=None):
    return lib.wkv6_forward(B, T, H, N, r, k, v, w, dt, u, y, si, sm, ns, so, algo, ds, None)


def v5(lib, B=2, T=8, H=2, N=64, r=P, k=P, v=P, dt=1, w=P, u=P, y=P, si=None, sm=None, ns=0, so=None,
       algo=0, ds=None):
    return lib.wkv5_forward(B, T, H, N, r, k, v, dt, w, u, y, si, sm, ns, so, algo, ds, None)


@pytest.mark.parametrize("fn", [v5, v6])
def test_dense_validation(lib, fn):
    E, U = nat.WKV_ERR_INVALID_ARG, nat.WKV_ERR_UNSUPPORTED
    assert fn(lib, N=32) == U and b"head size" in lib.wkv_last_error()
    assert fn(lib, N=128) == U
    assert fn(lib, dt=7) == U
    assert fn(lib, algo=9) == U
    assert fn(lib, B=0) == E
    assert fn(lib, H=0) == E
    assert fn(lib, T=-1) == E
    assert fn(lib, B=70000) == E
    assert fn(lib, r=None) == E
    assert fn(lib, y=None) == E
    assert fn(lib, u=None) == E
    assert fn(lib, k=MIS) == E and b"aligned" in lib.wkv_last_error()
    assert fn(lib, si=MIS, ns=2) == E
    assert fn(lib, si=P, ns=0) == E
    assert fn(lib, si=P, ns=3) == E          # no map: n_state must be 1 or B
    assert fn(lib, sm=P, ns=0) == E          # map without state
    assert fn(lib, si=P, sm=P, ns=2, so=P) == E   # in place with a map
    assert fn(lib, si=P, ns=1, so=P) == E    # in place needs n_state == B
    assert fn(lib, ds=0x10001) == E
    # T = 0 without a state to write is a no-op that launches nothing
    assert fn(lib, T=0, r=None, k=None, v=None, y=None) == nat.WKV_OK
    assert lib.wkv_last_error() == b""


def test_v4_validation(lib):
    E = nat.WKV_ERR_INVALID_ARG

    def call(B=2, T=8, C=64, tau=P, u=P, k=P, v=P, r=None, dt=0, y=P, si=None, so=None):
        return lib.wkv4_forward(B, T, C, tau, u, k, v, r, dt, y, si, so, None)

    assert call(B=0) == E
    assert call(C=0) == E
    assert call(T=-2) == E
    assert call(tau=None) == E
    assert call(k=None) == E
    assert call(r=MIS) == E
    assert call(si=MIS) == E
    assert call(dt=3) == nat.WKV_ERR_UNSUPPORTED
    assert call(T=0, k=None, v=None, y=None) == nat.WKV_OK
    assert call(T=0, k=None, v=None, y=None, si=P, so=P) == nat.WKV_OK


def test_varlen_validation(lib):
    E, U = nat.WKV_ERR_INVALID_ARG, nat.WKV_ERR_UNSUPPORTED

    def call(S=4, H=2, N=64, lens=P, max_len=16, total=32, r=P, k=P, v=P, w=P, dt=1, u=P, y=P, si=P, so=P,
             sm=None, ns=4, ds=None):
        return lib.wkv6_forward_varlen(S, H, N, lens, max_len, total, r, k, v, w, dt, u, y, si, so, sm, ns, ds,
                                       None)

    assert call(N=16) == U
    assert call(S=-1) == E
    assert call(max_len=-1) == E
    assert call(total=-1) == E
    assert call(lens=None) == E
    assert call(si=None) == E
    assert call(so=None) == E
    assert call(ns=3) == E                    # identity map needs n_state >= slots
    assert call(sm=MIS, ns=3) == E
    assert call(w=MIS) == E
    assert call(total=0, r=None, k=None, v=None, w=None, y=None, lens=None) == E  # lengths still required
    assert call(S=0, lens=None, si=None, so=None) == nat.WKV_OK   # no slots: no-op


def _rr_reference(remaining, budget):
    """One token at a time to every slot with tokens left, in slot order."""
    rem = list(remaining)
    take = [0] * len(rem)
    left = budget
    while left > 0 and any(x > 0 for x in rem):
        for s in range(len(rem)):
            if left == 0:
                break
            if rem[s] > 0:
                take[s] += 1
                rem[s] -= 1
                left -= 1
    return take


@pytest.mark.parametrize("seed", range(6))
def test_round_robin_scheduler(lib, seed):
    rng = np.random.default_rng(seed)
    S = int(rng.integers(1, 70))
    rem = rng.integers(0, 300, size=S).astype(np.int32)
    rem[rng.random(S) < 0.2] = 0
    budget = int(rng.integers(0, 600))
    take = np.zeros(S, dtype=np.int32)
    total = ctypes.c_int32(-1)
    i32p = ctypes.POINTER(ctypes.c_int32)
    st = lib.wkv_schedule_round_robin(S, rem.ctypes.data_as(i32p), budget, take.ctypes.data_as(i32p),
                                      ctypes.byref(total))
    assert st == nat.WKV_OK
    assert take.tolist() == _rr_reference(rem.tolist(), budget)
    assert total.value == int(take.sum()) == min(budget, int(rem.sum()))


def test_round_robin_rejects_negative(lib):
    rem = np.array([3, -1], dtype=np.int32)
    take = np.zeros(2, dtype=np.int32)
    i32p = ctypes.POINTER(ctypes.c_int32)
    assert lib.wkv_schedule_round_robin(2, rem.ctypes.data_as(i32p), 5, take.ctypes.data_as(i32p),
                                        None) == nat.WKV_ERR_INVALID_ARG


def test_resolve_algo(lib):
    A, S, C = nat.WKV_ALGO_AUTO, nat.WKV_ALGO_SCAN, nat.WKV_ALGO_CHUNKED
    bf, f32 = nat.WKV_BF16, nat.WKV_F32
    assert lib.wkv_resolve_algo(6, 8, 4096, 32, 64, bf, S) == S
    assert lib.wkv_resolve_algo(6, 8, 4096, 32, 64, bf, C) == C
    assert lib.wkv_resolve_algo(6, 8, 4096, 32, 64, bf, A) == C
    assert lib.wkv_resolve_algo(5, 8, 4096, 32, 64, bf, A) == C
    assert lib.wkv_resolve_algo(6, 8, 63, 32, 64, bf, A) == S          # no full chunk
    assert lib.wkv_resolve_algo(6, 8, 1, 32, 64, bf, A) == S           # decode stays on the scan
    assert lib.wkv_resolve_algo(6, 8, 4096, 32, 64, f32, A) == S       # fp32 inputs: scan
    assert lib.wkv_resolve_algo(4, 8, 4096, 32, 64, bf, A) == S


def v6x(lib, B=2, T=8, H=2, N=64, dt=1, lay=0, y=P, odt=0, algo=0):
    return lib.wkv6_forward_ex(B, T, H, N, P, P, P, P, dt, lay, P, y, odt, None, None, 0, None, algo, None, None)


def v5x(lib, B=2, T=8, H=2, N=64, dt=1, lay=0, y=P, odt=0, algo=0):
    return lib.wkv5_forward_ex(B, T, H, N, P, P, P, dt, lay, P, P, y, odt, None, None, 0, None, algo, None, None)


@pytest.mark.parametrize("fn", [v5x, v6x])
def test_ex_validation(lib, fn):
    """Layout and output-dtype checks of the _ex entry points (host only)."""
    E, U = nat.WKV_ERR_INVALID_ARG, nat.WKV_ERR_UNSUPPORTED
    assert fn(lib, lay=2) == U and b"layout" in lib.wkv_last_error()
    assert fn(lib, lay=-1) == U
    assert fn(lib, odt=5) == U and b"output dtype" in lib.wkv_last_error()
    assert fn(lib, N=32) == U
    assert fn(lib, y=None) == E
    assert fn(lib, y=MIS) == E
    assert fn(lib, B=0) == E
    # more channels per token than the chunked kernel's 32-bit row offsets take
    assert fn(lib, H=(1 << 23) // 64 + 1, algo=nat.WKV_ALGO_CHUNKED) == U
    for lay in (nat.WKV_LAYOUT_BTHN, nat.WKV_LAYOUT_BHTN):
        for odt in (nat.WKV_F32, nat.WKV_BF16):
            assert fn(lib, T=0, lay=lay, odt=odt) == nat.WKV_OK


def test_ex_v4_and_varlen_validation(lib):
    U = nat.WKV_ERR_UNSUPPORTED
    assert lib.wkv4_forward_ex(2, 8, 64, P, P, P, P, None, 0, P, 7, None, None, None) == U
    assert b"output dtype" in lib.wkv_last_error()
    assert lib.wkv4_forward_ex(2, 0, 64, P, P, None, None, None, 0, None, 1, None, None, None) == nat.WKV_OK
    assert lib.wkv6_forward_varlen_ex(4, 2, 64, P, 16, 32, P, P, P, P, 1, P, P, 9, P, P, None, 4, None,
                                      None) == U
    assert lib.wkv6_forward_varlen_ex(0, 2, 64, None, 16, 32, P, P, P, P, 1, P, P, 1, None, None, None, 4, None,
                                      None) == nat.WKV_OK


def test_v7_validation(lib):
    E, U = nat.WKV_ERR_INVALID_ARG, nat.WKV_ERR_UNSUPPORTED

    def call(B=2, T=8, H=2, N=64, r=P, w=P, k=P, v=P, a=P, b=P, dt=1, lay=0, y=P, odt=0, si=None, sm=None, ns=0,
             so=None, ds=None):
        return lib.wkv7_forward(B, T, H, N, r, w, k, v, a, b, dt, lay, y, odt, si, sm, ns, so, ds, None)

    assert call(N=32) == U and b"head size" in lib.wkv_last_error()
    assert call(dt=4) == U
    assert call(odt=3) == U and b"output dtype" in lib.wkv_last_error()
    assert call(lay=5) == U and b"layout" in lib.wkv_last_error()
    assert call(B=0) == E
    assert call(T=-1) == E
    assert call(a=None) == E
    assert call(b=MIS) == E and b"aligned" in lib.wkv_last_error()
    assert call(si=P, ns=3) == E
    assert call(sm=P) == E
    assert call(si=P, sm=P, ns=2, so=P) == E
    assert call(T=0, r=None, w=None, k=None, v=None, a=None, b=None, y=None) == nat.WKV_OK


def test_resolve_algo_wide_rows(lib):
    bf = nat.WKV_BF16
    assert lib.wkv_resolve_algo(6, 1, 4096, (1 << 23) // 64, 64, bf, nat.WKV_ALGO_AUTO) == nat.WKV_ALGO_CHUNKED
    assert lib.wkv_resolve_algo(6, 1, 4096, (1 << 23) // 64 + 1, 64, bf, nat.WKV_ALGO_AUTO) == nat.WKV_ALGO_SCAN


def test_chunked_needs_bf16(lib):
    assert v6(lib, dt=nat.WKV_F32, algo=nat.WKV_ALGO_CHUNKED) == nat.WKV_ERR_UNSUPPORTED
    assert b"bf16" in lib.wkv_last_error()


def bwd(lib, B=2, T=8, H=2, N=64, dt=1, dy=P, si=None, sm=None, ns=0, sf=None, dso=None, dr=P, dk=P, dv=P,
        dw=P, du=P, dur=P, dsi=None):
    return lib.wkv6_backward(B, T, H, N, P, P, P, P, dt, P, dy, si, sm, ns, sf, dso, dr, dk, dv, dw, du, dur, dsi,
                             None, None)


def test_v6_backward_validation(lib):
    """Host-side checks of wkv6_backward (no launch happens for any of these)."""
    assert bwd(lib, N=32) == 2                 # head size other than 64
    assert bwd(lib, dt=7) == 2                 # unknown dtype
    assert bwd(lib, B=0) == 1
    assert bwd(lib, dy=None) == 1              # dy needed when T > 0
    assert bwd(lib, dk=MIS) == 1               # dk must be 16-byte aligned
    assert bwd(lib, du=None) == 1
    assert bwd(lib, dur=None) == 1
    assert bwd(lib, dso=P) == 1                # d_state_out without the forward's final state
    assert b"state_final" in lib.wkv_last_error()
    assert bwd(lib, sm=P) == 1                 # state_map without state_in
    assert bwd(lib, si=P, ns=3) == 1           # n_state must be 1 or B without a map


def test_train_forward_and_saved_states_validation(lib):
    """wkv6_forward_train needs bf16 inputs and, past one chunk, an aligned chunk_states array;
    wkv6_backward_ex checks the alignment of the saved states it is handed (host only)."""
    E, U = nat.WKV_ERR_INVALID_ARG, nat.WKV_ERR_UNSUPPORTED

    def train(B=2, T=100, H=2, N=64, dt=1, y=P, odt=0, cs=P):
        return lib.wkv6_forward_train(B, T, H, N, P, P, P, P, dt, P, y, odt, None, None, 0, None, cs, None, None)

    assert train(dt=0) == U and b"bf16" in lib.wkv_last_error()
    assert train(cs=None) == E and b"chunk_states" in lib.wkv_last_error()
    assert train(cs=MIS) == E and b"chunk_states" in lib.wkv_last_error()
    assert train(odt=5) == U and b"output dtype" in lib.wkv_last_error()
    assert train(N=32) == U and b"head size" in lib.wkv_last_error()
    assert train(y=MIS) == E
    assert train(T=0, cs=None) == nat.WKV_OK  # no tokens, no states to save

    def bwd(T=100, dt=1, cs=P, algo=nat.WKV_ALGO_AUTO):
        return lib.wkv6_backward_ex(2, T, 2, 64, P, P, P, P, dt, P, P, None, None, 0, None, None, P, P, P, P, P, P,
                                    None, cs, algo, None, None)

    assert bwd(cs=MIS) == E and b"chunk_states" in lib.wkv_last_error()
    assert bwd(algo=7) == U and b"algorithm" in lib.wkv_last_error()
    assert bwd(dt=0, algo=nat.WKV_ALGO_CHUNKED) == U and b"bf16" in lib.wkv_last_error()
