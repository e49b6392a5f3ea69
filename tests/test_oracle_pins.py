"""Pins of the fp64 oracle against mathematics it does not itself contain.

Each pin is an independent route to the same number: closed-form weighted sums
with every weight computed directly (no running state), an O(T^2 N^2)
brute-force sum of explicit decay products, exact rational arithmetic, the
no-decay case written as causal linear attention with matrix products, the
full-decay case, and invariants that hold bitwise in the oracle (chunk-carry
splitting, scaling by 2, v5 == v6 with constant decay, slot permutation).

The v4 definition follows the RWKV-v4 walk-through page (RWKV_TimeMix.forward:
WKV over (time_decay, time_first, k, v), gated by sigmoid(r)); the v5/v6 one
follows the rwkv_ops page's RWKV6_OP call table (r, k, v, w, u, init_state,
state_map -> y, y_state).  Neither page prints the formula; the readings are
the standard RWKV-4 and RWKV-5/6 recurrences.
"""
import os
import shutil
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest

import oracle
from wkv_inputs import wkv4_inputs, wkv5_inputs, wkv6_inputs, varlen_inputs, stored_f32


def relerr(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = max(np.sqrt(np.mean(ref ** 2)), 1e-300)
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), scale)))


# ---------------------------------------------------------------- v4 pins

def v4_closed_form(tau, u, k, v, r=None, A0=None, B0=None):
    """Weighted average with each weight exp((t-1-i)*lambda + k_i) computed directly."""
    lam = -np.exp(tau.astype(np.float64))
    k = k.astype(np.float64)
    v = v.astype(np.float64)
    u = u.astype(np.float64)
    T, C = k.shape
    y = np.empty((T, C))
    for t in range(T):
        i = np.arange(t, dtype=np.float64)
        w = np.exp((t - 1 - i)[:, None] * lam[None, :] + k[:t])
        bonus = np.exp(u + k[t])
        num = (w * v[:t]).sum(axis=0) + bonus * v[t]
        den = w.sum(axis=0) + bonus
        if A0 is not None:
            num = num + np.exp(t * lam) * A0
            den = den + np.exp(t * lam) * B0
        y[t] = num / den
        if r is not None:
            y[t] = y[t] * (1.0 / (1.0 + np.exp(-r[t].astype(np.float64))))
    i = np.arange(T, dtype=np.float64)
    w = np.exp((T - 1 - i)[:, None] * lam[None, :] + k)
    A = (w * v).sum(axis=0)
    Bd = w.sum(axis=0)
    if A0 is not None:
        A = A + np.exp(T * lam) * A0
        Bd = Bd + np.exp(T * lam) * B0
    return y, A, Bd


def _v4_state_AB(state):
    a, b, p = (state[:, i].astype(np.float64) for i in range(3))
    return a * np.exp(p), b * np.exp(p)


@pytest.mark.parametrize("with_r,init", [(False, False), (True, False), (True, True)])
def test_v4_matches_closed_form(with_r, init):
    inp = wkv4_inputs(2, 40, 16, seed=3, with_r=with_r, init_state=init)
    A0 = B0 = None
    if init:
        A0, B0 = _v4_state_AB(inp["state"])
    y, A, Bd = oracle.wkv4(inp["tau"], inp["u"], inp["k"], inp["v"], inp["r"], A0, B0, threads=2)
    for b in range(2):
        yc, Ac, Bc = v4_closed_form(inp["tau"], inp["u"], inp["k"][b], inp["v"][b],
                                    None if inp["r"] is None else inp["r"][b],
                                    None if A0 is None else A0[b], None if B0 is None else B0[b])
        assert relerr(y[b], yc) < 1e-12
        assert relerr(A[b], Ac) < 1e-12
        assert relerr(Bd[b], Bc) < 1e-12


def test_v4_config0_closed_form():
    """The small v4 parity workload: B=1, T=64, C=32, zero state, seed 0."""
    inp = wkv4_inputs(1, 64, 32, seed=0)
    y, A, Bd = oracle.wkv4(inp["tau"], inp["u"], inp["k"], inp["v"])
    yc, Ac, Bc = v4_closed_form(inp["tau"], inp["u"], inp["k"][0], inp["v"][0])
    assert relerr(y[0], yc) < 1e-12
    assert relerr(A[0], Ac) < 1e-12 and relerr(Bd[0], Bc) < 1e-12


def test_v4_first_output_is_v0_and_constant_v_is_fixed_point():
    inp = wkv4_inputs(1, 24, 8, seed=5)
    y, _, _ = oracle.wkv4(inp["tau"], inp["u"], inp["k"], inp["v"])
    np.testing.assert_allclose(y[0, 0], inp["v"][0, 0].astype(np.float64), rtol=4e-16, atol=0)
    # a weighted average of a constant is that constant
    vc = np.full_like(inp["v"], 0.75)
    y, _, _ = oracle.wkv4(inp["tau"], inp["u"], inp["k"], vc)
    np.testing.assert_allclose(y, 0.75, rtol=1e-14)


def test_v4_equals_ratio_of_two_v5_runs():
    """v4 numerator and denominator are each a v5 recurrence with N=1.

    With r=1, k -> exp(k), u -> exp(u) and the same decay parameter, the v5
    output is the v4 numerator (for v) or denominator (for v = 1).
    """
    inp = wkv4_inputs(1, 30, 6, seed=9, init_state=True)
    A0, B0 = _v4_state_AB(inp["state"])
    y4, A4, B4 = oracle.wkv4(inp["tau"], inp["u"], inp["k"], inp["v"], None, A0, B0)
    C = 6
    ones = np.ones((C, 1, 30, 1))
    for c in range(C):
        kk = np.exp(inp["k"][:, :, c:c + 1].astype(np.float64))
        vv = inp["v"][:, :, c:c + 1].astype(np.float64)
        rr = np.ones_like(kk)
        x = inp["tau"][c:c + 1].astype(np.float64)
        uu = np.exp(inp["u"][c:c + 1].astype(np.float64))
        num, Sn = oracle.wkv56(rr, kk, vv, x, uu, 1, 1, state=A0[:, c].reshape(1, 1, 1, 1))
        den, Sd = oracle.wkv56(rr, kk, ones[c], x, uu, 1, 1, state=B0[:, c].reshape(1, 1, 1, 1))
        assert relerr(y4[0, :, c], (num / den)[0, :, 0]) < 1e-13
        assert relerr(A4[0, c], Sn.ravel()) < 1e-13
        assert relerr(B4[0, c], Sd.ravel()) < 1e-13


def test_v4_carry_split_is_bitwise():
    inp = wkv4_inputs(2, 50, 8, seed=11, with_r=True)
    y, A, Bd = oracle.wkv4(inp["tau"], inp["u"], inp["k"], inp["v"], inp["r"])
    y1, A1, B1 = oracle.wkv4(inp["tau"], inp["u"], inp["k"][:, :17], inp["v"][:, :17], inp["r"][:, :17])
    y2, A2, B2 = oracle.wkv4(inp["tau"], inp["u"], inp["k"][:, 17:], inp["v"][:, 17:], inp["r"][:, 17:], A1, B1)
    assert np.array_equal(np.concatenate([y1, y2], axis=1), y)
    assert np.array_equal(A2, A) and np.array_equal(B2, Bd)


# ---------------------------------------------------------------- v5 / v6 pins

def v56_closed_form(r, k, v, d, u, S0):
    """Explicit sum over earlier tokens with decay products formed term by term.

    y_t[j] = sum_i r_t[i] * ( P(0,t)[i] S0[i][j] + sum_{s<t} P(s+1,t)[i] k_s[i] v_s[j]
                              + u[i] k_t[i] v_t[j] ),   P(a,t)[i] = prod_{m=a}^{t-1} d_m[i].
    """
    T, N = r.shape
    y = np.zeros((T, N))
    for t in range(T):
        P = np.ones((t + 1, N))          # P[s] = prod_{m=s}^{t-1} d_m  (s = 0..t)
        for s in range(t + 1):
            for m in range(s, t):
                P[s] = P[s] * d[m]
        acc = (r[t] * P[0]) @ S0
        for s in range(t):
            acc = acc + np.dot(r[t] * P[s + 1], k[s]) * v[s]
        acc = acc + np.dot(r[t] * u, k[t]) * v[t]
        y[t] = acc
    Pend = np.ones((T + 1, N))
    for s in range(T + 1):
        for m in range(s, T):
            Pend[s] = Pend[s] * d[m]
    S = Pend[0][:, None] * S0
    for s in range(T):
        S = S + np.outer(Pend[s + 1] * k[s], v[s])
    return y, S


def _decay(x):
    return np.exp(-np.exp(np.asarray(x, dtype=np.float64)))


@pytest.mark.parametrize("N,T", [(4, 20), (8, 16), (64, 8)])
def test_v6_matches_bruteforce(N, T):
    H, B = 2, 2
    inp = wkv6_inputs(B, T, H, N, seed=N + T, init_state=B)
    y, S = oracle.wkv56(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], H, N, state=inp["state"])
    f = {n: stored_f32(inp[n]).astype(np.float64) for n in ("r", "k", "v", "x")}
    u = inp["u"].astype(np.float64)
    for b in range(B):
        for h in range(H):
            sl = slice(h * N, (h + 1) * N)
            yc, Sc = v56_closed_form(f["r"][b, :, sl], f["k"][b, :, sl], f["v"][b, :, sl],
                                     _decay(f["x"][b, :, sl]), u[sl], inp["state"][b, h].astype(np.float64))
            assert relerr(y[b, :, sl], yc) < 1e-12
            assert relerr(S[b, h], Sc) < 1e-12


def test_v5_matches_bruteforce_and_state_map():
    H, N, B, T = 2, 8, 3, 18
    inp = wkv5_inputs(B, T, H, N, seed=4, init_state=2)
    smap = np.array([1, 0, 1])
    y, S = oracle.wkv56(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], H, N,
                        state=inp["state"], state_map=smap)
    f = {n: stored_f32(inp[n]).astype(np.float64) for n in ("r", "k", "v")}
    d = _decay(inp["x"])
    u = inp["u"].astype(np.float64)
    for b in range(B):
        for h in range(H):
            sl = slice(h * N, (h + 1) * N)
            yc, Sc = v56_closed_form(f["r"][b, :, sl], f["k"][b, :, sl], f["v"][b, :, sl],
                                     np.broadcast_to(d[sl], (T, N)), u[sl],
                                     inp["state"][smap[b], h].astype(np.float64))
            assert relerr(y[b, :, sl], yc) < 1e-12
            assert relerr(S[b, h], Sc) < 1e-12


def test_exact_rational_tiny_case():
    """N=2, T=3 with decay exactly 1/2 everywhere, checked against exact fractions.

    x = ln(ln 2) gives exp(-exp(x)) = 1/2 up to one rounding in fp64.
    """
    F = Fraction
    r = [[F(1), F(2)], [F(-1), F(1, 2)], [F(3), F(-2)]]
    k = [[F(1, 2), F(-1)], [F(2), F(1)], [F(-1, 4), F(3)]]
    v = [[F(1), F(-3)], [F(2), F(1, 2)], [F(-1), F(4)]]
    u = [F(3, 2), F(-1, 2)]
    S0 = [[F(1, 4), F(-1)], [F(2), F(1, 8)]]
    half = F(1, 2)
    T, N = 3, 2

    def P(a, t):  # prod_{m=a}^{t-1} 1/2
        return half ** (t - a) if t > a else F(1)

    exact_y = [[sum(r[t][i] * (P(0, t) * S0[i][j]
                               + sum(P(s + 1, t) * k[s][i] * v[s][j] for s in range(t))
                               + u[i] * k[t][i] * v[t][j]) for i in range(N)) for j in range(N)]
               for t in range(T)]
    exact_S = [[P(0, T) * S0[i][j] + sum(P(s + 1, T) * k[s][i] * v[s][j] for s in range(T))
                for j in range(N)] for i in range(N)]
    to = lambda a: np.array(a, dtype=np.float64)[None]  # noqa: E731
    x = np.full((1, T, N), np.log(np.log(2.0)))
    y, S = oracle.wkv56(to(r), to(k), to(v), x, np.array(u, dtype=np.float64), 1, N,
                        state=np.array(S0, dtype=np.float64).reshape(1, 1, N, N))
    np.testing.assert_allclose(y[0], np.array(exact_y, dtype=np.float64), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(S[0, 0], np.array(exact_S, dtype=np.float64), rtol=1e-14, atol=1e-14)
    # one value by hand: y_0[0] = r0.(S0[:,0] + u*k0*v0[0]) = 1*(1/4+3/4) + 2*(2+1/2) = 6
    assert exact_y[0][0] == 6 and abs(y[0, 0, 0] - 6.0) < 1e-14


def test_no_decay_is_causal_linear_attention():
    """x = -100 gives decay exactly 1: y = (tril_-1(R K^T) + diag(R.(u*K))) V + R S0."""
    H, N, T = 1, 16, 24
    inp = wkv6_inputs(1, T, H, N, seed=21, init_state=1)
    x = np.full((1, T, N), -100.0)
    assert np.all(_decay(x) == 1.0)
    y, S = oracle.wkv56(inp["r"], inp["k"], inp["v"], x, inp["u"], H, N, state=inp["state"])
    R = stored_f32(inp["r"][0]).astype(np.float64)
    K = stored_f32(inp["k"][0]).astype(np.float64)
    V = stored_f32(inp["v"][0]).astype(np.float64)
    u = inp["u"].astype(np.float64)
    S0 = inp["state"][0, 0].astype(np.float64)
    A = np.tril(R @ K.T, -1) + np.diag(np.sum(R * u * K, axis=1))
    ref = A @ V + R @ S0
    assert relerr(y[0], ref) < 1e-12
    assert relerr(S[0, 0], S0 + K.T @ V) < 1e-12


def test_full_decay_keeps_only_previous_token():
    """x = +20 gives decay exactly 0: only the previous token and the bonus remain."""
    H, N, T = 1, 8, 10
    inp = wkv6_inputs(1, T, H, N, seed=22, init_state=1)
    x = np.full((1, T, N), 20.0)
    assert np.all(_decay(x) == 0.0)
    y, S = oracle.wkv56(inp["r"], inp["k"], inp["v"], x, inp["u"], H, N, state=inp["state"])
    R = stored_f32(inp["r"][0]).astype(np.float64)
    K = stored_f32(inp["k"][0]).astype(np.float64)
    V = stored_f32(inp["v"][0]).astype(np.float64)
    u = inp["u"].astype(np.float64)
    S0 = inp["state"][0, 0].astype(np.float64)
    ref = np.empty((T, N))
    ref[0] = R[0] @ S0 + np.dot(R[0] * u, K[0]) * V[0]
    for t in range(1, T):
        ref[t] = np.dot(R[t], K[t - 1]) * V[t - 1] + np.dot(R[t] * u, K[t]) * V[t]
    assert relerr(y[0], ref) < 1e-13
    assert relerr(S[0, 0], np.outer(K[-1], V[-1])) < 1e-15


def test_v6_carry_split_bitwise_and_scaling():
    H, N, B, T = 2, 16, 2, 33
    inp = wkv6_inputs(B, T, H, N, seed=30, init_state=B)
    args = lambda a, b: (inp["r"][:, a:b], inp["k"][:, a:b], inp["v"][:, a:b], inp["x"][:, a:b])  # noqa: E731
    y, S = oracle.wkv56(*args(0, T), inp["u"], H, N, state=inp["state"])
    y1, S1 = oracle.wkv56(*args(0, 13), inp["u"], H, N, state=inp["state"])
    y2, S2 = oracle.wkv56(*args(13, 14), inp["u"], H, N, state=S1)
    y3, S3 = oracle.wkv56(*args(14, T), inp["u"], H, N, state=S2)
    assert np.array_equal(np.concatenate([y1, y2, y3], axis=1), y)
    assert np.array_equal(S3, S)
    # doubling v and the initial state doubles y and the state exactly
    v2 = stored_f32(inp["v"]).astype(np.float64) * 2
    yd, Sd = oracle.wkv56(inp["r"], inp["k"], v2, inp["x"], inp["u"], H, N, state=inp["state"] * 2.0)
    assert np.array_equal(yd, 2 * y) and np.array_equal(Sd, 2 * S)
    # superposition in v (with zero initial state)
    va = stored_f32(inp["v"]).astype(np.float64)
    vb = np.random.default_rng(1).standard_normal(va.shape)
    ya, _ = oracle.wkv56(inp["r"], inp["k"], va, inp["x"], inp["u"], H, N)
    yb, _ = oracle.wkv56(inp["r"], inp["k"], vb, inp["x"], inp["u"], H, N)
    yab, _ = oracle.wkv56(inp["r"], inp["k"], va + vb, inp["x"], inp["u"], H, N)
    assert relerr(yab, ya + yb) < 1e-12


def test_v5_equals_v6_with_constant_decay():
    H, N, B, T = 2, 8, 2, 12
    inp = wkv5_inputs(B, T, H, N, seed=31)
    x6 = np.broadcast_to(inp["x"], (B, T, H * N)).copy()
    y5, S5 = oracle.wkv56(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], H, N)
    y6, S6 = oracle.wkv56(inp["r"], inp["k"], inp["v"], x6, inp["u"], H, N)
    assert np.array_equal(y5, y6) and np.array_equal(S5, S6)


# ---------------------------------------------------------------- varlen pins

def test_varlen_equals_independent_slots_and_permutation():
    H, N = 2, 8
    inp = varlen_inputs(5, H, N, seed=40, max_prompt=20, decode_steps=0, lengths=[3, 0, 7, 1, 12])
    lengths = inp["lengths"]
    off = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    y, st = oracle.wkv6_varlen(lengths, inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], H, N, inp["state"])
    for s in range(5):
        rows = slice(off[s], off[s] + lengths[s])
        if lengths[s] == 0:
            assert np.array_equal(st[s], inp["state"][s].astype(np.float64))
            continue
        ys, Ss = oracle.wkv56(inp["r"][None, rows], inp["k"][None, rows], inp["v"][None, rows],
                              inp["x"][None, rows], inp["u"], H, N, state=inp["state"][s:s + 1])
        assert np.array_equal(ys[0], y[rows])
        assert np.array_equal(Ss[0], st[s])
    # rows permuted through state_map move bitwise
    perm = np.array([3, 0, 4, 1, 2])
    state_p = np.empty_like(inp["state"])
    state_p[perm] = inp["state"]
    yp, stp = oracle.wkv6_varlen(lengths, inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], H, N,
                                 state_p, state_map=perm)
    assert np.array_equal(yp, y)
    assert np.array_equal(stp[perm], st)


def test_varlen_call_split_is_bitwise():
    H, N = 1, 8
    lengths = np.array([6, 2, 9], dtype=np.int32)
    inp = varlen_inputs(3, H, N, seed=41, decode_steps=0, lengths=lengths)
    off = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    y, st = oracle.wkv6_varlen(lengths, inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], H, N, inp["state"])
    # consume in two calls: first (2, 1, 4) tokens, then the rest
    first = np.array([2, 1, 4])
    rest = lengths - first
    pick = lambda a, lo, n: np.concatenate([a[off[s] + lo[s]: off[s] + lo[s] + n[s]] for s in range(3)])  # noqa: E731
    zeros = np.zeros(3, dtype=np.int64)
    arrs1 = [pick(inp[n], zeros, first) for n in ("r", "k", "v", "x")]
    arrs2 = [pick(inp[n], first, rest) for n in ("r", "k", "v", "x")]
    y1, st1 = oracle.wkv6_varlen(first, *arrs1, inp["u"], H, N, inp["state"])
    y2, st2 = oracle.wkv6_varlen(rest, *arrs2, inp["u"], H, N, st1)
    assert np.array_equal(st2, st)
    o1 = np.concatenate([[0], np.cumsum(first)[:-1]])
    o2 = np.concatenate([[0], np.cumsum(rest)[:-1]])
    for s in range(3):
        got = np.concatenate([y1[o1[s]:o1[s] + first[s]], y2[o2[s]:o2[s] + rest[s]]])
        assert np.array_equal(got, y[off[s]:off[s] + lengths[s]])


# ---------------------------------------------------------------- planted mistakes

_MUTANTS = {
    "dropped_bonus": ("rt[i] * (S[i * N + j] + u[i] * kt[i] * vt[j])", "rt[i] * (S[i * N + j])"),
    "transposed_state": ("rt[i] * (S[i * N + j] +", "rt[i] * (S[j * N + i] +"),
    "decay_sign": ("double d = exp(-exp(xt[i]));\n            for (int j = 0; j < N; j++)\n                S[i * N + j]",
                   "double d = exp(exp(xt[i]) * -0.5);\n            for (int j = 0; j < N; j++)\n                S[i * N + j]"),
    "decay_index": ("const double *xt = x + (long)t * xs;", "const double *xt = x + (long)(t > 0 ? t - 1 : 0) * xs;"),
    "v4_bonus_on_k": ("double bonus = exp(u[c] + kt);", "double bonus = exp(u[c]);"),
    "v4_decay_twice": ("A = decay * A + ek * vt;", "A = decay * decay * A + ek * vt;"),
}


@pytest.mark.parametrize("name", sorted(_MUTANTS))
def test_pins_catch_planted_mistakes(name):
    """A mistake planted in a copy of the oracle source must fail a pin."""
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(os.path.join(os.path.dirname(oracle.__file__), "wkv_oracle.c")).read()
    old, new = _MUTANTS[name]
    assert src.count(old) == 1, name
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        so = os.path.join(d, "mutant.so")
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", path, "-o", so, "-lm"])
        lib = oracle.load(so)
        caught = False
        # v4 pin
        inp4 = wkv4_inputs(1, 20, 4, seed=3, with_r=True)
        y, A, Bd = oracle.wkv4(inp4["tau"], inp4["u"], inp4["k"], inp4["v"], inp4["r"], lib=lib, threads=1)
        yc, Ac, Bc = v4_closed_form(inp4["tau"], inp4["u"], inp4["k"][0], inp4["v"][0], inp4["r"][0])
        caught |= relerr(y[0], yc) > 1e-9 or relerr(A[0], Ac) > 1e-9
        # v6 pin
        inp = wkv6_inputs(1, 10, 1, 4, seed=7, init_state=1)
        y, S = oracle.wkv56(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], 1, 4,
                            state=inp["state"], lib=lib, threads=1)
        f = {n: stored_f32(inp[n]).astype(np.float64) for n in ("r", "k", "v", "x")}
        yc, Sc = v56_closed_form(f["r"][0], f["k"][0], f["v"][0], _decay(f["x"][0]),
                                 inp["u"].astype(np.float64), inp["state"][0, 0].astype(np.float64))
        caught |= relerr(y[0], yc) > 1e-9 or relerr(S[0, 0], Sc) > 1e-9
        assert caught, f"mutant {name} passed every pin"


# ---------------------------------------------------------------- v6 backward pins

def _bwd_case(seed, B=2, H=1, N=4, T=7, shared_state=False):
    rng = np.random.default_rng(seed)
    C = H * N
    case = {
        "r": rng.standard_normal((B, T, C)), "k": rng.standard_normal((B, T, C)),
        "v": rng.standard_normal((B, T, C)), "x": rng.uniform(-3.0, 1.0, (B, T, C)),
        "u": rng.standard_normal(C) * 0.5,
        "state": rng.standard_normal((1 if shared_state else B, H, N, N)) * 0.3,
        "dy": rng.standard_normal((B, T, C)), "dso": rng.standard_normal((B, H, N, N)),
    }
    case["map"] = np.zeros(B, dtype=np.int64) if shared_state else np.arange(B)
    return case, H, N


def _loss(c, H, N):
    """L = sum(dy * y) + sum(dso * S_final) through the forward oracle."""
    y, S = oracle.wkv56(c["r"], c["k"], c["v"], c["x"], c["u"], H, N, state=c["state"],
                        state_map=c["map"], threads=1)
    return float(np.sum(c["dy"] * y) + np.sum(c["dso"] * S))


def _fd_grads(c, H, N, h=1e-6):
    """Central differences of the forward oracle's loss, element by element."""
    out = {}
    for name in ("r", "k", "v", "x", "u", "state"):
        g = np.zeros_like(c[name])
        flat = c[name].reshape(-1)
        gf = g.reshape(-1)
        for e in range(flat.size):
            keep = flat[e]
            flat[e] = keep + h
            lp = _loss(c, H, N)
            flat[e] = keep - h
            lm = _loss(c, H, N)
            flat[e] = keep
            gf[e] = (lp - lm) / (2 * h)
        out[name] = g
    return out


def _check_bwd_against_fd(c, H, N, lib=None, tol=1e-6):
    dr, dk, dv, dx, du, du_rows, dS = oracle.wkv6_backward(
        c["r"], c["k"], c["v"], c["x"], c["u"], H, N, c["dy"], state=c["state"], state_map=c["map"],
        d_state_out=c["dso"], threads=1, lib=lib)
    fd = _fd_grads(c, H, N)
    # the gradient of a shared initial state row is the sum over the batch rows that started from it
    dstate = np.zeros_like(c["state"])
    for b, row in enumerate(c["map"]):
        dstate[row] += dS[b]
    errs = {"r": relerr(dr, fd["r"]), "k": relerr(dk, fd["k"]), "v": relerr(dv, fd["v"]),
            "x": relerr(dx, fd["x"]), "u": relerr(du, fd["u"]), "state": relerr(dstate, fd["state"])}
    return errs, du_rows


@pytest.mark.parametrize("shared_state", [False, True])
def test_v6_backward_matches_finite_differences(shared_state):
    """Every gradient of the backward oracle equals central differences of the forward oracle's
    loss sum(dy * y) + sum(dS * S_final) (fp64, step 1e-6: agreement to about 1e-8)."""
    c, H, N = _bwd_case(5, shared_state=shared_state)
    errs, du_rows = _check_bwd_against_fd(c, H, N)
    assert max(errs.values()) < 1e-6, errs
    assert np.allclose(du_rows.sum(axis=0), oracle.wkv6_backward(
        c["r"], c["k"], c["v"], c["x"], c["u"], H, N, c["dy"], state=c["state"], state_map=c["map"],
        d_state_out=c["dso"], threads=1)[4], rtol=0, atol=0)


def test_v6_backward_two_heads_and_no_state():
    """Two heads (the per-head channel offsets) and a zero initial state with no state gradient in."""
    c, H, N = _bwd_case(8, B=1, H=2, N=3, T=5)
    c["state"] = np.zeros_like(c["state"])
    c["dso"] = np.zeros_like(c["dso"])
    errs, _ = _check_bwd_against_fd(c, H, N)
    assert max(errs.values()) < 1e-6, errs


def test_v6_backward_is_linear_in_upstream_gradients():
    c, H, N = _bwd_case(11, N=5, T=9)
    args = (c["r"], c["k"], c["v"], c["x"], c["u"], H, N)
    g1 = oracle.wkv6_backward(*args, c["dy"], state=c["state"], d_state_out=c["dso"], threads=1)
    g2 = oracle.wkv6_backward(*args, 2.0 * c["dy"], state=c["state"], d_state_out=2.0 * c["dso"], threads=1)
    for a, b2 in zip(g1, g2):
        assert np.array_equal(2.0 * a, b2)  # scaling by 2 is exact in binary floating point


_BWD_MUTANTS = {
    "dk_drops_bonus": ("dk[(long)t * ts + i] = b + u[i] * rt[i] * dyv;", "dk[(long)t * ts + i] = b;"),
    "G_not_decayed": ("G[i * N + j] = d * G[i * N + j] + rt[i] * dyt[j];", "G[i * N + j] = G[i * N + j] + rt[i] * dyt[j];"),
    "dx_missing_d": ("dx[(long)t * ts + i] = c * d * (-ex);", "dx[(long)t * ts + i] = c * (-ex);"),
    "dv_transposed": ("for (int i = 0; i < N; i++) a += G[i * N + j] * kt[i];", "for (int i = 0; i < N; i++) a += G[j * N + i] * kt[i];"),
    "dr_state_after": ("a += dyt[j] * (Sp[i * N + j] + u[i] * kt[i] * vt[j]);", "a += dyt[j] * (Sp[NN + i * N + j] + u[i] * kt[i] * vt[j]);"),
}


@pytest.mark.parametrize("name", sorted(_BWD_MUTANTS))
def test_backward_pins_catch_planted_mistakes(name):
    """A mistake planted in a copy of the backward oracle must fail the finite-difference pin."""
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(os.path.join(os.path.dirname(oracle.__file__), "wkv_oracle.c")).read()
    old, new = _BWD_MUTANTS[name]
    assert src.count(old) == 1, name
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        so = os.path.join(d, "mutant.so")
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", path, "-o", so, "-lm"])
        lib = oracle.load(so)
        c, H, N = _bwd_case(5)
        errs, _ = _check_bwd_against_fd(c, H, N, lib=lib)
        assert max(errs.values()) > 1e-4, f"mutant {name} passed the pin: {errs}"
