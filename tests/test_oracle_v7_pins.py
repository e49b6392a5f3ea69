"""Pins of the fp64 v7 oracle (the generalized delta rule) against mathematics it does not contain.

The rwkv_ops page gives the operator's interface (generalized_delta_rule: r, w, k, v, a, b of
shape [B, T, H, K], initial_state [N, H, K, V]) but no formula; the reading is the standard RWKV-7
recurrence on the state h[key][value]:
    h_t = A_t h_{t-1} + k_t v_t^T,   A_t = diag(d_t) + b_t a_t^T,   y_t = h_t^T r_t,
with the decay d_t = exp(-exp(w_t)) of rwkv6op: the page's padding note for this operator
(w += (1 - mask) * -1e9, left and right padding handled by the recurrent operator) needs a padded
token's decay to be exactly 1.

Pins:
  * the closed form h_t = sum_s (A_t ... A_{s+1}) k_s v_s^T + (A_t ... A_0) h_init, with every
    transition matrix built explicitly and multiplied out (no running state);
  * the delta rule's recall: with no decay (w = -1e9, the page's padding value), a = -kappa,
    b = kappa for a unit kappa and k = kappa, the state maps kappa to v_t exactly, so y_t = v_t
    for r_t = kappa;
  * padded tokens (w = -1e9, zero r, k, v, a, b) leave the state exactly as it was, on the left
    and on the right;
  * with a = 0 and a decay constant in time, v7 is the v5 oracle (itself pinned elsewhere) with
    r scaled by the decay and u = 1 / decay;
  * scaling v and the initial state by 2 scales y and the state exactly; splitting a sequence
    with the state carried over is bitwise equal to one pass;
  * planted mistakes in a copy of the oracle fail a pin.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from wkv_inputs import stored_f32, wkv7_inputs


def _f(inp, n):
    return stored_f32(inp[n]).astype(np.float64)


def v7_closed_form(r, w, k, v, a, b, S0):
    """One head, arrays [T, N]: outputs and final state from explicit transition products."""
    T, N = r.shape
    A = [np.diag(np.exp(-np.exp(w[t]))) + np.outer(b[t], a[t]) for t in range(T)]
    y = np.zeros((T, N))
    Ht = S0.copy()
    for t in range(T):
        P = np.eye(N)
        Ht = np.zeros((N, N))
        for s in range(t, -1, -1):
            Ht += P @ np.outer(k[s], v[s])
            P = P @ A[s]
        Ht += P @ S0
        y[t] = r[t] @ Ht
    return y, Ht


def _relerr(got, ref):
    scale = max(float(np.sqrt(np.mean(ref ** 2))), 1e-300)
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), scale)))


@pytest.mark.parametrize("N,T,dtype", [(4, 12, "f32"), (8, 10, "bf16"), (64, 5, "f32")])
def test_v7_matches_transition_products(N, T, dtype):
    inp = wkv7_inputs(2, T, 2, N, seed=N + T, dtype=dtype, init_state=3)
    smap = np.array([2, 0], dtype=np.int32)
    y, S = oracle.wkv7(*(inp[n] for n in ("r", "w", "k", "v", "a", "b")), 2, N, state=inp["state"],
                       state_map=smap)
    f = {n: _f(inp, n) for n in ("r", "w", "k", "v", "a", "b")}
    for bb in range(2):
        for h in range(2):
            sl = slice(h * N, (h + 1) * N)
            yc, Sc = v7_closed_form(*(f[n][bb, :, sl] for n in ("r", "w", "k", "v", "a", "b")),
                                    inp["state"][smap[bb], h].astype(np.float64))
            assert _relerr(y[bb, :, sl], yc) < 1e-12
            assert _relerr(S[bb, h], Sc) < 1e-12


def test_v7_delta_rule_recalls_the_written_value():
    """No decay, a = -kappa, b = kappa, k = kappa (unit): h <- (I - kappa kappa^T) h + kappa v^T,
    so kappa^T h = v^T after the token whatever the state was: reading with r = kappa gives v."""
    rng = np.random.default_rng(3)
    T, N = 6, 16
    kappa = rng.standard_normal((1, T, N))
    kappa /= np.linalg.norm(kappa, axis=-1, keepdims=True)
    v = rng.standard_normal((1, T, N))
    no_decay = np.full((1, T, N), -1e9)
    state = rng.standard_normal((1, 1, N, N))
    y, S = oracle.wkv7(kappa, no_decay, kappa, v, -kappa, kappa, 1, N, state=state)
    assert np.max(np.abs(y - v)) < 1e-12
    # the last written pair is stored in the final state
    assert np.max(np.abs(kappa[0, -1] @ S[0, 0] - v[0, -1])) < 1e-12


def test_v7_without_a_is_v5():
    """a = 0 and a decay d constant in time: y_t = sum_{s<=t} r_t . (d^(t-s) k_s) v_s + ..., which is
    v5 with r' = r d (one extra decay step), the bonus u = 1 / d and the same decay parameter."""
    B, T, H, N = 2, 9, 2, 8
    inp = wkv7_inputs(B, T, H, N, seed=11, dtype="f32", init_state=B)
    w = np.repeat(inp["w"][:, :1, :], T, axis=1)  # constant over time, per (row, channel)
    w = np.broadcast_to(w[:1], w.shape).copy()    # and the same in every row (v5 is per channel)
    d = np.exp(-np.exp(w[0, 0].astype(np.float64)))
    zeros = np.zeros_like(inp["a"])
    y7, S7 = oracle.wkv7(inp["r"], w, inp["k"], inp["v"], zeros, inp["b"], H, N, state=inp["state"])
    r5 = _f(inp, "r") * d
    x5 = w[0, 0].astype(np.float64)
    y5, S5 = oracle.wkv56(r5, inp["k"], inp["v"], x5, 1.0 / d, H, N, state=inp["state"])
    assert _relerr(y7, y5) < 1e-12
    assert _relerr(S7, S5) < 1e-12


@pytest.mark.parametrize("side", ["left", "right"])
def test_v7_padding_leaves_the_state(side):
    """The page's padding convention: padded tokens get w = -1e9 (decay exactly 1) and zero r, k, v,
    a, b, so they neither read nor change the state: the real tokens' outputs and the final state
    equal those of the unpadded call, bitwise."""
    inp = wkv7_inputs(1, 20, 2, 8, seed=19, dtype="f32", init_state=1)
    args = {n: _f(inp, n) for n in ("r", "w", "k", "v", "a", "b")}
    y, S = oracle.wkv7(*(args[n] for n in ("r", "w", "k", "v", "a", "b")), 2, 8, state=inp["state"])
    pad = {n: np.zeros((1, 7, 16)) for n in args}
    pad["w"] = np.full((1, 7, 16), -1e9)
    cat = (lambda x, q: np.concatenate([q, x], axis=1)) if side == "left" else (lambda x, q: np.concatenate([x, q], axis=1))
    yp, Sp = oracle.wkv7(*(cat(args[n], pad[n]) for n in ("r", "w", "k", "v", "a", "b")), 2, 8, state=inp["state"])
    real = slice(7, 27) if side == "left" else slice(0, 20)
    assert np.array_equal(yp[:, real], y) and np.array_equal(Sp, S)


def test_v7_scaling_and_carry_split():
    inp = wkv7_inputs(2, 40, 2, 8, seed=13, dtype="f32", init_state=2)
    args = [inp[n] for n in ("r", "w", "k", "v", "a", "b")]
    y, S = oracle.wkv7(*args, 2, 8, state=inp["state"])
    a2 = list(args)
    a2[3] = 2.0 * _f(inp, "v")
    y2, S2 = oracle.wkv7(*a2, 2, 8, state=2.0 * inp["state"].astype(np.float64))
    assert np.array_equal(y2, 2.0 * y) and np.array_equal(S2, 2.0 * S)
    cut = 17
    ya, Sa = oracle.wkv7(*(x[:, :cut] for x in args), 2, 8, state=inp["state"])
    yb, Sb = oracle.wkv7(*(x[:, cut:] for x in args), 2, 8, state=Sa)
    assert np.array_equal(np.concatenate([ya, yb], axis=1), y) and np.array_equal(Sb, S)


_V7_MUTANTS = {
    "no_sa_term": ("S[i * N + j] = d * S[i * N + j] + bt[i] * sa[j] + kt[i] * vt[j];",
                   "S[i * N + j] = d * S[i * N + j] + kt[i] * vt[j];"),
    "sa_uses_b": ("for (int i = 0; i < N; i++) acc += at[i] * S[i * N + j];",
                  "for (int i = 0; i < N; i++) acc += bt[i] * S[i * N + j];"),
    "sa_transposed": ("for (int i = 0; i < N; i++) acc += at[i] * S[i * N + j];",
                      "for (int i = 0; i < N; i++) acc += at[i] * S[j * N + i];"),
    "decay_sign": ("double d = exp(-exp(wt[i]));\n            for (int j = 0; j < N; j++)\n                S[i * N + j] = d * S[i * N + j] + bt[i]",
                   "double d = exp(-exp(-wt[i]));\n            for (int j = 0; j < N; j++)\n                S[i * N + j] = d * S[i * N + j] + bt[i]"),
    "outer_transposed": ("bt[i] * sa[j] + kt[i] * vt[j];", "bt[i] * sa[j] + kt[j] * vt[i];"),
    "output_transposed": ("for (int i = 0; i < N; i++) acc += rt[i] * S[i * N + j];",
                          "for (int i = 0; i < N; i++) acc += rt[i] * S[j * N + i];"),
}


@pytest.mark.parametrize("name", sorted(_V7_MUTANTS))
def test_v7_pins_catch_planted_mistakes(name):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(os.path.join(os.path.dirname(oracle.__file__), "wkv_oracle.c")).read()
    old, new = _V7_MUTANTS[name]
    assert src.count(old) == 1, name
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        so = os.path.join(d, "mutant.so")
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", path, "-o", so, "-lm"])
        lib = oracle.load(so)
        inp = wkv7_inputs(1, 8, 1, 4, seed=17, dtype="f32", init_state=1)
        y, S = oracle.wkv7(*(inp[n] for n in ("r", "w", "k", "v", "a", "b")), 1, 4, state=inp["state"],
                           lib=lib, threads=1)
        f = {n: _f(inp, n) for n in ("r", "w", "k", "v", "a", "b")}
        yc, Sc = v7_closed_form(*(f[n][0] for n in ("r", "w", "k", "v", "a", "b")),
                                inp["state"][0, 0].astype(np.float64))
        assert _relerr(y[0], yc) > 1e-9 or _relerr(S[0, 0], Sc) > 1e-9, f"mutant {name} passed the pin"
