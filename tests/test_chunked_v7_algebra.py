"""The chunk-level algebra of the chunked v7 forward, in fp64, against the oracle.

The rwkv_ops page names a chunkwise form of its generalized_delta_rule operator next to the
recurrent one.  The chunked kernel rewrites the standard RWKV-7 recurrence
  sa_t = a_t^T h_{t-1},  h_t = diag(d_t) h_{t-1} + b_t sa_t^T + k_t v_t^T,  y_t = h_t^T r_t
over chunks of up to 64 tokens from the chunk's start state H0.  With P_t the inclusive in-chunk
sum of the log decays -exp(w) and, as rows,
  Ab_t = e^{P_{t-1}} a_t,  Rb_t = e^{P_t} r_t,  Bt_s = e^{-P_s} b_s,  Kt_s = e^{-P_s} k_s,
  (I - M) SA = RHS,  M = tril_{-1}(Ab Bt^T),  RHS = Ab H0 + tril_{-1}(Ab Kt^T) V,
  Y = Rb H0 + tril_0(Rb Bt^T) SA + tril_0(Rb Kt^T) V,
  H1 = diag(e^{P_last}) (H0 + Bt^T SA + Kt^T V).
The kernel solves the triangular system in two blocks of rows: rows 0..31 by forward
substitution, then rows 32.. receive M[32.., 0..31] SA[0..31] as one product, then rows 32.. by
forward substitution.  This test writes that rewriting out in numpy, block split included, and
checks that it reproduces the oracle to rounding; a dropped term, a wrong mask or a wrong decay
exponent would show at far above the bound, as the planted omission of the cross-block product
does.
"""
import numpy as np
import pytest

import oracle
from wkv_inputs import stored_f32, wkv7_inputs

L = 64
HALF = 32


def forward_subst(M, R):
    """Rows of (I - M) X = R in order, M strictly lower triangular."""
    X = R.copy()
    for s in range(X.shape[0]):
        X[s + 1:] += np.outer(M[s + 1:, s], X[s])
    return X


def chunked_v7(r, w, k, v, a, b, H0, cross=True):
    """One (row, head): r, w, k, v, a, b [T, N] fp64, H0 [N, N] -> y [T, N], final state."""
    T, N = r.shape
    y = np.zeros((T, N))
    H = H0.copy()
    for c0 in range(0, T, L):
        sl = slice(c0, min(T, c0 + L))
        n = sl.stop - sl.start
        P = np.cumsum(-np.exp(w[sl]), axis=0)
        Pprev = np.vstack([np.zeros((1, N)), P[:-1]])
        Ab, Rb = np.exp(Pprev) * a[sl], np.exp(P) * r[sl]
        Bt, Kt = np.exp(-P) * b[sl], np.exp(-P) * k[sl]
        V = v[sl]
        M = np.tril(Ab @ Bt.T, -1)
        RHS = Ab @ H + np.tril(Ab @ Kt.T, -1) @ V
        h = min(HALF, n)
        SA = np.zeros((n, N))
        SA[:h] = forward_subst(M[:h, :h], RHS[:h])
        if n > h:
            rest = RHS[h:] + (M[h:, :h] @ SA[:h] if cross else 0.0)
            SA[h:] = forward_subst(M[h:, h:], rest)
        y[sl] = Rb @ H + np.tril(Rb @ Bt.T) @ SA + np.tril(Rb @ Kt.T) @ V
        H = np.exp(P[-1])[:, None] * (H + Bt.T @ SA + Kt.T @ V)
    return y, H


def _case(T, seed):
    H, N = 2, 64
    inp = wkv7_inputs(1, T, H, N, seed=seed, init_state=1)
    f = {n: stored_f32(inp[n]).astype(np.float64) for n in ("r", "w", "k", "v", "a", "b")}
    yo, So = oracle.wkv7(f["r"], f["w"], f["k"], f["v"], f["a"], f["b"], H, N, state=inp["state"])
    return f, inp["state"].astype(np.float64), yo, So, H, N


@pytest.mark.parametrize("T,seed", [(20, 1), (40, 2), (64, 3), (209, 4)])
def test_chunked_v7_algebra_matches_oracle(T, seed):
    f, S0, yo, So, H, N = _case(T, seed)
    for h in range(H):
        cs = slice(h * N, (h + 1) * N)
        y, S = chunked_v7(*(f[n][0, :, cs] for n in ("r", "w", "k", "v", "a", "b")), S0[0, h])
        scale = max(1.0, float(np.abs(yo[0, :, cs]).max()))
        assert np.abs(y - yo[0, :, cs]).max() <= 1e-10 * scale, (T, h)
        assert np.abs(S - So[0, h]).max() <= 1e-10 * max(1.0, float(np.abs(So[0, h]).max())), (T, h)


def test_chunked_v7_algebra_needs_the_cross_block_product():
    f, S0, yo, So, H, N = _case(130, 5)
    cs = slice(0, N)
    y, _ = chunked_v7(*(f[n][0, :, cs] for n in ("r", "w", "k", "v", "a", "b")), S0[0, 0], cross=False)
    assert np.abs(y - yo[0, :, cs]).max() > 1e-3
