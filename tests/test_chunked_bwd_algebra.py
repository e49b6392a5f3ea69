"""The chunk-level algebra of the chunked v6 backward, in fp64, against the oracle's gradients.

The chunked kernels rewrite the reverse-mode derivative of the token recurrence (the rwkv_ops
page's RWKV6_OP, the standard RWKV-6 recurrence) as 64-token matrix products.  This test writes
that rewriting out in numpy, chunk by chunk (forward states at the chunk starts, then the chunks
in reverse with the state gradient G carried between them), and checks that it reproduces the
oracle's gradients to rounding: a dropped term, a wrong mask or a wrong decay exponent in the
algebra would show here at the 1e-2 level.  Inside a chunk of L tokens starting from S_c, with
Lam_t the inclusive in-chunk sum of the log decays lam = -exp(x):
  rb_t = r_t exp(Lam_{t-1}),  kt_s = k_s exp(-Lam_s),  A = tril_{-1}(rb kt^T),
  dV = A^T dY + diag(b) dY + kt Gh,  dA = tril_{-1}(dY V^T),  drb = dY S_c^T + dA kt,
  dkt = dA^T rb + V Gh^T,  G_c = rb^T dY + Gh,  Gh = diag(exp(Lam_{L-1})) G,
  dlam_m = sum_{t>=m} (rb_{t+1} drb_{t+1} [t+1 < L] - kt_t dkt_t) + E_{c+1},  E = rowsum(S G).
"""
import numpy as np
import pytest

import oracle
from wkv_inputs import stored_f32, wkv6_inputs, wkv6_upstream

L = 64


def chunked_backward(r, k, v, x, u, dy, S0, dST, ST):
    """One (row, head): r, k, v, x, dy [T, N] fp64; u [N]; S0, dST, ST [N, N]."""
    T, N = r.shape
    lam = -np.exp(x)
    nch = (T + L - 1) // L
    S = [S0.copy()]  # the state at every chunk start
    for c in range(nch - 1):
        sl = slice(c * L, (c + 1) * L)
        Lam = np.cumsum(lam[sl], 0)
        kt = k[sl] * np.exp(-Lam)
        S.append(np.exp(Lam[-1])[:, None] * (S[c] + kt.T @ v[sl]))
    dr, dk, dv, dx = (np.zeros_like(r) for _ in range(4))
    du = np.zeros(N)
    G = dST.copy()
    E = (ST * dST).sum(1)
    for c in reversed(range(nch)):
        sl = slice(c * L, min((c + 1) * L, T))
        n = sl.stop - sl.start
        rr, kk, vv, dd = r[sl], k[sl], v[sl], dy[sl]
        Lam = np.cumsum(lam[sl], 0)
        Lex = Lam - lam[sl]
        rb, kt = rr * np.exp(Lex), kk * np.exp(-Lam)
        Gh = np.exp(Lam[-1])[:, None] * G
        b, db = (rr * u * kk).sum(1), (dd * vv).sum(1)
        mask = np.tril(np.ones((n, n)), -1)
        A = (rb @ kt.T) * mask
        dA = (dd @ vv.T) * mask
        dv[sl] = A.T @ dd + b[:, None] * dd + kt @ Gh
        drb = dd @ S[c].T + dA @ kt
        dkt = dA.T @ rb + vv @ Gh.T
        Gc = rb.T @ dd + Gh
        dr[sl] = np.exp(Lex) * drb + u * kk * db[:, None]
        dk[sl] = np.exp(-Lam) * dkt + u * rr * db[:, None]
        du += (rr * kk * db[:, None]).sum(0)
        t1 = np.zeros_like(rr)
        t1[:-1] = (rb * drb)[1:]
        dLam = t1 - kt * dkt
        dLam[-1] += E
        dx[sl] = -np.exp(x[sl]) * np.cumsum(dLam[::-1], 0)[::-1]
        E = (S[c] * Gc).sum(1)
        G = Gc
    return dr, dk, dv, dx, du, G


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_chunked_backward_algebra_matches_oracle(T):
    B, H, N = 2, 2, 64
    inp = wkv6_inputs(B, T, H, N, seed=800 + T, dtype="f32", init_state=B)
    up = wkv6_upstream(B, T, H, N, seed=900 + T)
    ref = oracle.wkv6_backward(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], H, N, up["dy"],
                               state=inp["state"], d_state_out=up["d_state"])
    _, SF = oracle.wkv56(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], H, N, state=inp["state"])
    SF = np.asarray(SF)
    got = [np.zeros_like(np.asarray(ref[i], dtype=np.float64)) for i in (0, 1, 2, 3)]
    du = np.zeros(H * N)
    dS = np.zeros((B, H, N, N))
    for b in range(B):
        for h in range(H):
            cols = slice(h * N, (h + 1) * N)
            r, k, v, x = (stored_f32(inp[n])[b][:, cols].astype(np.float64) for n in ("r", "k", "v", "x"))
            out = chunked_backward(r, k, v, x, inp["u"][cols].astype(np.float64),
                                   up["dy"][b][:, cols].astype(np.float64), inp["state"][b, h].astype(np.float64),
                                   up["d_state"][b, h].astype(np.float64), SF[b, h].astype(np.float64))
            for i in range(4):
                got[i][b][:, cols] = out[i]
            du[cols] += out[4]
            dS[b, h] = out[5]
    for name, g, o in zip(("dr", "dk", "dv", "dw", "du", "d_state"), got + [du, dS], list(ref[:5]) + [ref[6]]):
        o = np.asarray(o, dtype=np.float64)
        e = np.abs(g - o).max() / max(np.abs(o).max(), 1e-300)
        assert e < 1e-10, f"T={T} {name}: {e:.3e}"
