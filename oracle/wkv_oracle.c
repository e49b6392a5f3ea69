/*
 * fp64 CPU oracle of the RWKV WKV time-mixing recurrences.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, calls or
 * includes this file; only the tests, the smoke check and the benchmark's CPU
 * baseline load it.  It shares no code with the HIP kernels.
 *
 * Every function is the definition written out in double precision, one
 * token at a time, with no blocking, fusion or reordering.  Inputs arrive as
 * doubles holding the exact stored input values (bf16 / fp32 widen exactly).
 *
 * Sources.  The pages name the operators and their arguments but print no
 * formula:
 *   - RWKV-v4 walk-through blog ("代码连连看——RWKV"), RWKV_TimeMix.forward:
 *     the WKV call takes (B, T, C, time_decay, time_first, k, v) and its
 *     result is gated by sigmoid(r).  The v4 formula used here is the standard
 *     RWKV-4 weighted average with per-step decay exp(-exp(time_decay)) and
 *     the bonus exp(time_first) on the current token.
 *   - rwkv_ops package page, "rwkv6op 使用方法" call table: r, k, v, w of shape
 *     (batch, seq, hidden), u of shape (heads, head_size), init_state of shape
 *     (n_state, heads, head_size, head_size), state_map picking each row's
 *     initial state, y_state the final state.  The v5/v6 recurrence used here
 *     is the standard RWKV-5/6 one:
 *         y_t[j] = sum_i r_t[i] * (S[i][j] + u[i] * k_t[i] * v_t[j])
 *         S[i][j] <- d_t[i] * S[i][j] + k_t[i] * v_t[j]
 *     with d_t[i] = exp(-exp(x_t[i])) (x constant over t for v5), S indexed
 *     [key i][value j].
 *
  *   - rwkv_ops page, generalized_delta_rule interface (rwkv7 "generalized
 *     delta rule"): r, w, k, v, a, b of shape [B, T, H, K], initial_state
 *     [N, H, K, V].  The page prints no formula; the recurrence used here is
 *     the standard RWKV-7 one, with the state h indexed [key i][value j] as
 *     the page's [.., K, V] layout:
 *         sa[j]    = sum_i a_t[i] h[i][j]
 *         h[i][j] <- d_t[i] h[i][j] + b_t[i] sa[j] + k_t[i] v_t[j]
 *         y_t[j]   = sum_i r_t[i] h[i][j]          (after the update)
 *     with d_t = exp(-exp(w_t)), the rwkv6op parameterisation: the page's
 *     padding note for this operator (w += (1 - mask) * -1e9, handled for
 *     left and right padding by the recurrent operator) needs a padded
 *     token's decay to be exactly 1, which exp(-exp(-1e9)) is.
 *
 * Pins (tests/test_oracle_pins.py): closed-form weighted sums, O(T^2 N^2)
 * brute force, exact rational arithmetic on tiny cases, the no-decay case
 * equal to causal linear attention by matrix product, the full-decay case,
 * chunk-carry invariance, linearity, v5 == v6 with constant decay, and the
 * v4 <-> v5(N=1) mapping; for v7, products of explicit transition matrices,
 * the delta rule's exact recall, v7 with a = 0 against v5, linearity and
 * chunk-carry invariance.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no HIP headers).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

/*
 * v4, one batch row, channels [c0, c1).
 *
 * Definition (per channel c, lambda = -exp(tau[c])):
 *   A_t = sum_{i<t} exp((t-1-i)*lambda + k_i) * v_i + exp(t*lambda) * A_0
 *   B_t = sum_{i<t} exp((t-1-i)*lambda + k_i)       + exp(t*lambda) * B_0
 *   wkv_t = (A_t + exp(u + k_t) * v_t) / (B_t + exp(u + k_t))
 *   y_t = sigmoid(r_t) * wkv_t   if r is given, else wkv_t
 * evaluated through A_{t+1} = exp(lambda) * A_t + exp(k_t) * v_t (and the
 * same for B).  A_0, B_0 are the numerator and denominator carried in from a
 * previous call (zero for a fresh sequence); the final A_T, B_T are returned.
 *
 * k, v, r, y point at element [b, 0, 0] of a [B, T, C] row-major array.
 */
void oracle_wkv4_row(int T, int C, int c0, int c1,
                     const double *tau, const double *u,
                     const double *k, const double *v, const double *r,
                     const double *A0, const double *B0,
                     double *y, double *A_out, double *B_out)
{
    for (int c = c0; c < c1; c++) {
        double decay = exp(-exp(tau[c]));
        double A = A0 ? A0[c] : 0.0;
        double Bd = B0 ? B0[c] : 0.0;
        for (int t = 0; t < T; t++) {
            long e = (long)t * C + c;
            double kt = k[e], vt = v[e];
            double bonus = exp(u[c] + kt);
            double wkv = (A + bonus * vt) / (Bd + bonus);
            if (r)
                wkv = wkv / (1.0 + exp(-r[e]));
            y[e] = wkv;
            double ek = exp(kt);
            A = decay * A + ek * vt;
            Bd = decay * Bd + ek;
        }
        if (A_out) A_out[c] = A;
        if (B_out) B_out[c] = Bd;
    }
}

/*
 * v5 / v6, one (batch row, head) unit.
 *
 * r, k, v, y point at element [b, 0, h*N] of a [B, T, H*N] array whose token
 * stride is ts elements.  x points at the head's decay parameters: for v6 at
 * [b, 0, h*N] with token stride xs = ts, for v5 at [h*N] with xs = 0.
 * u points at [h*N].  S0 is the [N][N] initial state (NULL: zero), S_out
 * receives the state after the last token (NULL: not returned).
 */
void oracle_wkv56_head(int T, int N, long ts,
                       const double *r, const double *k, const double *v,
                       const double *x, long xs, const double *u,
                       const double *S0, double *y, double *S_out)
{
    double *S = (double *)malloc(sizeof(double) * (size_t)N * (size_t)N);
    if (!S) return;
    if (S0)
        memcpy(S, S0, sizeof(double) * (size_t)N * (size_t)N);
    else
        memset(S, 0, sizeof(double) * (size_t)N * (size_t)N);

    for (int t = 0; t < T; t++) {
        const double *rt = r + (long)t * ts;
        const double *kt = k + (long)t * ts;
        const double *vt = v + (long)t * ts;
        const double *xt = x + (long)t * xs;
        double *yt = y + (long)t * ts;
        /* output reads the state before this token's update, plus the bonus */
        for (int j = 0; j < N; j++) {
            double acc = 0.0;
            for (int i = 0; i < N; i++)
                acc += rt[i] * (S[i * N + j] + u[i] * kt[i] * vt[j]);
            yt[j] = acc;
        }
        /* decay every key row, then add this token's outer product */
        for (int i = 0; i < N; i++) {
            double d = exp(-exp(xt[i]));
            for (int j = 0; j < N; j++)
                S[i * N + j] = d * S[i * N + j] + kt[i] * vt[j];
        }
    }
    if (S_out)
        memcpy(S_out, S, sizeof(double) * (size_t)N * (size_t)N);
    free(S);
}

/*
 * v6 backward, one (batch row, head) unit: the gradients of
 *   L = sum_t sum_j dy_t[j] y_t[j] + sum_ij dS_T[i][j] S_T[i][j]
 * with respect to r, k, v, x, u and the initial state, where y and the final
 * state S_T come from oracle_wkv56_head (same arguments).  This is reverse-mode
 * differentiation of the forward definition, one token at a time: the forward
 * states before every token are kept, then the tokens are walked backwards
 * with G = dL/dS_t (G = dS_T after the last token):
 *   dr_t[i] = sum_j dy_t[j] (S_{t-1}[i][j] + u[i] k_t[i] v_t[j])
 *   dk_t[i] = sum_j G[i][j] v_t[j] + u[i] r_t[i] (dy_t . v_t)
 *   dv_t[j] = sum_i G[i][j] k_t[i] + (sum_i r_t[i] u[i] k_t[i]) dy_t[j]
 *   du[i]  += r_t[i] k_t[i] (dy_t . v_t)
 *   dx_t[i] = (sum_j G[i][j] S_{t-1}[i][j]) * d_t[i] * (-exp(x_t[i]))
 *   G[i][j] <- d_t[i] G[i][j] + r_t[i] dy_t[j]        (now dL/dS_{t-1})
 * and dS_0 = G at the end.  du accumulates (+=) into the caller's array.
 * dy, dr, dk, dv, dx use token stride ts like r; dST may be NULL (zero).
 * The gradient of the decay parameter is per token (v6: x of shape [B,T,C]).
 */
void oracle_wkv6_head_bwd(int T, int N, long ts,
                          const double *r, const double *k, const double *v,
                          const double *x, const double *u, const double *S0,
                          const double *dy, const double *dST,
                          double *dr, double *dk, double *dv, double *dx,
                          double *du, double *dS0)
{
    size_t NN = (size_t)N * (size_t)N;
    double *hist = (double *)malloc(sizeof(double) * NN * (size_t)(T + 1));
    double *G = (double *)malloc(sizeof(double) * NN);
    if (!hist || !G) { free(hist); free(G); return; }
    /* forward: hist[t] is the state before token t */
    if (S0) memcpy(hist, S0, sizeof(double) * NN);
    else memset(hist, 0, sizeof(double) * NN);
    for (int t = 0; t < T; t++) {
        const double *kt = k + (long)t * ts, *vt = v + (long)t * ts, *xt = x + (long)t * ts;
        const double *Sp = hist + (size_t)t * NN;
        double *Sn = hist + (size_t)(t + 1) * NN;
        for (int i = 0; i < N; i++) {
            double d = exp(-exp(xt[i]));
            for (int j = 0; j < N; j++)
                Sn[i * N + j] = d * Sp[i * N + j] + kt[i] * vt[j];
        }
    }
    if (dST) memcpy(G, dST, sizeof(double) * NN);
    else memset(G, 0, sizeof(double) * NN);
    for (int t = T - 1; t >= 0; t--) {
        const double *rt = r + (long)t * ts, *kt = k + (long)t * ts, *vt = v + (long)t * ts;
        const double *xt = x + (long)t * ts, *dyt = dy + (long)t * ts;
        const double *Sp = hist + (size_t)t * NN;
        double dyv = 0.0, bonus = 0.0;
        for (int j = 0; j < N; j++) dyv += dyt[j] * vt[j];
        for (int i = 0; i < N; i++) bonus += rt[i] * u[i] * kt[i];
        for (int i = 0; i < N; i++) {
            double a = 0.0, b = 0.0, c = 0.0;
            for (int j = 0; j < N; j++) {
                a += dyt[j] * (Sp[i * N + j] + u[i] * kt[i] * vt[j]);
                b += G[i * N + j] * vt[j];
                c += G[i * N + j] * Sp[i * N + j];
            }
            double ex = exp(xt[i]);
            double d = exp(-ex);
            dr[(long)t * ts + i] = a;
            dk[(long)t * ts + i] = b + u[i] * rt[i] * dyv;
            dx[(long)t * ts + i] = c * d * (-ex);
            du[i] += rt[i] * kt[i] * dyv;
        }
        for (int j = 0; j < N; j++) {
            double a = 0.0;
            for (int i = 0; i < N; i++) a += G[i * N + j] * kt[i];
            dv[(long)t * ts + j] = a + bonus * dyt[j];
        }
        for (int i = 0; i < N; i++) {
            double d = exp(-exp(xt[i]));
            for (int j = 0; j < N; j++)
                G[i * N + j] = d * G[i * N + j] + rt[i] * dyt[j];
        }
    }
    if (dS0) memcpy(dS0, G, sizeof(double) * NN);
    free(hist);
    free(G);
}

/*
 * v7 (generalized delta rule), one (batch row, head) unit.
 *
 * r, w, k, v, a, b, y point at element [b, 0, h*N] of [B, T, H*N] arrays with
 * token stride ts.  w is the raw decay parameter: the decay of key row i at
 * token t is exp(-exp(w_t[i])).  S0 is the [N][N] initial state h[i][j] (NULL:
 * zero), S_out receives the state after the last token (NULL: not returned).
 * Per token, in this order: sa = a_t^T h (over the key rows), the update
 *   h[i][j] <- d_t[i] h[i][j] + b_t[i] sa[j] + k_t[i] v_t[j],
 * then y_t = r_t^T h with the updated state.
 */
void oracle_wkv7_head(int T, int N, long ts,
                      const double *r, const double *w, const double *k,
                      const double *v, const double *a, const double *b,
                      const double *S0, double *y, double *S_out)
{
    size_t NN = (size_t)N * (size_t)N;
    double *S = (double *)malloc(sizeof(double) * NN);
    double *sa = (double *)malloc(sizeof(double) * (size_t)N);
    if (!S || !sa) { free(S); free(sa); return; }
    if (S0) memcpy(S, S0, sizeof(double) * NN);
    else memset(S, 0, sizeof(double) * NN);
    for (int t = 0; t < T; t++) {
        const double *rt = r + (long)t * ts, *wt = w + (long)t * ts, *kt = k + (long)t * ts;
        const double *vt = v + (long)t * ts, *at = a + (long)t * ts, *bt = b + (long)t * ts;
        double *yt = y + (long)t * ts;
        for (int j = 0; j < N; j++) {
            double acc = 0.0;
            for (int i = 0; i < N; i++) acc += at[i] * S[i * N + j];
            sa[j] = acc;
        }
        for (int i = 0; i < N; i++) {
            double d = exp(-exp(wt[i]));
            for (int j = 0; j < N; j++)
                S[i * N + j] = d * S[i * N + j] + bt[i] * sa[j] + kt[i] * vt[j];
        }
        for (int j = 0; j < N; j++) {
            double acc = 0.0;
            for (int i = 0; i < N; i++) acc += rt[i] * S[i * N + j];
            yt[j] = acc;
        }
    }
    if (S_out) memcpy(S_out, S, sizeof(double) * NN);
    free(S);
    free(sa);
}
