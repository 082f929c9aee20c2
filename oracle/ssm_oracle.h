/*
 * ssm_oracle.h -- fp64 CPU oracle for the selective state-space scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this code; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or constant with the
 * HIP library.
 *
 * What it computes (every array is fp64, C-contiguous, owned by the caller):
 *
 *   for every (b, d):                      channels are independent
 *     h[n] = h0[b,d,n]  (or 0)
 *     for t = 0 .. L-1:
 *       x      = delta[b,d,t] + bias[d]          (bias may be NULL -> 0)
 *       dt     = softplus(x) if delta_softplus else x
 *       for n:  dA    = exp(dt * A[d,n])
 *               dBu   = dt * B[b,n,t] * u[b,d,t]                 (zoh_b == 0)
 *                     = (exp(dt*A[d,n]) - 1) / A[d,n] * B[b,n,t] * u[b,d,t]
 *                                                               (zoh_b == 1)
 *               h[n]  = dA * h[n] + dBu
 *       yv = sum_n C[b,n,t] * h[n]  (+ D[d] * u[b,d,t])
 *       y[b,d,t] = yv * silu(z[b,d,t])   (z may be NULL -> no gate)
 *     h_final[b,d,:] = h
 *
 * Sources (web pages this follows):
 *  - "Mamba & State Space Models - Guide Complet", section 4 "Implementation du
 *    SSM selectif (S6)": per-token loop with A = -exp(A_log) fixed per channel,
 *    delta = softplus(dt_proj(x)) (bias inside the projection), A_bar =
 *    exp(delta*A), h = h*A_bar + (..)*x_t, readout y_t = h.C_t + D*x_t;
 *    section 1 "Discretisation": exact ZOH  B_bar = (exp(dA)-I) A^-1 B.
 *  - "Mamba и State Space Models: альтернатива Transformer", section "SSM as
 *    RNN": B_scaled = B*delta (Euler input discretisation), y = C*h_new
 *    (readout after the update); section "Selective SSM": y * silu(gate).
 *  - "Mamba: co potrafia modele przestrzeni stanow", section on selection:
 *    delta, B and C are functions of the current token; A stays fixed.
 */
#ifndef SSM_ORACLE_H
#define SSM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Full sequential scan.  Shapes:
 *   u, delta, z, y : (batch, dim, seqlen)     A : (dim, dstate)
 *   B, C           : (batch, dstate, seqlen)  D, delta_bias : (dim)
 *   h0, h_final    : (batch, dim, dstate)
 * Nullable: D, z, delta_bias, h0, h_final.  Returns 0, or -1 on a bad
 * argument (NULL required pointer, negative size, dstate > 4096). */
int oracle_scan_f64(const double *u, const double *delta, const double *A,
                    const double *B, const double *C, const double *D,
                    const double *z, const double *delta_bias,
                    int delta_softplus, int zoh_b, const double *h0,
                    double *y, double *h_final, int64_t batch, int64_t dim,
                    int64_t dstate, int64_t seqlen);

/* One token of the same recurrence (the recurrent / decoding mode).
 *   state : (batch, dim, dstate), read and written in place
 *   x, delta, z, y : (batch, dim)     B, C : (batch, dstate)
 * Nullable: D, z, delta_bias. */
int oracle_step_f64(double *state, const double *x, const double *delta,
                    const double *A, const double *B, const double *C,
                    const double *D, const double *z,
                    const double *delta_bias, int delta_softplus, int zoh_b,
                    double *y, int64_t batch, int64_t dim, int64_t dstate);

/* softplus(x) = log(1 + e^x), evaluated without overflow or cancellation. */
double oracle_softplus(double x);

/* Depthwise causal 1-D convolution followed by SiLU, the step before the
 * SSM in the Mamba block ("Mamba & State Space Models - Guide Complet",
 * section 4 architecture figure: Linear -> Conv1D -> SiLU -> SSM; the
 * convolution is depthwise (groups = channels) with padding d_conv - 1 and
 * its output trimmed to the first L positions, section 7; d_conv = 4 on the
 * inferownia.pl page, "Zrob to sam"):
 *   u[b,d,t] = silu(bias[d] + sum_{k=0}^{K-1} w[d,k] * x[b,d,t-(K-1)+k])
 * with x = 0 before t = 0.  x, u: (batch, dim, seqlen); w: (dim, K);
 * bias: (dim) or NULL.  Returns 0, or -1 on a bad argument. */
int oracle_causal_conv1d_silu_f64(const double *x, const double *w,
                                  const double *bias, int64_t K, double *u,
                                  int64_t batch, int64_t dim, int64_t seqlen);

/* Gradients of oracle_causal_conv1d_silu_f64 for a loss whose gradient
 * with respect to u is du: with pre_t = bias + sum_k w[k] x[t-(K-1)+k] and
 * g_t = du_t * silu'(pre_t),
 *   dx[s]   = sum_k w[k] g_{s+(K-1)-k}   (terms with s+(K-1)-k < seqlen)
 *   dw[d,k] = sum_{b,t} g_t x[t-(K-1)+k]  (x = 0 before t = 0)
 *   db[d]   = sum_{b,t} g_t
 * dx: (batch, dim, seqlen); dw: (dim, K), db: (dim) or NULL, overwritten.
 * Returns 0, or -1 on a bad argument. */
int oracle_causal_conv1d_silu_bwd_f64(const double *x, const double *w,
                                      const double *bias, int64_t K,
                                      const double *du, double *dx, double *dw,
                                      double *db, int64_t batch, int64_t dim,
                                      int64_t seqlen);

/* Gradients of the full scan, by the chain rule applied to the recurrence
 * above, token by token in reverse.  The loss is any scalar whose gradient
 * with respect to y is dy and with respect to h_final is dh_final (NULL ->
 * 0).  The inferownia.pl page ("Cena selekcji") states that the backward
 * pass recomputes the intermediate states rather than storing them; this
 * reference simply keeps the whole (L+1) x N state history of one channel,
 * which is the plain definition, not that optimisation.  With c the input
 * coefficient of oracle_scan_f64 (dt for Euler; (exp(dt A_n) - 1)/A_n for
 * exact zero-order hold, "Mamba & State Space Models - Guide Complet",
 * section 1), dc/ddt = 1 (Euler) or exp(dt A_n) (ZOH) and dc/dA_n = 0
 * (Euler) or (dt exp(dt A_n) - c)/A_n (ZOH; dt^2/2 at A_n = 0):
 *
 *   per (b, d): forward, keeping h_t for t = -1..L-1 and yc_t (pre-gate y);
 *   g = dh_final; for t = L-1 .. 0:
 *     s = silu(z_t), gc = dy_t * s;  dz_t = dy_t * yc_t * silu'(z_t)
 *     dD += gc * u_t;  du_t = gc * D
 *     for n: g[n] += gc * C[n,t];  dC[n,t] += gc * h_t[n]
 *            a = exp(dt A_n);  ddt += g[n] * (A_n a h_{t-1}[n] + dc/ddt B[n,t] u_t)
 *            dA[n] += g[n] (dt a h_{t-1}[n] + dc/dA_n B[n,t] u_t)
 *            dB[n,t] += g[n] c u_t;  du_t += g[n] c B[n,t];  g[n] *= a
 *     dx = ddt * sigmoid(x) (softplus) or ddt;  ddelta_t = dx;  dbias += dx
 *   dh0 = g.
 * Outputs (fp64): du, ddelta (batch, dim, seqlen); dA (dim, dstate);
 * dB, dC (batch, dstate, seqlen) summed over channels; dD, ddelta_bias
 * (dim) summed over batch and tokens; dz (batch, dim, seqlen); dh0 (batch,
 * dim, dstate).  Nullable inputs: D, z, delta_bias, h0, dh_final; nullable
 * outputs: dD (required when D is given), ddelta_bias, dz, dh0.  Summed
 * outputs are overwritten, not accumulated into.  Returns 0, or -1 on a bad
 * argument or when memory for the state history cannot be had. */
int oracle_scan_bwd_f64(const double *u, const double *delta, const double *A,
                        const double *B, const double *C, const double *D,
                        const double *z, const double *delta_bias,
                        int delta_softplus, int zoh_b, const double *h0,
                        const double *dy, const double *dh_final, double *du,
                        double *ddelta, double *dA, double *dB, double *dC,
                        double *dD, double *ddelta_bias, double *dz,
                        double *dh0, int64_t batch, int64_t dim,
                        int64_t dstate, int64_t seqlen);

/* Mamba-2 "SSD" (state space dual) form ("Mamba & State Space Models -
 * Guide Complet", section 5: d_state 64-256, y = (L o S) u with L the causal
 * mask (1 where t >= s) and S a structured semiseparable matrix).  Reading
 * taken (the page gives no more): one scalar decay A[h] per head, a step
 * dt[b,h,t] = softplus(dt_raw + dt_bias[h]) per head and token, B and C
 * shared by the heads of a group (nheads / ngroups heads per group), Euler
 * input term; then
 *   S[t,s]     = (sum_n C[b,g,n,t] B[b,g,n,s]) * exp(A[h] (cum_t - cum_s)) * dt_s,
 *                cum_t = sum_{r<=t} dt_r
 *   y[b,h,p,t] = sum_{s<=t} S[t,s] x[b,h,p,s]
 *              + sum_n C[b,g,n,t] exp(A[h] cum_t) h0[b,h,p,n]     (h0 given)
 *              + D[h] x[b,h,p,t],   then * silu(z[b,h,p,t])        (z given)
 *   h_final[b,h,p,n] = exp(A[h] cum_{L-1}) h0[b,h,p,n]
 *              + sum_s exp(A[h] (cum_{L-1} - cum_s)) dt_s x[b,h,p,s] B[b,g,n,s]
 * computed directly as the O(L^2) masked matrix product (the definition).
 * Shapes: x, z, y (batch, nheads, headdim, L); dt (batch, nheads, L);
 * A, D, dt_bias (nheads); B, C (batch, ngroups, N, L); h0, h_final (batch,
 * nheads, headdim, N).  Nullable: D, z, dt_bias, h0, h_final.  Returns 0,
 * or -1 on a bad argument. */
int oracle_ssd_f64(const double *x, const double *dt, const double *A,
                   const double *B, const double *C, const double *D,
                   const double *z, const double *dt_bias, int dt_softplus,
                   const double *h0, double *y, double *h_final,
                   int64_t batch, int64_t nheads, int64_t headdim,
                   int64_t ngroups, int64_t dstate, int64_t seqlen);

#ifdef __cplusplus
}
#endif
#endif /* SSM_ORACLE_H */
