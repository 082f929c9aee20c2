/*
 * ssm_oracle.c -- plain, slow fp64 reference of the selective SSM scan.
 *
 * TEST INFRASTRUCTURE ONLY (see ssm_oracle.h).  Deliberately naive: one
 * channel at a time, one token at a time, one state at a time, in the order
 * the pages write the recurrence.  No blocking, no reordering, no threads.
 * Callers that want several cores call it on disjoint channel ranges.
 */
#include "ssm_oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

/* softplus(x) = log(1 + exp(x)).  Written so neither branch overflows or
 * loses the small result: for x <= 0, log1p(e^x); for x > 0,
 * x + log1p(e^-x).  No threshold: the value is the mathematical one to
 * within libm's rounding. */
double oracle_softplus(double x)
{
    if (x <= 0.0)
        return log1p(exp(x));
    return x + log1p(exp(-x));
}

/* silu(z) = z * sigmoid(z) = z / (1 + e^-z).  For z very negative e^-z
 * overflows to +inf and the quotient is -0, which is the limit. */
static double oracle_silu(double z)
{
    return z / (1.0 + exp(-z));
}

/* Input discretisation of one state.
 *  zoh_b == 0: Euler, dB = dt * B ("SSM as RNN": B_scaled = B * delta).
 *  zoh_b == 1: exact zero-order hold for a diagonal A,
 *              dB = (exp(dt*a) - 1) / a * B  ("Discretisation", Guide
 *              Complet section 1); at a == 0 this is its limit dt * B.
 *              exp(dt*a) - 1 is evaluated by expm1, which does not lose the
 *              relative accuracy of the difference when dt*a is small. */
static double oracle_input_coeff(double dt, double a, int zoh_b)
{
    if (!zoh_b || a == 0.0)
        return dt;
    return expm1(dt * a) / a;
}

/* One token for one channel: updates h[0..N-1] in place and returns y.
 * This is the loop body of the S6 forward: discretise with the token's
 * delta, advance every state, read out through C, add the D skip, gate. */
static double oracle_token(double *h, int64_t N, double u, double draw,
                           const double *A_d, const double *B_t,
                           int64_t B_stride, const double *C_t,
                           int64_t C_stride, const double *D_d,
                           const double *z_t, const double *bias_d,
                           int delta_softplus, int zoh_b)
{
    double x = draw + (bias_d ? *bias_d : 0.0);
    double dt = delta_softplus ? oracle_softplus(x) : x;
    double yv = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        double a = A_d[n];
        double dA = exp(dt * a);
        double dBu = oracle_input_coeff(dt, a, zoh_b) * B_t[n * B_stride] * u;
        h[n] = dA * h[n] + dBu;
    }
    for (int64_t n = 0; n < N; ++n)
        yv += C_t[n * C_stride] * h[n];
    if (D_d)
        yv += (*D_d) * u;
    if (z_t)
        yv *= oracle_silu(*z_t);
    return yv;
}

int oracle_scan_f64(const double *u, const double *delta, const double *A,
                    const double *B, const double *C, const double *D,
                    const double *z, const double *delta_bias,
                    int delta_softplus, int zoh_b, const double *h0,
                    double *y, double *h_final, int64_t batch, int64_t dim,
                    int64_t dstate, int64_t seqlen)
{
    double h[4096];
    if (!u || !delta || !A || !B || !C || !y)
        return -1;
    if (batch < 0 || dim < 0 || dstate < 0 || seqlen < 0 || dstate > 4096)
        return -1;

    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < dim; ++d) {
            int64_t row = (b * dim + d) * seqlen;      /* (b, d, :) */
            int64_t srow = (b * dim + d) * dstate;     /* (b, d, :) state */
            for (int64_t n = 0; n < dstate; ++n)
                h[n] = h0 ? h0[srow + n] : 0.0;
            for (int64_t t = 0; t < seqlen; ++t) {
                /* B[b, n, t] and C[b, n, t]: stride seqlen between states */
                const double *B_t = B + b * dstate * seqlen + t;
                const double *C_t = C + b * dstate * seqlen + t;
                y[row + t] = oracle_token(
                    h, dstate, u[row + t], delta[row + t], A + d * dstate,
                    B_t, seqlen, C_t, seqlen, D ? D + d : NULL,
                    z ? z + row + t : NULL, delta_bias ? delta_bias + d : NULL,
                    delta_softplus, zoh_b);
            }
            if (h_final)
                for (int64_t n = 0; n < dstate; ++n)
                    h_final[srow + n] = h[n];
        }
    }
    return 0;
}

int oracle_step_f64(double *state, const double *x, const double *delta,
                    const double *A, const double *B, const double *C,
                    const double *D, const double *z,
                    const double *delta_bias, int delta_softplus, int zoh_b,
                    double *y, int64_t batch, int64_t dim, int64_t dstate)
{
    if (!state || !x || !delta || !A || !B || !C || !y)
        return -1;
    if (batch < 0 || dim < 0 || dstate < 0)
        return -1;

    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < dim; ++d) {
            int64_t e = b * dim + d;                   /* (b, d) */
            y[e] = oracle_token(state + e * dstate, dstate, x[e], delta[e],
                                A + d * dstate, B + b * dstate, 1,
                                C + b * dstate, 1, D ? D + d : NULL,
                                z ? z + e : NULL,
                                delta_bias ? delta_bias + d : NULL,
                                delta_softplus, zoh_b);
        }
    }
    return 0;
}

int oracle_causal_conv1d_silu_f64(const double *x, const double *w,
                                  const double *bias, int64_t K, double *u,
                                  int64_t batch, int64_t dim, int64_t seqlen)
{
    if (!x || !w || !u || K < 1 || batch < 0 || dim < 0 || seqlen < 0)
        return -1;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < dim; ++d) {
            const double *xr = x + (b * dim + d) * seqlen;
            double *ur = u + (b * dim + d) * seqlen;
            for (int64_t t = 0; t < seqlen; ++t) {
                double acc = bias ? bias[d] : 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    int64_t s = t - (K - 1) + k;   /* causal: past and present */
                    if (s >= 0)
                        acc += w[d * K + k] * xr[s];
                }
                ur[t] = oracle_silu(acc);
            }
        }
    }
    return 0;
}

/* sigmoid(x) = 1 / (1 + e^-x); the derivative of softplus. */
static double oracle_sigmoid(double x)
{
    return 1.0 / (1.0 + exp(-x));
}

/* d silu(z) / dz = sigmoid(z) * (1 + z * (1 - sigmoid(z))). */
static double oracle_dsilu(double z)
{
    double s = oracle_sigmoid(z);
    return s * (1.0 + z * (1.0 - s));
}

int oracle_causal_conv1d_silu_bwd_f64(const double *x, const double *w,
                                      const double *bias, int64_t K,
                                      const double *du, double *dx, double *dw,
                                      double *db, int64_t batch, int64_t dim,
                                      int64_t seqlen)
{
    if (!x || !w || !du || !dx || !dw || K < 1 || batch < 0 || dim < 0 || seqlen < 0)
        return -1;
    double *g = malloc(sizeof(double) * (size_t)(seqlen + 1));
    if (!g)
        return -1;
    memset(dw, 0, sizeof(double) * (size_t)(dim * K));
    if (db)
        memset(db, 0, sizeof(double) * (size_t)dim);
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < dim; ++d) {
            const double *xr = x + (b * dim + d) * seqlen;
            const double *dur = du + (b * dim + d) * seqlen;
            double *dxr = dx + (b * dim + d) * seqlen;
            /* g_t = du_t silu'(pre_t), the pre-activation recomputed */
            for (int64_t t = 0; t < seqlen; ++t) {
                double pre = bias ? bias[d] : 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    int64_t s = t - (K - 1) + k;
                    if (s >= 0)
                        pre += w[d * K + k] * xr[s];
                }
                g[t] = dur[t] * oracle_dsilu(pre);
            }
            for (int64_t s = 0; s < seqlen; ++s) {
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    int64_t t = s + (K - 1) - k;   /* the outputs x[s] feeds */
                    if (t < seqlen)
                        acc += w[d * K + k] * g[t];
                }
                dxr[s] = acc;
            }
            for (int64_t t = 0; t < seqlen; ++t) {
                for (int64_t k = 0; k < K; ++k) {
                    int64_t s = t - (K - 1) + k;
                    if (s >= 0)
                        dw[d * K + k] += g[t] * xr[s];
                }
                if (db)
                    db[d] += g[t];
            }
        }
    }
    free(g);
    return 0;
}

/* Derivatives of the input coefficient c(dt, a) of oracle_input_coeff:
 * *dc_ddt = dc/ddt and *dc_da = dc/da.  Euler: c = dt, so 1 and 0.  ZOH:
 * c = (exp(dt a) - 1)/a, dc/ddt = exp(dt a), dc/da = (dt exp(dt a) - c)/a;
 * where |dt a| < 1e-3 that difference cancels, so dc/da is taken from the
 * series dt^2 (1/2 + x/3 + x^2/8 + x^3/30 + x^4/144), x = dt a (the
 * derivative of c = dt sum_k x^k/(k+1)!; truncated below 1e-18 relative),
 * whose value at a = 0 is the limit dt^2/2. */
static void oracle_input_coeff_grad(double dt, double a, int zoh_b,
                                    double *dc_ddt, double *dc_da)
{
    if (!zoh_b) {
        *dc_ddt = 1.0;
        *dc_da = 0.0;
        return;
    }
    double x = dt * a;
    double e = exp(x);
    *dc_ddt = e;
    if (fabs(x) < 1e-3)
        *dc_da = dt * dt * (0.5 + x * (1.0 / 3.0 + x * (0.125 + x * (1.0 / 30.0 + x / 144.0))));
    else
        *dc_da = (dt * e - oracle_input_coeff(dt, a, zoh_b)) / a;
}

int oracle_scan_bwd_f64(const double *u, const double *delta, const double *A,
                        const double *B, const double *C, const double *D,
                        const double *z, const double *delta_bias,
                        int delta_softplus, int zoh_b, const double *h0,
                        const double *dy, const double *dh_final, double *du,
                        double *ddelta, double *dA, double *dB, double *dC,
                        double *dD, double *ddelta_bias, double *dz,
                        double *dh0, int64_t batch, int64_t dim, int64_t N,
                        int64_t L)
{
    if (!u || !delta || !A || !B || !C || !dy || !du || !ddelta || !dA ||
        !dB || !dC || (D && !dD))
        return -1;
    if (batch < 0 || dim < 0 || N < 0 || L < 0)
        return -1;
    double *hs = malloc(sizeof(double) * (size_t)((L + 1) * N + 2 * L + N + 1));
    if (!hs)
        return -1;
    double *yc = hs + (L + 1) * N;   /* pre-gate output per token */
    double *dts = yc + L;            /* dt per token */
    double *g = dts + L;             /* dL/dh, one channel */

    memset(dA, 0, sizeof(double) * (size_t)(dim * N));
    memset(dB, 0, sizeof(double) * (size_t)(batch * N * L));
    memset(dC, 0, sizeof(double) * (size_t)(batch * N * L));
    if (D)
        memset(dD, 0, sizeof(double) * (size_t)dim);
    if (ddelta_bias)
        memset(ddelta_bias, 0, sizeof(double) * (size_t)dim);

    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < dim; ++d) {
            int64_t row = (b * dim + d) * L;
            int64_t srow = (b * dim + d) * N;
            const double *Bb = B + b * N * L;   /* B[b, n, t] = Bb[n*L + t] */
            const double *Cb = C + b * N * L;
            const double *Ad = A + d * N;
            /* forward, keeping every state: hs[(t+1)*N + n] = h_t[n] */
            for (int64_t n = 0; n < N; ++n)
                hs[n] = h0 ? h0[srow + n] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                double x = delta[row + t] + (delta_bias ? delta_bias[d] : 0.0);
                double dt = delta_softplus ? oracle_softplus(x) : x;
                dts[t] = dt;
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    double h = exp(dt * Ad[n]) * hs[t * N + n] +
                               oracle_input_coeff(dt, Ad[n], zoh_b) *
                                   Bb[n * L + t] * u[row + t];
                    hs[(t + 1) * N + n] = h;
                    acc += Cb[n * L + t] * h;
                }
                if (D)
                    acc += D[d] * u[row + t];
                yc[t] = acc;
            }
            /* reverse */
            for (int64_t n = 0; n < N; ++n)
                g[n] = dh_final ? dh_final[srow + n] : 0.0;
            for (int64_t t = L - 1; t >= 0; --t) {
                double x = delta[row + t] + (delta_bias ? delta_bias[d] : 0.0);
                double dt = dts[t];
                double ut = u[row + t];
                double s = z ? oracle_silu(z[row + t]) : 1.0;
                double gc = dy[row + t] * s;
                if (z && dz)
                    dz[row + t] = dy[row + t] * yc[t] * oracle_dsilu(z[row + t]);
                double dut = 0.0, ddt = 0.0;
                if (D) {
                    dD[d] += gc * ut;
                    dut = gc * D[d];
                }
                for (int64_t n = 0; n < N; ++n) {
                    double a = exp(dt * Ad[n]);
                    double c = oracle_input_coeff(dt, Ad[n], zoh_b);
                    double dc_ddt, dc_da;
                    oracle_input_coeff_grad(dt, Ad[n], zoh_b, &dc_ddt, &dc_da);
                    double hprev = hs[t * N + n];
                    double Bn = Bb[n * L + t];
                    g[n] += gc * Cb[n * L + t];
                    dC[b * N * L + n * L + t] += gc * hs[(t + 1) * N + n];
                    ddt += g[n] * (Ad[n] * a * hprev + dc_ddt * Bn * ut);
                    dA[d * N + n] += g[n] * (dt * a * hprev + dc_da * Bn * ut);
                    dB[b * N * L + n * L + t] += g[n] * c * ut;
                    dut += g[n] * c * Bn;
                    g[n] *= a;
                }
                du[row + t] = dut;
                double dx = delta_softplus ? ddt * oracle_sigmoid(x) : ddt;
                ddelta[row + t] = dx;
                if (ddelta_bias)
                    ddelta_bias[d] += dx;
            }
            if (dh0)
                for (int64_t n = 0; n < N; ++n)
                    dh0[srow + n] = g[n];
        }
    }
    free(hs);
    return 0;
}

int oracle_ssd_f64(const double *x, const double *dt, const double *A,
                   const double *B, const double *C, const double *D,
                   const double *z, const double *dt_bias, int dt_softplus,
                   const double *h0, double *y, double *h_final,
                   int64_t batch, int64_t nheads, int64_t P, int64_t ngroups,
                   int64_t N, int64_t L)
{
    if (!x || !dt || !A || !B || !C || !y)
        return -1;
    if (batch < 0 || nheads < 1 || P < 1 || ngroups < 1 || N < 1 || L < 0 ||
        nheads % ngroups != 0)
        return -1;
    double *cum = malloc(sizeof(double) * (size_t)(2 * L + P + 1));
    if (!cum)
        return -1;
    double *dts = cum + L;
    double *acc = dts + L;   /* one output column, all rows of the head */
    const int64_t hpg = nheads / ngroups;   /* heads per group */
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t h = 0; h < nheads; ++h) {
            const int64_t g = h / hpg;
            const double *Bg = B + (b * ngroups + g) * N * L;  /* [n*L + t] */
            const double *Cg = C + (b * ngroups + g) * N * L;
            const double *dtr = dt + (b * nheads + h) * L;
            double run = 0.0;
            for (int64_t t = 0; t < L; ++t) {
                double v = dtr[t] + (dt_bias ? dt_bias[h] : 0.0);
                dts[t] = dt_softplus ? oracle_softplus(v) : v;
                run += dts[t];
                cum[t] = run;
            }
            /* y[:, t] = sum_{s <= t} S[t,s] x[:, s]: S[t,s] is formed once per
             * (t, s) and applied to every row p of the head */
            for (int64_t t = 0; t < L; ++t) {
                for (int64_t p = 0; p < P; ++p)
                    acc[p] = 0.0;
                for (int64_t s = 0; s <= t; ++s) {          /* the causal mask */
                    double cb = 0.0;
                    for (int64_t n = 0; n < N; ++n)
                        cb += Cg[n * L + t] * Bg[n * L + s];
                    double w = cb * exp(A[h] * (cum[t] - cum[s])) * dts[s];
                    for (int64_t p = 0; p < P; ++p)
                        acc[p] += w * x[((b * nheads + h) * P + p) * L + s];
                }
                for (int64_t p = 0; p < P; ++p) {
                    const int64_t row = ((b * nheads + h) * P + p) * L;
                    const int64_t srow = ((b * nheads + h) * P + p) * N;
                    double v = acc[p];
                    if (h0) {
                        double decay = exp(A[h] * cum[t]);
                        for (int64_t n = 0; n < N; ++n)
                            v += Cg[n * L + t] * decay * h0[srow + n];
                    }
                    if (D)
                        v += D[h] * x[row + t];
                    if (z)
                        v *= oracle_silu(z[row + t]);
                    y[row + t] = v;
                }
            }
            if (h_final) {
                for (int64_t p = 0; p < P; ++p) {
                    const int64_t row = ((b * nheads + h) * P + p) * L;
                    const int64_t srow = ((b * nheads + h) * P + p) * N;
                    for (int64_t n = 0; n < N; ++n) {
                        double st = h0 ? exp(A[h] * (L > 0 ? cum[L - 1] : 0.0)) * h0[srow + n]
                                       : 0.0;
                        for (int64_t s = 0; s < L; ++s)
                            st += exp(A[h] * (cum[L - 1] - cum[s])) * dts[s] *
                                  x[row + s] * Bg[n * L + s];
                        h_final[srow + n] = st;
                    }
                }
            }
        }
    }
    free(cum);
    return 0;
}
