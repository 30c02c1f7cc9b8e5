/*
 * oracle.c -- plain, slow, fp64 CPU reference of the selective state-space scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg do.  It shares no code, header, table or
 * helper with the HIP library.
 *
 * Every input arrives widened to double (bf16 and fp32 widen exactly), every
 * operation runs in double with the host libm, one (batch, channel) row at a
 * time, token by token, in the order the method defines.  No blocking, no
 * reassociation, no vector tricks.  Rows are independent, so OpenMP splits
 * the row loop (static schedule); that changes no arithmetic.
 *
 * Sources for what is computed (all are web pages about Mamba):
 *  - "Understanding Mamba and Selective State Space Models (SSMs)" (bqwf.cn
 *    practitioner blog), section 2.2 "first cut: selectivity": the state
 *    update h_n = exp(Delta_n A) h_{n-1} + Delta_n B_n x_n, with Delta, B, C
 *    depending on the token; section 2.2 "second cut": the recurrent scan
 *    starting from a zero state; the tip closing section 2.2: Delta passes
 *    through softplus log(1+exp(x)) to stay positive; section 2.1: the
 *    read-out y = C h + D x; section 4.3: A = -exp(A_log), diagonal.
 *  - The Mamba README embedded in the gittoolsai tool page for
 *    state-spaces/mamba, sections "Selective SSM", "Mamba-2" and
 *    "Initialization": the selective SSM layer, the Mamba-2 variant, and the
 *    Delta bias that places Delta in a target range.
 *  - The "model-architecture-mamba" skill page: Mamba-2 uses multiple heads,
 *    d_state 128 and headdim 64.
 * Readings where the pages are silent or garbled (sign of the exponent, the
 * sum over the state index in the read-out, the gate multiplying the D term,
 * the zero initial state) are the plainest ones consistent with those pages:
 *   y_t = (sum_n C_t[n] h_t[n] + D_d u_t) * silu(z_t),  h_{-1} = 0 (or h0).
 *
 * Parity pins: see tests/test_oracle_pins.py (closed forms, brute force,
 * invariants).  Every function here is pinned there.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <omp.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_NO_MEM 2

/* softplus(x) = log(1 + e^x), written so that e^x never overflows. */
static double sp64(double x) { return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x)); }

/* silu(z) = z * sigmoid(z) = z / (1 + e^-z). */
static double silu64(double z) { return z / (1.0 + exp(-z)); }

const char* oracle_version(void) { return "selscan-oracle fp64 1"; }

/* Number of threads of the calling thread's later parallel regions (the
 * timing of the oracle picks it; OMP_NUM_THREADS is read only once, when the
 * OpenMP runtime starts).  Values below 1 are ignored. */
void oracle_set_threads(int n) {
    if (n > 0) omp_set_num_threads(n);
}

/*
 * Mamba-1 selective scan, one channel row at a time.
 *   u, delta, z : [nb, nd, nl]   (z may be NULL: no gate)
 *   A           : [nd, nn]
 *   Bm, Cm      : [nb, nn, nl]
 *   Dv, bias    : [nd]           (either may be NULL: treated as 0)
 *   h0          : [nb, nd, nn]   (NULL: zero initial state)
 *   y           : [nb, nd, nl]   out
 *   last        : [nb, nd, nn]   out (may be NULL)
 */
int oracle_m1_f64(int64_t nb, int64_t nd, int64_t nn, int64_t nl,
                  const double* u, const double* delta, const double* A,
                  const double* Bm, const double* Cm, const double* Dv,
                  const double* z, const double* bias, int softplus,
                  const double* h0, double* y, double* last)
{
    if (nb < 0 || nd < 0 || nn < 1 || nl < 0) return ORACLE_BAD_ARG;
    if (!u || !delta || !A || !Bm || !Cm || !y) return ORACLE_BAD_ARG;
    const int64_t rows = nb * nd;
    int status = ORACLE_OK;

#pragma omp parallel
    {
        double* h = (double*)malloc((size_t)nn * sizeof(double));
        if (!h) {
#pragma omp atomic write
            status = ORACLE_NO_MEM;
        }
#pragma omp for schedule(static)
        for (int64_t row = 0; row < rows; ++row) {
            if (!h) continue;
            const int64_t b = row / nd;
            const int64_t d = row % nd;
            const double* urow = u + row * nl;
            const double* drow = delta + row * nl;
            const double* zrow = z ? z + row * nl : NULL;
            const double* Arow = A + d * nn;
            const double* Bb = Bm + b * nn * nl;   /* B[b, n, t] = Bb[n*nl + t] */
            const double* Cb = Cm + b * nn * nl;
            double* yrow = y + row * nl;
            for (int64_t n = 0; n < nn; ++n) h[n] = h0 ? h0[row * nn + n] : 0.0;
            for (int64_t t = 0; t < nl; ++t) {
                double xv = drow[t] + (bias ? bias[d] : 0.0);
                double dt = softplus ? sp64(xv) : xv;        /* Delta_t */
                double ut = urow[t];
                double acc = 0.0;
                for (int64_t n = 0; n < nn; ++n) {
                    double dA = exp(dt * Arow[n]);            /* exp(Delta A) */
                    h[n] = dA * h[n] + dt * Bb[n * nl + t] * ut;
                    acc += Cb[n * nl + t] * h[n];
                }
                double yv = acc + (Dv ? Dv[d] * ut : 0.0);
                if (zrow) yv *= silu64(zrow[t]);
                yrow[t] = yv;
            }
            if (last)
                for (int64_t n = 0; n < nn; ++n) last[row * nn + n] = h[n];
        }
        free(h);
    }
    return status;
}

/*
 * Mamba-2 multi-head selective scan: a scalar A per head, one Delta per
 * (batch, token, head) shared by the head's channels, B and C shared by the
 * heads of a group (head h belongs to group h / (nh / ng)).
 *   x, z        : [nb, nl, nh, np]   (z may be NULL)
 *   dt          : [nb, nl, nh]
 *   A, Dv, dtb  : [nh]               (Dv, dtb may be NULL: treated as 0)
 *   Bm, Cm      : [nb, nl, ng, nn]
 *   h0, last    : [nb, nh, np, nn]   (h0 NULL: zero state; last may be NULL)
 *   y           : [nb, nl, nh, np]
 */
int oracle_m2_f64(int64_t nb, int64_t nl, int64_t nh, int64_t np, int64_t ng,
                  int64_t nn, const double* x, const double* dt, const double* A,
                  const double* Bm, const double* Cm, const double* Dv,
                  const double* z, const double* dtb, int softplus,
                  const double* h0, double* y, double* last)
{
    if (nb < 0 || nl < 0 || nh < 1 || np < 1 || ng < 1 || nn < 1) return ORACLE_BAD_ARG;
    if (nh % ng != 0) return ORACLE_BAD_ARG;
    if (!x || !dt || !A || !Bm || !Cm || !y) return ORACLE_BAD_ARG;
    const int64_t units = nb * nh * np;   /* one (batch, head, channel) each */
    const int64_t heads_per_group = nh / ng;
    int status = ORACLE_OK;

#pragma omp parallel
    {
        double* s = (double*)malloc((size_t)nn * sizeof(double));
        if (!s) {
#pragma omp atomic write
            status = ORACLE_NO_MEM;
        }
#pragma omp for schedule(static)
        for (int64_t unit = 0; unit < units; ++unit) {
            if (!s) continue;
            const int64_t b = unit / (nh * np);
            const int64_t hh = (unit / np) % nh;
            const int64_t p = unit % np;
            const int64_t g = hh / heads_per_group;
            for (int64_t n = 0; n < nn; ++n) s[n] = h0 ? h0[unit * nn + n] : 0.0;
            for (int64_t t = 0; t < nl; ++t) {
                const int64_t bt = b * nl + t;
                double xv = dt[bt * nh + hh] + (dtb ? dtb[hh] : 0.0);
                double delt = softplus ? sp64(xv) : xv;
                double dA = exp(delt * A[hh]);
                double xt = x[(bt * nh + hh) * np + p];
                const double* Bt = Bm + (bt * ng + g) * nn;
                const double* Ct = Cm + (bt * ng + g) * nn;
                double acc = 0.0;
                for (int64_t n = 0; n < nn; ++n) {
                    s[n] = dA * s[n] + delt * Bt[n] * xt;
                    acc += Ct[n] * s[n];
                }
                double yv = acc + (Dv ? Dv[hh] * xt : 0.0);
                if (z) yv *= silu64(z[(bt * nh + hh) * np + p]);
                y[(bt * nh + hh) * np + p] = yv;
            }
            if (last)
                for (int64_t n = 0; n < nn; ++n) last[unit * nn + n] = s[n];
        }
        free(s);
    }
    return status;
}

/*
 * Causal depthwise convolution ahead of the scan (blog "Understanding Mamba
 * ..." section 3.3: a width-4 1-D convolution whose output at a position
 * sees that token and the three before it; the README's causal-conv1d layer
 * inside the Mamba block), one channel row at a time:
 *
 *   out[b,d,t] = act( bias[d] + sum_{k=0}^{nk-1} w[d,k] * x[b,d,t-(nk-1)+k] ),
 *
 * x before the first token taken as 0, act = silu when `silu` else identity.
 *   x, out : [nb, nd, nl];  w : [nd, nk];  bias : [nd] or NULL.
 */
int oracle_conv1d_f64(int64_t nb, int64_t nd, int64_t nl, int64_t nk, const double* x, const double* w,
                      const double* bias, int silu, double* out) {
    if (nb < 1 || nd < 1 || nl < 1 || nk < 1 || !x || !w || !out) return ORACLE_BAD_ARG;
    const int64_t rows = nb * nd;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t d = r % nd;
        const double* xr = x + r * nl;
        double* orow = out + r * nl;
        for (int64_t t = 0; t < nl; ++t) {
            double acc = bias ? bias[d] : 0.0;
            for (int64_t k = 0; k < nk; ++k) {
                const int64_t s = t - (nk - 1) + k;
                if (s >= 0) acc += w[d * nk + k] * xr[s];
            }
            orow[t] = silu ? silu64(acc) : acc;
        }
    }
    return ORACLE_OK;
}

/*
 * Gradients of the Mamba-1 scan (reverse-mode, fp64), for
 *   out_t = y_t * silu(z_t),  y_t = sum_n C_t[n] h_t[n] + D u_t,
 *   h_t = exp(Delta_t A) h_{t-1} + Delta_t B_t u_t,  Delta_t = sp(delta_t + bias),
 * given dout = d loss / d out.  The adjoint of the state runs backward in
 * time: lam_t = dy_t C_t + exp(Delta_{t+1} A) lam_{t+1}, and each input's
 * gradient collects lam_t times the partial derivative of h_t's update
 * (the chain rule through the recurrence, no shortcut).  h0 [nb,nd,nn] is
 * the state before the first token (NULL = 0); its gradient dh0 =
 * exp(Delta_0 A) lam_0 is written when dh0 is non-NULL.
 * Outputs (all written, all fp64): du, ddelta, dz [nb,nd,nl]; dA [nd,nn];
 * dB, dC [nb,nn,nl]; dD, dbias [nd].  z, D, bias may be NULL (then their
 * gradients are written as 0 and the corresponding terms vanish).
 * Rows are processed one after another so that the sums over channels of
 * dB, dC, dA, dD, dbias are plain sequential sums.
 */
int oracle_m1_bwd_f64(int64_t nb, int64_t nd, int64_t nn, int64_t nl, const double* u, const double* delta,
                      const double* A, const double* Bm, const double* Cm, const double* Dv, const double* z,
                      const double* bias, int softplus, const double* h0, const double* dout, double* du,
                      double* ddelta, double* dA, double* dBm, double* dCm, double* dD, double* dz, double* dbias,
                      double* dh0) {
    if (nb < 1 || nd < 1 || nn < 1 || nl < 1 || !u || !delta || !A || !Bm || !Cm || !dout || !du || !ddelta ||
        !dA || !dBm || !dCm || !dD || !dz || !dbias)
        return ORACLE_BAD_ARG;
    double* h = (double*)malloc(sizeof(double) * (size_t)(nl + 1) * (size_t)nn);   /* h_{-1} .. h_{L-1} */
    double* lam = (double*)malloc(sizeof(double) * (size_t)nn);
    double* dl = (double*)malloc(sizeof(double) * (size_t)nl);
    if (!h || !lam || !dl) {
        free(h); free(lam); free(dl);
        return ORACLE_NO_MEM;
    }
    for (int64_t i = 0; i < nd * nn; ++i) dA[i] = 0.0;
    for (int64_t i = 0; i < nd; ++i) { dD[i] = 0.0; dbias[i] = 0.0; }
    for (int64_t i = 0; i < nb * nn * nl; ++i) { dBm[i] = 0.0; dCm[i] = 0.0; }
    for (int64_t b = 0; b < nb; ++b) {
        for (int64_t d = 0; d < nd; ++d) {
            const int64_t row = b * nd + d;
            const double* ur = u + row * nl;
            const double* xr = delta + row * nl;
            const double* zr = z ? z + row * nl : NULL;
            const double* gr = dout + row * nl;
            /* forward, keeping every state */
            for (int64_t n = 0; n < nn; ++n) h[n] = h0 ? h0[row * nn + n] : 0.0;
            for (int64_t t = 0; t < nl; ++t) {
                const double x = xr[t] + (bias ? bias[d] : 0.0);
                dl[t] = softplus ? sp64(x) : x;
                for (int64_t n = 0; n < nn; ++n) {
                    const double a = exp(dl[t] * A[d * nn + n]);
                    h[(t + 1) * nn + n] = a * h[t * nn + n] + dl[t] * Bm[(b * nn + n) * nl + t] * ur[t];
                }
            }
            /* backward */
            for (int64_t n = 0; n < nn; ++n) lam[n] = 0.0;
            for (int64_t t = nl - 1; t >= 0; --t) {
                double y = Dv ? Dv[d] * ur[t] : 0.0;
                for (int64_t n = 0; n < nn; ++n) y += Cm[(b * nn + n) * nl + t] * h[(t + 1) * nn + n];
                double dy = gr[t];
                if (zr) {
                    const double zz = zr[t];
                    const double sg = 1.0 / (1.0 + exp(-zz));
                    dz[row * nl + t] = gr[t] * y * sg * (1.0 + zz * (1.0 - sg));
                    dy = gr[t] * zz * sg;
                } else {
                    dz[row * nl + t] = 0.0;
                }
                double dut = Dv ? dy * Dv[d] : 0.0;
                if (Dv) dD[d] += dy * ur[t];
                double ddl = 0.0;
                for (int64_t n = 0; n < nn; ++n) {
                    const double c = Cm[(b * nn + n) * nl + t];
                    const double bb = Bm[(b * nn + n) * nl + t];
                    /* lam_t = dy C_t + a_{t+1} lam_{t+1}; lam[] holds a_{t+1} lam_{t+1} */
                    const double l = dy * c + lam[n];
                    dCm[(b * nn + n) * nl + t] += dy * h[(t + 1) * nn + n];
                    dBm[(b * nn + n) * nl + t] += l * dl[t] * ur[t];
                    dut += l * dl[t] * bb;
                    const double a = exp(dl[t] * A[d * nn + n]);
                    const double hp = h[t * nn + n];
                    ddl += l * (bb * ur[t] + A[d * nn + n] * a * hp);
                    dA[d * nn + n] += l * dl[t] * a * hp;
                    lam[n] = a * l;   /* a_t lam_t, carried to token t-1 */
                }
                du[row * nl + t] = dut;
                const double x = xr[t] + (bias ? bias[d] : 0.0);
                const double dx = softplus ? ddl / (1.0 + exp(-x)) : ddl;   /* sp'(x) = sigmoid(x) */
                ddelta[row * nl + t] = dx;
                if (bias) dbias[d] += dx;
            }
            if (dh0)
                for (int64_t n = 0; n < nn; ++n) dh0[row * nn + n] = lam[n];
        }
    }
    free(h); free(lam); free(dl);
    return ORACLE_OK;
}

/*
 * Gradients of the Mamba-2 (multi-head) scan (reverse-mode, fp64).  The
 * forward is oracle_m2_f64: per (batch b, head hh, channel p), with the
 * group g = hh / (nh / ng) of the head,
 *   Delta_t = sp(dt[b,t,hh] + dtb[hh]),  a_t = exp(Delta_t A[hh]),
 *   h_t[n]  = a_t h_{t-1}[n] + Delta_t B[b,t,g,n] x[b,t,hh,p],
 *   out_t   = (sum_n C[b,t,g,n] h_t[n] + D[hh] x[b,t,hh,p]) * silu(z[b,t,hh,p]),
 * i.e. the Mamba-1 recurrence with one scalar decay per (token, head) and B,
 * C shared by the heads of a group (README section "Mamba-2"; skill page
 * "model-architecture-mamba").  Given dout = d loss / d out, the adjoint of
 * the state runs backward in time exactly as for Mamba-1,
 *   lam_t[n] = dy_t C_t[n] + a_{t+1} lam_{t+1}[n],
 * and the gradients that the Mamba-2 sharing ties together are sums: ddt
 * over the channels p of the head, dA, dD, ddt_bias over everything but the
 * head, dB and dC over the heads of the group and their channels.
 * Outputs (all written, fp64): dx, dz [nb,nl,nh,np]; ddt [nb,nl,nh];
 * dA, dD, ddtb [nh]; dB, dC [nb,nl,ng,nn]; dh0 [nb,nh,np,nn] when non-NULL
 * (dh0 = a_0 lam_0).  z, D, dtb, h0 may be NULL.  Units run one after
 * another, so every sum is a plain sequential sum.
 */
int oracle_m2_bwd_f64(int64_t nb, int64_t nl, int64_t nh, int64_t np, int64_t ng, int64_t nn,
                      const double* x, const double* dt, const double* A, const double* Bm, const double* Cm,
                      const double* Dv, const double* z, const double* dtb, int softplus, const double* h0,
                      const double* dout, double* dx, double* ddt, double* dA, double* dBm, double* dCm,
                      double* dD, double* dz, double* ddtb, double* dh0) {
    if (nb < 1 || nl < 1 || nh < 1 || np < 1 || ng < 1 || nn < 1 || nh % ng != 0) return ORACLE_BAD_ARG;
    if (!x || !dt || !A || !Bm || !Cm || !dout || !dx || !ddt || !dA || !dBm || !dCm || !dD || !dz || !ddtb)
        return ORACLE_BAD_ARG;
    double* h = (double*)malloc(sizeof(double) * (size_t)(nl + 1) * (size_t)nn);   /* h_{-1} .. h_{L-1} */
    double* lam = (double*)malloc(sizeof(double) * (size_t)nn);
    double* dl = (double*)malloc(sizeof(double) * (size_t)nl);
    if (!h || !lam || !dl) {
        free(h); free(lam); free(dl);
        return ORACLE_NO_MEM;
    }
    const int64_t hpg = nh / ng;
    for (int64_t i = 0; i < nh; ++i) { dA[i] = 0.0; dD[i] = 0.0; ddtb[i] = 0.0; }
    for (int64_t i = 0; i < nb * nl * nh; ++i) ddt[i] = 0.0;
    for (int64_t i = 0; i < nb * nl * ng * nn; ++i) { dBm[i] = 0.0; dCm[i] = 0.0; }
    for (int64_t b = 0; b < nb; ++b) {
        for (int64_t hh = 0; hh < nh; ++hh) {
            const int64_t g = hh / hpg;
            for (int64_t t = 0; t < nl; ++t) {
                const double v = dt[(b * nl + t) * nh + hh] + (dtb ? dtb[hh] : 0.0);
                dl[t] = softplus ? sp64(v) : v;
            }
            for (int64_t p = 0; p < np; ++p) {
                const int64_t unit = (b * nh + hh) * np + p;
                /* forward, keeping every state */
                for (int64_t n = 0; n < nn; ++n) h[n] = h0 ? h0[unit * nn + n] : 0.0;
                for (int64_t t = 0; t < nl; ++t) {
                    const double a = exp(dl[t] * A[hh]);
                    const double xt = x[((b * nl + t) * nh + hh) * np + p];
                    const double* Bt = Bm + ((b * nl + t) * ng + g) * nn;
                    for (int64_t n = 0; n < nn; ++n) h[(t + 1) * nn + n] = a * h[t * nn + n] + dl[t] * Bt[n] * xt;
                }
                /* backward */
                for (int64_t n = 0; n < nn; ++n) lam[n] = 0.0;
                for (int64_t t = nl - 1; t >= 0; --t) {
                    const int64_t e = ((b * nl + t) * nh + hh) * np + p;
                    const double xt = x[e];
                    const double* Bt = Bm + ((b * nl + t) * ng + g) * nn;
                    const double* Ct = Cm + ((b * nl + t) * ng + g) * nn;
                    double* dBt = dBm + ((b * nl + t) * ng + g) * nn;
                    double* dCt = dCm + ((b * nl + t) * ng + g) * nn;
                    double y = Dv ? Dv[hh] * xt : 0.0;
                    for (int64_t n = 0; n < nn; ++n) y += Ct[n] * h[(t + 1) * nn + n];
                    double dy = dout[e];
                    if (z) {
                        const double zz = z[e];
                        const double sg = 1.0 / (1.0 + exp(-zz));
                        dz[e] = dout[e] * y * sg * (1.0 + zz * (1.0 - sg));
                        dy = dout[e] * zz * sg;
                    } else {
                        dz[e] = 0.0;
                    }
                    double dxt = Dv ? dy * Dv[hh] : 0.0;
                    if (Dv) dD[hh] += dy * xt;
                    const double a = exp(dl[t] * A[hh]);
                    double ddl = 0.0;
                    for (int64_t n = 0; n < nn; ++n) {
                        /* lam_t = dy C_t + a_{t+1} lam_{t+1}; lam[] holds a_{t+1} lam_{t+1} */
                        const double l = dy * Ct[n] + lam[n];
                        const double hp = h[t * nn + n];
                        dCt[n] += dy * h[(t + 1) * nn + n];
                        dBt[n] += l * dl[t] * xt;
                        dxt += l * dl[t] * Bt[n];
                        ddl += l * (Bt[n] * xt + A[hh] * a * hp);
                        dA[hh] += l * dl[t] * a * hp;
                        lam[n] = a * l;   /* a_t lam_t, carried to token t-1 */
                    }
                    dx[e] = dxt;
                    const double v = dt[(b * nl + t) * nh + hh] + (dtb ? dtb[hh] : 0.0);
                    const double dv = softplus ? ddl / (1.0 + exp(-v)) : ddl;   /* sp'(v) = sigmoid(v) */
                    ddt[(b * nl + t) * nh + hh] += dv;
                    if (dtb) ddtb[hh] += dv;
                }
                if (dh0)
                    for (int64_t n = 0; n < nn; ++n) dh0[unit * nn + n] = lam[n];
            }
        }
    }
    free(h); free(lam); free(dl);
    return ORACLE_OK;
}
