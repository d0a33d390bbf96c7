/*
 * Plain, slow CPU oracle for the Vision-RWKV spatial-mix path (Bi-WKV and Q-Shift).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may include, link or call this file.
 * Only the test-suite, the smoke check and the benchmark's CPU-baseline leg use it, through the
 * ctypes wrapper in this folder. It shares no code, header, table or constant with the HIP
 * library; it depends on libc/libm (exp, fabs, floor) and OpenMP only.
 *
 * Sources (cited by page title and equation; the pages are the authority):
 *   [VRWKV]  "OpenGVLab&港中文&复旦&南大&清华提出Vision-RWKV Backbone" (cloud.tencent.com article
 *            rendering the Vision-RWKV paper), section "Linear Complexity Bidirectional
 *            Attention": Eq. (5) summation form, Eq. (6) four hidden states, Eq. (7) output,
 *            and the prose that each state update adds or removes one term and multiplies or
 *            divides by e^{-w/T}; section "Scale Up Stability": exponent divided by T.
 *   [NOTES]  "LinXin's Blog", Vision-RWKV notes: the q_shift function (token shift on the
 *            H x W patch grid, channel groups at int(C*gamma*j), zero fill, remainder copied).
 *
 * Everything is float64. Inputs are the exact kernel inputs widened to float64 (fp32 and bf16
 * widen exactly). Arrays are [B, T, C] contiguous, C fastest.
 *
 * Readings of the pages (each also listed in the design notes):
 *   - Eq. (5) exponent grouping: weight of token i != t is exp(-((|t-i|-1)/T) * w + k_i); the
 *     self term is exp(u + k_t). Adjacent tokens therefore carry no decay.
 *   - T in the exponent is the sequence length of the call.
 *   - A per-channel constant subtracted from every exponent is an exact identity of Eq. (5);
 *     the oracle uses one only to keep float64 finite.
 *   - Q-Shift follows the listing's direction order (right, left, down, up) and its
 *     int(C*gamma*j) group boundaries, not Eq. (9)'s order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_ARG -1
#define ORC_ERR_PARAM -2
#define ORC_ERR_NOMEM -3

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Gather one (b, c) column of a [B, T, C] array into a contiguous buffer of length T. */
static void gather_col(const double* x, int64_t b, int64_t c, int64_t T, int64_t C, double* col) {
    const double* base = x + b * T * C + c;
    for (int64_t t = 0; t < T; ++t) col[t] = base[t * C];
}

/*
 * O1 — Eq. (5) of [VRWKV], summation form, written out term by term.
 *   wkv_t = ( sum_{i != t} exp(-((|t-i|-1)/T) w + k_i) v_i + exp(u + k_t) v_t )
 *         / ( sum_{i != t} exp(-((|t-i|-1)/T) w + k_i)     + exp(u + k_t)     )
 * For each output the largest logit M is subtracted before exponentiating (an exact identity).
 * Also returns scale_t = sum p_i |v_i| / sum p_i, the magnitude the weighted mean is formed
 * from (used by the tests' error metric).
 * rows: NULL for every t, else nrows token indices; out/scale are then [B, nrows, C].
 */
int oracle_biwkv_sum(const double* k, const double* v, const double* w, const double* u,
                     int64_t B, int64_t T, int64_t C, const int64_t* rows, int64_t nrows,
                     double* out, double* scale, int nthreads) {
    if (!k || !v || !w || !u || !out || B < 0 || T < 0 || C < 0) return ORC_ERR_ARG;
    if (!rows) nrows = T;
    for (int64_t r = 0; rows && r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= T) return ORC_ERR_ARG;
    if (B == 0 || T == 0 || C == 0 || nrows == 0) return ORC_OK;
    set_threads(nthreads);
    int failed = 0;
#pragma omp parallel
    {
        double* kc = (double*)malloc(sizeof(double) * (size_t)T);
        double* vc = (double*)malloc(sizeof(double) * (size_t)T);
        double* s = (double*)malloc(sizeof(double) * (size_t)T);
        if (!kc || !vc || !s) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t bc = 0; bc < B * C; ++bc) {
                const int64_t b = bc / C, c = bc % C;
                gather_col(k, b, c, T, C, kc);
                gather_col(v, b, c, T, C, vc);
                const double wc = w[c], uc = u[c], Td = (double)T;
                for (int64_t r = 0; r < nrows; ++r) {
                    const int64_t t = rows ? rows[r] : r;
                    double M = -INFINITY;
                    for (int64_t i = 0; i < T; ++i) {
                        double si;
                        if (i == t) {
                            si = uc + kc[i];
                        } else {
                            const int64_t dist = (i > t) ? (i - t) : (t - i);
                            si = -(((double)(dist - 1)) / Td) * wc + kc[i];
                        }
                        s[i] = si;
                        if (si > M) M = si;
                    }
                    double num = 0.0, den = 0.0, mag = 0.0;
                    for (int64_t i = 0; i < T; ++i) {
                        const double p = exp(s[i] - M);
                        num += p * vc[i];
                        den += p;
                        mag += p * fabs(vc[i]);
                    }
                    const int64_t o = (b * nrows + r) * C + c;
                    out[o] = num / den;
                    if (scale) scale[o] = mag / den;
                }
            }
        }
        free(kc);
        free(vc);
        free(s);
    }
    return failed ? ORC_ERR_NOMEM : ORC_OK;
}

/*
 * O2 — Eq. (6)-(7) of [VRWKV], the RNN form with four hidden states, evaluated as two sweeps.
 * With lam = exp(-w/T) and e_i = exp(k_i - kappa) (kappa = max_i k_i, an exact identity shift):
 *   a: A_0 = 0, A_{t+1} = lam*A_t + e_t v_t      (A_t is Eq. (6)'s a_{t-1})
 *   c: C_0 = 0, C_{t+1} = lam*C_t + e_t          (c_{t-1})
 *   b: B_{T-1} = 0, B_{t-1} = lam*B_t + e_t v_t  (b_{t-1})
 *   d: D_{T-1} = 0, D_{t-1} = lam*D_t + e_t      (d_{t-1})
 *   wkv_t = (A_t + B_t + E_t v_t) / (C_t + D_t + E_t),  E_t = exp(u + k_t - kappa)   (Eq. (7))
 * Also returns the magnitude scale (same recurrences on |v|).
 * Valid while lam^T and exp(u + k - kappa) stay inside float64 (|w| and u of a few hundred).
 */
int oracle_biwkv_rnn(const double* k, const double* v, const double* w, const double* u,
                     int64_t B, int64_t T, int64_t C, double* out, double* scale, int nthreads) {
    if (!k || !v || !w || !u || !out || B < 0 || T < 0 || C < 0) return ORC_ERR_ARG;
    if (B == 0 || T == 0 || C == 0) return ORC_OK;
    set_threads(nthreads);
    int failed = 0;
#pragma omp parallel
    {
        double* kc = (double*)malloc(sizeof(double) * (size_t)T);
        double* vc = (double*)malloc(sizeof(double) * (size_t)T);
        double* aa = (double*)malloc(sizeof(double) * (size_t)T);
        double* cc = (double*)malloc(sizeof(double) * (size_t)T);
        double* am = (double*)malloc(sizeof(double) * (size_t)T);
        if (!kc || !vc || !aa || !cc || !am) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t bc = 0; bc < B * C; ++bc) {
                const int64_t b = bc / C, c = bc % C;
                gather_col(k, b, c, T, C, kc);
                gather_col(v, b, c, T, C, vc);
                double kappa = -INFINITY;
                for (int64_t t = 0; t < T; ++t)
                    if (kc[t] > kappa) kappa = kc[t];
                const double lam = exp(-w[c] / (double)T);
                /* forward sweep: states a, c (and |v| variant) */
                double A = 0.0, Cs = 0.0, Am = 0.0;
                for (int64_t t = 0; t < T; ++t) {
                    aa[t] = A;
                    cc[t] = Cs;
                    am[t] = Am;
                    const double e = exp(kc[t] - kappa);
                    A = lam * A + e * vc[t];
                    Cs = lam * Cs + e;
                    Am = lam * Am + e * fabs(vc[t]);
                }
                /* backward sweep: states b, d; output of Eq. (7) */
                double Bs = 0.0, D = 0.0, Bm = 0.0;
                for (int64_t t = T - 1; t >= 0; --t) {
                    const double E = exp(u[c] + kc[t] - kappa);
                    const double den = cc[t] + D + E;
                    const int64_t o = (b * T + t) * C + c;
                    out[o] = (aa[t] + Bs + E * vc[t]) / den;
                    if (scale) scale[o] = (am[t] + Bm + E * fabs(vc[t])) / den;
                    const double e = exp(kc[t] - kappa);
                    Bs = lam * Bs + e * vc[t];
                    D = lam * D + e;
                    Bm = lam * Bm + e * fabs(vc[t]);
                }
            }
        }
        free(kc);
        free(vc);
        free(aa);
        free(cc);
        free(am);
    }
    return failed ? ORC_ERR_NOMEM : ORC_OK;
}

/*
 * O2' — the prose recurrence of [VRWKV] §"Linear Complexity Bidirectional Attention" read
 * literally: one forward sweep in which a, c gain a term and are multiplied by e^{-w/T}, while
 * b, d (started from their full sums) lose a term and are divided by e^{-w/T}:
 *   a_t = e^{-w/T} a_{t-1} + e^{k_t} v_t
 *   b_t = (b_{t-1} - e^{k_{t+1}} v_{t+1}) / e^{-w/T}
 * It cancels badly for long sequences; it is a small-T pin only.
 */
int oracle_biwkv_rnn_literal(const double* k, const double* v, const double* w, const double* u,
                             int64_t B, int64_t T, int64_t C, double* out) {
    if (!k || !v || !w || !u || !out || B < 0 || T < 0 || C < 0) return ORC_ERR_ARG;
    if (B == 0 || T == 0 || C == 0) return ORC_OK;
    double* kc = (double*)malloc(sizeof(double) * (size_t)T);
    double* vc = (double*)malloc(sizeof(double) * (size_t)T);
    if (!kc || !vc) {
        free(kc);
        free(vc);
        return ORC_ERR_NOMEM;
    }
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t c = 0; c < C; ++c) {
            gather_col(k, b, c, T, C, kc);
            gather_col(v, b, c, T, C, vc);
            double kappa = -INFINITY;
            for (int64_t t = 0; t < T; ++t)
                if (kc[t] > kappa) kappa = kc[t];
            const double Td = (double)T, lam = exp(-w[c] / Td);
            /* b_{-1}, d_{-1}: the sums over i >= 1 for the first token (t = 0) */
            double a = 0.0, cs = 0.0, bs = 0.0, d = 0.0;
            for (int64_t i = 1; i < T; ++i) {
                const double wt = exp(-(((double)(i - 1)) / Td) * w[c] + kc[i] - kappa);
                bs += wt * vc[i];
                d += wt;
            }
            for (int64_t t = 0; t < T; ++t) {
                const double E = exp(u[c] + kc[t] - kappa);
                out[(b * T + t) * C + c] = (a + bs + E * vc[t]) / (cs + d + E);
                const double et = exp(kc[t] - kappa);
                a = lam * a + et * vc[t];
                cs = lam * cs + et;
                if (t + 1 < T) {
                    const double en = exp(kc[t + 1] - kappa);
                    bs = (bs - en * vc[t + 1]) / lam;
                    d = (d - en) / lam;
                }
            }
        }
    }
    free(kc);
    free(vc);
    return ORC_OK;
}

/*
 * O1c — the causal attention the pages compare against (the original RWKV attention, whose sum
 * stops at the token before the current one; [VRWKV] "Linear Complexity Bidirectional
 * Attention" describes Bi-WKV as raising that upper limit to T-1). Reading: Eq. (5) with the
 * decayed sum restricted to i < t, same exponent convention, self term exp(u + k_t):
 *   wkv_t = ( sum_{i < t} exp(-((t-1-i)/T) w + k_i) v_i + exp(u + k_t) v_t )
 *         / ( sum_{i < t} exp(-((t-1-i)/T) w + k_i)     + exp(u + k_t)     )
 * The original no-/T convention is the same formula with w replaced by T w. Term by term, with the
 * largest logit subtracted first (an exact identity); scale as in O1.
 */
int oracle_biwkv_causal_sum(const double* k, const double* v, const double* w, const double* u,
                            int64_t B, int64_t T, int64_t C, double* out, double* scale,
                            int nthreads) {
    if (!k || !v || !w || !u || !out || B < 0 || T < 0 || C < 0) return ORC_ERR_ARG;
    if (B == 0 || T == 0 || C == 0) return ORC_OK;
    set_threads(nthreads);
    int failed = 0;
#pragma omp parallel
    {
        double* kc = (double*)malloc(sizeof(double) * (size_t)T);
        double* vc = (double*)malloc(sizeof(double) * (size_t)T);
        double* s = (double*)malloc(sizeof(double) * (size_t)T);
        if (!kc || !vc || !s) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t bc = 0; bc < B * C; ++bc) {
                const int64_t b = bc / C, c = bc % C;
                gather_col(k, b, c, T, C, kc);
                gather_col(v, b, c, T, C, vc);
                const double wc = w[c], uc = u[c], Td = (double)T;
                for (int64_t t = 0; t < T; ++t) {
                    double M = -INFINITY;
                    for (int64_t i = 0; i <= t; ++i) {
                        const double si = (i == t) ? uc + kc[i]
                                                   : -(((double)(t - 1 - i)) / Td) * wc + kc[i];
                        s[i] = si;
                        if (si > M) M = si;
                    }
                    double num = 0.0, den = 0.0, mag = 0.0;
                    for (int64_t i = 0; i <= t; ++i) {
                        const double p = exp(s[i] - M);
                        num += p * vc[i];
                        den += p;
                        mag += p * fabs(vc[i]);
                    }
                    const int64_t o = (b * T + t) * C + c;
                    out[o] = num / den;
                    if (scale) scale[o] = mag / den;
                }
            }
        }
        free(kc);
        free(vc);
        free(s);
    }
    return failed ? ORC_ERR_NOMEM : ORC_OK;
}

/*
 * O2c — the causal attention in RNN form: Eq. (6)'s prefix states a, c only (one forward sweep)
 * and Eq. (7) with b = d = 0:
 *   A_0 = 0, A_{t+1} = lam*A_t + e_t v_t;  C_0 = 0, C_{t+1} = lam*C_t + e_t
 *   wkv_t = (A_t + E_t v_t) / (C_t + E_t),  E_t = exp(u + k_t - kappa)
 * with lam = exp(-w/T), e_i = exp(k_i - kappa), kappa = max_i k_i. Also returns the magnitude
 * scale (the same recurrence on |v|) when scale is not NULL.
 */
int oracle_biwkv_causal_rnn(const double* k, const double* v, const double* w, const double* u,
                            int64_t B, int64_t T, int64_t C, double* out, double* scale,
                            int nthreads) {
    if (!k || !v || !w || !u || !out || B < 0 || T < 0 || C < 0) return ORC_ERR_ARG;
    if (B == 0 || T == 0 || C == 0) return ORC_OK;
    set_threads(nthreads);
    int failed = 0;
#pragma omp parallel
    {
        double* kc = (double*)malloc(sizeof(double) * (size_t)T);
        double* vc = (double*)malloc(sizeof(double) * (size_t)T);
        if (!kc || !vc) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t bc = 0; bc < B * C; ++bc) {
                const int64_t b = bc / C, c = bc % C;
                gather_col(k, b, c, T, C, kc);
                gather_col(v, b, c, T, C, vc);
                double kappa = -INFINITY;
                for (int64_t t = 0; t < T; ++t)
                    if (kc[t] > kappa) kappa = kc[t];
                const double lam = exp(-w[c] / (double)T);
                double A = 0.0, Cs = 0.0, Am = 0.0;
                for (int64_t t = 0; t < T; ++t) {
                    const double E = exp(u[c] + kc[t] - kappa);
                    out[(b * T + t) * C + c] = (A + E * vc[t]) / (Cs + E);
                    if (scale) scale[(b * T + t) * C + c] = (Am + E * fabs(vc[t])) / (Cs + E);
                    const double e = exp(kc[t] - kappa);
                    A = lam * A + e * vc[t];
                    Cs = lam * Cs + e;
                    Am = lam * Am + e * fabs(vc[t]);
                }
            }
        }
        free(kc);
        free(vc);
    }
    return failed ? ORC_ERR_NOMEM : ORC_OK;
}

/*
 * OB1 — gradients of Eq. (5) of [VRWKV] (the pages state that the backward pass is an O(TC)
 * recurrence but do not print it), written out from the definition. With the weights
 * p_ti = exp(s_ti) / sum_j exp(s_tj) of Eq. (5) (s_ti = -((|t-i|-1)/T) w + k_i, s_tt = u + k_t)
 * and y_t = sum_i p_ti v_i, the upstream gradient g_t = dL/dy_t gives
 *   dv_i = sum_t g_t p_ti
 *   dk_i = sum_t g_t p_ti (v_i - y_t)
 *   du   = sum_t g_t p_tt (v_t - y_t)                                 (summed over b)
 *   dw   = sum_t sum_{i != t} g_t p_ti (v_i - y_t) * (-(|t-i|-1)/T)    (summed over b)
 * because dy_t/ds_ti = p_ti (v_i - y_t). Quadratic in T. Also returns magnitude scales for the
 * tests' error metric: |g_t| p_ti for dv, and |g_t| p_ti (|v_i| + |y_t|) in place of each term
 * g_t p_ti (v_i - y_t) (times |t-i|-1 over T for dw), since v_i - y_t of two nearly equal values
 * (T = 1, a dominant bonus term) is known only to the rounding of y_t, which is relative to
 * |y_t|; any scale pointer may be NULL.
 */
int oracle_biwkv_backward_sum(const double* k, const double* v, const double* w, const double* u,
                              const double* g, int64_t B, int64_t T, int64_t C, double* dk,
                              double* dv, double* dw, double* du, double* sdk, double* sdv,
                              double* sdw, double* sdu, int nthreads) {
    if (!k || !v || !w || !u || !g || !dk || !dv || !dw || !du || B < 0 || T < 0 || C < 0)
        return ORC_ERR_ARG;
    for (int64_t c = 0; c < C; ++c) {
        dw[c] = du[c] = 0.0;
        if (sdw) sdw[c] = 0.0;
        if (sdu) sdu[c] = 0.0;
    }
    if (B == 0 || T == 0 || C == 0) return ORC_OK;
    set_threads(nthreads);
    int failed = 0;
    /* per (c) accumulation of dw, du over b happens after the parallel loop, in b order */
    double* pw = (double*)calloc((size_t)(B * C), sizeof(double));
    double* pu = (double*)calloc((size_t)(B * C), sizeof(double));
    double* psw = (double*)calloc((size_t)(B * C), sizeof(double));
    double* psu = (double*)calloc((size_t)(B * C), sizeof(double));
    if (!pw || !pu || !psw || !psu) {
        free(pw); free(pu); free(psw); free(psu);
        return ORC_ERR_NOMEM;
    }
#pragma omp parallel
    {
        double* kc = (double*)malloc(sizeof(double) * (size_t)T);
        double* vc = (double*)malloc(sizeof(double) * (size_t)T);
        double* gc = (double*)malloc(sizeof(double) * (size_t)T);
        double* p = (double*)malloc(sizeof(double) * (size_t)(T * T));
        double* y = (double*)malloc(sizeof(double) * (size_t)T);
        if (!kc || !vc || !gc || !p || !y) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t bc = 0; bc < B * C; ++bc) {
                const int64_t b = bc / C, c = bc % C;
                gather_col(k, b, c, T, C, kc);
                gather_col(v, b, c, T, C, vc);
                gather_col(g, b, c, T, C, gc);
                const double wc = w[c], uc = u[c], Td = (double)T;
                /* the weights p_ti of every output t */
                for (int64_t t = 0; t < T; ++t) {
                    double* pt = p + t * T;
                    double M = -INFINITY;
                    for (int64_t i = 0; i < T; ++i) {
                        const int64_t dist = (i > t) ? (i - t) : (t - i);
                        pt[i] = (i == t) ? uc + kc[i] : -(((double)(dist - 1)) / Td) * wc + kc[i];
                        if (pt[i] > M) M = pt[i];
                    }
                    double den = 0.0, num = 0.0;
                    for (int64_t i = 0; i < T; ++i) {
                        pt[i] = exp(pt[i] - M);
                        den += pt[i];
                    }
                    for (int64_t i = 0; i < T; ++i) {
                        pt[i] /= den;
                        num += pt[i] * vc[i];
                    }
                    y[t] = num;
                }
                double dwc = 0.0, duc = 0.0, swc = 0.0, suc = 0.0;
                for (int64_t i = 0; i < T; ++i) {
                    double dvi = 0.0, dki = 0.0, svi = 0.0, ski = 0.0;
                    for (int64_t t = 0; t < T; ++t) {
                        const double gp = gc[t] * p[t * T + i];
                        const double term = gp * (vc[i] - y[t]);
                        const double mag = fabs(gp) * (fabs(vc[i]) + fabs(y[t]));
                        dvi += gp;
                        svi += fabs(gp);
                        dki += term;
                        ski += mag;
                        if (t == i) {
                            duc += term;
                            suc += mag;
                        } else {
                            const int64_t dist = (i > t) ? (i - t) : (t - i);
                            const double dterm = term * (-((double)(dist - 1)) / Td);
                            dwc += dterm;
                            swc += mag * (((double)(dist - 1)) / Td);
                        }
                    }
                    const int64_t o = (b * T + i) * C + c;
                    dv[o] = dvi;
                    dk[o] = dki;
                    if (sdv) sdv[o] = svi;
                    if (sdk) sdk[o] = ski;
                }
                pw[b * C + c] = dwc;
                pu[b * C + c] = duc;
                psw[b * C + c] = swc;
                psu[b * C + c] = suc;
            }
        }
        free(kc);
        free(vc);
        free(gc);
        free(p);
        free(y);
    }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < C; ++c) {
            dw[c] += pw[b * C + c];
            du[c] += pu[b * C + c];
            if (sdw) sdw[c] += psw[b * C + c];
            if (sdu) sdu[c] += psu[b * C + c];
        }
    free(pw);
    free(pu);
    free(psw);
    free(psu);
    return failed ? ORC_ERR_NOMEM : ORC_OK;
}

/*
 * OB2 — the same gradients in linear time, as decayed prefix / suffix sums (float64, valid while
 * lam^T and exp(u + k - kappa) stay inside float64, like O2). With lam = exp(-w/T),
 * e_i = exp(k_i - kappa), the forward states of Eq. (6)
 *   a_j = sum_{i<j} lam^{j-1-i} e_i v_i,  c_j = same with 1,  b_j = sum_{i>j} lam^{i-j-1} e_i v_i,  d_j
 * and D_j = c_j + d_j + e^{u} e_j, y_j from Eq. (7), put q_t = g_t / D_t and r_t = q_t y_t. Then
 *   dv_i = e_i (Qpre_i + Qsuf_i + e^{u} q_i),   dk_i = v_i dv_i - e_i (Rpre_i + Rsuf_i + e^{u} r_i)
 *   du   = sum_t e^{u} e_t (q_t v_t - r_t)
 * with Qpre_i = sum_{t<i} lam^{i-1-t} q_t and Qsuf_i = sum_{t>i} lam^{t-i-1} q_t (R alike), and,
 * writing |t-i|-1 as the number of tokens strictly between t and i and splitting lam^{|t-i|-1}
 * at each such token j,
 *   dw = -(lam / T) sum_j ( b_j Qpre_j - d_j Rpre_j + a_j Qsuf_j - c_j Rsuf_j ).
 * (kappa cancels: q carries 1/exp(kappa), the states exp(kappa).)
 */
int oracle_biwkv_backward_rnn(const double* k, const double* v, const double* w, const double* u,
                              const double* g, int64_t B, int64_t T, int64_t C, double* dk,
                              double* dv, double* dw, double* du, int nthreads) {
    if (!k || !v || !w || !u || !g || !dk || !dv || !dw || !du || B < 0 || T < 0 || C < 0)
        return ORC_ERR_ARG;
    for (int64_t c = 0; c < C; ++c) dw[c] = du[c] = 0.0;
    if (B == 0 || T == 0 || C == 0) return ORC_OK;
    set_threads(nthreads);
    int failed = 0;
    double* pw = (double*)calloc((size_t)(B * C), sizeof(double));
    double* pu = (double*)calloc((size_t)(B * C), sizeof(double));
    if (!pw || !pu) {
        free(pw);
        free(pu);
        return ORC_ERR_NOMEM;
    }
#pragma omp parallel
    {
        double* buf = (double*)malloc(sizeof(double) * (size_t)T * 14);
        if (!buf) {
#pragma omp atomic write
            failed = 1;
        } else {
            double *kc = buf, *vc = buf + T, *gc = buf + 2 * T, *e = buf + 3 * T;
            double *a = buf + 4 * T, *cc = buf + 5 * T, *bb = buf + 6 * T, *d = buf + 7 * T;
            double *q = buf + 8 * T, *r = buf + 9 * T, *qp = buf + 10 * T, *rp = buf + 11 * T;
            double *qs = buf + 12 * T, *rs = buf + 13 * T;
#pragma omp for schedule(dynamic, 1)
            for (int64_t bc = 0; bc < B * C; ++bc) {
                const int64_t b = bc / C, c = bc % C;
                gather_col(k, b, c, T, C, kc);
                gather_col(v, b, c, T, C, vc);
                gather_col(g, b, c, T, C, gc);
                double kappa = -INFINITY;
                for (int64_t t = 0; t < T; ++t)
                    if (kc[t] > kappa) kappa = kc[t];
                const double lam = exp(-w[c] / (double)T), eu = exp(u[c]);
                for (int64_t t = 0; t < T; ++t) e[t] = exp(kc[t] - kappa);
                double A = 0.0, Cs = 0.0;
                for (int64_t t = 0; t < T; ++t) {
                    a[t] = A;
                    cc[t] = Cs;
                    A = lam * A + e[t] * vc[t];
                    Cs = lam * Cs + e[t];
                }
                double Bs = 0.0, D = 0.0;
                for (int64_t t = T - 1; t >= 0; --t) {
                    bb[t] = Bs;
                    d[t] = D;
                    Bs = lam * Bs + e[t] * vc[t];
                    D = lam * D + e[t];
                }
                for (int64_t t = 0; t < T; ++t) {
                    const double den = cc[t] + d[t] + eu * e[t];
                    const double y = (a[t] + bb[t] + eu * e[t] * vc[t]) / den;
                    q[t] = gc[t] / den;
                    r[t] = q[t] * y;
                }
                double Q = 0.0, R = 0.0;
                for (int64_t t = 0; t < T; ++t) {
                    qp[t] = Q;
                    rp[t] = R;
                    Q = lam * Q + q[t];
                    R = lam * R + r[t];
                }
                Q = R = 0.0;
                for (int64_t t = T - 1; t >= 0; --t) {
                    qs[t] = Q;
                    rs[t] = R;
                    Q = lam * Q + q[t];
                    R = lam * R + r[t];
                }
                double dwc = 0.0, duc = 0.0;
                for (int64_t i = 0; i < T; ++i) {
                    const double dvi = e[i] * (qp[i] + qs[i] + eu * q[i]);
                    const int64_t o = (b * T + i) * C + c;
                    dv[o] = dvi;
                    dk[o] = vc[i] * dvi - e[i] * (rp[i] + rs[i] + eu * r[i]);
                    duc += eu * e[i] * (q[i] * vc[i] - r[i]);
                    dwc += bb[i] * qp[i] - d[i] * rp[i] + a[i] * qs[i] - cc[i] * rs[i];
                }
                pw[b * C + c] = -(lam / (double)T) * dwc;
                pu[b * C + c] = duc;
            }
        }
        free(buf);
    }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < C; ++c) {
            dw[c] += pw[b * C + c];
            du[c] += pu[b * C + c];
        }
    free(pw);
    free(pu);
    return failed ? ORC_ERR_NOMEM : ORC_OK;
}

/*
 * Channel-group boundaries of the q_shift function in [NOTES]: g_j = int(C * gamma * j),
 * j = 1..4, evaluated as the listing's Python does it: double product, left to right,
 * truncated toward zero.
 */
static int64_t group_bound(int64_t C, double gamma, int j) {
    const double x = (double)C * gamma * (double)j;
    return (int64_t)x;
}

/*
 * O3 — Q-Shift token shift X-dagger of [NOTES] (q_shift) on [B, H*W, C] data, token n = h*W + w.
 * Values are moved as raw 32-bit words (no floating-point operation touches them).
 *   c in [0, g1):   out[h, w] = x[h, w - s]  if w >= s      else 0   (shift right)
 *   c in [g1, g2):  out[h, w] = x[h, w + s]  if w <  W - s  else 0   (shift left)
 *   c in [g2, g3):  out[h, w] = x[h - s, w]  if h >= s      else 0   (shift down)
 *   c in [g3, g4):  out[h, w] = x[h + s, w]  if h <  H - s  else 0   (shift up)
 *   c >= g4:        out[h, w] = x[h, w]                             (copied)
 * Errors: gamma outside [0, 1/4] or NaN (the listing asserts gamma <= 1/4), shift < 0, or
 * shift > min(H, W) (the listing's slice assignment fails for such shifts).
 */
int oracle_qshift(const uint32_t* x, uint32_t* out, int64_t B, int64_t H, int64_t W, int64_t C,
                  int64_t shift, double gamma) {
    if (!x || !out || B < 0 || H < 0 || W < 0 || C < 0) return ORC_ERR_ARG;
    if (!(gamma >= 0.0 && gamma <= 0.25)) return ORC_ERR_PARAM;
    if (shift < 0 || shift > H || shift > W) return ORC_ERR_PARAM;
    const int64_t g1 = group_bound(C, gamma, 1), g2 = group_bound(C, gamma, 2);
    const int64_t g3 = group_bound(C, gamma, 3), g4 = group_bound(C, gamma, 4);
    const int64_t s = shift;
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t h = 0; h < H; ++h) {
            for (int64_t wc = 0; wc < W; ++wc) {
                for (int64_t c = 0; c < C; ++c) {
                    int64_t sh = h, sw = wc;
                    int valid = 1;
                    if (c < g1) {
                        sw = wc - s;
                        valid = wc >= s;
                    } else if (c < g2) {
                        sw = wc + s;
                        valid = wc < W - s;
                    } else if (c < g3) {
                        sh = h - s;
                        valid = h >= s;
                    } else if (c < g4) {
                        sh = h + s;
                        valid = h < H - s;
                    }
                    const int64_t o = ((b * H + h) * W + wc) * C + c;
                    out[o] = valid ? x[((b * H + sh) * W + sw) * C + c] : 0u;
                }
            }
        }
    }
    return ORC_OK;
}

/*
 * O3b — the bidirectional shift that the Vision-RWKV article's MAE paragraph puts in place of
 * Q-Shift for sparse inputs (only the visible tokens of a masked image are present, so there is
 * no H x W grid). Reading: the token sequence of length N replaces the grid, and each channel
 * group keeps the sense of its Q-Shift move: the groups that take an earlier raster token (shift
 * right, shift down) take token n - s, the groups that take a later one (left, up) take token
 * n + s. Same group bounds g_j, zero fill at the ends, remainder copied, raw 32-bit words:
 *   c in [0, g1) and [g2, g3):  out[n] = x[n - s]  if n >= s      else 0
 *   c in [g1, g2) and [g3, g4): out[n] = x[n + s]  if n <  N - s  else 0
 *   c >= g4:                    out[n] = x[n]
 * Errors: gamma outside [0, 1/4] or NaN, shift < 0 or shift > N.
 */
int oracle_qshift_bidir(const uint32_t* x, uint32_t* out, int64_t B, int64_t N, int64_t C,
                        int64_t shift, double gamma) {
    if (!x || !out || B < 0 || N < 0 || C < 0) return ORC_ERR_ARG;
    if (!(gamma >= 0.0 && gamma <= 0.25)) return ORC_ERR_PARAM;
    if (shift < 0 || shift > N) return ORC_ERR_PARAM;
    const int64_t g1 = group_bound(C, gamma, 1), g2 = group_bound(C, gamma, 2);
    const int64_t g3 = group_bound(C, gamma, 3), g4 = group_bound(C, gamma, 4);
    const int64_t s = shift;
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t c = 0; c < C; ++c) {
                int64_t src = n;
                int valid = 1;
                if (c < g4) {
                    const int earlier = c < g1 || (c >= g2 && c < g3);
                    if (earlier) {
                        src = n - s;
                        valid = n >= s;
                    } else {
                        src = n + s;
                        valid = n < N - s;
                    }
                }
                out[(b * N + n) * C + c] = valid ? x[(b * N + src) * C + c] : 0u;
            }
        }
    }
    return ORC_OK;
}
