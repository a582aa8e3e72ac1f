/*
 * Oracle: causal linear attention with per-head decay, recurrent form, fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this code; the product path never
 * does.  It shares no code with the GPU library.
 *
 * What it computes (per (batch, head) sequence of n tokens, head dim d,
 * decay lam in [0, 1]):
 *   O_t = sum_{j <= t} lam^(t-j) (q_t . k_j) v_j  [+ lam^(t+1) q_t S0]
 * Lightning Attention-2 (phantomic12.github.io, "Lightning Attention-2",
 * Tiling paragraph and the record's mechanism field) computes exactly this
 * causal linear attention, reorganised into blocks; the glossary page
 * ("Lightning Attention", features list: recurrent/parallel forms, fixed-size
 * state) states that a recurrent form with a fixed-size state computes the same
 * function.  This file is that recurrent form, token by token, with no
 * blocking:
 *   S <- lam S + k_t v_t^T  (S is d x d, rows indexed by key dim, columns by
 *   value dim), then o_t = q_t S.
 * The backward is for the loss L = <dO, O> with S0 held constant:
 *   forward sweep  S <- lam S + k_t v_t^T,  dq_t = S dO_t
 *   reverse sweep  dS <- lam dS + q_t dO_t^T,  dk_t = dS v_t,  dv_t = dS^T k_t.
 * The derivative of the same loss with respect to lam comes from differentiating
 * the recurrence forward in lam: T = dS/dlam is carried next to S.
 * Pinned by the CPU tests against exact rational brute force of the definition
 * (including exact gradients obtained from the definition by linearity),
 * closed forms for constant inputs, the quadratic masked form and a library
 * matrix product at lam = 1.
 *
 * Layout: each sequence is row-major [n][d]; state is row-major [d][d]
 * (key index, value index).  Batched entry points loop over `pairs`
 * independent sequences with OpenMP, each with its own lam.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* One sequence, recurrent forward.
 * s_init: d*d or NULL (zero).  o: n*d.  s_final: d*d or NULL.
 * s_bounds: if not NULL, receives the state before token b*bk for every
 * b = 0 .. ceil(n/bk) - 1 (ceil(n/bk) * d * d doubles). */
static void fwd_one(const double* q, const double* k, const double* v, int64_t n, int64_t d,
                    double lam, const double* s_init, double* o, double* s_final, double* s_bounds,
                    int64_t bk) {
    double* S = (double*)calloc((size_t)(d * d), sizeof(double));
    if (s_init) memcpy(S, s_init, sizeof(double) * (size_t)(d * d));
    for (int64_t t = 0; t < n; ++t) {
        if (s_bounds && bk > 0 && t % bk == 0)
            memcpy(s_bounds + (t / bk) * d * d, S, sizeof(double) * (size_t)(d * d));
        const double* kt = k + t * d;
        const double* vt = v + t * d;
        const double* qt = q + t * d;
        for (int64_t a = 0; a < d; ++a) {
            double* row = S + a * d;
            double ka = kt[a];
            for (int64_t c = 0; c < d; ++c) row[c] = lam * row[c] + ka * vt[c];
        }
        double* ot = o + t * d;
        for (int64_t c = 0; c < d; ++c) ot[c] = 0.0;
        for (int64_t a = 0; a < d; ++a) {
            double qa = qt[a];
            const double* row = S + a * d;
            for (int64_t c = 0; c < d; ++c) ot[c] += qa * row[c];
        }
    }
    if (s_final) memcpy(s_final, S, sizeof(double) * (size_t)(d * d));
    free(S);
}

/* One sequence, backward of L = <dO, O>.  Any of dq, dk, dv may be NULL. */
/* Backward of L = <dO, O> + <G, S_N> for one sequence (G = dkv_out, may be NULL
 * for zero).  The forward-order sweep gives dQ (S includes token t); the
 * reverse sweep carries the adjoint of the state after token t,
 *     A_t = q_t dO_t^T + lam A_{t+1},   A_{n-1} = q_{n-1} dO_{n-1}^T + G,
 * (the recurrence S_t = lam S_{t-1} + k_t v_t^T, o_t = q_t S_t run backwards),
 * so dk_t = A_t v_t, dv_t = A_t^T k_t, and the gradient of the initial state
 * S_{-1} = S0 is lam A_0 (ds_init, may be NULL). */
static void bwd_one(const double* q, const double* k, const double* v, const double* dout, int64_t n,
                    int64_t d, double lam, const double* s_init, const double* g_final, double* dq,
                    double* dk, double* dv, double* ds_init) {
    double* S = (double*)calloc((size_t)(d * d), sizeof(double));
    if (dq) {
        if (s_init) memcpy(S, s_init, sizeof(double) * (size_t)(d * d));
        for (int64_t t = 0; t < n; ++t) {
            const double* kt = k + t * d;
            const double* vt = v + t * d;
            const double* gt = dout + t * d;
            double* out = dq + t * d;
            for (int64_t a = 0; a < d; ++a) {
                double* row = S + a * d;
                double ka = kt[a], acc = 0.0;
                for (int64_t c = 0; c < d; ++c) {
                    row[c] = lam * row[c] + ka * vt[c];
                    acc += row[c] * gt[c];
                }
                out[a] = acc;
            }
        }
    }
    if (dk || dv || ds_init) {
        if (g_final)
            memcpy(S, g_final, sizeof(double) * (size_t)(d * d));
        else
            memset(S, 0, sizeof(double) * (size_t)(d * d));
        for (int64_t t = n - 1; t >= 0; --t) {
            const double* qt = q + t * d;
            const double* gt = dout + t * d;
            const double* kt = k + t * d;
            const double* vt = v + t * d;
            const double dec = (t == n - 1) ? 1.0 : lam;  /* A_{t+1} carries lam; G enters undecayed */
            for (int64_t a = 0; a < d; ++a) {
                double* row = S + a * d;
                double qa = qt[a];
                for (int64_t c = 0; c < d; ++c) row[c] = dec * row[c] + qa * gt[c];
            }
            if (dk) {
                double* out = dk + t * d;
                for (int64_t a = 0; a < d; ++a) {
                    const double* row = S + a * d;
                    double acc = 0.0;
                    for (int64_t c = 0; c < d; ++c) acc += row[c] * vt[c];
                    out[a] = acc;
                }
            }
            if (dv) {
                double* out = dv + t * d;
                for (int64_t c = 0; c < d; ++c) out[c] = 0.0;
                for (int64_t a = 0; a < d; ++a) {
                    const double* row = S + a * d;
                    double ka = kt[a];
                    for (int64_t c = 0; c < d; ++c) out[c] += ka * row[c];
                }
            }
        }
        if (ds_init) {
            if (n > 0)
                for (int64_t e = 0; e < d * d; ++e) ds_init[e] = lam * S[e];
            else
                for (int64_t e = 0; e < d * d; ++e) ds_init[e] = g_final ? g_final[e] : 0.0;
        }
    }
    free(S);
}

/* Derivative of L = <dO, O> + <G, S_N> with respect to lam for one sequence
 * (G = g_final, may be NULL for zero), by forward-mode differentiation of the
 * recurrence.  With T_t = dS_t/dlam (S_{-1} = S0 does not depend on lam):
 *     T_t = S_{t-1} + lam T_{t-1},   T_{-1} = 0,
 *     S_t = lam S_{t-1} + k_t v_t^T,
 *     d o_t / dlam = q_t T_t,
 * so dL/dlam = sum_t <dO_t, q_t T_t> + <G, T_{n-1}>. */
static double dlam_one(const double* q, const double* k, const double* v, const double* dout,
                       int64_t n, int64_t d, double lam, const double* s_init, const double* g_final) {
    double* S = (double*)calloc((size_t)(d * d), sizeof(double));
    double* T = (double*)calloc((size_t)(d * d), sizeof(double));
    double* u = (double*)calloc((size_t)d, sizeof(double));
    if (s_init) memcpy(S, s_init, sizeof(double) * (size_t)(d * d));
    double total = 0.0;
    for (int64_t t = 0; t < n; ++t) {
        const double* kt = k + t * d;
        const double* vt = v + t * d;
        const double* qt = q + t * d;
        const double* gt = dout + t * d;
        for (int64_t a = 0; a < d; ++a) {
            double* srow = S + a * d;
            double* trow = T + a * d;
            double ka = kt[a];
            for (int64_t c = 0; c < d; ++c) {
                trow[c] = srow[c] + lam * trow[c];
                srow[c] = lam * srow[c] + ka * vt[c];
            }
        }
        for (int64_t c = 0; c < d; ++c) u[c] = 0.0;
        for (int64_t a = 0; a < d; ++a) {
            double qa = qt[a];
            const double* trow = T + a * d;
            for (int64_t c = 0; c < d; ++c) u[c] += qa * trow[c];
        }
        for (int64_t c = 0; c < d; ++c) total += u[c] * gt[c];
    }
    if (g_final)
        for (int64_t e = 0; e < d * d; ++e) total += g_final[e] * T[e];
    free(S);
    free(T);
    free(u);
    return total;
}

/* Batched forward over `pairs` sequences laid out back to back ([pairs][n][d]).
 * lam: pairs entries.  s_init: [pairs][d][d] or NULL.  s_final: [pairs][d][d] or NULL.
 * s_bounds: [pairs][ceil(n/bk)][d][d] or NULL. */
void oracle_fwd_recurrent(const double* q, const double* k, const double* v, int64_t pairs,
                          int64_t n, int64_t d, const double* lam, const double* s_init, double* o,
                          double* s_final, double* s_bounds, int64_t bk) {
    int64_t nb = (bk > 0) ? (n + bk - 1) / bk : 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < pairs; ++p) {
        fwd_one(q + p * n * d, k + p * n * d, v + p * n * d, n, d, lam[p],
                s_init ? s_init + p * d * d : NULL, o + p * n * d, s_final ? s_final + p * d * d : NULL,
                s_bounds ? s_bounds + p * nb * d * d : NULL, bk);
    }
}

void oracle_bwd_recurrent(const double* q, const double* k, const double* v, const double* dout,
                          int64_t pairs, int64_t n, int64_t d, const double* lam, const double* s_init,
                          const double* g_final, double* dq, double* dk, double* dv, double* ds_init) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < pairs; ++p) {
        int64_t off = p * n * d, so = p * d * d;
        bwd_one(q + off, k + off, v + off, dout + off, n, d, lam[p], s_init ? s_init + so : NULL,
                g_final ? g_final + so : NULL, dq ? dq + off : NULL, dk ? dk + off : NULL,
                dv ? dv + off : NULL, ds_init ? ds_init + so : NULL);
    }
}

/* dL/dlam of every sequence (see dlam_one): out[p] for p < pairs. */
void oracle_dlam_recurrent(const double* q, const double* k, const double* v, const double* dout,
                           int64_t pairs, int64_t n, int64_t d, const double* lam, const double* s_init,
                           const double* g_final, double* out) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < pairs; ++p) {
        int64_t off = p * n * d, so = p * d * d;
        out[p] = dlam_one(q + off, k + off, v + off, dout + off, n, d, lam[p],
                          s_init ? s_init + so : NULL, g_final ? g_final + so : NULL);
    }
}

/* One recurrent decode step for `pairs` independent (sequence, head) states:
 * S <- lam S + k v^T, then o = q S.  state: [pairs][d][d] updated in place;
 * q, k, v, o: [pairs][d]. */
void oracle_decode_step(double* state, const double* q, const double* k, const double* v,
                        int64_t pairs, int64_t d, const double* lam, double* o) {
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < pairs; ++p) {
        double* S = state + p * d * d;
        const double *qp = q + p * d, *kp = k + p * d, *vp = v + p * d;
        double* op = o + p * d;
        for (int64_t a = 0; a < d; ++a)
            for (int64_t c = 0; c < d; ++c) S[a * d + c] = lam[p] * S[a * d + c] + kp[a] * vp[c];
        for (int64_t c = 0; c < d; ++c) op[c] = 0.0;
        for (int64_t a = 0; a < d; ++a)
            for (int64_t c = 0; c < d; ++c) op[c] += qp[a] * S[a * d + c];
    }
}
