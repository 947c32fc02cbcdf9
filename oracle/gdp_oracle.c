/*
 * gdp_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64 CPU reference for the chunked Gated Delta Product (GDP)
 * forward.  Only tests/, the package smoke check and the benchmark's CPU
 * baseline may load this library.  It shares no source with the HIP kernels
 * and the product path never calls it.
 *
 * What it computes (one sequence, one value head per call):
 *
 *   The gated delta rule (Yang, Kautz & Hatamizadeh, "Gated Delta Networks",
 *   ICLR 2025) run over the Householder-expanded stream.  The expanded stream
 *   holds M rows per token, row e = t*M + j for copy j (copies folded into the
 *   sequence dimension: core.ssm.ops.gdp.prepare, module description).  The
 *   token's decay acts on its first copy and its query is read after its last
 *   copy (core.ssm.ops.gdp.prepare, module description, the decode bullet that
 *   places the query on the last copy and the decay on the first).
 *
 *   State S is V x K.  For each expanded row e of token t, copy j:
 *       alpha_e = exp(g_t) if j == 0 else 1
 *       S_e     = alpha_e * S_{e-1} * (I - beta_e khat_e khat_e^T)
 *                 + beta_e * v_e * khat_e^T
 *   which is evaluated in the equivalent "corrected value" form
 *       delta_e = beta_e * (v_e - alpha_e * S_{e-1} khat_e)
 *       S_e     = alpha_e * S_{e-1} + delta_e khat_e^T
 *   (expand the product: alpha*S - alpha*beta*(S khat) khat^T + beta*v khat^T).
 *   Output after the last copy of token t:  o_t = scale * S_{tM+M-1} qhat_t.
 *   qhat and khat are L2-normalised per row, x / sqrt(sum x^2 + eps); the
 *   normalisation belongs to the chunk op, not to prepare
 *   (core.ssm.ops.gdp.prepare, gdp_prefill_prepare, Returns).
 *
 *   delta_e is what the chunk_o page calls the corrected values
 *   (core.ssm.ops.gdp.chunk_o, chunk_gated_delta_product_fwd_o, Parameters v);
 *   the state snapshot entering chunk c is S_{c*C-1} (S_{-1} = h0 or 0): the
 *   "state at each chunk boundary" of the same parameter list.
 *
 * gdp_oracle_wy computes the per-chunk WY factors by textbook forward
 * substitution (core.ssm.ops.gdp.wy_fast, module description and
 * recompute_w_u_fwd): with gamma_e the within-chunk cumulative log decay,
 *       L_ab = beta_a exp(gamma_a - gamma_b) khat_a . khat_b   (b < a)
 *       (I + L) U = diag(beta) V,   (I + L) W = diag(beta exp(gamma)) Khat
 * solved row by row; U is u (effective values), W is w (effective keys
 * carrying the decay).
 *
 * All arithmetic is double precision on the exact values of the inputs.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Row r of a row-major 2-D array with row stride rs (elements). */
#define ROW(p, r, rs) ((p) + (int64_t)(r) * (rs))

/* out[i] = x[i] / sqrt(sum_i x[i]^2 + eps) */
static void l2_normalise(const float *x, int n, double eps, double *out)
{
    double ss = 0.0;
    for (int i = 0; i < n; ++i)
        ss += (double)x[i] * (double)x[i];
    double inv = 1.0 / sqrt(ss + eps);
    for (int i = 0; i < n; ++i)
        out[i] = (double)x[i] * inv;
}

/*
 * Serial recurrence over one sequence of L tokens for one value head.
 *
 * Inputs (float32 values; bf16 data is widened exactly by the caller):
 *   q    [L][K]     row stride q_rs      (query of token t)
 *   k    [L*M][K]   row stride k_rs      (key of expanded row e)
 *   v    [L*M][V]   row stride v_rs
 *   beta [L*M]      stride beta_rs
 *   g    [L]        stride g_rs; natural-log decay of token t; NULL means 0
 *   h0   [V][K]     initial state, NULL means zero
 * Outputs (double, caller-owned, any may be NULL except o):
 *   o      [L][V]
 *   v_new  [L*M][V]      delta_e
 *   h      [nc][V][K]    S entering chunk c (rows [c*chunk, (c+1)*chunk)),
 *                        nc = ceil(L*M / chunk)
 *   h_final [V][K]       S after the last row
 * Returns 0, or -1 on bad sizes, -2 on allocation failure.
 */
int gdp_oracle_recurrence(int64_t L, int M, int K, int V,
                          const float *q, int64_t q_rs,
                          const float *k, int64_t k_rs,
                          const float *v, int64_t v_rs,
                          const float *beta, int64_t beta_rs,
                          const float *g, int64_t g_rs,
                          double scale, double eps, int chunk,
                          const double *h0,
                          double *o, double *v_new, double *h, double *h_final)
{
    if (L < 0 || M < 1 || K < 1 || V < 1 || chunk < 1 || o == NULL)
        return -1;
    double *S = (double *)calloc((size_t)V * K, sizeof(double));
    double *kh = (double *)malloc((size_t)K * sizeof(double));
    double *qh = (double *)malloc((size_t)K * sizeof(double));
    double *d = (double *)malloc((size_t)V * sizeof(double));
    if (!S || !kh || !qh || !d) {
        free(S); free(kh); free(qh); free(d);
        return -2;
    }
    if (h0)
        memcpy(S, h0, sizeof(double) * (size_t)V * K);

    const int64_t rows = L * (int64_t)M;
    for (int64_t e = 0; e < rows; ++e) {
        const int64_t t = e / M;
        const int j = (int)(e % M);

        /* state entering a chunk boundary */
        if (h && e % chunk == 0)
            memcpy(h + (e / chunk) * (int64_t)V * K, S, sizeof(double) * (size_t)V * K);

        const double alpha = (j == 0 && g) ? exp((double)*ROW(g, t, g_rs)) : 1.0;
        const double b = (double)*ROW(beta, e, beta_rs);
        l2_normalise(ROW(k, e, k_rs), K, eps, kh);
        const float *ve = ROW(v, e, v_rs);

        /* delta = beta * (v - alpha * S khat) */
        for (int i = 0; i < V; ++i) {
            double sk = 0.0;
            for (int c = 0; c < K; ++c)
                sk += S[(int64_t)i * K + c] * kh[c];
            d[i] = b * ((double)ve[i] - alpha * sk);
        }
        /* S = alpha * S + delta khat^T */
        for (int i = 0; i < V; ++i)
            for (int c = 0; c < K; ++c)
                S[(int64_t)i * K + c] = alpha * S[(int64_t)i * K + c] + d[i] * kh[c];

        if (v_new)
            for (int i = 0; i < V; ++i)
                v_new[e * V + i] = d[i];

        /* query of token t is read after its last copy */
        if (j == M - 1) {
            l2_normalise(ROW(q, t, q_rs), K, eps, qh);
            for (int i = 0; i < V; ++i) {
                double s = 0.0;
                for (int c = 0; c < K; ++c)
                    s += S[(int64_t)i * K + c] * qh[c];
                o[t * V + i] = scale * s;
            }
        }
    }
    if (h_final)
        memcpy(h_final, S, sizeof(double) * (size_t)V * K);
    free(S); free(kh); free(qh); free(d);
    return 0;
}

/*
 * Per-chunk WY factors for one sequence of L tokens and one value head.
 * Chunks are rows [c*chunk, min((c+1)*chunk, L*M)) of the expanded stream.
 * gamma_e = sum of log alpha over rows of the chunk up to and including e,
 * where log alpha_e = g_t on the first copy of token t and 0 otherwise.
 * Outputs w [L*M][K] and u [L*M][V] (double); either may be NULL.
 */
int gdp_oracle_wy(int64_t L, int M, int K, int V,
                  const float *k, int64_t k_rs,
                  const float *v, int64_t v_rs,
                  const float *beta, int64_t beta_rs,
                  const float *g, int64_t g_rs,
                  double eps, int chunk,
                  double *w, double *u)
{
    if (L < 0 || M < 1 || K < 1 || V < 1 || chunk < 1)
        return -1;
    const int64_t rows = L * (int64_t)M;
    double *kh = (double *)malloc(sizeof(double) * (size_t)chunk * K);
    double *gam = (double *)malloc(sizeof(double) * (size_t)chunk);
    double *Lm = (double *)malloc(sizeof(double) * (size_t)chunk * chunk);
    double *bu = (double *)malloc(sizeof(double) * (size_t)chunk);
    if (!kh || !gam || !Lm || !bu) {
        free(kh); free(gam); free(Lm); free(bu);
        return -2;
    }
    for (int64_t c0 = 0; c0 < rows; c0 += chunk) {
        const int n = (int)((rows - c0 < chunk) ? rows - c0 : chunk);
        double run = 0.0;
        for (int a = 0; a < n; ++a) {
            const int64_t e = c0 + a;
            if (e % M == 0 && g)
                run += (double)*ROW(g, e / M, g_rs);
            gam[a] = run;
            bu[a] = (double)*ROW(beta, e, beta_rs);
            l2_normalise(ROW(k, e, k_rs), K, eps, kh + (int64_t)a * K);
        }
        /* strictly lower transition block */
        for (int a = 0; a < n; ++a)
            for (int b = 0; b < n; ++b) {
                double val = 0.0;
                if (b < a) {
                    double dot = 0.0;
                    for (int c = 0; c < K; ++c)
                        dot += kh[(int64_t)a * K + c] * kh[(int64_t)b * K + c];
                    val = bu[a] * exp(gam[a] - gam[b]) * dot;
                }
                Lm[(int64_t)a * chunk + b] = val;
            }
        /* forward substitution, row by row: X_a = rhs_a - sum_{b<a} L_ab X_b */
        if (u)
            for (int a = 0; a < n; ++a) {
                const float *va = ROW(v, c0 + a, v_rs);
                double *ua = u + (c0 + a) * V;
                for (int i = 0; i < V; ++i) {
                    double s = bu[a] * (double)va[i];
                    for (int b = 0; b < a; ++b)
                        s -= Lm[(int64_t)a * chunk + b] * u[(c0 + b) * V + i];
                    ua[i] = s;
                }
            }
        if (w)
            for (int a = 0; a < n; ++a) {
                const double scale_a = bu[a] * exp(gam[a]);
                double *wa = w + (c0 + a) * K;
                for (int i = 0; i < K; ++i) {
                    double s = scale_a * kh[(int64_t)a * K + i];
                    for (int b = 0; b < a; ++b)
                        s -= Lm[(int64_t)a * chunk + b] * w[(c0 + b) * K + i];
                    wa[i] = s;
                }
            }
    }
    free(kh); free(gam); free(Lm); free(bu);
    return 0;
}
