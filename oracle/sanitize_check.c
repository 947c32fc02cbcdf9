/*
 * sanitize_check.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A driver that runs every entry point of gdp_oracle.c over small and edge
 * shapes (empty and one-token sequences, ragged last chunks, chunk sizes 1
 * and larger than the stream, M = 1..4, strided rows, absent optional
 * inputs and outputs) with exactly sized heap buffers, so that a build with
 * -fsanitize=address,undefined reports any out-of-bounds access, leak or
 * undefined operation in the oracle.  It checks return codes and that every
 * written output is finite; the values themselves are pinned by the Python
 * tests.  Prints "ok" and returns 0 when every case passes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int gdp_oracle_recurrence(int64_t L, int M, int K, int V, const float *q, int64_t q_rs, const float *k,
                          int64_t k_rs, const float *v, int64_t v_rs, const float *beta, int64_t beta_rs,
                          const float *g, int64_t g_rs, double scale, double eps, int chunk, const double *h0,
                          double *o, double *v_new, double *h, double *h_final);
int gdp_oracle_wy(int64_t L, int M, int K, int V, const float *k, int64_t k_rs, const float *v, int64_t v_rs,
                  const float *beta, int64_t beta_rs, const float *g, int64_t g_rs, double eps, int chunk,
                  double *w, double *u);

static uint64_t state = 0x9e3779b97f4a7c15ull;

/* uniform in [lo, hi) from a 64-bit linear congruential step */
static float uni(float lo, float hi) {
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return lo + (hi - lo) * (float)((state >> 40) * (1.0 / 16777216.0));
}

/* an n-element array (NULL for n == 0, like a caller with nothing to pass) */
static float *arr(int64_t n, float lo, float hi) {
    if (n == 0) return NULL;
    float *p = (float *)malloc(sizeof(float) * (size_t)n);
    if (!p) exit(2);
    for (int64_t i = 0; i < n; ++i) p[i] = uni(lo, hi);
    return p;
}

static double *darr(int64_t n) {
    if (n == 0) return NULL;
    double *p = (double *)calloc((size_t)n, sizeof(double));
    if (!p) exit(2);
    return p;
}

static int finite_all(const double *p, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) return 0;
    return 1;
}

static int failures = 0;

static void expect(int cond, const char *what, int64_t L, int M, int K, int V, int chunk) {
    if (!cond) {
        fprintf(stderr, "FAIL %s: L=%lld M=%d K=%d V=%d chunk=%d\n", what, (long long)L, M, K, V, chunk);
        ++failures;
    }
}

/* One shape: row strides wider than the rows (pad columns), with or without
 * gates, initial state and each optional output. */
static void run_case(int64_t L, int M, int K, int V, int chunk, int pad, int with_g, int with_h0, int with_opt) {
    const int64_t rows = L * M;
    const int64_t q_rs = K + pad, k_rs = K + pad, v_rs = V + pad, b_rs = 1 + pad, g_rs = 1 + pad;
    /* each strided array holds exactly (n - 1) * stride + width elements */
    const int64_t nq = L ? (L - 1) * q_rs + K : 0, nk = rows ? (rows - 1) * k_rs + K : 0;
    const int64_t nv = rows ? (rows - 1) * v_rs + V : 0, nb = rows ? (rows - 1) * b_rs + 1 : 0;
    const int64_t ng = L ? (L - 1) * g_rs + 1 : 0;
    float *q = arr(nq, -1.f, 1.f), *k = arr(nk, -1.f, 1.f), *v = arr(nv, -1.f, 1.f);
    float *beta = arr(nb, 0.f, 2.f), *g = with_g ? arr(ng, -3.f, 0.f) : NULL;
    const int64_t nc = (rows + chunk - 1) / chunk;
    double *h0 = with_h0 ? darr((int64_t)V * K) : NULL;
    if (h0)
        for (int64_t i = 0; i < (int64_t)V * K; ++i) h0[i] = uni(-0.5f, 0.5f);
    double *o = darr(L * V + 1);  /* o is required even for L = 0 */
    double *vn = with_opt ? darr(rows * V) : NULL, *h = with_opt ? darr(nc * V * K) : NULL;
    double *hf = with_opt ? darr((int64_t)V * K) : NULL;
    int rc = gdp_oracle_recurrence(L, M, K, V, q, q_rs, k, k_rs, v, v_rs, beta, b_rs, g, g_rs, 0.125, 1e-6,
                                   chunk, h0, o, vn, h, hf);
    expect(rc == 0, "recurrence rc", L, M, K, V, chunk);
    expect(finite_all(o, L * V), "recurrence o finite", L, M, K, V, chunk);
    if (with_opt) {
        expect(finite_all(vn, rows * V), "recurrence v_new finite", L, M, K, V, chunk);
        expect(finite_all(h, nc * V * K), "recurrence h finite", L, M, K, V, chunk);
        expect(finite_all(hf, (int64_t)V * K), "recurrence h_final finite", L, M, K, V, chunk);
    }
    double *w = darr(rows * K), *u = with_opt ? darr(rows * V) : NULL;
    rc = gdp_oracle_wy(L, M, K, V, k, k_rs, v, v_rs, beta, b_rs, g, g_rs, 1e-6, chunk, w, u);
    expect(rc == 0, "wy rc", L, M, K, V, chunk);
    expect(finite_all(w, rows * K), "wy w finite", L, M, K, V, chunk);
    if (u) expect(finite_all(u, rows * V), "wy u finite", L, M, K, V, chunk);
    free(q); free(k); free(v); free(beta); free(g); free(h0); free(o); free(vn); free(h); free(hf);
    free(w); free(u);
}

int main(void) {
    static const int64_t Ls[] = {0, 1, 2, 7, 33, 70};
    static const int Ms[] = {1, 2, 3, 4};
    static const int chunks[] = {1, 16, 64, 512};
    for (size_t a = 0; a < sizeof(Ls) / sizeof(Ls[0]); ++a)
        for (size_t b = 0; b < sizeof(Ms) / sizeof(Ms[0]); ++b)
            for (size_t c = 0; c < sizeof(chunks) / sizeof(chunks[0]); ++c) {
                const int variant = (int)((a + b + c) % 4);
                run_case(Ls[a], Ms[b], 8, 12, chunks[c], variant == 1 ? 3 : 0, variant != 2, variant == 3,
                         variant != 0);
            }
    run_case(5, 2, 64, 64, 64, 1, 1, 1, 1);
    run_case(40, 3, 128, 32, 64, 0, 1, 0, 1);
    /* rejected sizes return -1 without touching anything */
    double o1 = 0.0;
    expect(gdp_oracle_recurrence(-1, 1, 8, 8, NULL, 0, NULL, 0, NULL, 0, NULL, 0, NULL, 0, 1.0, 1e-6, 64, NULL,
                                 &o1, NULL, NULL, NULL) == -1, "recurrence rejects L < 0", -1, 1, 8, 8, 64);
    expect(gdp_oracle_recurrence(1, 0, 8, 8, NULL, 0, NULL, 0, NULL, 0, NULL, 0, NULL, 0, 1.0, 1e-6, 64, NULL,
                                 &o1, NULL, NULL, NULL) == -1, "recurrence rejects M < 1", 1, 0, 8, 8, 64);
    expect(gdp_oracle_recurrence(1, 1, 8, 8, NULL, 0, NULL, 0, NULL, 0, NULL, 0, NULL, 0, 1.0, 1e-6, 64, NULL,
                                 NULL, NULL, NULL, NULL) == -1, "recurrence rejects o == NULL", 1, 1, 8, 8, 64);
    expect(gdp_oracle_wy(1, 1, 8, 8, NULL, 0, NULL, 0, NULL, 0, NULL, 0, 1e-6, 0, NULL, NULL) == -1,
           "wy rejects chunk < 1", 1, 1, 8, 8, 0);
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
