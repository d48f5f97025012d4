/*
 * Driver for sanitizer builds of the CPU oracle (tests/test_sanitizers.py):
 * runs the fp64 and fp32 recurrences on small seeded inputs (several threads,
 * empty and one-token sequences, absent gates/beta/state, with and without
 * the L2 norm) and checks one closed form (beta = 0: the state only decays,
 * S_T = (prod a) S_0).  Exit status 0 when every run succeeds and the closed
 * form holds; sanitizer reports are the test's real subject.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int gdn_oracle_run_f64(const double *q, const double *k, const double *v, const double *g, const double *beta,
                       double scale, const int64_t *cu, int64_t N, int64_t Hqk, int64_t Hv, int64_t K, int64_t V,
                       const double *s0, int l2, double *out, double *sN, int nthreads);
int gdn_oracle_run_f32(const float *q, const float *k, const float *v, const float *g, const float *beta,
                       double scale, const int64_t *cu, int64_t N, int64_t Hqk, int64_t Hv, int64_t K, int64_t V,
                       const float *s0, int l2, float *out, float *sN, int nthreads);

static uint64_t rng = 88172645463325252ull;
static double uni(void) {   /* xorshift64, uniform in [0, 1) */
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0;
}

int main(void) {
    const int64_t lens[] = {37, 0, 1, 130, 64};
    const int64_t N = 5, Hqk = 2, Hv = 4, K = 128, V = 128;
    int64_t cu[6] = {0};
    for (int i = 0; i < N; ++i) cu[i + 1] = cu[i] + lens[i];
    const int64_t T = cu[N];
    const size_t nq = (size_t)(T * Hqk * K), nv = (size_t)(T * Hv * V), ng = (size_t)(T * Hv), ns = (size_t)(N * Hv * V * K);
    double *q = malloc(nq * 8), *k = malloc(nq * 8), *v = malloc(nv * 8), *g = malloc(ng * 8), *b = malloc(ng * 8);
    double *s0 = malloc(ns * 8), *out = malloc(nv * 8), *sN = malloc(ns * 8), *zero = calloc(ng, 8);
    float *qf = malloc(nq * 4), *kf = malloc(nq * 4), *vf = malloc(nv * 4), *gf = malloc(ng * 4), *bf = malloc(ng * 4);
    float *s0f = malloc(ns * 4), *outf = malloc(nv * 4), *sNf = malloc(ns * 4);
    if (!q || !k || !v || !g || !b || !s0 || !out || !sN || !zero || !qf || !kf || !vf || !gf || !bf || !s0f || !outf || !sNf)
        return 2;
    for (size_t i = 0; i < nq; ++i) { q[i] = uni() - 0.5; k[i] = uni() - 0.5; qf[i] = (float)q[i]; kf[i] = (float)k[i]; }
    for (size_t i = 0; i < nv; ++i) { v[i] = uni() - 0.5; vf[i] = (float)v[i]; }
    for (size_t i = 0; i < ng; ++i) { g[i] = 0.9 + 0.1 * uni(); b[i] = uni(); gf[i] = (float)g[i]; bf[i] = (float)b[i]; }
    for (size_t i = 0; i < ns; ++i) { s0[i] = 0.01 * (uni() - 0.5); s0f[i] = (float)s0[i]; }
    int bad = 0;
    for (int l2 = 0; l2 < 2; ++l2) {
        bad |= gdn_oracle_run_f64(q, k, v, g, b, 0.0, cu, N, Hqk, Hv, K, V, s0, l2, out, sN, 4) != 0;
        bad |= gdn_oracle_run_f32(qf, kf, vf, gf, bf, 0.0, cu, N, Hqk, Hv, K, V, s0f, l2, outf, sNf, 3) != 0;
        bad |= gdn_oracle_run_f64(q, k, v, NULL, NULL, 0.5, cu, N, Hqk, Hv, K, V, NULL, l2, out, NULL, 8) != 0;
        bad |= gdn_oracle_run_f32(qf, kf, vf, NULL, bf, -1.0, cu, N, Hqk, Hv, K, V, NULL, l2, outf, sNf, 1) != 0;
    }
    /* beta = 0: S_T = (prod of a over the sequence) S_0 */
    bad |= gdn_oracle_run_f64(q, k, v, g, zero, 0.0, cu, N, Hqk, Hv, K, V, s0, 1, out, sN, 4) != 0;
    double worst = 0.0;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t h = 0; h < Hv; ++h) {
            double prod = 1.0;
            for (int64_t t = cu[n]; t < cu[n + 1]; ++t) prod *= g[t * Hv + h];
            for (int64_t e = 0; e < V * K; ++e) {
                const size_t i = (size_t)((n * Hv + h) * V * K + e);
                worst = fmax(worst, fabs(sN[i] - prod * s0[i]));
            }
        }
    bad |= !(worst < 1e-15);
    /* invalid arguments are refused */
    bad |= gdn_oracle_run_f64(q, k, v, g, b, 0.0, cu, N, 3, Hv, K, V, s0, 0, out, sN, 2) != -1;
    printf("oracle driver: %s (beta = 0 closed form, worst |S_T - prod(a) S_0| = %.3g)\n", bad ? "FAILED" : "ok", worst);
    free(q); free(k); free(v); free(g); free(b); free(s0); free(out); free(sN); free(zero);
    free(qf); free(kf); free(vf); free(gf); free(bf); free(s0f); free(outf); free(sNf);
    return bad;
}
