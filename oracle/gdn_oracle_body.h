/*
 * Body of the reference recurrence, instantiated twice by gdn_oracle.c
 * (REAL = double, REAL = float).  TEST INFRASTRUCTURE ONLY: nothing on the
 * product path may include, link or call this.
 *
 * Expected macros: REAL (arithmetic type), SFX(name) (name suffixer),
 * RSQRT_EPS(x) (1/sqrt(x + eps) in REAL).
 *
 * What is computed (the gated delta rule that the pages name as "Chunked
 * Gated Delta Rule" without printing it):
 *
 *     S_t = a_t * S_{t-1} * (I - b_t k_t k_t^T) + b_t v_t k_t^T
 *     o_t = scale * S_t q_t
 *
 * with the conventions fixed by the pages:
 *   - a_t is the forget gate in linear space, all ones when absent
 *     ("flashinfer.cudnn.cudnn_chunk_gated_delta_rule", Parameters: g);
 *   - b_t is the post-sigmoid update gate, all ones when absent
 *     (same page, Parameters: beta);
 *   - scale = 1/sqrt(head_dim) when given as 0 (same page, Parameters: scale);
 *   - S is V-major, S[v][k] ("flashinfer.cudnn", section Linear attention;
 *     cudnn_chunk_gated_delta_rule, Parameters: initial_state);
 *   - optional q/k L2 normalisation before use (Parameters:
 *     use_qk_l2norm_in_kernel), read as x / sqrt(sum x^2 + 1e-6);
 *   - packed varlen batches delimited by cu_seqlens (Parameters: cu_seqlens);
 *   - v-head h reads q/k head h / (Hv/Hqk) (consecutive grouping; the pages
 *     leave the head relation to the engine).
 *
 * The expansion used per token is an exact rearrangement of the formula:
 *   S <- a S;  p = S k;  u = b (v - p);  S <- S + u k^T;  o = scale S q.
 * Each row v of S is updated on its own; per row the order of operations is
 * fixed, so results do not depend on the thread count.
 */

typedef struct {
    const REAL *q, *k, *v, *g, *beta, *s0;
    const int64_t *cu;
    REAL *out, *sN;
    int64_t N, Hqk, Hv, K, V;
    REAL scale;
    int l2;
    int64_t next;          /* shared work counter (atomic) */
} SFX(job);

static void SFX(run_item)(SFX(job) *J, int64_t item, REAL *qn, REAL *kn, REAL *S)
{
    const int64_t n = item / J->Hv, h = item % J->Hv;
    const int64_t K = J->K, V = J->V;
#if ORACLE_MUTANT == 6
    const int64_t hq = h % J->Hqk;                      /* planted: wrong head map */
#else
    const int64_t hq = h / (J->Hv / J->Hqk);
#endif
    const int64_t bos = J->cu[n], eos = J->cu[n + 1];

    /* step 1: initial state (zero when absent) */
    for (int64_t e = 0; e < V * K; ++e)
        S[e] = J->s0 ? J->s0[(n * J->Hv + h) * V * K + e] : (REAL)0;

    for (int64_t t = bos; t < eos; ++t) {
        const REAL *qt = J->q + (t * J->Hqk + hq) * K;
        const REAL *kt = J->k + (t * J->Hqk + hq) * K;
        const REAL *vt = J->v + (t * J->Hv + h) * V;
        /* (a) q and k, optionally L2-normalised */
        REAL sq = 0, sk = 0;
        for (int64_t i = 0; i < K; ++i) { sq += qt[i] * qt[i]; sk += kt[i] * kt[i]; }
#if ORACLE_MUTANT == 8
        const REAL fq = (REAL)1;                        /* planted: q not normalised */
#else
        const REAL fq = J->l2 ? RSQRT_EPS(sq) : (REAL)1;
#endif
        const REAL fk = J->l2 ? RSQRT_EPS(sk) : (REAL)1;
        for (int64_t i = 0; i < K; ++i) { qn[i] = qt[i] * fq; kn[i] = kt[i] * fk; }
        /* (b) gates */
#if ORACLE_MUTANT == 1
        const REAL a = (REAL)1;                         /* planted: gate dropped */
#else
        const REAL a = J->g ? J->g[t * J->Hv + h] : (REAL)1;
#endif
        const REAL b = J->beta ? J->beta[t * J->Hv + h] : (REAL)1;
        REAL *ot = J->out + (t * J->Hv + h) * V;
        for (int64_t r = 0; r < V; ++r) {
            REAL *row = S + r * K;
#if ORACLE_MUTANT == 9
            REAL p = 0;                                 /* planted: predict before decay */
            for (int64_t i = 0; i < K; ++i) p += row[i] * kn[i];
            for (int64_t i = 0; i < K; ++i) row[i] = a * row[i];
#else
            /* (c) decay */
            for (int64_t i = 0; i < K; ++i) row[i] = a * row[i];
            /* (d) prediction p = S k */
            REAL p = 0;
            for (int64_t i = 0; i < K; ++i) p += row[i] * kn[i];
#endif
            /* (e) delta u = b (v - p) */
#if ORACLE_MUTANT == 2
            const REAL u = b * (vt[r] + p);             /* planted: sign */
#elif ORACLE_MUTANT == 5
            const REAL u = (vt[r] - p);                 /* planted: beta dropped */
#else
            const REAL u = b * (vt[r] - p);
#endif
#if ORACLE_MUTANT == 3
            REAL o_pre = 0;                             /* planted: readout before update */
            for (int64_t i = 0; i < K; ++i) o_pre += row[i] * qn[i];
#endif
            /* (f) rank-one update S += u k^T */
            for (int64_t i = 0; i < K; ++i) row[i] = row[i] + u * kn[i];
            /* (g) readout o = scale S q, with the updated state */
            REAL o = 0;
#if ORACLE_MUTANT == 4
            (void)row;                                  /* planted: transposed readout */
            for (int64_t i = 0; i < K; ++i) o += S[i * K + r] * qn[i];
#else
            for (int64_t i = 0; i < K; ++i) o += row[i] * qn[i];
#endif
#if ORACLE_MUTANT == 3
            o = o_pre;
#endif
            ot[r] = J->scale * o;
        }
    }
    /* step 3: final state */
    if (J->sN)
        for (int64_t e = 0; e < V * K; ++e) J->sN[(n * J->Hv + h) * V * K + e] = S[e];
}

static void *SFX(worker)(void *arg)
{
    SFX(job) *J = (SFX(job) *)arg;
    REAL *qn = (REAL *)malloc(sizeof(REAL) * (size_t)J->K);
    REAL *kn = (REAL *)malloc(sizeof(REAL) * (size_t)J->K);
    REAL *S = (REAL *)malloc(sizeof(REAL) * (size_t)(J->K * J->V));
    if (!qn || !kn || !S) { free(qn); free(kn); free(S); return (void *)1; }
    const int64_t items = J->N * J->Hv;
    for (;;) {
        const int64_t it = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
        if (it >= items) break;
        SFX(run_item)(J, it, qn, kn, S);
    }
    free(qn); free(kn); free(S);
    return NULL;
}

/*
 * Runs the recurrence over every (sequence, v-head) item.
 * Layouts (all contiguous, row-major):
 *   q, k  [T, Hqk, K];  v, out [T, Hv, V];  g, beta [T, Hv] (NULL = ones);
 *   initial_state, final_state [N, Hv, V, K] (NULL = zero / not written);
 *   cu_seqlens [N+1], cu[0] = 0, non-decreasing, cu[N] = T.
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int SFX(gdn_oracle_run)(const REAL *q, const REAL *k, const REAL *v,
                        const REAL *g, const REAL *beta, double scale,
                        const int64_t *cu_seqlens, int64_t N,
                        int64_t Hqk, int64_t Hv, int64_t K, int64_t V,
                        const REAL *initial_state, int use_qk_l2norm,
                        REAL *out, REAL *final_state, int nthreads)
{
    if (N < 0 || Hqk <= 0 || Hv <= 0 || K <= 0 || V <= 0 || Hv % Hqk != 0 || !cu_seqlens)
        return -1;
    SFX(job) J;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta;
    J.s0 = initial_state; J.cu = cu_seqlens; J.out = out; J.sN = final_state;
    J.N = N; J.Hqk = Hqk; J.Hv = Hv; J.K = K; J.V = V;
#if ORACLE_MUTANT == 7
    J.scale = (REAL)(scale == 0.0 ? 1.0 / (double)K : scale);   /* planted: default scale */
#else
    J.scale = (REAL)(scale == 0.0 ? 1.0 / sqrt((double)K) : scale);
#endif
    J.l2 = use_qk_l2norm;
    J.next = 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int started = 0, rc = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[started], NULL, SFX(worker), &J) != 0) break;
        ++started;
    }
    if (SFX(worker)(&J) != NULL) rc = -1;
    for (int i = 0; i < started; ++i) {
        void *res = NULL;
        pthread_join(th[i], &res);
        if (res != NULL) rc = -1;
    }
    return rc;
}
