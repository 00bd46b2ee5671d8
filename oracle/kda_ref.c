/*
 * Reference (oracle) for the Kimi Delta Attention recurrence: plain, slow,
 * sequential, fp64, on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no source with the HIP library.
 *
 * What it computes (page "Notations mathematiques", table "Attention et KDA"):
 *   the transition of one token is  M_t = (I - beta_t k_t k_t^T) Diag(alpha_t),
 *   the state update is             S_t = M_t S_{t-1} + beta_t k_t v_t^T,
 *   with alpha_t = exp(g_t) per key channel (rows "alpha_t" and "g_t"), and the
 *   raw output read after the write is o_t = S_t^T q_t (row "o~_t").
 * The chunkwise form is, per the "Glossaire" entry "Chunkwise", an exact
 * rewrite of this recurrence, so the reference is the recurrence itself, one
 * token after another, with no chunking at all.
 *
 * The update is evaluated in the order the definition of M_t gives:
 *   1. decay every key row of S by alpha (the Diag(alpha_t) factor);
 *   2. read what the decayed state returns for k_t:  y = S^T k_t;
 *   3. delta correction ("Glossaire", entry "Delta rule"): u = beta (v_t - y);
 *   4. rank-one write S += k_t u^T
 *      (together 2-4 are (I - beta k k^T) S + beta k v^T);
 *   5. o_t = S^T q_t.
 *
 * Layouts (row-major, last index fastest), all fp64:
 *   q, k, g : [total_tokens][H][dk]     v, o : [total_tokens][H][dv]
 *   beta    : [total_tokens][H]         states : [num_seqs][H][dk][dv]
 *   cu_seqlens : [num_seqs + 1], cu[0] = 0, non-decreasing, cu[N] = total.
 * A NULL initial state means zeros.  final_state may be NULL (not written).
 *
 * Parity status: every step above is pinned by the CPU tests against values
 * the pages print (two-channel trace of the course page, sections 2, 3 and
 * 12.1), closed forms (exact recall, linear-attention reduction) and a
 * brute-force product of explicit M_t matrices.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v, *g, *beta, *s0;
    const int64_t *cu;
    int num_seqs, H, dk, dv;
    double *o, *sf;
    /* work distribution */
    pthread_mutex_t lock;
    int64_t next;
    int failed;
} job_t;

/* One (sequence, head): advance the state over tokens [t0, t1). */
static int run_one(const job_t *J, int n, int h)
{
    const int H = J->H, dk = J->dk, dv = J->dv;
    const int64_t t0 = J->cu[n], t1 = J->cu[n + 1];
    double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
    double *u = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!S || !u) { free(S); free(u); return 1; }

    const size_t soff = ((size_t)n * H + h) * (size_t)dk * dv;
    if (J->s0) memcpy(S, J->s0 + soff, sizeof(double) * (size_t)dk * dv);
    else memset(S, 0, sizeof(double) * (size_t)dk * dv);

    for (int64_t t = t0; t < t1; ++t) {
        const double *qt = J->q + ((size_t)t * H + h) * dk;
        const double *kt = J->k + ((size_t)t * H + h) * dk;
        const double *vt = J->v + ((size_t)t * H + h) * dv;
        const double *gt = J->g + ((size_t)t * H + h) * dk;
        const double bt = J->beta[(size_t)t * H + h];

        /* 1. S <- Diag(alpha_t) S, alpha_t = exp(g_t) */
        for (int c = 0; c < dk; ++c) {
            const double a = exp(gt[c]);
            for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] *= a;
        }
        /* 2-3. u = beta (v - S^T k) */
        for (int j = 0; j < dv; ++j) {
            double y = 0.0;
            for (int c = 0; c < dk; ++c) y += S[(size_t)c * dv + j] * kt[c];
            u[j] = bt * (vt[j] - y);
        }
        /* 4. S <- S + k u^T */
        for (int c = 0; c < dk; ++c)
            for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] += kt[c] * u[j];
        /* 5. o_t = S^T q */
        double *ot = J->o + ((size_t)t * H + h) * dv;
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int c = 0; c < dk; ++c) acc += S[(size_t)c * dv + j] * qt[c];
            ot[j] = acc;
        }
    }
    if (J->sf) memcpy(J->sf + soff, S, sizeof(double) * (size_t)dk * dv);
    free(S);
    free(u);
    return 0;
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    const int64_t total = (int64_t)J->num_seqs * J->H;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int64_t w = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (w >= total) break;
        if (run_one(J, (int)(w / J->H), (int)(w % J->H))) {
            pthread_mutex_lock(&J->lock);
            J->failed = 1;
            pthread_mutex_unlock(&J->lock);
        }
    }
    return NULL;
}

/* Returns 0 on success, 1 on bad arguments, 2 on allocation failure. */
int kda_oracle_forward_f64(const double *q, const double *k, const double *v,
                           const double *g, const double *beta,
                           const double *initial_state, const int64_t *cu_seqlens,
                           int num_seqs, int H, int dk, int dv,
                           double *o, double *final_state, int nthreads)
{
    if (!q || !k || !v || !g || !beta || !cu_seqlens || !o) return 1;
    if (num_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0) return 1;
    if (cu_seqlens[0] != 0) return 1;
    for (int n = 0; n < num_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return 1;

    job_t J;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.s0 = initial_state;
    J.cu = cu_seqlens; J.num_seqs = num_seqs; J.H = H; J.dk = dk; J.dv = dv;
    J.o = o; J.sf = final_state; J.next = 0; J.failed = 0;
    pthread_mutex_init(&J.lock, NULL);

    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int started = 0;
    for (int i = 1; i < nthreads; ++i)
        if (pthread_create(&th[started], NULL, worker, &J) == 0) ++started;
    worker(&J);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&J.lock);
    return J.failed ? 2 : 0;
}

/*
 * One decode step ("Glossaire", entry "Decode"): every request advances its
 * own state by exactly one token.  This is the forward above with sequences
 * of length one whose initial and final states are the same buffer.
 *   q, k, g : [N][H][dk]  v, o : [N][H][dv]  beta : [N][H]
 *   state   : [N][H][dk][dv], read and overwritten.
 */
int kda_oracle_decode_f64(const double *q, const double *k, const double *v,
                          const double *g, const double *beta, double *state,
                          int N, int H, int dk, int dv, double *o, int nthreads)
{
    if (N < 0) return 1;
    int64_t *cu = (int64_t *)malloc(sizeof(int64_t) * ((size_t)N + 1));
    if (!cu) return 2;
    for (int n = 0; n <= N; ++n) cu[n] = n;
    /* each (request, head) reads its own slice before writing it */
    const int rc = kda_oracle_forward_f64(q, k, v, g, beta, state, cu, N, H, dk, dv,
                                          o, state, nthreads);
    free(cu);
    return rc;
}
