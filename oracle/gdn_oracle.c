/*
 * gdn_oracle.c -- fp64 token-by-token reference for the Gated DeltaNet layer.
 *
 * TEST INFRASTRUCTURE ONLY. This file is compiled into liboracle.so, which
 * only the tests, the smoke check and the benchmark's CPU-baseline leg load.
 * It shares no code, header or constant with the HIP library.
 *
 * What it computes (the plain definition, token by token, in double):
 *
 *   The layer keeps one fixed-size matrix state S (dv x dk) per sequence and
 *   value head; a learned gate decides how much of S survives each token and
 *   a delta update writes the current token into it ("Optimiser l'inference
 *   sur appareil pour Apple Silicon", section "Qwen cree trois formes de
 *   charges de travail distinctes"; the state and gate are kept in 32-bit or
 *   wider floats because rounding accumulates over the sequential updates,
 *   section "Maintenir l'etat recurrent sur la puce"). The gated delta rule:
 *
 *       a_t = exp(g_t)
 *       S_t = a_t * S_{t-1} * (I - b_t k_t k_t^T) + b_t v_t k_t^T
 *       o_t = scale * S_t q_t
 *
 *   Expanding the product gives the same S_t as
 *       S_t[i][j] = a_t S_{t-1}[i][j] + b_t (v_t[i] - a_t (S_{t-1} k_t)[i]) k_t[j],
 *   which is what the loop below evaluates. The literal matrix form is
 *   evaluated separately (numpy, tiny inputs) and compared with this loop.
 *
 * Layouts (row-major, contiguous):
 *   q, k   [T][hk][dk]      v, out  [T][hv][dv]      g, beta [T][hv]
 *   cu     [num_seqs + 1]   int64 token offsets, sequence n = [cu[n], cu[n+1])
 *   s0, s_final  [num_seqs][hv][dv][dk]  (s0 may be NULL = zero state;
 *                                         s_final may be NULL = not written)
 *   value head h reads query/key head h / (hv / hk) (consecutive value heads
 *   share one query/key head).
 *   heads: optional list of value heads to compute (NULL = all); outputs of
 *   other heads are left untouched.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v, *g, *beta;
    const int64_t *cu;
    int64_t num_seqs, hk, hv, dk, dv;
    double scale;
    const double *s0;
    double *out, *s_final;
    const int64_t *heads;
    int64_t n_heads;
    int64_t next; /* shared work counter */
} oracle_job;

/* Scan one (sequence, value head) pair from its initial state to the end. */
static void scan_pair(const oracle_job *J, int64_t n, int64_t h, double *S, double *sk)
{
    const int64_t dk = J->dk, dv = J->dv;
    const int64_t group = J->hv / J->hk;
    const int64_t kh = h / group;
    const size_t state_off = ((size_t)n * J->hv + h) * dv * dk;

    if (J->s0)
        memcpy(S, J->s0 + state_off, sizeof(double) * dv * dk);
    else
        memset(S, 0, sizeof(double) * dv * dk);

    for (int64_t t = J->cu[n]; t < J->cu[n + 1]; ++t) {
        const double a = exp(J->g[t * J->hv + h]);
        const double b = J->beta[t * J->hv + h];
        const double *kk = J->k + ((size_t)t * J->hk + kh) * dk;
        const double *qq = J->q + ((size_t)t * J->hk + kh) * dk;
        const double *vv = J->v + ((size_t)t * J->hv + h) * dv;
        double *oo = J->out + ((size_t)t * J->hv + h) * dv;

        /* sk = S_{t-1} k_t */
        for (int64_t i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < dk; ++j)
                acc += S[i * dk + j] * kk[j];
            sk[i] = acc;
        }
        /* S_t = a S_{t-1} + b (v - a S_{t-1} k) k^T */
        for (int64_t i = 0; i < dv; ++i) {
            const double u = b * (vv[i] - a * sk[i]);
            for (int64_t j = 0; j < dk; ++j)
                S[i * dk + j] = a * S[i * dk + j] + u * kk[j];
        }
        /* o_t = scale * S_t q_t */
        for (int64_t i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < dk; ++j)
                acc += S[i * dk + j] * qq[j];
            oo[i] = J->scale * acc;
        }
    }
    if (J->s_final)
        memcpy(J->s_final + state_off, S, sizeof(double) * dv * dk);
}

static void *worker(void *arg)
{
    oracle_job *J = (oracle_job *)arg;
    const int64_t nh = J->heads ? J->n_heads : J->hv;
    const int64_t total = J->num_seqs * nh;
    double *S = (double *)malloc(sizeof(double) * (size_t)J->dv * J->dk);
    double *sk = (double *)malloc(sizeof(double) * (size_t)J->dv);
    if (!S || !sk) {
        free(S);
        free(sk);
        return (void *)1;
    }
    for (;;) {
        const int64_t w = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
        if (w >= total)
            break;
        const int64_t n = w / nh;
        const int64_t h = J->heads ? J->heads[w % nh] : (w % nh);
        scan_pair(J, n, h, S, sk);
    }
    free(S);
    free(sk);
    return NULL;
}

/*
 * Returns 0 on success, -1 on invalid arguments, -2 if memory or threads
 * could not be obtained.
 */
int gdn_oracle_scan(const double *q, const double *k, const double *v,
                    const double *g, const double *beta,
                    const int64_t *cu, int64_t num_seqs,
                    int64_t hk, int64_t hv, int64_t dk, int64_t dv, double scale,
                    const double *s0, double *out, double *s_final,
                    const int64_t *heads, int64_t n_heads, int n_threads)
{
    if (!cu || !out || num_seqs < 0 || hk <= 0 || hv <= 0 || dk <= 0 || dv <= 0)
        return -1;
    if (hv % hk != 0)
        return -1;
    if (cu[num_seqs] > 0 && (!q || !k || !v || !g || !beta))
        return -1;
    for (int64_t n = 0; n < num_seqs; ++n)
        if (cu[n + 1] < cu[n])
            return -1;
    if (heads) {
        for (int64_t i = 0; i < n_heads; ++i)
            if (heads[i] < 0 || heads[i] >= hv)
                return -1;
    }
    oracle_job J = {q, k, v, g, beta, cu, num_seqs, hk, hv, dk, dv, scale,
                    s0, out, s_final, heads, n_heads, 0};
    if (n_threads < 1)
        n_threads = 1;
    const int64_t work = num_seqs * (heads ? n_heads : hv);
    if (n_threads > work)
        n_threads = work > 0 ? (int)work : 1;

    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    if (!tid)
        return -2;
    /* Workers drain a shared counter, so any number of started threads
     * (including none: the calling thread then does all the work) covers
     * every pair. */
    int started = 0, failed = 0;
    for (int i = 0; i < n_threads; ++i) {
        if (pthread_create(&tid[i], NULL, worker, &J) != 0)
            break;
        ++started;
    }
    if (started == 0 && worker(&J) != NULL)
        failed = 1;
    for (int i = 0; i < started; ++i) {
        void *rc = NULL;
        pthread_join(tid[i], &rc);
        if (rc != NULL)
            failed = 1;
    }
    free(tid);
    return failed ? -2 : 0;
}
