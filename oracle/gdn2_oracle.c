/*
 * Oracle for the Gated DeltaNet-2 token mixer: a plain, sequential,
 * token-by-token fp64 CPU implementation of the Gated Delta Rule-2.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or
 * load this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do. It shares no code with the HIP kernels.
 *
 * What it computes (snilld.dk, "Gated DeltaNet-2 fra NVIDIA ...", section
 * "Hvad Gated DeltaNet-2 ændrer", the compact update equation), per sequence
 * and head, with the state S in R^{dk x dv} (rows = key channels):
 *
 *     S_t = (I - k_t (b_t * k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t * v_t)^T
 *     o_t = S_t^T q_t
 *
 * The decay Diag(alpha_t) acts before the rank-one edit (same section: the
 * channel-wise decay is applied ahead of the active edit). The readout uses
 * the updated state, as in the layer diagram's step 4 ("Memory Readout") and
 * the per-token loop of the PyTorch layer on aifetchly-blog.pages.dev, "Gated
 * DeltaNet-2 Guide", section "End-to-End PyTorch Implementation". The decay
 * arrives as log(alpha), so alpha = exp(log_alpha); -inf means alpha = 0.
 *
 * The product (I - k (b*k)^T) D S is applied in rank-one form:
 *     S~ = D S;  e = S~^T (b*k);  S = S~ + k (w*v - e)^T
 * which equals the matrix product exactly in real arithmetic
 * ((I - k (b*k)^T) S~ = S~ - k ((b*k)^T S~) = S~ - k e^T).
 *
 * Layouts (row-major, contiguous): token tensors [tokens, H, d] where the
 * token index runs over all sequences back to back; S0 / ST / decode state
 * [N, H, dk, dv]. Sequence i covers tokens [cu[i], cu[i+1]); cu == NULL
 * means N = B equal sequences of T tokens.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v, *la, *b, *w, *S0;
    double *o, *ST;
    const int64_t *cu;
    int64_t T;
    int N, H, dk, dv, nthreads, tid;
} job_t;

/* One (sequence, head) chain: the recurrence above, token by token. */
static void run_chain(const job_t *J, int seq, int h, double *S, double *e)
{
    const int H = J->H, dk = J->dk, dv = J->dv;
    const int64_t t0 = J->cu ? J->cu[seq] : (int64_t)seq * J->T;
    const int64_t t1 = J->cu ? J->cu[seq + 1] : (int64_t)(seq + 1) * J->T;
    const size_t sofs = ((size_t)seq * H + h) * (size_t)dk * dv;

    if (J->S0)
        memcpy(S, J->S0 + sofs, sizeof(double) * (size_t)dk * dv);
    else
        memset(S, 0, sizeof(double) * (size_t)dk * dv);

    for (int64_t t = t0; t < t1; ++t) {
        const size_t ik = ((size_t)t * H + h) * (size_t)dk;
        const size_t iv = ((size_t)t * H + h) * (size_t)dv;
        const double *q = J->q + ik, *k = J->k + ik, *la = J->la + ik, *b = J->b + ik;
        const double *v = J->v + iv, *w = J->w + iv;

        /* S~ = Diag(alpha_t) S_{t-1}: scale row c by alpha_c. */
        for (int c = 0; c < dk; ++c) {
            const double a = exp(la[c]);
            for (int j = 0; j < dv; ++j)
                S[(size_t)c * dv + j] = a * S[(size_t)c * dv + j];
        }
        /* e = S~^T (b * k) */
        for (int j = 0; j < dv; ++j)
            e[j] = 0.0;
        for (int c = 0; c < dk; ++c) {
            const double bk = b[c] * k[c];
            for (int j = 0; j < dv; ++j)
                e[j] += S[(size_t)c * dv + j] * bk;
        }
        /* S_t = S~ + k (w * v - e)^T */
        for (int j = 0; j < dv; ++j)
            e[j] = w[j] * v[j] - e[j];
        for (int c = 0; c < dk; ++c)
            for (int j = 0; j < dv; ++j)
                S[(size_t)c * dv + j] += k[c] * e[j];
        /* o_t = S_t^T q_t */
        if (J->o) {
            double *o = J->o + iv;
            for (int j = 0; j < dv; ++j)
                o[j] = 0.0;
            for (int c = 0; c < dk; ++c)
                for (int j = 0; j < dv; ++j)
                    o[j] += S[(size_t)c * dv + j] * q[c];
        }
    }
    if (J->ST)
        memcpy(J->ST + sofs, S, sizeof(double) * (size_t)dk * dv);
}

static void *worker(void *arg)
{
    const job_t *J = (const job_t *)arg;
    double *S = (double *)malloc(sizeof(double) * (size_t)J->dk * J->dv);
    double *e = (double *)malloc(sizeof(double) * (size_t)J->dv);
    if (S && e) {
        const int64_t chains = (int64_t)J->N * J->H;
        for (int64_t c = J->tid; c < chains; c += J->nthreads)
            run_chain(J, (int)(c / J->H), (int)(c % J->H), S, e);
    }
    free(S);
    free(e);
    return NULL;
}

/*
 * Forward over a packed batch. o may be NULL (only ST wanted), ST may be
 * NULL, S0 NULL means zeros. Chains are spread over nthreads threads
 * (nthreads <= 0: one). Returns 0, or -1 on bad arguments.
 */
int gdn2_oracle_forward(const double *q, const double *k, const double *v,
                        const double *log_alpha, const double *b, const double *w,
                        const double *S0, double *o, double *ST,
                        const int64_t *cu_seqlens, int64_t T, int N, int H,
                        int dk, int dv, int nthreads)
{
    if (!q || !k || !v || !log_alpha || !b || !w || N < 0 || H <= 0 || dk <= 0 || dv <= 0)
        return -1;
    if (nthreads <= 0)
        nthreads = 1;
    if ((int64_t)nthreads > (int64_t)N * H)
        nthreads = (int)((int64_t)N * H > 0 ? (int64_t)N * H : 1);
    job_t *jobs = (job_t *)calloc((size_t)nthreads, sizeof(job_t));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -1;
    }
    for (int i = 0; i < nthreads; ++i) {
        job_t J = {q, k, v, log_alpha, b, w, S0, o, ST, cu_seqlens, T, N, H, dk, dv, nthreads, i};
        jobs[i] = J;
    }
    for (int i = 1; i < nthreads; ++i)
        pthread_create(&th[i], NULL, worker, &jobs[i]);
    worker(&jobs[0]);
    for (int i = 1; i < nthreads; ++i)
        pthread_join(th[i], NULL);
    free(jobs);
    free(th);
    return 0;
}

/*
 * One decode step for N independent sequences: each (sequence, head) state
 * S [dk, dv] advances by one token in place and o [N, H, dv] receives the
 * readout. This is the forward above with one token per sequence and the
 * state carried through S.
 */
int gdn2_oracle_decode_step(const double *q, const double *k, const double *v,
                            const double *log_alpha, const double *b, const double *w,
                            double *S, double *o, int N, int H, int dk, int dv, int nthreads)
{
    if (!S)
        return -1;
    return gdn2_oracle_forward(q, k, v, log_alpha, b, w, S, o, S, NULL, 1, N, H, dk, dv,
                               nthreads);
}
