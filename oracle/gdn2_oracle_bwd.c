/*
 * Oracle for the gradients of the Gated DeltaNet-2 token mixer: reverse-mode
 * differentiation of the token recurrence in gdn2_oracle.c, token by token,
 * in fp64 on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY, like gdn2_oracle.c: only the tests and the
 * benchmark's CPU-baseline leg use it; it shares no code with the HIP path.
 *
 * Forward step for token t (snilld.dk, "Gated DeltaNet-2 fra NVIDIA ...",
 * section "Hvad Gated DeltaNet-2 ændrer", update equation; readout after the
 * update as in aifetchly-blog.pages.dev, "Gated DeltaNet-2 Guide", layer
 * workflow step 4), with D = Diag(exp(log_alpha_t)), bk = b_t * k_t,
 * u = w_t * v_t:
 *
 *     S~ = D S_{t-1};   e = S~^T bk;   d = u - e;   S_t = S~ + k_t d^T;
 *     o_t = S_t^T q_t
 *
 * Given the gradient G of a scalar loss with respect to S_t (from the later
 * tokens, or dS_T for the last one) and dO_t, the chain rule through those
 * five lines, last line first:
 *
 *     G    += q_t dO_t^T                    (o_t = S_t^T q_t)
 *     dq_t  = S_t dO_t
 *     dd    = G^T k_t;   dk_t = G d         (S_t = S~ + k d^T)
 *     du    = dd;        de   = -dd         (d = u - e)
 *     dw_t  = du * v_t;  dv_t = du * w_t    (u = w * v)
 *     dS~   = G + bk de^T;  dbk = S~ de     (e = S~^T bk)
 *     db_t  = dbk * k_t;  dk_t += dbk * b_t (bk = b * k)
 *     dlog_alpha_t[c] = sum_j dS~[c][j] S~[c][j];   G <- D dS~   (S~ = D S)
 *
 * and dS0 is the final G. The states the backward sweep needs are recomputed
 * from checkpoints kept every 64 tokens during a forward sweep (plain
 * recomputation; nothing is reordered).
 *
 * Layouts as in gdn2_oracle.c; gradients have the layouts of their inputs.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define CKPT 64

typedef struct {
    const double *q, *k, *v, *la, *b, *w, *S0, *dO, *dST;
    double *dq, *dk, *dv, *dla, *db, *dw, *dS0;
    const int64_t *cu;
    int64_t T;
    int N, H, dk_, dv_, nthreads, tid;
} bjob_t;

/* One token of the forward recurrence: S <- S_t from S_{t-1} (in place). */
static void fwd_token(const double *k, const double *la, const double *b, const double *v,
                      const double *w, double *S, double *e, int dk, int dv)
{
    for (int c = 0; c < dk; ++c) {
        const double a = exp(la[c]);
        for (int j = 0; j < dv; ++j)
            S[(size_t)c * dv + j] *= a;
    }
    for (int j = 0; j < dv; ++j)
        e[j] = 0.0;
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j)
            e[j] += S[(size_t)c * dv + j] * b[c] * k[c];
    for (int j = 0; j < dv; ++j)
        e[j] = w[j] * v[j] - e[j];
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j)
            S[(size_t)c * dv + j] += k[c] * e[j];
}

typedef struct {
    double *ckpt, *seg, *St, *Sd, *G, *dSd, *e, *d, *dd, *dbk;
} scratch_t;

static void run_chain_bwd(const bjob_t *J, int seq, int h, scratch_t *W)
{
    const int H = J->H, dk = J->dk_, dv = J->dv_;
    const size_t SZ = (size_t)dk * dv;
    const int64_t t0 = J->cu ? J->cu[seq] : (int64_t)seq * J->T;
    const int64_t t1 = J->cu ? J->cu[seq + 1] : (int64_t)(seq + 1) * J->T;
    const int64_t L = t1 - t0;
    const size_t sofs = ((size_t)seq * H + h) * SZ;
#define IK(t) (((size_t)(t) * H + h) * (size_t)dk)
#define IV(t) (((size_t)(t) * H + h) * (size_t)dv)

    /* forward sweep: checkpoint m holds the state before token t0 + m*CKPT */
    double *S = W->St;
    if (J->S0) memcpy(S, J->S0 + sofs, sizeof(double) * SZ);
    else memset(S, 0, sizeof(double) * SZ);
    for (int64_t i = 0; i < L; ++i) {
        if (i % CKPT == 0) memcpy(W->ckpt + (size_t)(i / CKPT) * SZ, S, sizeof(double) * SZ);
        const int64_t t = t0 + i;
        fwd_token(J->k + IK(t), J->la + IK(t), J->b + IK(t), J->v + IV(t), J->w + IV(t), S, W->e, dk, dv);
    }

    /* backward sweep */
    double *G = W->G;
    if (J->dST) memcpy(G, J->dST + sofs, sizeof(double) * SZ);
    else memset(G, 0, sizeof(double) * SZ);
    const int64_t nseg = (L + CKPT - 1) / CKPT;
    for (int64_t m = nseg - 1; m >= 0; --m) {
        const int64_t a = m * CKPT, n = (L - a < CKPT) ? L - a : CKPT;
        /* seg[i] = state before token t0 + a + i, i = 0..n */
        memcpy(W->seg, W->ckpt + (size_t)m * SZ, sizeof(double) * SZ);
        for (int64_t i = 0; i < n; ++i) {
            const int64_t t = t0 + a + i;
            memcpy(W->seg + (size_t)(i + 1) * SZ, W->seg + (size_t)i * SZ, sizeof(double) * SZ);
            fwd_token(J->k + IK(t), J->la + IK(t), J->b + IK(t), J->v + IV(t), J->w + IV(t),
                      W->seg + (size_t)(i + 1) * SZ, W->e, dk, dv);
        }
        for (int64_t i = n - 1; i >= 0; --i) {
            const int64_t t = t0 + a + i;
            const double *q = J->q + IK(t), *k = J->k + IK(t), *la = J->la + IK(t), *b = J->b + IK(t);
            const double *v = J->v + IV(t), *w = J->w + IV(t), *dO = J->dO + IV(t);
            const double *Sprev = W->seg + (size_t)i * SZ, *Snew = W->seg + (size_t)(i + 1) * SZ;
            double *Sd = W->Sd, *dSd = W->dSd, *e = W->e, *d = W->d, *dd = W->dd, *dbk = W->dbk;
            /* recompute S~, e, d of this token */
            for (int c = 0; c < dk; ++c) {
                const double al = exp(la[c]);
                for (int j = 0; j < dv; ++j)
                    Sd[(size_t)c * dv + j] = al * Sprev[(size_t)c * dv + j];
            }
            for (int j = 0; j < dv; ++j)
                e[j] = 0.0;
            for (int c = 0; c < dk; ++c)
                for (int j = 0; j < dv; ++j)
                    e[j] += Sd[(size_t)c * dv + j] * b[c] * k[c];
            for (int j = 0; j < dv; ++j)
                d[j] = w[j] * v[j] - e[j];
            /* G += q dO^T; dq = S_t dO */
            for (int c = 0; c < dk; ++c)
                for (int j = 0; j < dv; ++j)
                    G[(size_t)c * dv + j] += q[c] * dO[j];
            double *dq = J->dq + IK(t), *dkk = J->dk + IK(t), *dla = J->dla + IK(t), *db = J->db + IK(t);
            double *dvv = J->dv + IV(t), *dw = J->dw + IV(t);
            for (int c = 0; c < dk; ++c) {
                double s = 0.0;
                for (int j = 0; j < dv; ++j)
                    s += Snew[(size_t)c * dv + j] * dO[j];
                dq[c] = s;
            }
            /* dd = G^T k; dk = G d */
            for (int j = 0; j < dv; ++j) {
                double s = 0.0;
                for (int c = 0; c < dk; ++c)
                    s += G[(size_t)c * dv + j] * k[c];
                dd[j] = s;
            }
            for (int c = 0; c < dk; ++c) {
                double s = 0.0;
                for (int j = 0; j < dv; ++j)
                    s += G[(size_t)c * dv + j] * d[j];
                dkk[c] = s;
            }
            /* du = dd, de = -dd; dw, dv */
            for (int j = 0; j < dv; ++j) {
                dw[j] = dd[j] * v[j];
                dvv[j] = dd[j] * w[j];
            }
            /* dS~ = G + bk de^T; dbk = S~ de */
            for (int c = 0; c < dk; ++c)
                for (int j = 0; j < dv; ++j)
                    dSd[(size_t)c * dv + j] = G[(size_t)c * dv + j] - b[c] * k[c] * dd[j];
            for (int c = 0; c < dk; ++c) {
                double s = 0.0;
                for (int j = 0; j < dv; ++j)
                    s -= Sd[(size_t)c * dv + j] * dd[j];
                dbk[c] = s;
            }
            for (int c = 0; c < dk; ++c) {
                db[c] = dbk[c] * k[c];
                dkk[c] += dbk[c] * b[c];
            }
            /* dlog_alpha; G <- D dS~ */
            for (int c = 0; c < dk; ++c) {
                const double al = exp(la[c]);
                double s = 0.0;
                for (int j = 0; j < dv; ++j) {
                    s += dSd[(size_t)c * dv + j] * Sd[(size_t)c * dv + j];
                    G[(size_t)c * dv + j] = al * dSd[(size_t)c * dv + j];
                }
                dla[c] = s;
            }
        }
    }
    if (J->dS0) memcpy(J->dS0 + sofs, G, sizeof(double) * SZ);
#undef IK
#undef IV
}

static void *bworker(void *arg)
{
    const bjob_t *J = (const bjob_t *)arg;
    const size_t SZ = (size_t)J->dk_ * J->dv_;
    int64_t maxL = 0;
    for (int i = 0; i < J->N; ++i) {
        const int64_t L = J->cu ? J->cu[i + 1] - J->cu[i] : J->T;
        if (L > maxL) maxL = L;
    }
    scratch_t W;
    W.ckpt = (double *)malloc(sizeof(double) * SZ * (size_t)((maxL + CKPT - 1) / CKPT + 1));
    W.seg = (double *)malloc(sizeof(double) * SZ * (CKPT + 1));
    W.St = (double *)malloc(sizeof(double) * SZ);
    W.Sd = (double *)malloc(sizeof(double) * SZ);
    W.G = (double *)malloc(sizeof(double) * SZ);
    W.dSd = (double *)malloc(sizeof(double) * SZ);
    W.e = (double *)malloc(sizeof(double) * (size_t)J->dv_);
    W.d = (double *)malloc(sizeof(double) * (size_t)J->dv_);
    W.dd = (double *)malloc(sizeof(double) * (size_t)J->dv_);
    W.dbk = (double *)malloc(sizeof(double) * (size_t)J->dk_);
    if (W.ckpt && W.seg && W.St && W.Sd && W.G && W.dSd && W.e && W.d && W.dd && W.dbk) {
        const int64_t chains = (int64_t)J->N * J->H;
        for (int64_t c = J->tid; c < chains; c += J->nthreads)
            run_chain_bwd(J, (int)(c / J->H), (int)(c % J->H), &W);
    }
    free(W.ckpt); free(W.seg); free(W.St); free(W.Sd); free(W.G); free(W.dSd);
    free(W.e); free(W.d); free(W.dd); free(W.dbk);
    return NULL;
}

/*
 * Gradients of a loss L with dL/do = dO [tokens, H, dv] and dL/dS_T = dST
 * [N, H, dk, dv] (NULL: zero). Outputs dq, dk, dlog_alpha, db [tokens, H, dk],
 * dv, dw [tokens, H, dv] and dS0 [N, H, dk, dv] (NULL: not written). S0 NULL
 * means zeros. Returns 0, or -1 on bad arguments.
 */
int gdn2_oracle_backward(const double *q, const double *k, const double *v,
                         const double *log_alpha, const double *b, const double *w,
                         const double *S0, const double *dO, const double *dST,
                         double *dq, double *dk, double *dv, double *dlog_alpha,
                         double *db, double *dw, double *dS0,
                         const int64_t *cu_seqlens, int64_t T, int N, int H,
                         int dk_, int dv_, int nthreads)
{
    if (!q || !k || !v || !log_alpha || !b || !w || !dO || !dq || !dk || !dv || !dlog_alpha || !db || !dw ||
        N < 0 || H <= 0 || dk_ <= 0 || dv_ <= 0)
        return -1;
    if (nthreads <= 0)
        nthreads = 1;
    if ((int64_t)nthreads > (int64_t)N * H)
        nthreads = (int)((int64_t)N * H > 0 ? (int64_t)N * H : 1);
    bjob_t *jobs = (bjob_t *)calloc((size_t)nthreads, sizeof(bjob_t));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -1;
    }
    for (int i = 0; i < nthreads; ++i) {
        bjob_t J = {q, k, v, log_alpha, b, w, S0, dO, dST, dq, dk, dv, dlog_alpha, db, dw, dS0,
                    cu_seqlens, T, N, H, dk_, dv_, nthreads, i};
        jobs[i] = J;
    }
    for (int i = 1; i < nthreads; ++i)
        pthread_create(&th[i], NULL, bworker, &jobs[i]);
    bworker(&jobs[0]);
    for (int i = 1; i < nthreads; ++i)
        pthread_join(th[i], NULL);
    free(jobs);
    free(th);
    return 0;
}
