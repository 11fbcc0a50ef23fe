/*
 * Runs the fp64 oracle (forward, decode step, gradients) on small seeded
 * inputs under AddressSanitizer and UndefinedBehaviorSanitizer: packed
 * sequences with an empty one and ragged lengths, with and without S0, on
 * several threads. Checks that every output is finite and that T decode
 * steps reproduce the forward pass; exits non-zero otherwise.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int gdn2_oracle_forward(const double *q, const double *k, const double *v, const double *la, const double *b,
                        const double *w, const double *S0, double *o, double *ST, const int64_t *cu, int64_t T,
                        int N, int H, int dk, int dv, int nthreads);
int gdn2_oracle_decode_step(const double *q, const double *k, const double *v, const double *la,
                            const double *b, const double *w, double *S, double *o, int N, int H, int dk, int dv,
                            int nthreads);
int gdn2_oracle_backward(const double *q, const double *k, const double *v, const double *la, const double *b,
                         const double *w, const double *S0, const double *dO, const double *dST, double *dq,
                         double *dk, double *dv, double *dla, double *db, double *dw, double *dS0,
                         const int64_t *cu, int64_t T, int N, int H, int dk_, int dv_, int nthreads);

static uint64_t rs = 0x9E3779B97F4A7C15ull;
static double urand(void)   /* xorshift64*, uniform in [0, 1) */
{
    rs ^= rs >> 12; rs ^= rs << 25; rs ^= rs >> 27;
    return (double)((rs * 0x2545F4914F6CDD1Dull) >> 11) / 9007199254740992.0;
}
static double *arr(size_t n, double lo, double hi)
{
    double *x = malloc(n * sizeof *x);
    for (size_t i = 0; i < n; ++i) x[i] = lo + (hi - lo) * urand();
    return x;
}
static int finite_all(const double *x, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

int main(void)
{
    enum { N = 4, H = 3, DK = 8, DV = 6 };
    const int64_t cu[N + 1] = {0, 37, 37, 102, 103};   /* one empty, one single-token sequence */
    const int64_t T = cu[N];
    const size_t nk = (size_t)T * H * DK, nv = (size_t)T * H * DV, ns = (size_t)N * H * DK * DV;
    double *q = arr(nk, -0.4, 0.4), *k = arr(nk, -0.4, 0.4), *la = arr(nk, -0.3, 0.0), *b = arr(nk, 0, 1);
    double *v = arr(nv, -1, 1), *w = arr(nv, 0, 1), *S0 = arr(ns, -0.1, 0.1), *dO = arr(nv, -1, 1);
    double *dST = arr(ns, -1, 1);
    double *o = calloc(nv, sizeof *o), *ST = calloc(ns, sizeof *ST), *o2 = calloc(nv, sizeof *o2);
    double *ST2 = calloc(ns, sizeof *ST2);
    int bad = 0;

    for (int nt = 1; nt <= 5; nt += 4) {
        if (gdn2_oracle_forward(q, k, v, la, b, w, S0, o, ST, cu, 0, N, H, DK, DV, nt)) bad |= 1;
        if (gdn2_oracle_forward(q, k, v, la, b, w, NULL, o2, ST2, cu, 0, N, H, DK, DV, nt)) bad |= 1;
    }
    if (!finite_all(o, nv) || !finite_all(ST, ns) || !finite_all(o2, nv) || !finite_all(ST2, ns)) bad |= 2;
    /* uniform batch form: two sequences of 51 tokens */
    if (gdn2_oracle_forward(q, k, v, la, b, w, NULL, o2, ST2, NULL, 51, 2, H, DK, DV, 2)) bad |= 1;

    /* decode: sequence 2 (65 tokens) token by token equals its forward pass */
    {
        const int64_t t0 = cu[2], L = cu[3] - cu[2];
        double *S = malloc((size_t)H * DK * DV * sizeof *S), *od = malloc((size_t)H * DV * sizeof *od);
        memcpy(S, S0 + (size_t)2 * H * DK * DV, (size_t)H * DK * DV * sizeof *S);
        double err = 0.0;
        for (int64_t t = 0; t < L; ++t) {
            const size_t ok = (size_t)(t0 + t) * H * DK, ov = (size_t)(t0 + t) * H * DV;
            if (gdn2_oracle_decode_step(q + ok, k + ok, v + ov, la + ok, b + ok, w + ov, S, od, 1, H, DK, DV, 1))
                bad |= 4;
            for (int x = 0; x < H * DV; ++x) err = fmax(err, fabs(od[x] - o[ov + x]));
        }
        for (int x = 0; x < H * DK * DV; ++x) err = fmax(err, fabs(S[x] - ST[(size_t)2 * H * DK * DV + x]));
        if (!(err < 1e-12)) { fprintf(stderr, "decode vs forward: %g\n", err); bad |= 8; }
        free(S);
        free(od);
    }

    /* gradients */
    double *g[7];
    const size_t gn[7] = {nk, nk, nv, nk, nk, nv, ns};
    for (int i = 0; i < 7; ++i) g[i] = calloc(gn[i], sizeof(double));
    for (int nt = 1; nt <= 3; nt += 2) {
        if (gdn2_oracle_backward(q, k, v, la, b, w, S0, dO, dST, g[0], g[1], g[2], g[3], g[4], g[5], g[6], cu, 0, N,
                                 H, DK, DV, nt))
            bad |= 16;
        if (gdn2_oracle_backward(q, k, v, la, b, w, NULL, dO, NULL, g[0], g[1], g[2], g[3], g[4], g[5], g[6], cu, 0,
                                 N, H, DK, DV, nt))
            bad |= 16;
    }
    for (int i = 0; i < 7; ++i) {
        if (!finite_all(g[i], gn[i])) bad |= 32;
        free(g[i]);
    }
    free(q); free(k); free(la); free(b); free(v); free(w); free(S0); free(dO); free(dST);
    free(o); free(ST); free(o2); free(ST2);
    if (bad) fprintf(stderr, "oracle driver failed: flags %d\n", bad);
    else printf("oracle driver: ok\n");
    return bad;
}
