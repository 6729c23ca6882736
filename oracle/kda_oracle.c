/*
 * kda_oracle.c — plain, sequential CPU oracle for KDA / CKDA.
 *
 * TEST INFRASTRUCTURE ONLY (see kda_oracle.h): never linked into, called by or
 * used as a fallback for the HIP library.  Built with gcc -O2, no fast-math,
 * no intrinsics.  Parallel only over independent (b, h) recurrences.
 *
 * Every function follows a definition on the pages, in the pages' order:
 *   one token = decay first, then the delta correction, then the read-out
 *   ("Semidirect Fourier Delta Attention", §1 eq. (1) and §3 eq. (14);
 *    the per-channel decay S' = diag(a) S of "Kimi Delta Attention: a bounded
 *    case study", Chapter 12 §12.1; the read-compare-correct step of the same
 *    page, Exercise 2's reasoned solution).
 */
#include "kda_oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/*
 * One token of eq. (1) followed by eq. (14), on a double state S [Dk][Dv]:
 *   S <- diag(alpha) S                          (channel-wise decay)
 *   S <- (I - beta k k^T) S + beta k v^T         (delta correction of the
 *                                                 decayed state)
 *   o  = S^T q                                   (post-update read-out)
 * The correction is evaluated as S + beta k (v - S^T k)^T, which is the same
 * matrix expression expanded by distributivity.  pred is Dv doubles of
 * scratch.  o may be NULL.
 */
static void token_update(double* S, const float* q, const float* k,
                         const float* v, const float* alpha, double beta,
                         double* o, int Dk, int Dv, double* pred)
{
    for (int c = 0; c < Dk; ++c) {
        const double a = (double)alpha[c];
        double* row = S + (size_t)c * Dv;
        for (int j = 0; j < Dv; ++j) row[j] *= a;
    }
    for (int j = 0; j < Dv; ++j) pred[j] = 0.0;
    for (int c = 0; c < Dk; ++c) {
        const double kc = (double)k[c];
        const double* row = S + (size_t)c * Dv;
        for (int j = 0; j < Dv; ++j) pred[j] += kc * row[j];
    }
    for (int c = 0; c < Dk; ++c) {
        const double bk = beta * (double)k[c];
        double* row = S + (size_t)c * Dv;
        for (int j = 0; j < Dv; ++j) row[j] += bk * ((double)v[j] - pred[j]);
    }
    if (o) {
        for (int j = 0; j < Dv; ++j) o[j] = 0.0;
        for (int c = 0; c < Dk; ++c) {
            const double qc = (double)q[c];
            const double* row = S + (size_t)c * Dv;
            for (int j = 0; j < Dv; ++j) o[j] += qc * row[j];
        }
    }
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int kda_oracle_forward(const float* q, const float* k, const float* v,
                       const float* alpha, const float* beta, const float* S0,
                       double* out, double* ST, double* CS, int chunk,
                       int B, int T, int H, int Dk, int Dv, int nthreads)
{
    if (!q || !k || !v || !alpha || !beta || !out) return -1;
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return -1;
    if (CS && chunk <= 0) return -1;
    const long nchunks = CS ? (T + chunk - 1) / chunk : 0;
    set_threads(nthreads);
    const long nbh = (long)B * H;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < nbh; ++bh) {
        const int b = (int)(bh / H), h = (int)(bh % H);
        double* S = (double*)malloc(sizeof(double) * ((size_t)Dk * Dv + Dv));
        if (!S) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        double* pred = S + (size_t)Dk * Dv;
        if (S0) {
            const float* s0 = S0 + (size_t)bh * Dk * Dv;
            for (size_t e = 0; e < (size_t)Dk * Dv; ++e) S[e] = (double)s0[e];
        } else {
            memset(S, 0, sizeof(double) * (size_t)Dk * Dv);
        }
        for (int t = 0; t < T; ++t) {
            const size_t tok = ((size_t)b * T + t) * H + h;
            if (CS && t % chunk == 0)
                memcpy(CS + ((size_t)bh * nchunks + t / chunk) * Dk * Dv, S,
                       sizeof(double) * (size_t)Dk * Dv);
            token_update(S, q + tok * Dk, k + tok * Dk, v + tok * Dv,
                         alpha + tok * Dk, (double)beta[tok], out + tok * Dv,
                         Dk, Dv, pred);
        }
        if (ST) memcpy(ST + (size_t)bh * Dk * Dv, S, sizeof(double) * (size_t)Dk * Dv);
        free(S);
    }
    return failed ? -1 : 0;
}

int kda_oracle_decode(const float* q, const float* k, const float* v,
                      const float* alpha, const float* beta, double* S,
                      double* out, int nsteps, int B, int H, int Dk, int Dv,
                      int nthreads)
{
    if (!q || !k || !v || !alpha || !beta || !S || !out) return -1;
    if (nsteps < 0 || B < 0 || H < 0 || Dk <= 0 || Dv <= 0) return -1;
    set_threads(nthreads);
    const long nbh = (long)B * H;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < nbh; ++bh) {
        double* pred = (double*)malloc(sizeof(double) * (size_t)Dv);
        if (!pred) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        double* Sbh = S + (size_t)bh * Dk * Dv;
        for (int s = 0; s < nsteps; ++s) {
            const size_t tok = (size_t)s * nbh + bh;
            token_update(Sbh, q + tok * Dk, k + tok * Dk, v + tok * Dv,
                         alpha + tok * Dk, (double)beta[tok], out + tok * Dv,
                         Dk, Dv, pred);
        }
        free(pred);
    }
    return failed ? -1 : 0;
}

/*
 * Chunk-local gate summary.  The chunkwise execution carries the state from
 * block to block and only needs decay products inside one block
 * ("Kimi Delta Attention: a bounded case study", Exercise 2's reasoned
 * solution; "Semidirect Fourier Delta Attention", §2.2).  Per channel, the
 * product of gates from the chunk start to token r is
 *   prod_{j<=r} alpha_j = [zpos_r == 0] * (-1)^{parity_r} * 2^{L_r},
 * with the sum, count and index below taken straight from their definitions.
 */
int kda_oracle_gate_prep(const float* alpha, double* L, unsigned char* parity,
                         int* zpos, double* gend, int B, int T, int H, int Dk,
                         int C)
{
    if (!alpha || !L || !parity || !zpos || !gend) return -1;
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || C <= 0) return -1;
    const int NC = (T + C - 1) / C;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int n = 0; n < NC; ++n)
                for (int c = 0; c < Dk; ++c) {
                    double lsum = 0.0, prod = 1.0;
                    int neg = 0, last_zero = 0;
                    for (int r = 0; r < C; ++r) {
                        const int t = n * C + r;
                        if (t >= T) break;
                        const double a =
                            (double)alpha[(((size_t)b * T + t) * H + h) * Dk + c];
                        if (a == 0.0) last_zero = r + 1;
                        else lsum += log2(fabs(a));
                        if (a < 0.0) neg += 1;
                        prod *= a;
                        const size_t idx =
                            ((((size_t)b * H + h) * NC + n) * C + r) * Dk + c;
                        L[idx] = lsum;
                        parity[idx] = (unsigned char)(neg & 1);
                        zpos[idx] = last_zero;
                    }
                    gend[(((size_t)b * H + h) * NC + n) * Dk + c] = prod;
                }
    return 0;
}
