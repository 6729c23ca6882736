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
 *   S <- diag(alpha) S                          (channel-wise decay; with
 *                                                theta, the phase decay of
 *                                                eq. (13): see below)
 *   S <- (I - beta k k^T) S + beta k v^T         (delta correction of the
 *                                                 decayed state)
 *   o  = S^T q                                   (post-update read-out)
 * The correction is evaluated as S + beta k (v - S^T k)^T, which is the same
 * matrix expression expanded by distributivity.  pred is Dv doubles of
 * scratch.  o may be NULL.
 */
static void token_update(double* S, const double* q, const double* k,
                         const double* v, const double* alpha, const double* theta,
                         double beta, double* o, int Dk, int Dv, double* pred)
{
    if (!theta) {
        for (int c = 0; c < Dk; ++c) {
            const double a = alpha[c];
            double* row = S + (size_t)c * Dv;
            for (int j = 0; j < Dv; ++j) row[j] *= a;
        }
    } else {
        /* phase variant: channels 2p, 2p+1 form one complex coordinate and the
         * decay is alpha_p e^{i theta_p}, the 2x2 block alpha_p R(theta_p)
         * with R = [[cos, -sin], [sin, cos]] acting on that pair of rows */
        for (int p = 0; p < Dk / 2; ++p) {
            const double c = alpha[p] * cos(theta[p]), sn = alpha[p] * sin(theta[p]);
            double* r0 = S + (size_t)(2 * p) * Dv;
            double* r1 = r0 + Dv;
            for (int j = 0; j < Dv; ++j) {
                const double x = r0[j], y = r1[j];
                r0[j] = c * x - sn * y;
                r1[j] = sn * x + c * y;
            }
        }
    }
    for (int j = 0; j < Dv; ++j) pred[j] = 0.0;
    for (int c = 0; c < Dk; ++c) {
        const double kc = k[c];
        const double* row = S + (size_t)c * Dv;
        for (int j = 0; j < Dv; ++j) pred[j] += kc * row[j];
    }
    for (int c = 0; c < Dk; ++c) {
        const double bk = beta * k[c];
        double* row = S + (size_t)c * Dv;
        for (int j = 0; j < Dv; ++j) row[j] += bk * (v[j] - pred[j]);
    }
    if (o) {
        for (int j = 0; j < Dv; ++j) o[j] = 0.0;
        for (int c = 0; c < Dk; ++c) {
            const double qc = q[c];
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

/* Logistic function, 1 / (1 + e^{-x}), written so that exp never overflows. */
static double sigmoid(double x)
{
    if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
    const double e = exp(x);
    return e / (1.0 + e);
}

/* Per-token input parameterisation, or NULL for inputs taken as given. */
struct prologue {
    double amin, amax, bmax, eps;
    int normalize_q;
};

/*
 * One token's inputs in double.  With a prologue ("Semidirect Fourier Delta
 * Attention", §3, the stable parameterisation):
 *   alpha = amin + (amax - amin) * sigmoid(a)          eq. (15)
 *   beta  = bmax * sigmoid(c)                           eq. (17) (bmax = 1; 2 for
 *                                                       the CKDA beta range)
 *   k     = k_raw / (||k_raw||_2 + eps)                 eq. (18); q likewise
 *                                                       when normalize_q
 * A zero vector with eps = 0 stays zero (the quotient is read as 0).
 */
static double load_token(const struct prologue* pro, const float* q, const float* k,
                         const float* v, const float* alpha, float beta, double* qd,
                         double* kd, double* vd, double* ad, int Dk, int Dv, int na)
{
    for (int c = 0; c < Dk; ++c) {
        qd[c] = (double)q[c];
        kd[c] = (double)k[c];
    }
    for (int c = 0; c < na; ++c) ad[c] = (double)alpha[c];
    for (int j = 0; j < Dv; ++j) vd[j] = (double)v[j];
    if (!pro) return (double)beta;
    double nk = 0.0, nq = 0.0;
    for (int c = 0; c < Dk; ++c) {
        nk += kd[c] * kd[c];
        nq += qd[c] * qd[c];
    }
    nk = sqrt(nk) + pro->eps;
    nq = sqrt(nq) + pro->eps;
    for (int c = 0; c < Dk; ++c) {
        kd[c] = nk > 0.0 ? kd[c] / nk : 0.0;
        if (pro->normalize_q) qd[c] = nq > 0.0 ? qd[c] / nq : 0.0;
        ad[c] = pro->amin + (pro->amax - pro->amin) * sigmoid(ad[c]);
    }
    return pro->bmax * sigmoid((double)beta);
}

static int forward_impl(const struct prologue* pro, const float* q, const float* k,
                        const float* v, const float* alpha, const float* theta,
                        const float* beta, const float* S0, double* out, double* ST,
                        double* CS, int chunk, int B, int T, int H, int Dk, int Dv,
                        int nthreads)
{
    if (!q || !k || !v || !alpha || !beta || !out) return -1;
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return -1;
    if (theta && Dk % 2 != 0) return -1;
    const int na = theta ? Dk / 2 : Dk;      /* gates per token */
    if (CS && chunk <= 0) return -1;
    const long nchunks = CS ? (T + chunk - 1) / chunk : 0;
    set_threads(nthreads);
    const long nbh = (long)B * H;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < nbh; ++bh) {
        const int b = (int)(bh / H), h = (int)(bh % H);
        const size_t nscr = (size_t)Dk * Dv + 2 * (size_t)Dv + 4 * (size_t)Dk;
        double* S = (double*)malloc(sizeof(double) * nscr);
        if (!S) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        double* pred = S + (size_t)Dk * Dv;
        double* vd = pred + Dv;
        double* qd = vd + Dv;
        double* kd = qd + Dk;
        double* ad = kd + Dk;
        double* td = ad + Dk;
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
            const double bt = load_token(pro, q + tok * Dk, k + tok * Dk, v + tok * Dv,
                                         alpha + tok * na, beta[tok], qd, kd, vd, ad, Dk, Dv, na);
            if (theta)
                for (int p = 0; p < na; ++p) td[p] = (double)theta[tok * na + p];
            token_update(S, qd, kd, vd, ad, theta ? td : NULL, bt, out + tok * Dv, Dk, Dv, pred);
        }
        if (ST) memcpy(ST + (size_t)bh * Dk * Dv, S, sizeof(double) * (size_t)Dk * Dv);
        free(S);
    }
    return failed ? -1 : 0;
}

int kda_oracle_forward(const float* q, const float* k, const float* v,
                       const float* alpha, const float* beta, const float* S0,
                       double* out, double* ST, double* CS, int chunk,
                       int B, int T, int H, int Dk, int Dv, int nthreads)
{
    return forward_impl(NULL, q, k, v, alpha, NULL, beta, S0, out, ST, CS, chunk, B, T, H, Dk,
                        Dv, nthreads);
}

int kda_oracle_forward_prologue(const float* q_raw, const float* k_raw, const float* v,
                                const float* gate, const float* beta_logit, const float* S0,
                                double amin, double amax, double bmax, double eps,
                                int normalize_q, double* out, double* ST,
                                int B, int T, int H, int Dk, int Dv, int nthreads)
{
    if (!(eps >= 0.0)) return -1;
    const struct prologue pro = {amin, amax, bmax, eps, normalize_q};
    return forward_impl(&pro, q_raw, k_raw, v, gate, NULL, beta_logit, S0, out, ST, NULL, 0, B,
                        T, H, Dk, Dv, nthreads);
}

int kda_oracle_forward_phase(const float* q, const float* k, const float* v,
                             const float* alpha, const float* theta, const float* beta,
                             const float* S0, double* out, double* ST,
                             int B, int T, int H, int Dk, int Dv, int nthreads)
{
    if (!theta) return -1;
    return forward_impl(NULL, q, k, v, alpha, theta, beta, S0, out, ST, NULL, 0, B, T, H, Dk,
                        Dv, nthreads);
}

/*
 * One token's gradients with respect to the inputs as the recurrence uses
 * them (dqt, dkt, dat, db for q, k, alpha, beta) stored as gradients of the
 * given inputs: unchanged without a prologue; with one, by the chain rule
 * through eqs. (15), (17), (18):
 *   d gate_c       = dalpha_c (amax - amin) s_c (1 - s_c),  s_c = sigmoid(gate_c)
 *   d beta_logit   = dbeta bmax s (1 - s),                   s = sigmoid(beta_logit)
 *   d k_raw        = dk / (n + eps) - k_raw <k_raw, dk> / (n (n + eps)^2),  n = ||k_raw||
 *                    (the second term absent for n = 0; zero when n + eps = 0)
 *   d q_raw        likewise when q is normalised, else dq.
 */
static void store_token_grads(const struct prologue* pro, const float* q, const float* k,
                              const float* alpha, float beta, const double* qd,
                              const double* kd, const double* dqt, const double* dkt,
                              const double* dat, double db, double* dq, double* dk,
                              double* dalpha, double* dbeta, int Dk)
{
    (void)qd;
    (void)kd;
    if (!pro) {
        for (int c = 0; c < Dk; ++c) {
            dq[c] = dqt[c];
            dk[c] = dkt[c];
            dalpha[c] = dat[c];
        }
        *dbeta = db;
        return;
    }
    for (int c = 0; c < Dk; ++c) {
        const double sg = sigmoid((double)alpha[c]);
        dalpha[c] = dat[c] * (pro->amax - pro->amin) * sg * (1.0 - sg);
    }
    const double sb = sigmoid((double)beta);
    *dbeta = db * pro->bmax * sb * (1.0 - sb);
    for (int pass = 0; pass < 2; ++pass) {
        const float* raw = pass == 0 ? k : q;
        const double* g = pass == 0 ? dkt : dqt;
        double* out = pass == 0 ? dk : dq;
        if (pass == 1 && !pro->normalize_q) {
            for (int c = 0; c < Dk; ++c) out[c] = g[c];
            continue;
        }
        double n = 0.0, dot = 0.0;
        for (int c = 0; c < Dk; ++c) {
            n += (double)raw[c] * (double)raw[c];
            dot += (double)raw[c] * g[c];
        }
        n = sqrt(n);
        const double den = n + pro->eps;
        for (int c = 0; c < Dk; ++c) {
            if (den <= 0.0) {
                out[c] = 0.0;
            } else {
                out[c] = g[c] / den - (n > 0.0 ? (double)raw[c] * dot / (n * den * den) : 0.0);
            }
        }
    }
}

/*
 * Reverse-mode derivative of the forward above (inputs taken as given, no
 * prologue, no phase), for the scalar loss
 *   L = sum_t <o_t, dO_t> + <S_T, dST>
 * so dO and dST are the loss gradients of the outputs and the final state.
 * It is the chain rule applied to one token of eq. (1) + eq. (14) at a time,
 * from the last token back to the first, with G the gradient of the state the
 * token leaves behind (from later tokens and dST):
 *   o_t = S_t^T q_t            ->  dq_t = S_t dO_t,   G += q_t dO_t^T
 *   S_t = St + k_t delta^T,  St = diag(alpha_t) S_{t-1},
 *         delta = beta_t u,  u = v_t - St^T k_t
 *        y = G^T k_t          ->  dv_t = beta_t y,   dbeta_t = <u, y>
 *                                 dk_t = G delta - beta_t St y
 *                                 dSt  = G - beta_t k_t y^T
 *   St = diag(alpha_t) S_{t-1} -> dalpha_t[c] = <dSt[c,:], S_{t-1}[c,:]>,
 *                                 G_{t-1} = diag(alpha_t) dSt
 * and dS0 is the last G.  With theta (the phase variant, §3 eq. (13)) the
 * decay of the row pair (2p, 2p+1) is the block alpha_p R(theta_p); with
 * (x, y) that pair of S_{t-1}, (gx, gy) the same rows of dSt, c = cos theta_p,
 * s = sin theta_p:
 *   St = alpha_p [c x - s y ; s x + c y]
 *     -> dalpha_p = <gx, c x - s y> + <gy, s x + c y>,
 *        dtheta_p = alpha_p (<gx, -s x - c y> + <gy, c x - s y>),
 *        G_{t-1} = alpha_p R(theta_p)^T dSt = alpha_p [c gx + s gy ; -s gx + c gy].
 * The states S_{t-1} are recomputed forward from checkpoints taken every 64
 * tokens (the same forward arithmetic).
 */
static void decay_copy(double* St, const double* Sp, const double* ad, const double* td, int Dk,
                       int Dv)
{
    if (!td) {
        for (int c = 0; c < Dk; ++c)
            for (int j = 0; j < Dv; ++j) St[(size_t)c * Dv + j] = ad[c] * Sp[(size_t)c * Dv + j];
        return;
    }
    for (int p = 0; p < Dk / 2; ++p) {
        const double c = ad[p] * cos(td[p]), sn = ad[p] * sin(td[p]);
        const double* x = Sp + (size_t)(2 * p) * Dv;
        const double* y = x + Dv;
        double* r0 = St + (size_t)(2 * p) * Dv;
        double* r1 = r0 + Dv;
        for (int j = 0; j < Dv; ++j) {
            r0[j] = c * x[j] - sn * y[j];
            r1[j] = sn * x[j] + c * y[j];
        }
    }
}

static int backward_impl(const struct prologue* pro, const float* q, const float* k,
                         const float* v, const float* alpha, const float* theta,
                         const float* beta, const float* S0, const float* dO, const float* dST,
                         double* dq, double* dk, double* dv, double* dalpha, double* dtheta,
                         double* dbeta, double* dS0, int B, int T, int H, int Dk, int Dv,
                         int nthreads)
{
    if (!q || !k || !v || !alpha || !beta || !dO || !dq || !dk || !dv || !dalpha || !dbeta)
        return -1;
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return -1;
    if (theta && (Dk % 2 != 0 || pro || !dtheta)) return -1;
    const int na = theta ? Dk / 2 : Dk;      /* gates per token */
    const int K = 64;
    const long nseg = (T + K - 1) / K;
    const size_t SZ = (size_t)Dk * Dv;
    set_threads(nthreads);
    const long nbh = (long)B * H;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < nbh; ++bh) {
        const int b = (int)(bh / H), h = (int)(bh % H);
        /* checkpoints [nseg][SZ], states of one segment [K + 1][SZ], G, dSt,
         * and per-token vectors */
        const size_t nd = (size_t)(nseg > 0 ? nseg : 1) * SZ + (size_t)(K + 1) * SZ + 3 * SZ +
                          5 * (size_t)Dv + 8 * (size_t)Dk;
        double* ck = (double*)malloc(sizeof(double) * nd);
        if (!ck) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        double* buf = ck + (size_t)(nseg > 0 ? nseg : 1) * SZ;
        double* G = buf + (size_t)(K + 1) * SZ;
        double* dSt = G + SZ;
        double* St = dSt + SZ;      /* the decayed state of the token */
        double* pred = St + SZ;
        double* vd = pred + Dv;
        double* u = vd + Dv;
        double* y = u + Dv;
        double* dod = y + Dv;
        double* qd = dod + Dv;
        double* kd = qd + Dk;
        double* ad = kd + Dk;
        double* dqt = ad + Dk;      /* this token's gradients of q, k, alpha as used */
        double* dkt = dqt + Dk;
        double* dat = dkt + Dk;
        double* td = dat + Dk;      /* phases of the token, and their gradients */
        double* dtt = td + Dk;

        /* forward: checkpoint the state before tokens 0, K, 2K, ... */
        double* S = buf;
        if (S0) {
            const float* s0 = S0 + (size_t)bh * SZ;
            for (size_t e = 0; e < SZ; ++e) S[e] = (double)s0[e];
        } else {
            memset(S, 0, sizeof(double) * SZ);
        }
        for (int t = 0; t < T; ++t) {
            const size_t tok = ((size_t)b * T + t) * H + h;
            if (t % K == 0) memcpy(ck + (size_t)(t / K) * SZ, S, sizeof(double) * SZ);
            const double bt = load_token(pro, q + tok * Dk, k + tok * Dk, v + tok * Dv,
                                         alpha + tok * na, beta[tok], qd, kd, vd, ad, Dk, Dv, na);
            if (theta)
                for (int p = 0; p < na; ++p) td[p] = (double)theta[tok * na + p];
            token_update(S, qd, kd, vd, ad, theta ? td : NULL, bt, NULL, Dk, Dv, pred);
        }

        /* backward */
        if (dST) {
            const float* g = dST + (size_t)bh * SZ;
            for (size_t e = 0; e < SZ; ++e) G[e] = (double)g[e];
        } else {
            memset(G, 0, sizeof(double) * SZ);
        }
        for (long sgi = nseg - 1; sgi >= 0; --sgi) {
            const int a = (int)(sgi * K), e_ = (a + K < T) ? a + K : T;
            /* buf[i] = state before token a + i, i = 0 .. e_ - a */
            memcpy(buf, ck + (size_t)sgi * SZ, sizeof(double) * SZ);
            for (int t = a; t < e_; ++t) {
                const size_t tok = ((size_t)b * T + t) * H + h;
                double* nx = buf + (size_t)(t - a + 1) * SZ;
                memcpy(nx, buf + (size_t)(t - a) * SZ, sizeof(double) * SZ);
                const double bt = load_token(pro, q + tok * Dk, k + tok * Dk, v + tok * Dv,
                                             alpha + tok * na, beta[tok], qd, kd, vd, ad, Dk, Dv, na);
                if (theta)
                    for (int p = 0; p < na; ++p) td[p] = (double)theta[tok * na + p];
                token_update(nx, qd, kd, vd, ad, theta ? td : NULL, bt, NULL, Dk, Dv, pred);
            }
            for (int t = e_ - 1; t >= a; --t) {
                const size_t tok = ((size_t)b * T + t) * H + h;
                const double* Sp = buf + (size_t)(t - a) * SZ;       /* S_{t-1} */
                const double* Sn = Sp + SZ;                          /* S_t */
                const double bt = load_token(pro, q + tok * Dk, k + tok * Dk, v + tok * Dv,
                                             alpha + tok * na, beta[tok], qd, kd, vd, ad, Dk, Dv, na);
                if (theta)
                    for (int p = 0; p < na; ++p) td[p] = (double)theta[tok * na + p];
                decay_copy(St, Sp, ad, theta ? td : NULL, Dk, Dv);
                for (int j = 0; j < Dv; ++j) dod[j] = (double)dO[tok * Dv + j];
                /* read-out o_t = S_t^T q_t */
                for (int c = 0; c < Dk; ++c) {
                    double s = 0.0;
                    for (int j = 0; j < Dv; ++j) s += Sn[(size_t)c * Dv + j] * dod[j];
                    dqt[c] = s;
                    for (int j = 0; j < Dv; ++j) G[(size_t)c * Dv + j] += qd[c] * dod[j];
                }
                /* delta correction of the decayed state St */
                for (int j = 0; j < Dv; ++j) {
                    double p = 0.0, yy = 0.0;
                    for (int c = 0; c < Dk; ++c) {
                        p += kd[c] * St[(size_t)c * Dv + j];
                        yy += G[(size_t)c * Dv + j] * kd[c];
                    }
                    u[j] = vd[j] - p;
                    y[j] = yy;
                }
                double db = 0.0;
                for (int j = 0; j < Dv; ++j) {
                    dv[tok * Dv + j] = bt * y[j];
                    db += u[j] * y[j];
                }
                for (int c = 0; c < Dk; ++c) {
                    double s1 = 0.0, s2 = 0.0;
                    for (int j = 0; j < Dv; ++j) {
                        s1 += G[(size_t)c * Dv + j] * bt * u[j];
                        s2 += St[(size_t)c * Dv + j] * y[j];
                    }
                    dkt[c] = s1 - bt * s2;
                }
                for (int c = 0; c < Dk; ++c)
                    for (int j = 0; j < Dv; ++j)
                        dSt[(size_t)c * Dv + j] = G[(size_t)c * Dv + j] - bt * kd[c] * y[j];
                if (!theta) {
                    /* decay: St = diag(alpha) S_{t-1} */
                    for (int c = 0; c < Dk; ++c) {
                        double s = 0.0;
                        for (int j = 0; j < Dv; ++j) s += dSt[(size_t)c * Dv + j] * Sp[(size_t)c * Dv + j];
                        dat[c] = s;
                        for (int j = 0; j < Dv; ++j) G[(size_t)c * Dv + j] = ad[c] * dSt[(size_t)c * Dv + j];
                    }
                    store_token_grads(pro, q + tok * Dk, k + tok * Dk, alpha + tok * Dk, beta[tok],
                                      qd, kd, dqt, dkt, dat, db, dq + tok * Dk, dk + tok * Dk,
                                      dalpha + tok * Dk, dbeta + tok, Dk);
                    continue;
                }
                /* decay: the rows (2p, 2p+1) of St are alpha_p R(theta_p) of those of S_{t-1} */
                for (int p = 0; p < na; ++p) {
                    const double c = cos(td[p]), sn = sin(td[p]);
                    const double* x = Sp + (size_t)(2 * p) * Dv;
                    const double* yv = x + Dv;
                    double* gx = dSt + (size_t)(2 * p) * Dv;
                    double* gy = gx + Dv;
                    double da = 0.0, dth = 0.0;
                    for (int j = 0; j < Dv; ++j) {
                        da += gx[j] * (c * x[j] - sn * yv[j]) + gy[j] * (sn * x[j] + c * yv[j]);
                        dth += gx[j] * (-sn * x[j] - c * yv[j]) + gy[j] * (c * x[j] - sn * yv[j]);
                    }
                    dat[p] = da;
                    dtt[p] = ad[p] * dth;
                    double* G0 = G + (size_t)(2 * p) * Dv;
                    double* G1 = G0 + Dv;
                    for (int j = 0; j < Dv; ++j) {
                        G0[j] = ad[p] * (c * gx[j] + sn * gy[j]);
                        G1[j] = ad[p] * (-sn * gx[j] + c * gy[j]);
                    }
                }
                for (int c = 0; c < Dk; ++c) {
                    dq[tok * Dk + c] = dqt[c];
                    dk[tok * Dk + c] = dkt[c];
                }
                for (int p = 0; p < na; ++p) {
                    dalpha[tok * na + p] = dat[p];
                    dtheta[tok * na + p] = dtt[p];
                }
                dbeta[tok] = db;
            }
        }
        if (dS0) memcpy(dS0 + (size_t)bh * SZ, G, sizeof(double) * SZ);
        free(ck);
    }
    return failed ? -1 : 0;
}

int kda_oracle_backward(const float* q, const float* k, const float* v, const float* alpha,
                        const float* beta, const float* S0, const float* dO, const float* dST,
                        double* dq, double* dk, double* dv, double* dalpha, double* dbeta,
                        double* dS0, int B, int T, int H, int Dk, int Dv, int nthreads)
{
    return backward_impl(NULL, q, k, v, alpha, NULL, beta, S0, dO, dST, dq, dk, dv, dalpha, NULL,
                         dbeta, dS0, B, T, H, Dk, Dv, nthreads);
}

int kda_oracle_backward_phase(const float* q, const float* k, const float* v, const float* alpha,
                              const float* theta, const float* beta, const float* S0,
                              const float* dO, const float* dST, double* dq, double* dk,
                              double* dv, double* dalpha, double* dtheta, double* dbeta,
                              double* dS0, int B, int T, int H, int Dk, int Dv, int nthreads)
{
    if (!theta) return -1;
    return backward_impl(NULL, q, k, v, alpha, theta, beta, S0, dO, dST, dq, dk, dv, dalpha,
                         dtheta, dbeta, dS0, B, T, H, Dk, Dv, nthreads);
}

int kda_oracle_backward_prologue(const float* q_raw, const float* k_raw, const float* v,
                                 const float* gate, const float* beta_logit, const float* S0,
                                 const float* dO, const float* dST, double amin, double amax,
                                 double bmax, double eps, int normalize_q, double* dq_raw,
                                 double* dk_raw, double* dv, double* dgate, double* dbeta_logit,
                                 double* dS0, int B, int T, int H, int Dk, int Dv, int nthreads)
{
    if (!(eps >= 0.0)) return -1;
    const struct prologue pro = {amin, amax, bmax, eps, normalize_q};
    return backward_impl(&pro, q_raw, k_raw, v, gate, NULL, beta_logit, S0, dO, dST, dq_raw,
                         dk_raw, dv, dgate, NULL, dbeta_logit, dS0, B, T, H, Dk, Dv, nthreads);
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
        double* pred = (double*)malloc(sizeof(double) * (2 * (size_t)Dv + 4 * (size_t)Dk));
        if (!pred) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        double* vd = pred + Dv;
        double* qd = vd + Dv;
        double* kd = qd + Dk;
        double* ad = kd + Dk;
        double* Sbh = S + (size_t)bh * Dk * Dv;
        for (int s = 0; s < nsteps; ++s) {
            const size_t tok = (size_t)s * nbh + bh;
            const double bt = load_token(NULL, q + tok * Dk, k + tok * Dk, v + tok * Dv,
                                         alpha + tok * Dk, beta[tok], qd, kd, vd, ad, Dk, Dv, Dk);
            token_update(Sbh, qd, kd, vd, ad, NULL, bt, out + tok * Dv, Dk, Dv, pred);
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
