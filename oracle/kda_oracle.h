/*
 * kda_oracle.h — CPU oracle for the Kimi Delta Attention (KDA) recurrence and
 * its Complex-KDA (CKDA) range extension.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no source
 * with the HIP library and must never be used as a fallback for it.
 *
 * What it computes (plain definitions, fp64 state and accumulation):
 *   S_t = (I - beta_t k_t k_t^T) diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *       — "Semidirect Fourier Delta Attention" (arXiv 2607.11897), §1 eq. (1),
 *         restated per token as an affine map in §2.2 eq. (9);
 *   o_t = S_t^T q_t  (post-update state, no scale factor)
 *       — same page, §3 eq. (14) (SFDA reduces to KDA at zero phase, Prop. 2.1).
 * Range extension (alpha in [-1,1], beta in [0,2]) — "Complex KDA: Understanding
 * and Enhancing the Expressivity of Kimi Delta Attention", the abstract.  The
 * mathematics is the same for both ranges; the oracle takes any real inputs.
 *
 * Layouts (all row-major, contiguous):
 *   q, k, alpha : [B, T, H, Dk]      v : [B, T, H, Dv]      beta : [B, T, H]
 *   S0, ST      : [B, H, Dk, Dv]     out : [B, T, H, Dv]
 * Inputs are float (bf16 and fp32 values widen to double exactly); the state
 * and every accumulation are double; outputs are double.
 *
 * Return value: 0 on success, -1 on a bad argument (null pointer or size < 0).
 */
#ifndef KDA_ORACLE_H
#define KDA_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Sequential token-by-token forward over T tokens.  S0 may be NULL (zero
 * initial state); ST may be NULL (final state not wanted).  CS may be NULL;
 * otherwise chunk > 0 and CS [B, H, ceil(T/chunk), Dk, Dv] receives, for every
 * n, the state before token n*chunk (the state a chunk of the chunkwise form
 * starts from; "Kimi Delta Attention: a bounded case study", Exercise 2).
 * nthreads <= 0 uses the OpenMP default.  Parallelism is over independent
 * (b, h) pairs only. */
int kda_oracle_forward(const float* q, const float* k, const float* v,
                       const float* alpha, const float* beta, const float* S0,
                       double* out, double* ST, double* CS, int chunk,
                       int B, int T, int H, int Dk, int Dv, int nthreads);

/* The same forward from raw inputs through the stable parameterisation of
 * "Semidirect Fourier Delta Attention" §3: per token, in double,
 *   alpha = amin + (amax - amin) * sigmoid(gate)                eq. (15)
 *   beta  = bmax * sigmoid(beta_logit)                           eq. (17)
 *   k     = k_raw / (||k_raw||_2 + eps), and q likewise when normalize_q
 *                                                                eq. (18)
 * (a zero vector with eps = 0 stays zero).  gate has alpha's layout,
 * beta_logit beta's.  eps < 0 or NaN is a bad argument. */
int kda_oracle_forward_prologue(const float* q_raw, const float* k_raw, const float* v,
                                const float* gate, const float* beta_logit, const float* S0,
                                double amin, double amax, double bmax, double eps,
                                int normalize_q, double* out, double* ST,
                                int B, int T, int H, int Dk, int Dv, int nthreads);

/* Phase variant ("Semidirect Fourier Delta Attention", §3 eq. (13), real
 * form eq. (2) with the 2x2 rotation blocks of eq. (12)): channels 2p, 2p+1
 * form complex coordinate p and the decay is Lambda_t = diag(alpha_t e^{i
 * theta_t}), i.e. the block alpha_p R(theta_p), R = [[cos, -sin], [sin, cos]],
 * on that pair of state rows, then the same delta correction and read-out.
 * alpha, theta: [B, T, H, Dk/2] (one per pair); Dk must be even. */
int kda_oracle_forward_phase(const float* q, const float* k, const float* v,
                             const float* alpha, const float* theta, const float* beta,
                             const float* S0, double* out, double* ST,
                             int B, int T, int H, int Dk, int Dv, int nthreads);

/* Gradients of the scalar loss L = sum_t <o_t, dO_t> + <S_T, dST> with
 * respect to every input of kda_oracle_forward (reverse-mode chain rule
 * through each token of eq. (1) and eq. (14), last token first; dST may be
 * NULL = zero).  dO has out's layout; dq, dk, dalpha [B, T, H, Dk],
 * dv [B, T, H, Dv], dbeta [B, T, H], dS0 [B, H, Dk, Dv] (may be NULL).
 * The states are recomputed from checkpoints every 64 tokens. */
int kda_oracle_backward(const float* q, const float* k, const float* v, const float* alpha,
                        const float* beta, const float* S0, const float* dO, const float* dST,
                        double* dq, double* dk, double* dv, double* dalpha, double* dbeta,
                        double* dS0, int B, int T, int H, int Dk, int Dv, int nthreads);

/* The same gradients for the phase variant (kda_oracle_forward_phase,
 * "Semidirect Fourier Delta Attention" §3 eq. (13)): alpha, theta, dalpha and
 * dtheta are [B, T, H, Dk/2], one decay and one phase per channel pair; every
 * other layout as kda_oracle_backward.  The decay step's gradients take the
 * 2x2 block alpha_p R(theta_p) in place of the diagonal. */
int kda_oracle_backward_phase(const float* q, const float* k, const float* v, const float* alpha,
                              const float* theta, const float* beta, const float* S0,
                              const float* dO, const float* dST, double* dq, double* dk,
                              double* dv, double* dalpha, double* dtheta, double* dbeta,
                              double* dS0, int B, int T, int H, int Dk, int Dv, int nthreads);

/* The same gradients for the forward from raw inputs
 * (kda_oracle_forward_prologue): with respect to q_raw, k_raw, v, the gate
 * logits, the beta logits and S0, by the chain rule through eqs. (15), (17)
 * and (18) after the reverse pass.  Layouts as the forward's. */
int kda_oracle_backward_prologue(const float* q_raw, const float* k_raw, const float* v,
                                 const float* gate, const float* beta_logit, const float* S0,
                                 const float* dO, const float* dST, double amin, double amax,
                                 double bmax, double eps, int normalize_q, double* dq_raw,
                                 double* dk_raw, double* dv, double* dgate, double* dbeta_logit,
                                 double* dS0, int B, int T, int H, int Dk, int Dv, int nthreads);

/* nsteps single-token updates applied to a resident double state in place.
 * Per-step inputs are stacked: q, k, alpha [nsteps, B, H, Dk],
 * v [nsteps, B, H, Dv], beta [nsteps, B, H]; out [nsteps, B, H, Dv];
 * S [B, H, Dk, Dv] (double, read and written). */
int kda_oracle_decode(const float* q, const float* k, const float* v,
                      const float* alpha, const float* beta, double* S,
                      double* out, int nsteps, int B, int H, int Dk, int Dv,
                      int nthreads);

/* Chunk-local gate summary, from its definition, per (b, h, chunk n, local
 * token r, channel c) with chunk length C (last chunk may be short):
 *   L[.]      = sum over j <= r in the chunk with alpha_j != 0 of log2|alpha_j|
 *   parity[.] = (number of j <= r in the chunk with alpha_j < 0) mod 2
 *   zpos[.]   = 1 + (largest j <= r in the chunk with alpha_j == 0), 0 if none
 *   gend[b,h,n,c] = product of alpha over the whole chunk (plain product)
 * L, parity, zpos : [B, H, NC, C, Dk] (entries past T are left untouched);
 * gend : [B, H, NC, Dk];  NC = ceil(T / C). */
int kda_oracle_gate_prep(const float* alpha, double* L, unsigned char* parity,
                         int* zpos, double* gend, int B, int T, int H, int Dk,
                         int C);

#ifdef __cplusplus
}
#endif
#endif
