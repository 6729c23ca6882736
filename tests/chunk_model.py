"""fp64 numpy model of the chunkwise (WY) form of the KDA / CKDA forward.

Test-side only: it pins the oracle (chunked must equal sequential, "Kimi Delta
Attention: a bounded case study", Exercise 2's reasoned solution: chunking
changes cost, never the numbers) and documents the algebra the HIP kernels
implement.  It shares no code with either the oracle or the HIP library.

Within one chunk of C tokens (local index r = 0..C-1, S = state at chunk
start), with rho(r, i) = prod_{j=i+1..r} alpha_j (per channel, rho(r, r) = 1)
and Gamma_r = prod_{j<=r} alpha_j:
  A[r, i] = beta_r * sum_c k[r,c] k[i,c] rho(r,i)_c        (i < r, else 0)
  Tinv    = (I + A)^{-1}                                   (unit lower triangular)
  W = Tinv diag(beta) (K * Gamma),   U = Tinv diag(beta) V
  Delta = U - W S                    (row r = the delta actually written by token r)
  P[r, i] = sum_c q[r,c] k[i,c] rho(r,i)_c                  (i <= r, else 0)
  O = (Q * Gamma) S + P Delta
  S_next = diag(Gamma_{C-1}) S + Ktil^T Delta,   Ktil[i] = k_i * rho(C-1, i)
Derivation: unrolling S_r = diag(alpha_r) S_{r-1} + k_r Delta_r^T (eq. (1) of
"Semidirect Fourier Delta Attention" rewritten) inside a chunk gives a unit
lower-triangular system for the deltas (the triangular solve / UT transform of
that page's §2.2); the read-out is eq. (14).
"""
from __future__ import annotations

import numpy as np


def _rho_table(alpha):
    """rho[r, i, c] = prod_{j=i+1..r} alpha[j, c] for i <= r, else 0."""
    C, Dk = alpha.shape
    rho = np.zeros((C, C, Dk))
    for i in range(C):
        p = np.ones(Dk)
        rho[i, i] = p
        for r in range(i + 1, C):
            p = p * alpha[r]
            rho[r, i] = p
    return rho


def chunk_step(S, q, k, v, alpha, beta):
    """One chunk.  S [Dk,Dv]; q,k,alpha [C,Dk]; v [C,Dv]; beta [C].
    Returns (O [C,Dv], S_next [Dk,Dv])."""
    C = q.shape[0]
    rho = _rho_table(alpha)
    gamma = np.cumprod(alpha, axis=0)                      # Gamma_r
    A = np.zeros((C, C))
    P = np.zeros((C, C))
    for r in range(C):
        for i in range(r + 1):
            kk = np.sum(k[r] * k[i] * rho[r, i])
            if i < r:
                A[r, i] = beta[r] * kk
            P[r, i] = np.sum(q[r] * k[i] * rho[r, i])
    M = np.eye(C) + A
    W = np.linalg.solve(M, beta[:, None] * (k * gamma))
    U = np.linalg.solve(M, beta[:, None] * v)
    delta = U - W @ S
    O = (q * gamma) @ S + P @ delta
    ktil = k * rho[C - 1, :, :]
    S_next = gamma[C - 1][:, None] * S + ktil.T @ delta
    return O, S_next


def forward(q, k, v, alpha, beta, S0=None, chunk=16):
    """Chunked forward, same layouts as the oracle: q,k,alpha [B,T,H,Dk],
    v [B,T,H,Dv], beta [B,T,H], S0 [B,H,Dk,Dv] or None.  Returns (out, ST)."""
    q, k, v, alpha, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, alpha, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    out = np.zeros((B, T, H, Dv))
    ST = np.zeros((B, H, Dk, Dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((Dk, Dv)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
            for t0 in range(0, T, chunk):
                t1 = min(T, t0 + chunk)
                O, S = chunk_step(S, q[b, t0:t1, h], k[b, t0:t1, h], v[b, t0:t1, h],
                                  alpha[b, t0:t1, h], beta[b, t0:t1, h])
                out[b, t0:t1, h] = O
            ST[b, h] = S
    return out, ST
