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


# ---- backward --------------------------------------------------------------
# Gradients of L = sum <O, dO> + <S_T, dST>, chunk by chunk, in the form the
# HIP backward computes them.  With S the state entering a chunk, dS_next the
# loss gradient of the state leaving it (from later chunks and dST only),
# Delta the chunk's deltas and X = P^T dO + Ktil dS_next:
#   reverse chain:  dS = diag(Gamma_{C-1}) dS_next + (Q * Gamma)^T dO - W^T X
#   y = Tinv^T X,  dv = diag(beta) y  (y_r = G_r^T k_r, G_r the gradient of the
#       state after token r)
#   B1 = dO Delta^T, B3 = Y Delta^T;  F1 = dO S^T, F2 = Y S^T, F3 = Delta dS_next^T
#   LQ1_r = sum_{i<r} B1[r,i] rho(r,i) k_i     LK3_r = sum_{i<r} B3[r,i] rho(r,i) k_i
#   UQ1_r = sum_{j>r} B1[j,r] rho(j,r) q_j     UK2_r = sum_{j>r} beta_j B3[j,r] rho(j,r) k_j
#   dq = Gamma F1 + LQ1 + diag(B1) k
#   dk = rho(C-1, .) F3 + UQ1 + diag(B1) q - UK2 - beta Gamma F2 - beta LK3
#   dbeta_r = v_r . y_r - (k_r Gamma_r) . F2_r - k_r . LK3_r
#   alpha_r dalpha_r = Gamma_{C-1} sigma + sum_{i<r} (Ktil F3)_i
#                      + sum_{j>=r} Gamma_j (q_j F1_j - beta_j k_j F2_j)
#                      + sum_{t>=r} (R_t - Cs_t),   sigma_c = <dS_next[c], S[c]>,
#       R = q LQ1 - beta k LK3,  Cs = k (UQ1 - UK2)
# and, where |alpha_r| < TINY (a zero gate included), the direct form
#   dalpha_r[c] = <H_r[c,:], S_{r-1}[c,:]>,  H_r = G_r - beta_r k_r y_r^T.
TINY = 2.0 ** -6


def _chunk_operands(S, q, k, v, alpha, beta):
    C = q.shape[0]
    rho = _rho_table(alpha)
    gamma = np.cumprod(alpha, axis=0)
    A = np.zeros((C, C))
    P = np.zeros((C, C))
    for r in range(C):
        for i in range(r + 1):
            if i < r:
                A[r, i] = beta[r] * np.sum(k[r] * k[i] * rho[r, i])
            P[r, i] = np.sum(q[r] * k[i] * rho[r, i])
    Tinv = np.linalg.inv(np.eye(C) + A)
    W = Tinv @ (beta[:, None] * (k * gamma))
    U = Tinv @ (beta[:, None] * v)
    delta = U - W @ S
    ktil = k * rho[C - 1]
    return dict(rho=rho, gamma=gamma, Tinv=Tinv, W=W, P=P, delta=delta, ktil=ktil)


def chunk_local_backward(S, dSn, X, q, k, v, alpha, beta, dO, ops):
    """dq, dk, dv, dalpha, dbeta of one chunk from its start state S, the
    gradient dSn of its end state (later chunks only) and X."""
    C, Dk = q.shape
    rho, gamma, delta, ktil = ops["rho"], ops["gamma"], ops["delta"], ops["ktil"]
    y = ops["Tinv"].T @ X
    dv = beta[:, None] * y
    B1 = dO @ delta.T
    B3 = y @ delta.T
    F1 = dO @ S.T
    F2 = y @ S.T
    F3 = delta @ dSn.T
    sigma = np.sum(dSn * S, axis=1)
    LQ1 = np.zeros((C, Dk)); LK3 = np.zeros((C, Dk)); UQ1 = np.zeros((C, Dk)); UK2 = np.zeros((C, Dk))
    for r in range(C):
        for i in range(r):
            LQ1[r] += B1[r, i] * rho[r, i] * k[i]
            LK3[r] += B3[r, i] * rho[r, i] * k[i]
        for j in range(r + 1, C):
            UQ1[r] += B1[j, r] * rho[j, r] * q[j]
            UK2[r] += beta[j] * B3[j, r] * rho[j, r] * k[j]
    dB1 = np.diag(B1)[:, None]
    gend = rho[C - 1]                          # rho(C-1, r)
    dq = gamma * F1 + LQ1 + dB1 * k
    dk = gend * F3 + UQ1 + dB1 * q - UK2 - beta[:, None] * (gamma * F2) - beta[:, None] * LK3
    dbeta = np.sum(v * y, axis=1) - np.sum(k * gamma * F2, axis=1) - np.sum(k * LK3, axis=1)
    R = q * LQ1 - beta[:, None] * k * LK3
    Cs = k * (UQ1 - UK2)
    pre = np.cumsum(np.vstack([np.zeros((1, Dk)), (ktil * F3)[:-1]]), axis=0)     # sum_{i<r}
    suf1 = np.cumsum((gamma * (q * F1 - beta[:, None] * k * F2))[::-1], axis=0)[::-1]
    suf2 = np.cumsum((R - Cs)[::-1], axis=0)[::-1]
    Z = gamma[C - 1] * sigma + pre + suf1 + suf2
    dalpha = np.zeros((C, Dk))
    big = np.abs(alpha) >= TINY
    dalpha[big] = Z[big] / alpha[big]
    if not big.all():
        # direct form: states before each token and the gradients after it
        Sprev = np.zeros((C, Dk, S.shape[1]))
        cur = S.copy()
        for r in range(C):
            Sprev[r] = cur
            cur = alpha[r][:, None] * cur + np.outer(k[r], delta[r])
        G = dSn + np.outer(q[C - 1], dO[C - 1])
        for r in range(C - 1, -1, -1):
            Hm = G - np.outer(k[r], dv[r])
            for c in range(Dk):
                if not big[r, c]:
                    dalpha[r, c] = Hm[c] @ Sprev[r][c]
            if r > 0:
                G = alpha[r][:, None] * Hm + np.outer(q[r - 1], dO[r - 1])
    return dq, dk, dv, dalpha, dbeta


def backward(q, k, v, alpha, beta, dO, S0=None, dST=None, chunk=16):
    """Chunked backward, layouts as the oracle's.  Returns the same dict."""
    q, k, v, alpha, beta, dO = (np.asarray(x, dtype=np.float64) for x in (q, k, v, alpha, beta, dO))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    res = {"dq": np.zeros((B, T, H, Dk)), "dk": np.zeros((B, T, H, Dk)),
           "dv": np.zeros((B, T, H, Dv)), "dalpha": np.zeros((B, T, H, Dk)),
           "dbeta": np.zeros((B, T, H)), "dS0": np.zeros((B, H, Dk, Dv))}
    for b in range(B):
        for h in range(H):
            S = np.zeros((Dk, Dv)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
            sl = [(t0, min(T, t0 + chunk)) for t0 in range(0, T, chunk)]
            starts, opsl = [], []
            for t0, t1 in sl:
                a = [x[b, t0:t1, h] for x in (q, k, v, alpha)]
                ops = _chunk_operands(S, a[0], a[1], a[2], a[3], beta[b, t0:t1, h])
                starts.append(S)
                opsl.append(ops)
                S = ops["gamma"][-1][:, None] * S + ops["ktil"].T @ ops["delta"]
            dS = np.zeros((Dk, Dv)) if dST is None else np.array(dST[b, h], dtype=np.float64)
            for n in range(len(sl) - 1, -1, -1):
                t0, t1 = sl[n]
                ops = opsl[n]
                do = dO[b, t0:t1, h]
                X = ops["P"].T @ do + ops["ktil"] @ dS
                g = chunk_local_backward(starts[n], dS, X, q[b, t0:t1, h], k[b, t0:t1, h],
                                         v[b, t0:t1, h], alpha[b, t0:t1, h], beta[b, t0:t1, h],
                                         do, ops)
                for name, val in zip(("dq", "dk", "dv", "dalpha", "dbeta"), g):
                    res[name][b, t0:t1, h] = val
                qg = q[b, t0:t1, h] * ops["gamma"]
                dS = ops["gamma"][-1][:, None] * dS + qg.T @ do - ops["W"].T @ X
            res["dS0"][b, h] = dS
    return res
