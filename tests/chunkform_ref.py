"""Chunkwise schedule of the KDA recurrence in fp64 NumPy (test-only).

This is the derivation the GPU prefill implements, written out plainly so a
CPU test can show that it reaches the token-by-token result exactly (up to
rounding).  It follows page "Kimi Delta Attention (KDA)" (brain.bigb.es),
section "Two schedules for one recurrence":

 * provisional errors  ebar_i = beta_i (v_i - S_c D_{0:i} k_i),
 * coupling            rho_ij = beta_i k_j^T D_{j+1:i} k_i  (j < i),
 * true errors         E = (I + R)^{-1} Ebar  (rows e_i), a unit-lower
                       triangular solve,
 * state advance       S_{c+1} = S_c D_{0:C-1} + E^T K^end,
 * outputs             O = s Q^bnd S_c^T + A E,  chi_ij = s k_j^T D_{j+1:i} q_i
                       for j <= i (diagonal included: the read follows the
                       write).

Reading of the decay products (the page leaves the endpoints implicit):
D_{a:b} = Diag(prod_{m=a..b} alpha_m) over chunk-local indices, empty product
= identity; a token's own gate is applied before its write, so a write at j
reaches i >= j through alpha_{j+1..i}.

The errors are split as E = U - W S_c^T with U = T diag(beta) V and
W = T diag(beta) K^bnd, T = (I + R)^{-1}: the same factorisation the GPU
kernels use.  A partial last chunk is padded with q = k = v = 0, beta = 0 and
alpha = 1, which adds nothing and leaves the state untouched.

Nothing here is used by the GPU library, and it does not use the oracle.
"""
from __future__ import annotations

import numpy as np


def _decay_between(alpha_c, a, b):
    """prod_{m=a..b} alpha_m per channel (identity for an empty range)."""
    if b < a:
        return np.ones(alpha_c.shape[1])
    return np.prod(alpha_c[a:b + 1], axis=0)


def chunk_head(q, k, v, alpha, beta, S0, C, scale):
    """One head of one sequence.  q,k,alpha [T,dk], v [T,dv], beta [T],
    S0 [dv,dk].  Returns (o [T,dv], S_final [dv,dk])."""
    T, dk = q.shape
    dv = v.shape[1]
    S = S0.copy()
    o = np.zeros((T, dv))
    for c0 in range(0, T, C):
        L = min(C, T - c0)
        Q = np.zeros((C, dk)); K = np.zeros((C, dk)); V = np.zeros((C, dv))
        A_ = np.ones((C, dk)); b = np.zeros(C)
        Q[:L], K[:L], V[:L] = q[c0:c0 + L], k[c0:c0 + L], v[c0:c0 + L]
        A_[:L], b[:L] = alpha[c0:c0 + L], beta[c0:c0 + L]

        Kbnd = np.stack([_decay_between(A_, 0, i) * K[i] for i in range(C)])
        Qbnd = np.stack([_decay_between(A_, 0, i) * Q[i] for i in range(C)])
        Kend = np.stack([_decay_between(A_, j + 1, C - 1) * K[j] for j in range(C)])
        R = np.zeros((C, C))
        Aqk = np.zeros((C, C))
        for i in range(C):
            for j in range(i + 1):
                d = _decay_between(A_, j + 1, i)
                if j < i:
                    R[i, j] = b[i] * (K[j] * d) @ K[i]
                Aqk[i, j] = scale * (K[j] * d) @ Q[i]
        Tm = np.linalg.solve(np.eye(C) + R, np.eye(C))
        W = Tm @ (b[:, None] * Kbnd)
        U = Tm @ (b[:, None] * V)
        E = U - W @ S.T
        O = scale * Qbnd @ S.T + Aqk @ E
        S = S * _decay_between(A_, 0, C - 1)[None, :] + E.T @ Kend
        o[c0:c0 + L] = O[:L]
    return o, S


def chunk_fwd(q, k, v, alpha, beta, S0=None, C=64, scale=None):
    """Dense batch: q,k,alpha [B,T,H,dk], v [B,T,H,dv], beta [B,T,H]."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    scale = dk ** -0.5 if scale is None else scale
    o = np.zeros((B, T, H, dv))
    Sf = np.zeros((B, H, dv, dk))
    for bb in range(B):
        for h in range(H):
            s0 = np.zeros((dv, dk)) if S0 is None else S0[bb, h]
            o[bb, :, h], Sf[bb, h] = chunk_head(
                q[bb, :, h], k[bb, :, h], v[bb, :, h], alpha[bb, :, h],
                beta[bb, :, h], s0, C, scale)
    return o, Sf
