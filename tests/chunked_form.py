"""An fp64 chunked rewrite of the gated delta rule, used only to pin the oracle.

It reaches the sequential recurrence's result by a different route (per-chunk
triangular solve instead of a token-by-token loop).  Agreement to rounding pins
the oracle's recurrence and also fixes, before any GPU code, the chunk algebra the
GPU kernels implement.  It shares no code with the oracle.

Per chunk of C positions with S0 the state at the chunk start (key axis decays):
    Gam_i  = sum_{s<=i} g_s (chunk-local, per channel),  Lam_i = exp(Gam_i)
    A_ij   = beta_i * sum_c k_ic k_jc exp(Gam_ic - Gam_jc)    (j < i)
    Tm     = (I + A)^-1
    W      = Tm diag(beta) (K * Lam),   Ut = Tm diag(beta) V,   U = Ut - W S0
    P_ij   = sum_c q_ic k_jc exp(Gam_ic - Gam_jc)             (j <= i)
    O      = (Q * Lam) S0 + P U
    S_next = Diag(Lam_C) S0 + Ktil^T U,   Ktil = K * exp(Gam_C - Gam)
"""
from __future__ import annotations

import numpy as np


def chunk_quantities(q, k, v, g, beta):
    """Chunk-local matrices for one head: q, k, g [C, dk]; v [C, dv]; beta [C]."""
    C = k.shape[0]
    Gam = np.cumsum(g, axis=0)
    Lam = np.exp(Gam)
    # pairwise decay factors exp(Gam_i - Gam_j), only used where j <= i (<= 1 there)
    diff = Gam[:, None, :] - Gam[None, :, :]
    lower = np.tril(np.ones((C, C), dtype=bool))
    E = np.where(lower[:, :, None], np.exp(np.where(lower[:, :, None], diff, 0.0)), 0.0)
    A = beta[:, None] * np.einsum("ic,jc,ijc->ij", k, k, E)
    A = np.tril(A, -1)
    P = np.einsum("ic,jc,ijc->ij", q, k, E)
    Tm = np.linalg.inv(np.eye(C) + A)
    W = Tm @ (beta[:, None] * (k * Lam))
    Ut = Tm @ (beta[:, None] * v)
    Ktil = k * np.exp(Gam[-1][None, :] - Gam)
    return dict(Gam=Gam, Lam=Lam, A=A, P=P, Tm=Tm, W=W, Ut=Ut, Ktil=Ktil, LamC=Lam[-1])


def chunked_head(q, k, v, g, beta, S0, C, scale=1.0):
    """Whole sequence of one head in chunks of C (last chunk may be short)."""
    T = q.shape[0]
    S = np.array(S0, dtype=np.float64)
    o = np.zeros((T, v.shape[1]))
    for s in range(0, T, C):
        e = min(T, s + C)
        m = chunk_quantities(q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e])
        U = m["Ut"] - m["W"] @ S
        o[s:e] = scale * ((q[s:e] * m["Lam"]) @ S + m["P"] @ U)
        S = m["LamC"][:, None] * S + m["Ktil"].T @ U
    return o, S
