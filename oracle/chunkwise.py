"""Chunkwise fp64 reference of the KLA forward pass -- TEST INFRASTRUCTURE ONLY.

A second, independent route to the function the tokenwise oracle computes, taken
from the paper "Kaczmarz Linear Attention" (arXiv 2605.08587), section 4
"Chunkwise Parallelism", Proposition 3 (Eq. (7)) and Proposition 4 (Eq. (8),
(9)), with the matrix form of Appendix B.2/B.3.  For one chunk of C tokens with
incoming state S0 (row-vector convention, S is d_k x d_v):

    b_i   = eta_i / (||k_i||^2 + eps)           (b_i = 0 if the denominator is 0)
    G_i   = g_1 + ... + g_i                      chunk-local inclusive sum of log-decays
    gam_i = exp(G_i)                             gamma_i = alpha_1 ... alpha_i
    A_ij  = exp(G_i - G_j) for j <= i, else 0    the decay mask (A^- = its strict part)
    L     = Diag(b) (A^- o K K^T)                strictly lower triangular
    (I + L) U = Diag(b) (V - Diag(gam) K S0)     Eq. (7): forward substitution
    O     = Diag(gam) Q S0 + (A o Q K^T) U       Eq. (8)
    S_out = gam_C S0 + K^T Diag(exp(G_C - G)) U  Eq. (9)

The chain of chunks passes S_out of one chunk as S0 of the next; chunks restart
at every sequence start and the last chunk of a sequence may be short.  The
mask is built from differences G_i - G_j (never a ratio gam_i / gam_j) and is set
to zero above the diagonal before any exponential is taken.

Also returned, for unit checks of the device kernels: b, G and
T = (I + L)^{-1} Diag(b) per chunk, so that U = T (V - Diag(gam) K S0).
"""
from __future__ import annotations

import numpy as np


def _beta(k: np.ndarray, eta: np.ndarray, eps: float) -> np.ndarray:
    den = np.einsum("ti,ti->t", k, k) + eps
    out = np.zeros_like(den)
    nz = den != 0.0
    out[nz] = eta[nz] / den[nz]
    return out


def _forward_substitution(L: np.ndarray, rhs: np.ndarray) -> np.ndarray:
    """Solve (I + L) X = rhs for strictly lower-triangular L, one row at a time."""
    X = np.zeros_like(rhs)
    for i in range(rhs.shape[0]):
        X[i] = rhs[i] - L[i, :i] @ X[:i]
    return X


def chunk_step(S0, q, k, v, g, eta, eps):
    """One chunk of one head: returns (O, S_out, b, G, T) in fp64.

    S0 [d_k, d_v]; q, k [C, d_k]; v [C, d_v]; g, eta [C].
    """
    C = k.shape[0]
    b = _beta(k, eta, eps)
    G = np.cumsum(g)
    gam = np.exp(G)
    diff = G[:, None] - G[None, :]
    lower = np.tril(np.ones((C, C), dtype=bool))
    A = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)
    A_strict = np.tril(A, -1)
    L = b[:, None] * (A_strict * (k @ k.T))
    rhs = b[:, None] * (v - gam[:, None] * (k @ S0))
    U = _forward_substitution(L, rhs)
    O = gam[:, None] * (q @ S0) + (A * (q @ k.T)) @ U
    S_out = gam[-1] * S0 + k.T @ (np.exp(G[-1] - G)[:, None] * U)
    T = _forward_substitution(L, np.diag(b))
    return O, S_out, b, G, T


def prefill(q, k, v, g, eta, eps, S0=None, cu_seqlens=None, chunk=64):
    """Chunkwise fp64 prefill over packed sequences.

    Arrays as in the tokenwise oracle: q, k [n_tok, H, d_k]; v [n_tok, H, d_v];
    g, eta [n_tok, H]; S0 [n_seq, H, d_k, d_v] or None; cu_seqlens [n_seq+1] or
    None (one sequence).  Returns (o, S_T, inter) where inter maps
    (seq, head, chunk_index) -> dict(b=..., G=..., T=...).
    """
    q, k, v, g, eta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, eta))
    n_tok, H, dk = q.shape
    dv = v.shape[-1]
    cu = np.array([0, n_tok]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    ns = len(cu) - 1
    S0 = np.zeros((ns, H, dk, dv)) if S0 is None else np.asarray(S0, dtype=np.float64)
    o = np.zeros((n_tok, H, dv))
    ST = np.zeros((ns, H, dk, dv))
    inter = {}
    for n in range(ns):
        for h in range(H):
            S = S0[n, h].copy()
            for c, t0 in enumerate(range(int(cu[n]), int(cu[n + 1]), chunk)):
                t1 = min(t0 + chunk, int(cu[n + 1]))
                O, S, b, G, T = chunk_step(S, q[t0:t1, h], k[t0:t1, h], v[t0:t1, h],
                                           g[t0:t1, h], eta[t0:t1, h], eps)
                o[t0:t1, h] = O
                inter[(n, h, c)] = dict(b=b, G=G, T=T)
            ST[n, h] = S
    return o, ST, inter


# ------------------------------------------------------------------ diagonal gating
# Appendix B.5 ("Extension to diagonal gating"): with D_t = Diag(alpha_t), the scalar gamma
# of Propositions 3-4 becomes a vector per token and every decay product acts per key
# channel.  Working the chunk through the same way (row-vector convention, G the per-channel
# chunk-local cumulative log-decay, C x d_k):
#     A_ij  = sum_c k_i[c] k_j[c] exp(G_i[c] - G_j[c])      (j < i)
#     L     = Diag(b) A                                      strictly lower triangular
#     (I + L) U = Diag(b) (V - (K o exp(G)) S0)
#     P_ij  = sum_c q_i[c] k_j[c] exp(G_i[c] - G_j[c])      (j <= i)
#     O     = (Q o exp(G)) S0 + P U
#     S_out = Diag(exp(G_C)) S0 + (K o exp(G_C - G))^T U
# Every exponent is a difference G_i - G_j with j <= i, or G_C - G_j, so none is positive.


def chunk_step_diag(S0, q, k, v, g, eta, eps):
    """One chunk of one head under diagonal gating: returns (O, S_out, b, G, T) in fp64.

    S0 [d_k, d_v]; q, k [C, d_k]; v [C, d_v]; g [C, d_k]; eta [C].
    """
    C = k.shape[0]
    b = _beta(k, eta, eps)
    G = np.cumsum(g, axis=0)                                  # [C, d_k]
    D = G[:, None, :] - G[None, :, :]                         # D[i, j, c] = G_i[c] - G_j[c]
    lower = np.tril(np.ones((C, C), dtype=bool))
    E = np.where(lower[:, :, None], np.exp(np.where(lower[:, :, None], D, 0.0)), 0.0)
    A = np.einsum("ic,jc,ijc->ij", k, k, E)
    L = b[:, None] * np.tril(A, -1)
    rhs = b[:, None] * (v - (k * np.exp(G)) @ S0)
    U = _forward_substitution(L, rhs)
    P = np.einsum("ic,jc,ijc->ij", q, k, E)
    O = (q * np.exp(G)) @ S0 + P @ U
    S_out = np.exp(G[-1])[:, None] * S0 + (k * np.exp(G[-1][None, :] - G)).T @ U
    T = _forward_substitution(L, np.diag(b))
    return O, S_out, b, G, T


def prefill_diag(q, k, v, g, eta, eps, S0=None, cu_seqlens=None, chunk=64):
    """Chunkwise fp64 prefill under diagonal gating (g [n_tok, H, d_k]); as prefill."""
    q, k, v, g, eta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, eta))
    n_tok, H, dk = q.shape
    dv = v.shape[-1]
    cu = np.array([0, n_tok]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    ns = len(cu) - 1
    S0 = np.zeros((ns, H, dk, dv)) if S0 is None else np.asarray(S0, dtype=np.float64)
    o = np.zeros((n_tok, H, dv))
    ST = np.zeros((ns, H, dk, dv))
    for n in range(ns):
        for h in range(H):
            S = S0[n, h].copy()
            for t0 in range(int(cu[n]), int(cu[n + 1]), chunk):
                t1 = min(t0 + chunk, int(cu[n + 1]))
                O, S, _, _, _ = chunk_step_diag(S, q[t0:t1, h], k[t0:t1, h], v[t0:t1, h],
                                                g[t0:t1, h], eta[t0:t1, h], eps)
                o[t0:t1, h] = O
            ST[n, h] = S
    return o, ST
