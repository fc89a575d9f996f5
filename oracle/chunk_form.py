"""Chunkwise-parallel WY/UT form of the gated Q-Delta rule in fp64 numpy.
TEST INFRASTRUCTURE ONLY (see the ``oracle`` package docstring).

This is the chunk algebra of the Q-Delta reading notes, §2.6 ("分块并行"), in the
row-stacked convention that section uses (Q, K, X are C x d_k, V is C x d_v, the
entry state S_in is d_v x d_k), written out step by step in the section's order:

  gamma_i = prod_{j<=i} alpha_j,  B = diag(beta),  D_gamma = diag(gamma),
  H_ij = gamma_i / gamma_j for j <= i, else 0            (causal decay matrix)
  L       = sl(B X K^T)                                  (strictly lower part)
  L_gamma = sl(B (H o X K^T))
  W       = (I + L)^{-1} B X           (triangular solve, UT transform, Eq. 27)
  U~      = (I + L_gamma)^{-1} B V
  Z       = U~ - D_gamma W S_in^T
  K_out   = diag(gamma_C / gamma_1, ..., gamma_C / gamma_C) K
  S_out   = gamma_C S_in + Z^T K_out
  O       = D_gamma Q S_in^T + (H o Q K^T) Z

The section itself flags three misprints in the paper's v1 formulas (K X^T vs
X K^T in App. D.2, S vs S^T in Eq. 26, and the missing gamma_r/gamma_i decay in
Eq. 26); the unified Z/H form above is the notes' corrected statement and is what
is written here.  A short last chunk (T not a multiple of C) is simply a chunk
of fewer rows.

Library primitives used as single steps: matrix products and
``scipy.linalg.solve_triangular``.  Nothing here is blocked, fused or reordered
beyond the formulas above.  The recurrence in ``oracle.qdelta_fwd`` is the
definition; this module is checked against it, never the reverse.
"""
import numpy as np
from scipy.linalg import solve_triangular


def _chunk(Q, K, V, a, be, la, S_in):
    """One chunk.  Returns (O [c, dv], S_out [dv, dk])."""
    c = Q.shape[0]
    X = K + la[:, None] * Q                         # x_r = k_r + lambda_r q_r
    gamma = np.cumprod(a)                           # gamma_i = prod_{j<=i} alpha_j
    Hm = np.tril(gamma[:, None] / gamma[None, :])   # H_ij = gamma_i / gamma_j, j <= i
    Bm = np.diag(be)
    XK = X @ K.T                                    # (X K^T)_ri = k_i . x_r
    L = np.tril(Bm @ XK, -1)
    Lg = np.tril(Bm @ (Hm * XK), -1)
    I = np.eye(c)
    W = solve_triangular(I + L, Bm @ X, lower=True, unit_diagonal=True)
    U = solve_triangular(I + Lg, Bm @ V, lower=True, unit_diagonal=True)
    Z = U - np.diag(gamma) @ W @ S_in.T
    K_out = np.diag(gamma[-1] / gamma) @ K
    S_out = gamma[-1] * S_in + Z.T @ K_out
    O = np.diag(gamma) @ Q @ S_in.T + (Hm * (Q @ K.T)) @ Z
    return O, S_out


def chunk_fwd(q, k, v, alpha, beta, lam, S0, C: int):
    """Chunked forward over [B,T,H,*] inputs (same layout as ``oracle.qdelta_fwd``).
    alpha None means 1, lam None means 0, S0 None means zeros.
    Returns (o, S_T) as fp64 numpy arrays."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    alpha = np.ones((B, T, H)) if alpha is None else np.asarray(alpha, dtype=np.float64)
    lam = np.zeros((B, T, H)) if lam is None else np.asarray(lam, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    o = np.zeros((B, T, H, dv))
    S_T = np.zeros((B, H, dv, dk))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dv, dk)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
            for t0 in range(0, T, C):
                sl = slice(t0, min(t0 + C, T))
                O, S = _chunk(q[b, sl, h], k[b, sl, h], v[b, sl, h], alpha[b, sl, h],
                              beta[b, sl, h], lam[b, sl, h], S)
                o[b, sl, h] = O
            S_T[b, h] = S
    return o, S_T
