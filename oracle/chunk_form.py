"""fp64 chunkwise (UT/WY) rewrite of the gated delta-rule loop.  Test infrastructure only.

The pages give the token recurrence ("Linear Attention Architectures" notes,
sections 2.3-2.5, Eqs. 9-10, 15-17, 18-20) and only name a chunked kernel with a
triangular inverse (NextTransformer "method sources" page, backend and numerics
section).  The chunk algebra below is derived from the recurrence; in exact
arithmetic it equals the token loop, and the tests check that in fp64.

For one chunk of tokens r = 0..C-1 with entry state S_n (d_v x d_k):

  Gam_r        = D_0 D_1 ... D_r                 cumulative decay inside the chunk
  R(r, j)      = D_{j+1} ... D_r  (j <= r)       decay between two tokens
  A[r, j]      = beta_r k_r^T R(r, j) k_j        for j < r, else 0
  Tm           = (I + A)^{-1} diag(beta)         unit-lower-triangular solve
  W            = Tm (K Gam),   Ut = Tm V         rows of K Gam are Gam_r k_r
  U            = Ut - W S_n^T                    rows u_r = beta_r (v_r - S_{r-1} D_r k_r)
  P[r, j]      = q_r^T R(r, j) k_j               for j <= r, else 0
  O            = (Q Gam) S_n^T + P U
  S_{n+1}      = S_n Gam_{C-1} + sum_r u_r k_r^T R(C-1, r)

Derivation: unrolling the loop inside the chunk gives
S_r = S_n Gam_r + sum_{j<=r} u_j k_j^T R(r, j); substituting it into
u_r = beta_r (v_r - S_{r-1} D_r k_r) gives (I + A) U = diag(beta) (V - (K Gam) S_n^T),
and o_r = S_r q_r gives the two terms of O.

All decay ratios are formed as explicit products of the per-token gates (no
division, no logarithm), so gates equal to 0 or 1 are handled exactly.
"""
from __future__ import annotations

import numpy as np

MODE_NONE, MODE_SCALAR, MODE_CHANNEL = 0, 1, 2


def _decay_vectors(alpha_c, mode, C, dk):
    """Per-token diagonal of D_r as a (C, dk) array."""
    if mode == MODE_NONE:
        return np.ones((C, dk))
    if mode == MODE_SCALAR:
        return np.repeat(np.asarray(alpha_c, dtype=np.float64)[:, None], dk, axis=1)
    return np.asarray(alpha_c, dtype=np.float64)


def _ratio(dec, r, j):
    """R(r, j) = D_{j+1} ... D_r as a vector (empty product = ones)."""
    out = np.ones(dec.shape[1])
    for i in range(j + 1, r + 1):
        out = out * dec[i]
    return out


def chunk_step(S, Q, K, V, beta_c, alpha_c, mode):
    """One chunk: returns (O (C, dv), S_next (dv, dk)).  All fp64."""
    C, dk = K.shape
    dec = _decay_vectors(alpha_c, mode, C, dk)
    gam = np.stack([_ratio(dec, r, -1) for r in range(C)])         # Gam_r, (C, dk)
    A = np.zeros((C, C))
    P = np.zeros((C, C))
    for r in range(C):
        for j in range(r + 1):
            rr = _ratio(dec, r, j)
            if j < r:
                A[r, j] = beta_c[r] * np.dot(K[r] * rr, K[j])
            P[r, j] = np.dot(Q[r] * rr, K[j])
    Tm = np.linalg.solve(np.eye(C) + A, np.diag(beta_c))
    W = Tm @ (K * gam)
    Ut = Tm @ V
    U = Ut - W @ S.T
    O = (Q * gam) @ S.T + P @ U
    Ktail = np.stack([K[r] * _ratio(dec, C - 1, r) for r in range(C)])
    S_next = S * gam[C - 1][None, :] + U.T @ Ktail
    return O, S_next


def gdn_fwd(q, k, v, alpha, beta, S0=None, mode=MODE_SCALAR, chunk=64):
    """Chunked prefill, same layouts and meaning as ``oracle.gdn_fwd``."""
    q, k, v, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    alpha = None if mode == MODE_NONE else np.asarray(alpha, dtype=np.float64)
    o = np.zeros((B, T, H, dv))
    S_final = np.zeros((B, H, dv, dk))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dv, dk)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
            for n0 in range(0, T, chunk):
                sl = slice(n0, min(n0 + chunk, T))
                a_c = None if alpha is None else alpha[b, sl, h]
                O, S = chunk_step(S, q[b, sl, h], k[b, sl, h], v[b, sl, h],
                                  beta[b, sl, h], a_c, mode)
                o[b, sl, h] = O
            S_final[b, h] = S
    return o, S_final
