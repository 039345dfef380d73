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

Gated DeltaNet-2 (mode 3; "Linear Attention Architectures" notes, section 2.6)
changes two things: the prediction reads the erase direction e_r = b_r * k_r
and the target is z_r = w_r * v_r, with no beta.  The same unrolling gives
(I + A) U = Z - (E Gam) S_n^T with A[r, j] = e_r^T R(r, j) k_j, so Tm = (I + A)^{-1},
W = Tm (E Gam), Ut = Tm Z; the output and the state update keep k.
"""
from __future__ import annotations

import numpy as np

MODE_NONE, MODE_SCALAR, MODE_CHANNEL, MODE_GDN2 = 0, 1, 2, 3


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


def chunk_step(S, Q, K, V, beta_c, alpha_c, mode, erase_c=None, write_c=None):
    """One chunk: returns (O (C, dv), S_next (dv, dk)).  All fp64."""
    C, dk = K.shape
    dec = _decay_vectors(alpha_c, MODE_CHANNEL if mode == MODE_GDN2 else mode, C, dk)
    gdn2 = mode == MODE_GDN2
    Er = K * erase_c if gdn2 else K * np.asarray(beta_c)[:, None]   # row side of A
    gam = np.stack([_ratio(dec, r, -1) for r in range(C)])         # Gam_r, (C, dk)
    A = np.zeros((C, C))
    P = np.zeros((C, C))
    for r in range(C):
        for j in range(r + 1):
            rr = _ratio(dec, r, j)
            if j < r:
                A[r, j] = np.dot(Er[r] * rr, K[j])
            P[r, j] = np.dot(Q[r] * rr, K[j])
    if gdn2:
        Tm = np.linalg.solve(np.eye(C) + A, np.eye(C))
        W = Tm @ (Er * gam)
        Ut = Tm @ (V * write_c)
    else:
        Tm = np.linalg.solve(np.eye(C) + A, np.diag(beta_c))
        W = Tm @ (K * gam)
        Ut = Tm @ V
    U = Ut - W @ S.T
    O = (Q * gam) @ S.T + P @ U
    Ktail = np.stack([K[r] * _ratio(dec, C - 1, r) for r in range(C)])
    S_next = S * gam[C - 1][None, :] + U.T @ Ktail
    return O, S_next


def gdn_fwd(q, k, v, alpha, beta, S0=None, mode=MODE_SCALAR, chunk=64, erase=None, write=None):
    """Chunked prefill, same layouts and meaning as ``oracle.gdn_fwd``."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    beta = None if beta is None else np.asarray(beta, dtype=np.float64)
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
                b_c = None if beta is None else beta[b, sl, h]
                e_c = None if erase is None else np.asarray(erase[b, sl, h], dtype=np.float64)
                w_c = None if write is None else np.asarray(write[b, sl, h], dtype=np.float64)
                O, S = chunk_step(S, q[b, sl, h], k[b, sl, h], v[b, sl, h], b_c, a_c, mode, e_c, w_c)
                o[b, sl, h] = O
            S_final[b, h] = S
    return o, S_final
