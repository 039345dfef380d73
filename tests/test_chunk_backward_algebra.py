"""The chunk-level reverse mode that the bf16 backward kernels implement
(gdn_bwd_chunk.hip), written out in fp64 NumPy from its equations and checked
against the reference gradients (oracle/backward.py, itself pinned to finite
differences of the C loop).  This pins the algebra, not the kernels: the GPU
parity tests cover those.

Per chunk (G the running sum of log alpha inside it, E[r][s] = exp(G_r - G_s),
K~ = diag(exp(G_C - G)) K, dS the gradient at the chunk's end):
  dU = P^T dO + K~ dS^T,   dX = T^T dU = dV,   dS_n = gamma_C dS + dO^T Gamma Q - dX^T Gamma K
  dT = dU X^T,  N1 = M^T dT,  dA = -tril_-1(N1 T^T),  dP = tril_0(dO U^T)
  dbeta = diag(N1) + rows(dA o E o K K^T)
  dQ = (dP o E) K + Gamma dO S
  dK = (W + W^T) K + (dP o E)^T Q - Gamma dX S + diag(exp(G_C - G)) U dS,  W = diag(beta)(dA o E)
  dG = rows(Z) - cols(Z) + rows(Y) - cols(Y) + rows(Q o Gamma dO S) - rows(K o Gamma dX S)
       - rows(K~ o U dS),  Z = dA o A,  Y = dP o P;  dG_C += <dS, S_{n+1}>
  dlog alpha_t = sum_{r >= t} dG_r inside the chunk
"""
import numpy as np
import pytest

from oracle import backward as OB


def _chunk_states(q, k, v, la, beta, S0, C):
    T = q.shape[0]
    S, states = S0.copy(), []
    for t0 in range(0, T, C):
        states.append(S.copy())
        sl = slice(t0, min(T, t0 + C))
        K, V, b, G = k[sl], v[sl], beta[sl], np.cumsum(la[sl])
        E = np.exp(G[:, None] - G[None, :])
        M = np.linalg.inv(np.eye(len(b)) + np.tril(b[:, None] * E * (K @ K.T), -1))
        U = (M * b[None, :]) @ (V - np.exp(G)[:, None] * (K @ S.T))
        S = np.exp(G[-1]) * S + U.T @ (np.exp(G[-1] - G)[:, None] * K)
    states.append(S)
    return states


def _chunk_backward(q, k, v, la, beta, S0, do, dSf, C):
    """Gradients of one head by the chunk-level reverse mode (fp64)."""
    T = q.shape[0]
    st = _chunk_states(q, k, v, la, beta, S0, C)
    g = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
             dbeta=np.zeros(T), dla=np.zeros(T))
    dS = dSf.copy()
    for n in reversed(range(len(st) - 1)):
        sl = slice(n * C, min(T, n * C + C))
        K, Q, V, b, dO = k[sl], q[sl], v[sl], beta[sl], do[sl]
        S, Sn, G = st[n], st[n + 1], np.cumsum(la[sl])
        gam, E = np.exp(G), np.exp(G[:, None] - G[None, :])
        KK = K @ K.T
        A = np.tril(b[:, None] * E * KK, -1)
        M = np.linalg.inv(np.eye(len(b)) + A)
        Tm = M * b[None, :]
        X = V - gam[:, None] * (K @ S.T)
        U = Tm @ X
        Kt = np.exp(G[-1] - G)[:, None] * K
        P = np.tril(E * (Q @ K.T))
        dU = P.T @ dO + Kt @ dS.T
        dX = Tm.T @ dU
        N1 = M.T @ (dU @ X.T)
        dA = -np.tril(N1 @ Tm.T, -1)
        dP = np.tril(dO @ U.T)
        W = b[:, None] * dA * E
        dPE = dP * E
        dQi, P1, P2 = gam[:, None] * (dO @ S), gam[:, None] * (dX @ S), np.exp(G[-1] - G)[:, None] * (U @ dS)
        g['dq'][sl] = dPE @ K + dQi
        g['dk'][sl] = (W + W.T) @ K + dPE.T @ Q - P1 + P2
        g['dv'][sl] = dX
        g['dbeta'][sl] = np.diag(N1) + np.sum(dA * E * KK, 1)
        Z, Y = dA * A, dP * P
        dG = Z.sum(1) - Z.sum(0) + Y.sum(1) - Y.sum(0)
        dG += np.sum(Q * dQi, 1) - np.sum(K * P1, 1) - np.sum(K * P2, 1)
        dG[-1] += np.sum(dS * Sn)
        g['dla'][sl] = np.cumsum(dG[::-1])[::-1]
        dS = np.exp(G[-1]) * dS + dO.T @ (gam[:, None] * Q) - dX.T @ (gam[:, None] * K)
    g['dS0'] = dS
    return g


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("T,C", [(1, 64), (37, 16), (64, 64), (130, 64), (200, 16)])
def test_chunk_reverse_mode_matches_reference(mode, T, C):
    rng = np.random.default_rng(1000 * mode + T + C)
    dk, dv = 24, 16
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    beta[::5] = 0.0   # tokens that write nothing (diag(beta) singular)
    alpha = np.exp(-0.3 * np.log1p(np.exp(rng.standard_normal(T)))) if mode else np.ones(T)
    S0 = 0.2 * rng.standard_normal((dv, dk))
    do = rng.standard_normal((T, dv))
    dSf = 0.5 * rng.standard_normal((dv, dk))
    ref = OB.gdn_bwd(q[None, :, None], k[None, :, None], v[None, :, None],
                     alpha[None, :, None] if mode else None, beta[None, :, None], S0[None, None],
                     do[None, :, None], dSf[None, None], mode=mode)
    got = _chunk_backward(q, k, v, np.log(alpha), beta, S0, do, dSf, C)
    for name in ("dq", "dk", "dv", "dbeta", "dS0"):
        r = ref[name].reshape(got[name].shape)
        assert np.abs(got[name] - r).max() <= 1e-10 * max(1.0, np.abs(r).max()), name
    if mode:
        r = ref["dalpha"].reshape(T)
        assert np.abs(got["dla"] / alpha - r).max() <= 1e-10 * max(1.0, np.abs(r).max())
