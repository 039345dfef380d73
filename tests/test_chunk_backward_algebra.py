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


# ---------------------------------------------------------------------------
# Per-channel decay (G the running sum of log alpha per key channel inside the
# chunk, a [C, d_k] array; E3[r][s][c] = exp(G[r][c] - G[s][c]) <= 1 for s <= r).
# The forward's operands are K (.) Gamma, Q (.) Gamma and K (.) exp(G_C - G),
# gamma_C = exp(G_C) per channel, and the two C x C matrices contract the
# channels with the weights E3:
#   A = tril_-1(diag(beta) At),  At[r][s] = sum_c k_r[c] k_s[c] E3[r][s][c]
#   P = tril_0(Pt),              Pt[r][s] = sum_c q_r[c] k_s[c] E3[r][s][c]
# Reverse mode: dU, dX, dT, N1, dA, dP as above, then with W = diag(beta) dA
#   R_Pq[r] = sum_s dP[r][s] k_s (.) E3[r][s]     R_Pk[s] = sum_r dP[r][s] q_r (.) E3[r][s]
#   R_Ar[r] = sum_s W[r][s] k_s (.) E3[r][s]      R_Ac[s] = sum_r W[r][s] k_r (.) E3[r][s]
#   dq = R_Pq + Gamma (.) dO S
#   dk = R_Pk + R_Ar + R_Ac - Gamma (.) dX S + exp(G_C - G) (.) U dS
#   dbeta = diag(N1) + rows(dA o At)
#   dG = q (.) R_Pq - k (.) R_Pk + k (.) R_Ar - k (.) R_Ac
#        + (Q (.) Gamma) (.) dO S - (K (.) Gamma) (.) dX S - (K (.) exp(G_C - G)) (.) U dS,
#   dG[last] += sum_i dS[i] (.) S_{n+1}[i]   (per channel)
#   dS_n = dS diag(gamma_C) + dO^T (Q (.) Gamma) - dX^T (K (.) Gamma)
# ---------------------------------------------------------------------------

def _kda_chunk(Q, K, V, la, b, S):
    """One chunk's forward quantities (fp64), per-channel decay."""
    G = np.cumsum(la, 0)
    gam, gC = np.exp(G), np.exp(G[-1])
    E3 = np.exp(G[:, None, :] - G[None, :, :])          # [r][s][c]
    mask = np.tril(np.ones((len(b), len(b))), 0)[:, :, None]
    E3 = np.where(mask > 0, E3, 0.0)                     # only s <= r is ever used
    At = np.einsum("rc,sc,rsc->rs", K, K, E3)
    Pt = np.einsum("rc,sc,rsc->rs", Q, K, E3)
    A = np.tril(b[:, None] * At, -1)
    M = np.linalg.inv(np.eye(len(b)) + A)
    Tm = M * b[None, :]
    Kg, Qg, Kc = K * gam, Q * gam, K * np.exp(G[-1] - G)
    X = V - Kg @ S.T
    U = Tm @ X
    Sn = S * gC[None, :] + U.T @ Kc
    return dict(G=G, gam=gam, gC=gC, E3=E3, At=At, P=np.tril(Pt), M=M, Tm=Tm, Kg=Kg, Qg=Qg, Kc=Kc, X=X, U=U,
                Sn=Sn)


def _kda_chunk_backward(q, k, v, la, beta, S0, do, dSf, C):
    T = q.shape[0]
    states, S = [], S0.copy()
    for t0 in range(0, T, C):
        sl = slice(t0, min(T, t0 + C))
        states.append(S.copy())
        S = _kda_chunk(q[sl], k[sl], v[sl], la[sl], beta[sl], S)["Sn"]
    g = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v), dbeta=np.zeros(T),
             dla=np.zeros_like(la))
    dS = dSf.copy()
    for n in reversed(range(len(states))):
        sl = slice(n * C, min(T, n * C + C))
        Q, K, b, dO, S = q[sl], k[sl], beta[sl], do[sl], states[n]
        f = _kda_chunk(Q, K, v[sl], la[sl], b, S)
        E3 = f["E3"]
        dU = f["P"].T @ dO + f["Kc"] @ dS.T
        dX = f["Tm"].T @ dU
        N1 = f["M"].T @ (dU @ f["X"].T)
        dA = -np.tril(N1 @ f["Tm"].T, -1)
        dP = np.tril(dO @ f["U"].T)
        W = b[:, None] * dA
        R_Pq = np.einsum("rs,sc,rsc->rc", dP, K, E3)
        R_Pk = np.einsum("rs,rc,rsc->sc", dP, Q, E3)
        R_Ar = np.einsum("rs,sc,rsc->rc", W, K, E3)
        R_Ac = np.einsum("rs,rc,rsc->sc", W, K, E3)
        dQg, dKg, dKc = dO @ S, -(dX @ S), f["U"] @ dS
        g["dq"][sl] = R_Pq + f["gam"] * dQg
        g["dk"][sl] = R_Pk + R_Ar + R_Ac + f["gam"] * dKg + np.exp(f["G"][-1] - f["G"]) * dKc
        g["dv"][sl] = dX
        g["dbeta"][sl] = np.diag(N1) + np.sum(dA * f["At"], 1)
        dG = Q * R_Pq - K * R_Pk + K * R_Ar - K * R_Ac + f["Qg"] * dQg + f["Kg"] * dKg - f["Kc"] * dKc
        dG[-1] += np.sum(dS * f["Sn"], 0)
        g["dla"][sl] = np.cumsum(dG[::-1], 0)[::-1]
        dS = dS * f["gC"][None, :] + dO.T @ f["Qg"] - dX.T @ f["Kg"]
    g["dS0"] = dS
    return g


@pytest.mark.parametrize("T,C", [(1, 64), (37, 16), (64, 64), (130, 64), (200, 16)])
def test_chunk_reverse_mode_matches_reference_per_channel(T, C):
    rng = np.random.default_rng(7000 + T + C)
    dk, dv = 24, 16
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    beta[::5] = 0.0
    alpha = np.exp(-0.3 * np.log1p(np.exp(rng.standard_normal((T, dk)))))
    alpha[3::7, ::3] = np.exp(-6.0)   # strong single-channel decay
    S0 = 0.2 * rng.standard_normal((dv, dk))
    do = rng.standard_normal((T, dv))
    dSf = 0.5 * rng.standard_normal((dv, dk))
    ref = OB.gdn_bwd(q[None, :, None], k[None, :, None], v[None, :, None], alpha[None, :, None],
                     beta[None, :, None], S0[None, None], do[None, :, None], dSf[None, None], mode=2)
    got = _kda_chunk_backward(q, k, v, np.log(alpha), beta, S0, do, dSf, C)
    for name in ("dq", "dk", "dv", "dbeta", "dS0"):
        r = ref[name].reshape(got[name].shape)
        assert np.abs(got[name] - r).max() <= 1e-10 * max(1.0, np.abs(r).max()), name
    r = ref["dalpha"].reshape(T, dk)
    assert np.abs(got["dla"] / alpha - r).max() <= 1e-10 * max(1.0, np.abs(r).max())
