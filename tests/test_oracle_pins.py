"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these checks re-types the oracle's loop: each one compares it with a
value printed on the pages, a closed form, an exact rational evaluation of a
different formulation (the history-unrolled matrix product), an autograd
gradient step, or an invariant.  ``test_planted_mistakes_are_caught`` compiles
copies of the oracle with one plausible mistake each and checks that some pin
fails for every one of them.

Pages cited:
  LAA  = "Linear Attention Architectures: Mechanisms, Trade-offs, and Cross-Layer
         Routing" reading notes
  RLA  = "Enhancing Linear Attention with Residual Learning" reading notes
  SR   = "On State Reduction in Linear Attention" reading notes
  NT   = NextTransformer "method sources and implementation" page
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import MODE_CHANNEL, MODE_NONE, MODE_SCALAR, chunk_form

HERE = os.path.dirname(os.path.abspath(__file__))
MODES = [MODE_NONE, MODE_SCALAR, MODE_CHANNEL]


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _inputs(rng, B, T, H, dk, dv, mode, s0=True, lo=0.5):
    q = _unit(rng.standard_normal((B, T, H, dk)))
    k = _unit(rng.standard_normal((B, T, H, dk)))
    v = rng.standard_normal((B, T, H, dv))
    beta = rng.uniform(0.05, 0.95, (B, T, H))
    if mode == MODE_SCALAR:
        alpha = rng.uniform(lo, 1.0, (B, T, H))
    elif mode == MODE_CHANNEL:
        alpha = rng.uniform(lo, 1.0, (B, T, H, dk))
    else:
        alpha = None
    S0 = rng.standard_normal((B, H, dv, dk)) * 0.3 if s0 else None
    return q, k, v, alpha, beta, S0


def _decay_diag(alpha_t, mode, dk):
    if mode == MODE_NONE:
        return np.ones(dk)
    if mode == MODE_SCALAR:
        return np.full(dk, float(alpha_t))
    return np.asarray(alpha_t, dtype=np.float64)


def _rel(x, ref):
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(x - ref)) / (den if den > 0 else 1.0))


# ----------------------------------------------------------------------------------
# individual pins; each takes an oracle build so the mutation test can reuse them
# ----------------------------------------------------------------------------------

def _golden_worked_example():
    vals = {}
    with open(os.path.join(HERE, "golden", "delta_write_worked_example.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                key, val = line.split()
                vals[key] = float(val)
    return vals


def pin_worked_example(orc):
    """LAA section 2.3: unit key, prediction 2, target 5, beta 0.5 -> 3.5; and
    W_new k = (1 - beta) W_old k + beta v for a unit key."""
    g = _golden_worked_example()
    rng = np.random.default_rng(11)
    dk = 6
    kk = _unit(rng.standard_normal(dk))
    for mode in MODES:
        S0 = (g["prediction"] * kk)[None, :]                       # S0 k = prediction
        q = kk[None, None, None, :]
        k = kk[None, None, None, :]
        v = np.array([[[[g["target"]]]]])
        beta = np.array([[[g["beta"]]]])
        alpha = None if mode == MODE_NONE else (
            np.ones((1, 1, 1)) if mode == MODE_SCALAR else np.ones((1, 1, 1, dk)))
        o, S = orc.gdn_fwd(q, k, v, alpha, beta, S0[None, None], mode=mode)
        assert abs(o[0, 0, 0, 0] - g["new_prediction"]) < 1e-13
        assert abs((S[0, 0] @ kk)[0] - g["new_prediction"]) < 1e-13
    # general statement with a random memory (several value rows) and a random beta
    dv = 4
    S0 = rng.standard_normal((1, 1, dv, dk))
    v = rng.standard_normal((1, 1, 1, dv))
    b = 0.37
    _, S = orc.gdn_fwd(kk[None, None, None], kk[None, None, None], v, None,
                       np.array([[[b]]]), S0, mode=MODE_NONE)
    want = (1 - b) * (S0[0, 0] @ kk) + b * v[0, 0, 0]
    assert np.max(np.abs(S[0, 0] @ kk - want)) < 1e-13


def pin_exact_recall(orc):
    """LAA section 2.3: with a unit key and beta = 1 the write makes S_t k_t = v_t,
    whatever the decay and the earlier state.  Read back with q_t = k_t."""
    rng = np.random.default_rng(12)
    B, T, H, dk, dv = 2, 9, 2, 5, 3
    for mode in MODES:
        q, k, v, alpha, beta, S0 = _inputs(rng, B, T, H, dk, dv, mode)
        beta = np.ones_like(beta)
        o, _ = orc.gdn_fwd(k, k, v, alpha, beta, S0, mode=mode)
        assert np.max(np.abs(o - v)) < 1e-12


def pin_orthonormal_closed_form(orc):
    """SR section 2.1 / 2.2: with orthonormal keys, S0 = 0 and scalar decay the
    erase term vanishes (S_{t-1} k_t = 0 since the rows of S_{t-1} lie in the span
    of the earlier keys), so S_T = sum_t beta_t (prod_{i>t} alpha_i) v_t k_t^T and
    o_t = sum_{j<=t} beta_j (prod_{j<i<=t} alpha_i) v_j (k_j . q_t)."""
    rng = np.random.default_rng(13)
    dk, dv, T = 8, 5, 7
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm.T[:T]                                  # T orthonormal rows
    q = _unit(rng.standard_normal((T, dk)))
    v = rng.standard_normal((T, dv))
    beta = rng.uniform(0.1, 1.0, T)
    for mode in (MODE_NONE, MODE_SCALAR):
        a = np.ones(T) if mode == MODE_NONE else rng.uniform(0.3, 1.0, T)
        alpha = None if mode == MODE_NONE else a[None, :, None]
        o, S = orc.gdn_fwd(q[None, :, None], keys[None, :, None], v[None, :, None], alpha,
                           beta[None, :, None], None, mode=mode)
        S_want = sum(beta[t] * np.prod(a[t + 1:]) * np.outer(v[t], keys[t]) for t in range(T))
        assert _rel(S[0, 0], S_want) < 1e-13
        for t in range(T):
            o_want = sum(beta[j] * np.prod(a[j + 1:t + 1]) * v[j] * (keys[j] @ q[t])
                         for j in range(t + 1))
            assert np.max(np.abs(o[0, t, 0] - o_want)) < 1e-13
        if mode == MODE_NONE:  # beta = 1 recalls every stored value exactly
            _, S1 = orc.gdn_fwd(q[None, :, None], keys[None, :, None], v[None, :, None], None,
                                np.ones((1, T, 1)), None, mode=mode)
            assert np.max(np.abs(S1[0, 0] @ keys.T - v.T)) < 1e-13


def pin_kda_axis_keys_closed_form(orc):
    """LAA section 2.5 (Eqs. 18-20): KDA decays key channels, Diag(alpha) on the
    right of S.  With keys equal to distinct basis vectors e_{c_t} and S0 = 0, the
    decayed state never overlaps the new key, so column c_t of S_T equals
    beta_t v_t prod_{i>t} alpha_i[c_t] and o_t = sum_{j<=t} beta_j v_j
    prod_{j<i<=t} alpha_i[c_j] q_t[c_j]."""
    rng = np.random.default_rng(14)
    dk, dv, T = 9, 4, 6
    cols = rng.permutation(dk)[:T]
    keys = np.zeros((T, dk))
    keys[np.arange(T), cols] = 1.0
    q = _unit(rng.standard_normal((T, dk)))
    v = rng.standard_normal((T, dv))
    beta = rng.uniform(0.1, 1.0, T)
    a = rng.uniform(0.2, 1.0, (T, dk))
    o, S = orc.gdn_fwd(q[None, :, None], keys[None, :, None], v[None, :, None], a[None, :, None],
                       beta[None, :, None], None, mode=MODE_CHANNEL)
    S_want = np.zeros((dv, dk))
    for t in range(T):
        S_want[:, cols[t]] = beta[t] * v[t] * np.prod(a[t + 1:, cols[t]])
    assert _rel(S[0, 0], S_want) < 1e-13
    for t in range(T):
        o_want = sum(beta[j] * v[j] * np.prod(a[j + 1:t + 1, cols[j]]) * q[t, cols[j]]
                     for j in range(t + 1))
        assert np.max(np.abs(o[0, t, 0] - o_want)) < 1e-13


def pin_no_write(orc):
    """beta = 0 writes nothing: S_t = S0 D_1 ... D_t (alpha = 1 leaves S unchanged)
    and o_t = S_t q_t (LAA section 2.1, Eq. 8: the query reads the state)."""
    rng = np.random.default_rng(15)
    B, T, H, dk, dv = 1, 6, 2, 4, 3
    for mode in MODES:
        q, k, v, alpha, beta, S0 = _inputs(rng, B, T, H, dk, dv, mode)
        beta = np.zeros_like(beta)
        o, S = orc.gdn_fwd(q, k, v, alpha, beta, S0, mode=mode)
        for h in range(H):
            St = S0[0, h].copy()
            for t in range(T):
                a = None if alpha is None else alpha[0, t, h]
                St = St * _decay_diag(a, mode, dk)[None, :]
                assert np.max(np.abs(o[0, t, h] - St @ q[0, t, h])) < 1e-13
            assert np.max(np.abs(S[0, h] - St)) < 1e-13
        if mode != MODE_NONE:  # alpha = 1 and beta = 0: the state is returned unchanged
            one = np.ones_like(alpha)
            _, S1 = orc.gdn_fwd(q, k, v, one, beta, S0, mode=mode)
            assert np.array_equal(S1, S0)


def _exact_product_form(q, k, v, alpha, beta, S0, mode):
    """History-unrolled product S_t = S_{t-1} D_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    o_t = S_t q_t, in exact rational arithmetic (LAA Eqs. 14, 17, 20 expanded; NT's
    history-unrolled reference).  Inputs are lists of Fractions for one head."""
    T, dk, dv = len(q), len(q[0]), len(v[0])
    S = [row[:] for row in S0]
    outs = []
    for t in range(T):
        if mode == MODE_NONE:
            d = [Fraction(1)] * dk
        elif mode == MODE_SCALAR:
            d = [alpha[t]] * dk
        else:
            d = list(alpha[t])
        M = [[d[i] * ((1 if i == j else 0) - beta[t] * k[t][i] * k[t][j]) for j in range(dk)]
             for i in range(dk)]                                      # D_t (I - b k k^T)
        S = [[sum(S[r][i] * M[i][c] for i in range(dk)) + beta[t] * v[t][r] * k[t][c]
              for c in range(dk)] for r in range(dv)]
        outs.append([sum(S[r][c] * q[t][c] for c in range(dk)) for r in range(dv)])
    return outs, S


def pin_exact_rational(orc):
    """Exact rational evaluation of the product form on tiny dyadic inputs (exactly
    representable in fp64), including d_k != d_v both ways, against the oracle."""
    rng = np.random.default_rng(16)
    for mode in MODES:
        for dk, dv in ((3, 2), (2, 3)):
            T = 5
            dy = lambda *s: rng.integers(-8, 9, s) / 8.0
            q, k, v, S0 = dy(T, dk), dy(T, dk), dy(T, dv), dy(dv, dk)
            beta = rng.integers(0, 9, T) / 8.0
            alpha = (rng.integers(1, 9, T) / 8.0 if mode == MODE_SCALAR else
                     rng.integers(1, 9, (T, dk)) / 8.0 if mode == MODE_CHANNEL else None)
            Fr = lambda a: [[Fraction(x) for x in row] for row in np.atleast_2d(a)]
            oq, Sq = _exact_product_form(
                Fr(q), Fr(k), Fr(v),
                None if alpha is None else (Fr(alpha) if mode == MODE_CHANNEL else
                                            [Fraction(x) for x in alpha]),
                [Fraction(x) for x in beta], Fr(S0), mode)
            a_in = None if alpha is None else (alpha[None, :, None] if mode == MODE_SCALAR
                                               else alpha[None, :, None, :])
            o, S = orc.gdn_fwd(q[None, :, None], k[None, :, None], v[None, :, None], a_in,
                               beta[None, :, None], S0[None, None], mode=mode)
            o_ex = np.array([[float(x) for x in row] for row in oq])
            S_ex = np.array([[float(x) for x in row] for row in Sq])
            assert np.max(np.abs(o[0, :, 0] - o_ex)) <= 1e-12 * max(1.0, np.max(np.abs(o_ex)))
            assert np.max(np.abs(S[0, 0] - S_ex)) <= 1e-12 * max(1.0, np.max(np.abs(S_ex)))


def pin_gradient_step(orc):
    """RLA section 1.1 / SR section 2.1: the delta rule is one gradient step of
    0.5 ||S k - v||^2 with step beta, taken from the decayed state S' = S_{t-1} D_t
    (LAA Eqs. 15-17: decay first).  The gradient comes from torch autograd."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(17)
    T, dk, dv = 6, 5, 4
    for mode in MODES:
        q, k, v, alpha, beta, S0 = _inputs(rng, 1, T, 1, dk, dv, mode)
        o, S = orc.gdn_fwd(q, k, v, alpha, beta, S0, mode=mode)
        St = torch.tensor(S0[0, 0], dtype=torch.float64)
        for t in range(T):
            a = None if alpha is None else alpha[0, t, 0]
            Sp = (St * torch.tensor(_decay_diag(a, mode, dk))[None, :]).detach().requires_grad_(True)
            kt = torch.tensor(k[0, t, 0])
            vt = torch.tensor(v[0, t, 0])
            loss = 0.5 * torch.sum((Sp @ kt - vt) ** 2)
            (g,) = torch.autograd.grad(loss, Sp)
            St = (Sp - float(beta[0, t, 0]) * g).detach()
            o_t = (St @ torch.tensor(q[0, t, 0])).numpy()
            assert np.max(np.abs(o[0, t, 0] - o_t)) < 1e-12
        assert np.max(np.abs(S[0, 0] - St.numpy())) < 1e-12


def pin_orthogonal_invariance(orc):
    """SR section 2.5 (Eq. 8, Prop. 3.1): k' = T k, q' = T q, S' = S T^T with T
    orthogonal leaves every output unchanged and maps S_T to S_T T^T; scalar decay
    keeps this.  For per-channel decay only channel permutations (alpha permuted
    alike) commute with Diag(alpha)."""
    rng = np.random.default_rng(18)
    B, T, H, dk, dv = 1, 11, 2, 6, 4
    for mode in MODES:
        q, k, v, alpha, beta, S0 = _inputs(rng, B, T, H, dk, dv, mode)
        if mode == MODE_CHANNEL:
            Tm = np.eye(dk)[rng.permutation(dk)]
        else:
            Tm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
        o, S = orc.gdn_fwd(q, k, v, alpha, beta, S0, mode=mode)
        a2 = alpha if mode != MODE_CHANNEL else alpha @ Tm.T
        o2, S2 = orc.gdn_fwd(q @ Tm.T, k @ Tm.T, v, a2, beta, S0 @ Tm.T, mode=mode)
        assert _rel(o2, o) < 1e-12
        assert _rel(S2, S @ Tm.T) < 1e-12


def pin_rank_bound(orc):
    """SR section 2.2 (Eq. 3): from S0 = 0, rank S_T <= min(rank K_T, rank V_T) <= T."""
    rng = np.random.default_rng(19)
    dk = dv = 10
    for mode in MODES:
        for T in (1, 3, 6):
            q, k, v, alpha, beta, _ = _inputs(rng, 1, T, 1, dk, dv, mode)
            _, S = orc.gdn_fwd(q, k, v, alpha, beta, None, mode=mode)
            assert np.linalg.matrix_rank(S[0, 0], tol=1e-10) <= T
        # values of rank 2 over 6 tokens
        T = 6
        q, k, v, alpha, beta, _ = _inputs(rng, 1, T, 1, dk, dv, mode)
        basis = rng.standard_normal((2, dv))
        v = (rng.standard_normal((T, 2)) @ basis)[None, :, None]
        _, S = orc.gdn_fwd(q, k, v, alpha, beta, None, mode=mode)
        assert np.linalg.matrix_rank(S[0, 0], tol=1e-10) <= 2


def pin_value_channel_independence(orc):
    """SR section 2.5: each value channel (row of S) is its own linear system sharing
    the key-side transition, so rows I of S_T and channels I of o depend only on
    v[..., I] and rows I of S0."""
    rng = np.random.default_rng(20)
    B, T, H, dk, dv = 1, 13, 2, 5, 6
    I = [0, 2, 3]
    notI = [1, 4, 5]
    for mode in MODES:
        q, k, v, alpha, beta, S0 = _inputs(rng, B, T, H, dk, dv, mode)
        o, S = orc.gdn_fwd(q, k, v, alpha, beta, S0, mode=mode)
        v2, S02 = v.copy(), S0.copy()
        v2[..., notI] = rng.standard_normal(v2[..., notI].shape) * 5
        S02[:, :, notI] = rng.standard_normal(S02[:, :, notI].shape) * 5
        o2, S2 = orc.gdn_fwd(q, k, v2, alpha, beta, S02, mode=mode)
        assert np.max(np.abs(o2[..., I] - o[..., I])) < 1e-13
        assert np.max(np.abs(S2[:, :, I] - S[:, :, I])) < 1e-13
        assert np.max(np.abs(o2[..., notI] - o[..., notI])) > 1e-3


def pin_linearity(orc):
    """For fixed keys, queries and gates, (S0, V) -> (S_T, O) is linear (the state
    update is affine in S with the v-term linear: SR section 2.2)."""
    rng = np.random.default_rng(21)
    B, T, H, dk, dv = 1, 10, 1, 4, 3
    for mode in MODES:
        q, k, v, alpha, beta, S0 = _inputs(rng, B, T, H, dk, dv, mode)
        v2 = rng.standard_normal(v.shape)
        S02 = rng.standard_normal(S0.shape)
        c1, c2 = 0.7, -1.3
        o1, S1 = orc.gdn_fwd(q, k, v, alpha, beta, S0, mode=mode)
        o2, S2 = orc.gdn_fwd(q, k, v2, alpha, beta, S02, mode=mode)
        o3, S3 = orc.gdn_fwd(q, k, c1 * v + c2 * v2, alpha, beta, c1 * S0 + c2 * S02, mode=mode)
        assert _rel(o3, c1 * o1 + c2 * o2) < 1e-12
        assert _rel(S3, c1 * S1 + c2 * S2) < 1e-12


def pin_contraction(orc):
    """RLA section 2.4: for a unit key I - beta k k^T has eigenvalues 1 - beta and 1,
    so ||S_t||_2 <= max(alpha_t) ||S_{t-1}||_2 + beta_t ||v_t|| ||k_t||."""
    rng = np.random.default_rng(22)
    dk, dv, T = 6, 5, 12
    for mode in MODES:
        q, k, v, alpha, beta, S0 = _inputs(rng, 1, T, 1, dk, dv, mode)
        prev = np.linalg.norm(S0[0, 0], 2)
        S = S0
        for t in range(T):
            a = None if alpha is None else alpha[:, t:t + 1]
            _, S = orc.gdn_fwd(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], a,
                               beta[:, t:t + 1], S, mode=mode)
            amax = 1.0 if alpha is None else float(np.max(alpha[0, t]))
            bound = amax * prev + beta[0, t, 0] * np.linalg.norm(v[0, t, 0]) * np.linalg.norm(k[0, t, 0])
            now = np.linalg.norm(S[0, 0], 2)
            assert now <= bound * (1 + 1e-12)
            prev = now


def pin_mode_reductions(orc):
    """LAA section 2.5: alpha_t 1 turns KDA into GDN; GDN with alpha = 1 is DeltaNet."""
    rng = np.random.default_rng(23)
    B, T, H, dk, dv = 1, 9, 2, 4, 3
    q, k, v, a, beta, S0 = _inputs(rng, B, T, H, dk, dv, MODE_SCALAR)
    o_g, S_g = orc.gdn_fwd(q, k, v, a, beta, S0, mode=MODE_SCALAR)
    o_k, S_k = orc.gdn_fwd(q, k, v, np.repeat(a[..., None], dk, -1), beta, S0, mode=MODE_CHANNEL)
    assert np.array_equal(o_g, o_k) and np.array_equal(S_g, S_k)
    o_1, S_1 = orc.gdn_fwd(q, k, v, np.ones_like(a), beta, S0, mode=MODE_SCALAR)
    o_n, S_n = orc.gdn_fwd(q, k, v, None, beta, S0, mode=MODE_NONE)
    assert np.array_equal(o_1, o_n) and np.array_equal(S_1, S_n)


def pin_zero_gate_resets(orc):
    """alpha = 0 forgets everything: S_t = beta_t v_t k_t^T (LAA Eqs. 15-17 at the
    boundary value the gate range allows)."""
    rng = np.random.default_rng(24)
    B, T, H, dk, dv = 1, 4, 1, 5, 3
    for mode in (MODE_SCALAR, MODE_CHANNEL):
        q, k, v, alpha, beta, S0 = _inputs(rng, B, T, H, dk, dv, mode)
        alpha = np.zeros_like(alpha)
        o, S = orc.gdn_fwd(q, k, v, alpha, beta, S0, mode=mode)
        want = beta[0, -1, 0] * np.outer(v[0, -1, 0], k[0, -1, 0])
        assert np.max(np.abs(S[0, 0] - want)) < 1e-14


def pin_decode_matches_prefill(orc):
    """T decode steps equal one prefill over T tokens; a prefill split in two with
    the state handed over equals the whole prefill (the hand-off between calls)."""
    rng = np.random.default_rng(25)
    B, T, H, dk, dv = 2, 7, 3, 4, 5
    for mode in MODES:
        q, k, v, alpha, beta, S0 = _inputs(rng, B, T, H, dk, dv, mode)
        o, S = orc.gdn_fwd(q, k, v, alpha, beta, S0, mode=mode)
        St = S0
        for t in range(T):
            a = None if alpha is None else alpha[:, t]
            ot, St = orc.gdn_decode(q[:, t], k[:, t], v[:, t], a, beta[:, t], St, mode=mode)
            assert np.array_equal(ot, o[:, t])
        assert np.array_equal(St, S)
        t1 = 3
        sl = lambda x, s: None if x is None else x[:, s]
        oa, Sa = orc.gdn_fwd(q[:, :t1], k[:, :t1], v[:, :t1], sl(alpha, slice(0, t1)),
                             beta[:, :t1], S0, mode=mode)
        ob, Sb = orc.gdn_fwd(q[:, t1:], k[:, t1:], v[:, t1:], sl(alpha, slice(t1, None)),
                             beta[:, t1:], Sa, mode=mode)
        assert np.array_equal(np.concatenate([oa, ob], 1), o) and np.array_equal(Sb, S)


def pin_varlen_resets_at_sequence_starts(orc):
    """A packed batch (sequences back to back on one token axis) equals separate
    runs of the sequences, each from its own initial state: the state restarts
    at the first token of every sequence and nowhere else (NT, baseline section:
    the recurrent mixers reset their state at the start of each packed row).
    Covers empty sequences, lengths of one token, and a single sequence."""
    rng = np.random.default_rng(27)
    H, dk, dv = 2, 4, 3
    for mode in MODES:
        for lens in ([5, 0, 1, 7, 0, 3], [9], [0, 4], [3, 3, 3]):
            cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
            T, N = int(cu[-1]), len(lens)
            q, k, v, alpha, beta, _ = _inputs(rng, 1, T, H, dk, dv, mode)
            S0 = rng.standard_normal((N, H, dv, dk))
            sq = lambda x: None if x is None else x[0]
            for s0 in (S0, None):
                o, S = orc.gdn_fwd_varlen(q[0], k[0], v[0], sq(alpha), beta[0], cu, s0, mode=mode)
                assert o.shape == (T, H, dv) and S.shape == (N, H, dv, dk)
                for s in range(N):
                    a, b = int(cu[s]), int(cu[s + 1])
                    sl = lambda x: None if x is None else x[:, a:b]
                    init = None if s0 is None else s0[s:s + 1]
                    os_, Ss = orc.gdn_fwd(q[:, a:b], k[:, a:b], v[:, a:b], sl(alpha), beta[:, a:b],
                                          init, mode=mode)
                    assert np.array_equal(o[a:b], os_[0])
                    assert np.array_equal(S[s], Ss[0])
        # equal lengths: the same as a batch of rows
        L, N = 4, 3
        q, k, v, alpha, beta, S0 = _inputs(rng, N, L, H, dk, dv, mode)
        cu = np.arange(0, N * L + 1, L, dtype=np.int32)
        flat = lambda x: None if x is None else x.reshape((N * L,) + x.shape[2:])
        o, S = orc.gdn_fwd_varlen(flat(q), flat(k), flat(v), flat(alpha), flat(beta), cu, S0,
                                  mode=mode)
        ob, Sb = orc.gdn_fwd(q, k, v, alpha, beta, S0, mode=mode)
        assert np.array_equal(o, flat(ob)) and np.array_equal(S, Sb)


def _gdn2_inputs(rng, B, T, H, dk, dv, lo=0.5):
    q, k, v, alpha, beta, S0 = _inputs(rng, B, T, H, dk, dv, MODE_CHANNEL, lo=lo)
    erase = rng.uniform(0.0, 1.0, (B, T, H, dk))
    write = rng.uniform(0.0, 1.0, (B, T, H, dv))
    return q, k, v, alpha, erase, write, S0


def pin_gdn2_reduces_to_kda(orc):
    """Gated DeltaNet-2 with erase gate b = beta 1 and write gate w = beta 1 is the
    per-channel (KDA) recurrence (LAA section 2.6), and with equal channels the
    scalar-gate one (up to the rounding order of beta (v - p) against
    beta v - beta p)."""
    rng = np.random.default_rng(28)
    B, T, H, dk, dv = 2, 9, 2, 5, 4
    q, k, v, alpha, beta, S0 = _inputs(rng, B, T, H, dk, dv, MODE_CHANNEL)
    erase = np.repeat(beta[..., None], dk, axis=-1)
    write = np.repeat(beta[..., None], dv, axis=-1)
    o2, S2 = orc.gdn_fwd(q, k, v, alpha, None, S0, mode=oracle.MODE_GDN2, erase=erase, write=write)
    o1, S1 = orc.gdn_fwd(q, k, v, alpha, beta, S0, mode=MODE_CHANNEL)
    assert _rel(o2, o1) < 1e-13 and _rel(S2, S1) < 1e-13
    a1 = alpha[..., 0]
    o2, S2 = orc.gdn_fwd(q, k, v, np.repeat(a1[..., None], dk, axis=-1), None, S0,
                         mode=oracle.MODE_GDN2, erase=erase, write=write)
    o1, S1 = orc.gdn_fwd(q, k, v, a1, beta, S0, mode=MODE_SCALAR)
    assert _rel(o2, o1) < 1e-13 and _rel(S2, S1) < 1e-13


def pin_gdn2_orthonormal_closed_form(orc):
    """Orthonormal keys, no decay, S0 = 0, an erase gate equal over the channels
    (b_t = c_t 1): every erase read-out S e_t = c_t S k_t is zero (the state's rows
    lie in the span of the earlier keys), so S_T = sum_t (w_t * v_t) k_t^T and
    o_t = sum_{j<=t} (w_j * v_j)(k_j . q_t): the write gate alone scales what is
    stored, along the key itself."""
    rng = np.random.default_rng(29)
    T, dk, dv = 5, 6, 3
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:T][None, :, None, :]
    q = rng.standard_normal((1, T, 1, dk))
    v = rng.standard_normal((1, T, 1, dv))
    alpha = np.ones((1, T, 1, dk))
    erase = np.repeat(rng.uniform(0.1, 2.0, (1, T, 1, 1)), dk, axis=-1)
    write = rng.uniform(0.1, 1.0, (1, T, 1, dv))
    o, S = orc.gdn_fwd(q, k, v, alpha, None, None, mode=oracle.MODE_GDN2, erase=erase, write=write)
    z = (write * v)[0, :, 0]
    kk = k[0, :, 0]
    assert np.max(np.abs(S[0, 0] - z.T @ kk)) < 1e-14
    for t in range(T):
        want = sum(z[j] * float(kk[j] @ q[0, t, 0]) for j in range(t + 1))
        assert np.max(np.abs(o[0, t, 0] - want)) < 1e-13


def pin_gdn2_product_form(orc):
    """The unrolled form of the page's expansion S_t = S_{t-1} D_t (I - e_t k_t^T)
    + z_t k_t^T (LAA section 2.6): S_T = S0 prod_t D_t (I - e_t k_t^T)
    + sum_t z_t k_t^T prod_{j>t} D_j (I - e_j k_j^T), as matrix products."""
    rng = np.random.default_rng(30)
    T, dk, dv = 6, 4, 3
    q, k, v, alpha, erase, write, S0 = _gdn2_inputs(rng, 1, T, 1, dk, dv)
    o, S = orc.gdn_fwd(q, k, v, alpha, None, S0, mode=oracle.MODE_GDN2, erase=erase, write=write)
    M = [np.diag(alpha[0, t, 0]) @ (np.eye(dk) - np.outer(erase[0, t, 0] * k[0, t, 0], k[0, t, 0]))
         for t in range(T)]
    want = S0[0, 0].copy()
    for t in range(T):
        want = want @ M[t]
    for t in range(T):
        term = np.outer(write[0, t, 0] * v[0, t, 0], k[0, t, 0])
        for j in range(t + 1, T):
            term = term @ M[j]
        want = want + term
    assert _rel(S[0, 0], want) < 1e-13


PINS = [pin_worked_example, pin_exact_recall, pin_orthonormal_closed_form,
        pin_kda_axis_keys_closed_form, pin_no_write, pin_exact_rational, pin_gradient_step,
        pin_orthogonal_invariance, pin_rank_bound, pin_value_channel_independence,
        pin_linearity, pin_contraction, pin_mode_reductions, pin_zero_gate_resets,
        pin_decode_matches_prefill, pin_varlen_resets_at_sequence_starts, pin_gdn2_reduces_to_kda,
        pin_gdn2_orthonormal_closed_form, pin_gdn2_product_form]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle.loop.default())


def test_oracle_empty_sequence_returns_initial_state():
    """T = 0: no token, the state is S0 (zeros without S0)."""
    rng = np.random.default_rng(26)
    S0 = rng.standard_normal((2, 3, 4, 5))
    z = np.zeros((2, 0, 3, 5))
    o, S = oracle.gdn_fwd(z, z, np.zeros((2, 0, 3, 4)), np.zeros((2, 0, 3)), np.zeros((2, 0, 3)),
                          S0, mode=MODE_SCALAR)
    assert o.shape == (2, 0, 3, 4) and np.array_equal(S, S0)
    _, S = oracle.gdn_fwd(z, z, np.zeros((2, 0, 3, 4)), None, np.zeros((2, 0, 3)), None,
                          mode=MODE_NONE)
    assert np.array_equal(S, np.zeros((2, 3, 4, 5)))


def test_oracle_varlen_rejects_bad_offsets():
    """Offsets must run from 0 to T without decreasing."""
    z, v, b = np.zeros((6, 1, 4)), np.zeros((6, 1, 3)), np.zeros((6, 1))
    for cu in ([0, 4, 2, 6], [1, 6], [0, 5], [0, 3, 7]):
        with pytest.raises(RuntimeError):
            oracle.gdn_fwd_varlen(z, z, v, None, b, np.array(cu), mode=MODE_NONE)


# ----------------------------------------------------------------------------------
# chunk form (the algebra the GPU kernels follow) against the pinned loop
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("T,C", [(1, 64), (63, 16), (65, 64), (37, 3)])
def test_chunk_form_gdn2_equals_loop(T, C):
    rng = np.random.default_rng(2000 + T * 7 + C)
    q, k, v, alpha, erase, write, S0 = _gdn2_inputs(rng, 1, T, 2, 8, 6, lo=0.6)
    o, S = oracle.gdn_fwd(q, k, v, alpha, None, S0, mode=oracle.MODE_GDN2, erase=erase, write=write)
    oc, Sc = chunk_form.gdn_fwd(q, k, v, alpha, None, S0, mode=oracle.MODE_GDN2, chunk=C,
                                erase=erase, write=write)
    assert _rel(oc, o) < 1e-12 and _rel(Sc, S) < 1e-12


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("T,C", [(1, 64), (2, 1), (63, 16), (64, 64), (65, 64), (130, 64),
                                 (37, 3), (100, 16)])
def test_chunk_form_equals_loop(mode, T, C):
    rng = np.random.default_rng(1000 + T * 7 + C)
    B, H, dk, dv = 1, 2, 8, 6
    q, k, v, alpha, beta, S0 = _inputs(rng, B, T, H, dk, dv, mode, lo=0.6)
    o, S = oracle.gdn_fwd(q, k, v, alpha, beta, S0, mode=mode)
    oc, Sc = chunk_form.gdn_fwd(q, k, v, alpha, beta, S0, mode=mode, chunk=C)
    assert _rel(oc, o) < 1e-12
    assert _rel(Sc, S) < 1e-12


def test_chunk_form_zero_gates_and_strong_decay():
    """Gates at 0 and strong per-channel decay (product far below fp32 range inside a
    chunk) are exact in the chunk form because ratios are products of gates."""
    rng = np.random.default_rng(31)
    B, T, H, dk, dv = 1, 40, 1, 6, 4
    q, k, v, alpha, beta, S0 = _inputs(rng, B, T, H, dk, dv, MODE_CHANNEL)
    alpha = rng.uniform(0.0, 0.05, alpha.shape)
    alpha[0, 5] = 0.0
    o, S = oracle.gdn_fwd(q, k, v, alpha, beta, S0, mode=MODE_CHANNEL)
    oc, Sc = chunk_form.gdn_fwd(q, k, v, alpha, beta, S0, mode=MODE_CHANNEL, chunk=16)
    assert _rel(oc, o) < 1e-12 and _rel(Sc, S) < 1e-12


# ----------------------------------------------------------------------------------
# planted mistakes: each mutated copy of the oracle must fail at least one pin
# ----------------------------------------------------------------------------------

MUTATIONS = {
    "drop_scalar_decay": ("S[i] *= alpha[0];", "S[i] *= 1.0;"),
    "drop_channel_decay": ("S[i * dk + c] *= alpha[c];", "S[i * dk + c] *= 1.0;"),
    "kda_decay_on_value_rows": ("S[i * dk + c] *= alpha[c];", "S[i * dk + c] *= alpha[i % dk];"),
    "write_sign_flipped": ("S[i * dk + c] += u * k[c];", "S[i * dk + c] -= u * k[c];"),
    "beta_on_prediction_only": ("double u = beta * (v[i] - p[i]);",
                                "double u = (v[i] - beta * p[i]);"),
    "prediction_uses_query": ("acc += S[i * dk + c] * k[c];", "acc += S[i * dk + c] * q[c];"),
    "read_uses_key": ("acc += S[i * dk + c] * q[c];", "acc += S[i * dk + c] * k[c];"),
    "write_uses_query": ("S[i * dk + c] += u * k[c];", "S[i * dk + c] += u * q[c];"),
    "error_without_beta": ("double u = beta * (v[i] - p[i]);", "double u = (v[i] - p[i]);"),
    "gdn2_write_along_erase": ("W[i * dk + c] += res[i] * kappa[c];",
                               "W[i * dk + c] += res[i] * b[c] * kappa[c];"),
    "gdn2_no_write_gate": ("res[i] = w[i] * v[i] - read;", "res[i] = v[i] - read;"),
    "gdn2_erase_without_gate": ("read += W[i * dk + c] * (b[c] * kappa[c]);",
                                "read += W[i * dk + c] * kappa[c];"),
    "gdn2_decay_on_value_rows": ("for (c = 0; c < dk; ++c) W[i * dk + c] *= alpha[c];",
                                 "for (c = 0; c < dk; ++c) W[i * dk + c] *= alpha[i % dk];"),
    "varlen_wrong_initial_state": ("memcpy(S, S0 + ((size_t)seq * H + h) * sz",
                                   "memcpy(S, S0 + ((size_t)(seq - 1) * H + h) * sz"),
    "varlen_boundary_one_late": ("while (seq < N && cu[seq + 1] == t) {",
                                 "while (seq < N && t > 0 && cu[seq + 1] == t - 1) {"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, "mutation anchor not found once: %r" % old
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = oracle.compile_library(str(path), str(tmp_path / "libmutant.so"))
    mutant = oracle.Oracle(lib)
    failed = []
    for pin in PINS:
        try:
            pin(mutant)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "planted mistake %s escaped every pin" % name


# ----------------------------------------------------------------------------------
# the per-token prologue (oracle/prologue.py): closed forms
# ----------------------------------------------------------------------------------

def test_prologue_l2norm_closed_forms():
    """(3, 4) has norm 5: eps = 0 gives (0.6, 0.8); eps = 11 gives (3, 4) / 6.
    Every normalised vector has unit norm at eps = 0; scaling the input does
    not change the result."""
    from oracle import prologue as P
    assert np.array_equal(P.l2norm(np.array([3.0, 4.0]), 0.0), [0.6, 0.8])
    assert np.allclose(P.l2norm(np.array([3.0, 4.0]), 11.0), [0.5, 4.0 / 6.0], rtol=0, atol=1e-16)
    x = np.random.default_rng(3).standard_normal((5, 7, 16))
    n = np.linalg.norm(P.l2norm(x, 0.0), axis=-1)
    assert np.max(np.abs(n - 1)) < 1e-15
    assert np.max(np.abs(P.l2norm(7.5 * x, 0.0) - P.l2norm(x, 0.0))) < 1e-15


def test_prologue_sigmoid_softplus_closed_forms():
    """sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, sigmoid(x) + sigmoid(-x) = 1;
    softplus(0) = ln 2, softplus(y) - softplus(-y) = y, softplus(ln 3) = ln 4,
    and no overflow at |y| = 800."""
    from oracle import prologue as P
    assert P.sigmoid(np.array(0.0)) == 0.5
    assert abs(P.sigmoid(np.array(np.log(3.0))) - 0.75) < 1e-15
    y = np.linspace(-30, 30, 61)
    assert np.max(np.abs(P.sigmoid(y) + P.sigmoid(-y) - 1)) < 1e-15
    assert abs(P.softplus(np.array(0.0)) - np.log(2.0)) < 1e-16
    assert abs(P.softplus(np.array(np.log(3.0))) - np.log(4.0)) < 1e-15
    assert np.max(np.abs(P.softplus(y) - P.softplus(-y) - y)) < 1e-13
    big = P.softplus(np.array([800.0, -800.0]))
    assert big[0] == 800.0 and big[1] == 0.0


def test_prologue_decay_closed_forms():
    """exp(-a softplus(y)) = (1 + e^y)^(-a): a = 1 gives sigmoid(-y), a = 2 its
    square; the bias shifts the argument (per head for a scalar gate, per head
    and key channel for a per-channel gate); a -> 0 gives no decay."""
    from oracle import prologue as P
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 5, 2))                      # [B, T, H]
    b = np.array([0.5, -1.5])
    A = np.array([1.0, 2.0])
    al = P.decay_from_logits(x, A, b, MODE_SCALAR)
    s = 1.0 / (1.0 + np.exp(x + b))                         # sigmoid(-(x + b))
    assert np.max(np.abs(al[..., 0] - s[..., 0])) < 1e-15
    assert np.max(np.abs(al[..., 1] - s[..., 1] ** 2)) < 1e-15
    xc = rng.standard_normal((2, 4, 2, 3))                  # [B, T, H, dk]
    bc = rng.standard_normal((2, 3))
    alc = P.decay_from_logits(xc, A, bc, MODE_CHANNEL)
    sc = 1.0 / (1.0 + np.exp(xc + bc))
    assert np.max(np.abs(alc[:, :, 0] - sc[:, :, 0])) < 1e-15
    assert np.max(np.abs(alc[:, :, 1] - sc[:, :, 1] ** 2)) < 1e-15
    assert np.array_equal(P.decay_from_logits(x, np.zeros(2), None, MODE_SCALAR), np.ones_like(x))


def test_prologue_feeds_the_loop():
    """The prologue's outputs are exactly what the loop receives: with unit
    keys, beta logit +inf (beta = 1) and no decay the key is recalled exactly
    (exact-recall pin of the loop), whatever the keys' scale before the
    normalisation."""
    from oracle import prologue as P
    rng = np.random.default_rng(5)
    B, T, H, dk, dv = 1, 3, 1, 4, 2
    q = rng.standard_normal((B, T, H, dk)) * 5
    k = rng.standard_normal((B, T, H, dk)) * 3
    v = rng.standard_normal((B, T, H, dv))
    beta = np.full((B, T, H), 800.0)
    o, S = P.gdn_fwd(q, k, v, None, beta, None, mode=MODE_NONE, l2norm_qk=True, eps=0.0,
                     beta_logits=True)
    kn = k[0, -1, 0] / np.linalg.norm(k[0, -1, 0])
    assert np.max(np.abs(S[0, 0] @ kn - v[0, -1, 0])) < 1e-12


# ----------------------------------------------------------------------------------
# reference gradients (oracle/backward.py) against finite differences of the C loop
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("mode", MODES)
def test_backward_matches_finite_differences(mode):
    """Every entry of dq, dk, dv, dalpha, dbeta and dS0 equals the central
    difference of L = sum(do * o) + sum(dS_T * S_T) computed with the C loop
    (step 1e-6, fp64): the reverse-mode gradients are pinned to the pinned
    forward, not to a retyped copy of it."""
    from oracle import backward
    rng = np.random.default_rng(300 + mode)
    B, T, H, dk, dv = 1, 5, 2, 3, 2
    q, k, v, alpha, beta, S0 = _inputs(rng, B, T, H, dk, dv, mode, lo=0.3)
    do = rng.standard_normal((B, T, H, dv))
    dST = rng.standard_normal((B, H, dv, dk))
    g = backward.gdn_bwd(q, k, v, alpha, beta, S0, do, dST, mode=mode)

    def loss(**kw):
        args = dict(q=q, k=k, v=v, alpha=alpha, beta=beta, S0=S0)
        args.update(kw)
        o, S = oracle.gdn_fwd(args["q"], args["k"], args["v"], args["alpha"], args["beta"],
                              args["S0"], mode=mode)
        return float(np.sum(o * do) + np.sum(S * dST))

    h = 1e-6
    names = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("beta", "dbeta"), ("S0", "dS0")]
    if mode != MODE_NONE:
        names.append(("alpha", "dalpha"))
    base = dict(q=q, k=k, v=v, alpha=alpha, beta=beta, S0=S0)
    for name, gname in names:
        x = base[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            fd[idx] = (loss(**{name: xp}) - loss(**{name: xm})) / (2 * h)
        err = np.max(np.abs(g[gname] - fd)) / max(1.0, np.max(np.abs(fd)))
        assert err < 1e-7, (name, err)
