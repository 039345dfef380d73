"""fp64 reference of the per-token prologue the mixer layers apply before the
recurrence.  Test infrastructure only (see the package docstring).

What the pages fix:
  - q and k are L2-normalised per head before the recurrence ("Don't Read
    Everything" notes, section 2.1, symbol table; "Enhancing Linear Attention
    with Residual Learning" notes, section 2.2, symbol table; NextTransformer
    "method sources" page, baseline section: DeltaNet, KDA).
  - beta = sigmoid(x_beta) (NextTransformer page, DeltaNet entry; residual-
    learning notes, section 2.2).
  - alpha = exp(-a softplus(x_alpha + b)), a Mamba2-style decay with a positive
    rate a per head and a bias b (residual-learning notes, section 2.2; the
    NextTransformer page gives KDA a learnable decay bias, here one bias per
    head and key channel).
The pages leave the normaliser's epsilon open; here q / sqrt(|q|^2 + eps).
Everything is evaluated in fp64 on the exact values the kernels receive; the
recurrence then runs on the results through :mod:`oracle.loop`.
"""
from __future__ import annotations

import numpy as np

from .loop import _f64, MODE_NONE, MODE_SCALAR, MODE_CHANNEL, default


def l2norm(x, eps: float):
    """x / sqrt(sum(x^2) + eps) over the last axis."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def sigmoid(x):
    x = _f64(x)
    return 1.0 / (1.0 + np.exp(-x))


def softplus(y):
    """log(1 + e^y), written so that neither branch overflows."""
    y = _f64(y)
    return np.maximum(y, 0.0) + np.log1p(np.exp(-np.abs(y)))


def decay_from_logits(x, A, dt_bias, mode: int):
    """alpha = exp(-A[h] softplus(x + dt_bias)).

    Scalar decay: x [..., H], dt_bias [H] or None.  Per-channel decay:
    x [..., H, dk], dt_bias [H, dk] or None.  A [H] (positive)."""
    x = _f64(x)
    A = _f64(A)
    if mode == MODE_SCALAR:
        y = x + (0.0 if dt_bias is None else _f64(dt_bias))
        return np.exp(-A * softplus(y))
    if mode == MODE_CHANNEL:
        y = x + (0.0 if dt_bias is None else _f64(dt_bias))
        return np.exp(-A[:, None] * softplus(y))
    raise ValueError("decay_from_logits needs a decay mode")


def apply(q, k, alpha, beta, mode: int, l2norm_qk=False, eps=0.0, beta_logits=False,
          alpha_logits=False, A=None, dt_bias=None):
    """The recurrence's inputs after the prologue, in fp64: (q, k, alpha, beta)."""
    q, k, beta = _f64(q), _f64(k), _f64(beta)
    alpha = _f64(alpha)
    if l2norm_qk:
        q, k = l2norm(q, eps), l2norm(k, eps)
    if beta_logits:
        beta = sigmoid(beta)
    if alpha_logits and mode != MODE_NONE:
        alpha = decay_from_logits(alpha, A, dt_bias, mode)
    return q, k, alpha, beta


def gdn_fwd(q, k, v, alpha, beta, S0=None, mode: int = MODE_SCALAR, cu_seqlens=None, **pro):
    """Prefill with the prologue: the plain loop (batched rows, or packed rows
    when ``cu_seqlens`` is given) on the inputs :func:`apply` returns."""
    q, k, alpha, beta = apply(q, k, alpha, beta, mode, **pro)
    orc = default()
    if cu_seqlens is None:
        return orc.gdn_fwd(q, k, v, alpha, beta, S0, mode=mode)
    return orc.gdn_fwd_varlen(q, k, v, alpha, beta, cu_seqlens, S0, mode=mode)


def gdn_decode(q, k, v, alpha, beta, S, mode: int = MODE_SCALAR, **pro):
    """One decode step with the prologue."""
    q, k, alpha, beta = apply(q, k, alpha, beta, mode, **pro)
    return default().gdn_decode(q, k, v, alpha, beta, S, mode=mode)
