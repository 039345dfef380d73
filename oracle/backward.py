"""fp64 reference gradients of the gated delta-rule prefill.  Test infrastructure only.

The pages train these mixers with a custom first-order backward (NextTransformer
"method sources" page, KDA entry: it keeps the full state history and is
checked by an FP64 gradient check over every input and the initial state).
Here the gradients are those of the plain token loop (the same recurrence as
``gdn_oracle.c``: decay first, error against the decayed state, output from the
updated state), written with torch operations in fp64 on the CPU and
differentiated by torch's reverse mode.  The loop is retyped here only because
reverse mode needs it as torch operations; ``tests/test_oracle_pins.py`` pins
these gradients to central finite differences of the C loop itself.

For a scalar loss L = sum(do * o) + sum(dS_final * S_final) the function returns
dL/dq, dL/dk, dL/dv, dL/dalpha, dL/dbeta and dL/dS0.
"""
from __future__ import annotations

import numpy as np
import torch

from .loop import _f64, MODE_NONE, MODE_SCALAR, MODE_CHANNEL


def _t(x):
    return None if x is None else torch.from_numpy(_f64(x)).requires_grad_(True)


def gdn_bwd(q, k, v, alpha, beta, S0, do, dS_final=None, mode: int = MODE_SCALAR):
    """q, k [B, T, H, dk]; v, do [B, T, H, dv]; alpha [B, T, H] (scalar),
    [B, T, H, dk] (per channel) or None; beta [B, T, H]; S0 [B, H, dv, dk] or
    None (zeros; its gradient is then still returned); dS_final [B, H, dv, dk]
    or None.  Returns a dict of fp64 ndarrays: dq, dk, dv, dalpha (None without
    decay), dbeta, dS0."""
    qt, kt, vt, bt = _t(q), _t(k), _t(v), _t(beta)
    at = _t(alpha) if mode != MODE_NONE else None
    B, T, H, dk = qt.shape
    dv = vt.shape[-1]
    s0 = _f64(S0) if S0 is not None else np.zeros((B, H, dv, dk))
    S0t = torch.from_numpy(np.array(s0)).requires_grad_(True)
    S = S0t
    outs = []
    for t in range(T):
        if mode == MODE_SCALAR:
            S = S * at[:, t][:, :, None, None]
        elif mode == MODE_CHANNEL:
            S = S * at[:, t][:, :, None, :]
        kk = kt[:, t]                                     # [B, H, dk]
        p = torch.einsum("bhic,bhc->bhi", S, kk)          # prediction from the decayed state
        u = bt[:, t][:, :, None] * (vt[:, t] - p)         # pseudo-value
        S = S + u[..., None] * kk[:, :, None, :]          # delta write
        outs.append(torch.einsum("bhic,bhc->bhi", S, qt[:, t]))   # read of the updated state
    o = torch.stack(outs, dim=1) if T > 0 else torch.zeros(B, 0, H, dv, dtype=torch.float64)
    loss = (o * torch.from_numpy(_f64(do))).sum()
    if dS_final is not None:
        loss = loss + (S * torch.from_numpy(_f64(dS_final))).sum()
    inputs = [qt, kt, vt, bt, S0t] + ([at] if at is not None else [])
    grads = torch.autograd.grad(loss, inputs, allow_unused=True)

    def np_(g, like):
        return torch.zeros_like(like).numpy() if g is None else g.detach().numpy()

    return dict(dq=np_(grads[0], qt), dk=np_(grads[1], kt), dv=np_(grads[2], vt),
                dbeta=np_(grads[3], bt), dS0=np_(grads[4], S0t),
                dalpha=None if at is None else np_(grads[5], at))
