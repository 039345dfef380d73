"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle on the
same CPU inputs, compare per (b, h) slice as max|x - ref| / max|ref|."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads as W

# Tolerances (max relative error per (b, h) slice, outputs and final state).
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def to_dev(d: dict) -> dict:
    return {k: (None if v is None else v.cuda()) for k, v in d.items()}


def gpu_prefill(gdn, inp: dict, mode: int, **kw):
    dv_ = to_dev(inp)
    o, S = gdn.chunk_fwd(dv_["q"], dv_["k"], dv_["v"], dv_["alpha"], dv_["beta"], dv_["S0"],
                         mode=mode, **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), None if S is None else S.cpu().numpy()


def oracle_prefill(inp: dict, mode: int):
    return oracle.gdn_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"],
                          mode=mode)


def select_heads(inp: dict, heads) -> dict:
    """Inputs of the listed (b, h) heads stacked along B (H = 1): the oracle then
    runs only those heads (heads are independent)."""
    out = {}
    for key, t in inp.items():
        if t is None:
            out[key] = None
        elif key == "S0":
            out[key] = torch.stack([t[b, h] for b, h in heads])[:, None]
        else:
            out[key] = torch.stack([t[b, :, h] for b, h in heads])[:, :, None]
    return out


def rel_o(o, ref):       # o [B, T, H, dv]
    return W.per_head_rel_err(o, ref, (0, 2))


def rel_S(S, ref):       # S [B, H, dv, dk]
    return W.per_head_rel_err(S, ref, (0, 1))


def check_prefill(gdn, inp, mode, dtype, heads=None, tol=None, **kw):
    """Run the GPU path on all heads; compare with the oracle (on ``heads`` only if
    given).  Returns (rel_err_o, rel_err_S)."""
    tol = TOL[dtype] if tol is None else tol
    o, S = gpu_prefill(gdn, inp, mode, **kw)
    if heads is None:
        ro, rS = oracle_prefill(inp, mode)
    else:
        ro, rS = oracle_prefill(select_heads(inp, heads), mode)
        o = np.stack([o[b, :, h] for b, h in heads])[:, :, None]
        S = np.stack([S[b, h] for b, h in heads])[:, None]
    eo, eS = rel_o(o, ro), rel_S(S, rS)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    assert eo <= tol, "o rel err %.3e > %.1e" % (eo, tol)
    assert eS <= tol, "S_final rel err %.3e > %.1e" % (eS, tol)
    return eo, eS
