"""Decode step on the GPU against the fp64 oracle, step by step (o and S)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gdn_testlib import TOL

pytestmark = pytest.mark.gpu

GATE_OF_MODE = {0: "none", 1: "exp01", 2: "exp01_channel"}


def _run_steps(gdn, inp, steps, mode, heads=None):
    """All steps on the GPU in place; returns (o [steps, B, H, dv], S_final) on the CPU."""
    S = inp["S"].cuda().clone()
    dev = {k: (None if v is None else v.cuda()) for k, v in inp.items() if k != "S"}
    outs = []
    for s in range(steps):
        a = None if dev["alpha"] is None else dev["alpha"][s]
        outs.append(gdn.decode_step(dev["q"][s], dev["k"][s], dev["v"][s], a, dev["beta"][s], S,
                                    mode=mode))
    o = torch.stack(outs).float().cpu().numpy()
    torch.cuda.synchronize()
    return o, S.cpu().numpy()


def _oracle_steps(inp, steps, mode, heads=None):
    sel = (lambda t: t) if heads is None else (
        lambda t: torch.stack([t[:, b, h] for b, h in heads], 1)[:, :, None])
    selS = (lambda t: t) if heads is None else (
        lambda t: torch.stack([t[b, h] for b, h in heads])[:, None])
    q, k, v, beta = sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), sel(inp["beta"])
    alpha = None if inp["alpha"] is None else sel(inp["alpha"])
    S = selS(inp["S"])
    outs = []
    for s in range(steps):
        o, S = oracle.gdn_decode(q[s], k[s], v[s], None if alpha is None else alpha[s], beta[s], S,
                                 mode=mode)
        outs.append(o)
    return np.stack(outs), S


def _compare(o, S, ro, rS, tol):
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    eo = W.per_head_rel_err(o.transpose(1, 0, 2, 3), ro.transpose(1, 0, 2, 3), (0, 2))
    eS = W.per_head_rel_err(S, rS, (0, 1))
    assert eo <= tol, "o rel err %.3e" % eo
    assert eS <= tol, "S rel err %.3e" % eS
    return eo, eS


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_decode_small(gpu, dtype, mode, dk, dv):
    w = W.Decode("small", 3, 2, dk, dv, 6, dtype, GATE_OF_MODE[mode], 0.3, seed=70 + mode)
    inp = W.make_decode(w)
    o, S = _run_steps(gpu, inp, w.steps, mode)
    ro, rS = _oracle_steps(inp, w.steps, mode)
    _compare(o, S, ro, rS, TOL[dtype])


@pytest.mark.parametrize("w", [W.DECODE_DK128, W.DECODE_DK64], ids=lambda w: w.name)
def test_decode_full_size_sampled_heads(gpu, w):
    """All 1024 in-place steps at batch 64 x 16 heads; the oracle follows four heads."""
    inp = W.make_decode(w)
    heads = [(0, 0), (17, 5), (40, 11), (63, 15)]
    o, S = _run_steps(gpu, inp, w.steps, w.mode)
    ro, rS = _oracle_steps(inp, w.steps, w.mode, heads)
    o_s = np.stack([o[:, b, h] for b, h in heads], 1)[:, :, None]
    S_s = np.stack([S[b, h] for b, h in heads])[:, None]
    _compare(o_s, S_s, ro, rS, TOL[w.dtype])


def test_decode_zero_gates_and_beta(gpu):
    """beta = 0, alpha = 1 leaves S unchanged bit for bit; o = S q."""
    w = W.Decode("id", 4, 3, 128, 128, 1, torch.float32, "exp01", 0.5, seed=79)
    inp = W.make_decode(w)
    S = inp["S"].cuda().clone()
    one = torch.ones_like(inp["alpha"][0]).cuda()
    zero = torch.zeros_like(inp["beta"][0]).cuda()
    o = gpu.decode_step(inp["q"][0].cuda(), inp["k"][0].cuda(), inp["v"][0].cuda(), one, zero, S)
    torch.cuda.synchronize()
    assert torch.equal(S.cpu(), inp["S"])
    ref = torch.einsum("bhij,bhj->bhi", inp["S"].double(), inp["q"][0].double())
    assert float((o.cpu().double() - ref).abs().max()) < 1e-5
