"""GPU parity of the prefill backward (gdn_chunk_bwd) against the fp64 reference
gradients (oracle/backward.py, pinned to finite differences of the C loop).
Per (b, h) slice max|x - ref| / max|ref| for every gradient."""
import numpy as np
import pytest
import torch

import workloads as W
from gdn_testlib import TOL
from oracle import backward as OB

pytestmark = pytest.mark.gpu

GATE = {0: "none", 1: "exp01", 2: "exp01_channel"}


def _inputs(B, T, H, dk, dv, dtype, mode, seed, s0=True):
    w = W.Prefill("bwd", B, H, T, dk, dv, dtype, GATE[mode], 0.2 if s0 else 0.0, seed=seed)
    d = W.make_prefill(w)
    g = torch.Generator().manual_seed(seed + 7)
    d["do"] = torch.randn(B, T, H, dv, generator=g).to(dtype)
    d["dST"] = 0.5 * torch.randn(B, H, dv, dk, generator=g)
    return d


def _gpu(gdn, d, mode, with_dST=True):
    c = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    g = gdn.chunk_bwd(c["q"], c["k"], c["v"], c["alpha"], c["beta"], c["S0"], c["do"],
                      c["dST"] if with_dST else None, mode=mode)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.float().cpu().numpy()) for k, v in g.items()}


def _ref(d, mode, with_dST=True):
    return OB.gdn_bwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["do"],
                      d["dST"] if with_dST else None, mode=mode)


def _check(g, r, mode, tol):
    errs = {}
    for name, axes in (("dq", (0, 2)), ("dk", (0, 2)), ("dv", (0, 2)), ("dbeta", None),
                       ("dS0", (0, 1)), ("dalpha", None)):
        if name == "dalpha" and mode == 0:
            continue
        x, ref = g[name], r[name]
        assert np.all(np.isfinite(x)), name
        if axes is None:   # [B, T, H] or [B, T, H, dk]: per (b, h) slice
            if x.ndim == 3:
                x, ref = x[..., None], ref[..., None]
            axes = (0, 2)
        errs[name] = W.per_head_rel_err(x, ref, axes)
    bad = {k: v for k, v in errs.items() if v > tol}
    assert not bad, (bad, errs)
    return errs


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 64), (64, 128)])
@pytest.mark.parametrize("T", [1, 7, 64, 65, 130])
def test_backward_small(gpu, dtype, mode, dk, dv, T):
    d = _inputs(2, T, 2, dk, dv, dtype, mode, seed=110 + T)
    print("backward %s mode %d dk %d dv %d T %d" % (dtype, mode, dk, dv, T), flush=True)
    _check(_gpu(gpu, d, mode), _ref(d, mode), mode, TOL[dtype])


@pytest.mark.parametrize("mode", [1, 2])
def test_backward_without_initial_state_or_final_gradient(gpu, mode):
    d = _inputs(1, 70, 3, 128, 128, torch.float32, mode, seed=120, s0=False)
    _check(_gpu(gpu, d, mode, with_dST=False), _ref(d, mode, with_dST=False), mode, 1e-4)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_backward_zero_beta_rows(gpu, mode):
    """Every third token writes nothing (beta = 0): diag(beta) is singular, so
    the chunk-level kernels must take M = (I + A)^-1 from the solve itself."""
    d = _inputs(2, 130, 2, 128, 128, torch.bfloat16, mode, seed=125)
    d["beta"][:, ::3] = 0.0
    print("backward bf16 mode %d zero-beta rows" % mode, flush=True)
    _check(_gpu(gpu, d, mode), _ref(d, mode), mode, TOL[torch.bfloat16])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_backward_strong_decay(gpu, dtype):
    """alpha in [0.05, 0.5]: the decay inside a chunk spans ~190 e-folds."""
    d = _inputs(2, 150, 2, 128, 64, dtype, 1, seed=126)
    g = torch.Generator().manual_seed(127)
    d["alpha"] = 0.05 + 0.45 * torch.rand(d["alpha"].shape, generator=g)
    print("backward %s strong decay" % dtype, flush=True)
    _check(_gpu(gpu, d, 1), _ref(d, 1), 1, TOL[dtype])


@pytest.mark.parametrize("gate", ["kda_literal", "kda_clamped"])
def test_backward_per_channel_gates(gpu, gate):
    """bf16 per-channel decay (the chunk-level path): the literal gate (median
    alpha about 0.05, single channels decaying by hundreds of e-folds inside a
    chunk) and the clamped one; 200 tokens over four chunks."""
    w = W.Prefill("bwd", 2, 2, 200, 128, 128, torch.bfloat16, gate, 0.2, seed=131)
    d = W.make_prefill(w)
    g = torch.Generator().manual_seed(132)
    d["do"] = torch.randn(2, 200, 2, 128, generator=g).to(torch.bfloat16)
    d["dST"] = 0.5 * torch.randn(2, 2, 128, 128, generator=g)
    print("backward bf16 per-channel gate %s" % gate, flush=True)
    errs = _check(_gpu(gpu, d, 2), _ref(d, 2), 2, TOL[torch.bfloat16])
    print({k: "%.2e" % v for k, v in errs.items()}, flush=True)


def test_backward_empty_sequence(gpu):
    """T = 0: dS0 = dS_final, nothing else."""
    d = _inputs(2, 0, 2, 64, 64, torch.float32, 1, seed=121)
    g = _gpu(gpu, d, 1)
    assert np.array_equal(g["dS0"], d["dST"].numpy())


@pytest.mark.parametrize("mode", [1, 2], ids=["scalar", "per_channel"])
def test_backward_is_deterministic(gpu, mode):
    d = _inputs(2, 150, 2, 128, 128, torch.bfloat16, mode, seed=122)
    a, b = _gpu(gpu, d, mode), _gpu(gpu, d, mode)
    for k in a:
        assert a[k] is None or np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_backward_eight_heads(gpu, mode):
    """B * H a multiple of 8 (the chains group a head's value slices by XCD):
    every head against the reference, several chunks and a ragged tail."""
    d = _inputs(2, 200, 4, 128, 128, torch.bfloat16, mode, seed=124)
    print("backward bf16 mode %d B 2 H 4 T 200" % mode, flush=True)
    _check(_gpu(gpu, d, mode), _ref(d, mode), mode, TOL[torch.bfloat16])


def test_backward_workload_sampled(gpu):
    """B=8, H=16, T=4096, d=128, bf16 (the prefill workload's inputs): two heads
    of every gradient against the reference."""
    w = W.GDN_BF16_PREFILL
    d = W.make_prefill(w)
    g = torch.Generator().manual_seed(123)
    d["do"] = torch.randn(w.B, w.T, w.H, w.dv, generator=g).to(w.dtype)
    d["dST"] = 0.5 * torch.randn(w.B, w.H, w.dv, w.dk, generator=g)
    out = _gpu(gpu, d, 1)
    heads = [(2, 5), (7, 11)]
    sub = {}
    for key, t in d.items():
        if key in ("S0", "dST"):
            sub[key] = torch.stack([t[b, h] for b, h in heads])[:, None]
        else:
            sub[key] = torch.stack([t[b, :, h] for b, h in heads])[:, :, None]
    ref = _ref(sub, 1)
    picked = {}
    for key, x in out.items():
        if key == "dS0":
            picked[key] = np.stack([x[b, h] for b, h in heads])[:, None]
        else:
            picked[key] = np.stack([x[b, :, h] for b, h in heads])[:, :, None]
    errs = _check(picked, ref, 1, 2e-2)
    print("backward gdn bf16 b8 h16 t4096: %s" % {k: "%.2e" % v for k, v in errs.items()}, flush=True)


def test_backward_per_channel_workload_sampled(gpu):
    """B=4, H=16, T=8192, d=128, bf16, per-channel decay (the per-channel
    prefill workload's inputs): two heads of every gradient against the
    reference."""
    w = W.KDA_BF16_PREFILL
    d = W.make_prefill(w)
    g = torch.Generator().manual_seed(133)
    d["do"] = torch.randn(w.B, w.T, w.H, w.dv, generator=g).to(w.dtype)
    d["dST"] = 0.5 * torch.randn(w.B, w.H, w.dv, w.dk, generator=g)
    out = _gpu(gpu, d, 2)
    heads = [(0, 3), (3, 14)]
    sub = {}
    for key, t in d.items():
        if t is None:
            sub[key] = None
        elif key in ("S0", "dST"):
            sub[key] = torch.stack([t[b, h] for b, h in heads])[:, None]
        else:
            sub[key] = torch.stack([t[b, :, h] for b, h in heads])[:, :, None]
    ref = _ref(sub, 2)
    picked = {}
    for key, x in out.items():
        if key == "dS0":
            picked[key] = np.stack([x[b, h] for b, h in heads])[:, None]
        else:
            picked[key] = np.stack([x[b, :, h] for b, h in heads])[:, :, None]
    errs = _check(picked, ref, 2, 2e-2)
    print("backward kda bf16 b4 h16 t8192: %s" % {k: "%.2e" % v for k, v in errs.items()}, flush=True)
