"""GPU parity of the output epilogue (gdn_gated_rmsnorm) against the fp64
oracle (oracle/epilogue.py): y = o / sqrt(mean(o^2) + eps) * w * silu(g) per
row of d_v values.  Per-tensor max|x - ref| / max|ref|."""
import numpy as np
import pytest
import torch

import workloads as W
from gdn_testlib import TOL, check_prefill, gpu_prefill, oracle_prefill, to_dev
from oracle import epilogue as OE

pytestmark = pytest.mark.gpu


def _data(shape, dtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    o = (scale * torch.randn(*shape, generator=g)).to(dtype)
    gate = (2.0 * torch.randn(*shape, generator=g)).to(dtype)
    w = 1.0 + 0.5 * torch.randn(shape[-1], generator=g)
    return o, gate, w


def _rel(x, ref):
    return float(np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-30))


def _run(gdn, o, gate, w, eps, inplace=False):
    od, gd, wd = o.cuda(), gate.cuda(), w.cuda()
    y = gdn.gated_rmsnorm(od, gd, wd, eps=eps, out=od if inplace else None)
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("dv", [64, 128])
@pytest.mark.parametrize("lead", [(1,), (7,), (2, 5, 3), (4, 33, 2), (1000,)])
def test_gated_rmsnorm_matches_oracle(gpu, dtype, dv, lead):
    o, gate, w = _data(lead + (dv,), dtype, seed=dv + len(lead) + lead[0])
    y = _run(gpu, o, gate, w, 1e-6)
    assert _rel(y, OE.gated_rmsnorm(o, gate, w, 1e-6)) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_gated_rmsnorm_in_place_and_edge_rows(gpu, dtype):
    o, gate, w = _data((6, 4, 128), dtype, seed=3)
    o[0, 0] = 0.0                       # a zero row: zero out (eps > 0)
    o[1, 1] = 1e4                       # large and small magnitudes normalise alike
    o[2, 2] = 1e-20
    ref = OE.gated_rmsnorm(o, gate, w, 1e-6)
    y = _run(gpu, o.clone(), gate, w, 1e-6, inplace=True)
    assert np.all(np.isfinite(y))
    assert np.array_equal(y[0, 0], np.zeros(128))
    assert _rel(y, ref) <= TOL[dtype]
    for eps in (0.0, 0.5):
        assert _rel(_run(gpu, o, gate, w, eps)[1:], OE.gated_rmsnorm(o[1:], gate[1:], w, eps)) <= TOL[dtype]


def test_gated_rmsnorm_full_size_sampled(gpu):
    """[B=8, T=4096, H=16, d_v=128] bf16 (the prefill workload's output shape):
    every row on the GPU, 2048 sampled rows against the oracle."""
    o, gate, w = _data((8, 4096, 16, 128), torch.bfloat16, seed=11)
    y = _run(gpu, o, gate, w, 1e-6)
    rng = np.random.default_rng(12)
    idx = (rng.integers(0, 8, 2048), rng.integers(0, 4096, 2048), rng.integers(0, 16, 2048))
    ref = OE.gated_rmsnorm(o[idx], gate[idx], w, 1e-6)
    assert _rel(y[idx], ref) <= TOL[torch.bfloat16]


def test_prefill_then_epilogue(gpu):
    """The mixer's output path: prefill, then the epilogue on its output,
    against the oracle's prefill followed by the oracle's epilogue."""
    w = W.Prefill("epi", 2, 3, 200, 128, 128, torch.bfloat16, "exp01", 0.1, seed=17)
    inp = W.make_prefill(w)
    d = to_dev(inp)
    o, _ = gpu.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], mode=w.mode)
    gate, wt = _data((2, 200, 3, 128), torch.bfloat16, seed=18)[1:]
    y = gpu.gated_rmsnorm(o, gate.cuda(), wt.cuda(), eps=1e-6)
    torch.cuda.synchronize()
    ro, _ = oracle_prefill(inp, w.mode)
    ref = OE.gated_rmsnorm(ro, gate, wt, 1e-6)
    assert _rel(y.float().cpu().numpy(), ref) <= TOL[torch.bfloat16]
