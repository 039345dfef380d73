"""GPU parity of the fused per-token prologue (q, k L2 normalisation, beta and
alpha from logits) against the fp64 oracle: ``oracle.prologue`` applied to the
same raw inputs, then the plain loop.  Per (b, h) slice max|x - ref| / max|ref|,
worst slice within the dtype's tolerance.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gdn_testlib import TOL
from oracle import prologue as P

pytestmark = pytest.mark.gpu

EPS = 1e-6


def _dev(d):
    return {k: (None if v is None else v.cuda()) for k, v in d.items()}


def _flags(which):
    return dict(l2norm_qk="norm" in which, beta_logits="gates" in which,
                alpha_logits="gates" in which)


def _inputs(B, T, H, dk, dv, dtype, mode, seed, which):
    """Raw inputs for the parts of the prologue named in ``which``; the other
    parts get the plain generator's values (unit q, k; gates in (0, 1)): the
    delta rule with keys of norm above sqrt(2 / beta) diverges, in the oracle
    as on the GPU."""
    d = W.make_prologue(B, T, H, dk, dv, dtype, mode, seed)
    plain = W.make_prefill(W.Prefill("g", B, H, T, dk, dv, dtype,
                                     {0: "none", 1: "exp01", 2: "exp01_channel"}[mode], 0.0,
                                     seed=seed))
    if "gates" not in which:
        d["alpha"], d["beta"] = plain["alpha"], plain["beta"]
    if "norm" not in which:
        d["q"], d["k"] = plain["q"], plain["k"]
    return d


def _oracle_fwd(d, mode, which, cu=None):
    f = _flags(which)
    A = None if d["A"] is None else d["A"].numpy()
    b = None if d["dt_bias"] is None else d["dt_bias"].numpy()
    return P.gdn_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], mode=mode,
                     cu_seqlens=cu, eps=EPS, A=A, dt_bias=b, **f)


def _gpu_fwd(gdn, d, mode, which, cu=None):
    g = _dev(d)
    o, S = gdn.chunk_fwd_fused(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["S0"],
                               cu_seqlens=None if cu is None else cu.cuda(), mode=mode, eps=EPS,
                               A=g["A"], dt_bias=g["dt_bias"], **_flags(which))
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy()


@pytest.mark.parametrize("which", ["norm+gates", "norm", "gates"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 64)])
@pytest.mark.parametrize("T", [1, 65, 130])
def test_fused_prefill_small(gpu, which, dtype, mode, dk, dv, T):
    if mode == 0 and which == "gates" and T != 65:
        pytest.skip("no decay gate: beta alone is covered at T = 65")
    d = _inputs(2, T, 3, dk, dv, dtype, mode, 60 + T, which)
    print("fused prefill %s %s mode %d dk %d dv %d T %d" % (which, dtype, mode, dk, dv, T), flush=True)
    o, S = _gpu_fwd(gpu, d, mode, which)
    ro, rS = _oracle_fwd(d, mode, which)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    eo = W.per_head_rel_err(o, ro, (0, 2))
    eS = W.per_head_rel_err(S, rS, (0, 1))
    assert eo <= TOL[dtype] and eS <= TOL[dtype], (eo, eS)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_fused_all_off_is_the_plain_call(gpu, mode):
    """A prologue with every flag off gives bitwise what gdn_chunk_fwd gives."""
    w = W.Prefill("plain", 2, 3, 130, 128, 128, torch.bfloat16,
                  {0: "none", 1: "exp01", 2: "exp01_channel"}[mode], 0.1, seed=70)
    g = _dev(W.make_prefill(w))
    o1, S1 = gpu.chunk_fwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["S0"], mode=mode)
    o2, S2 = gpu.chunk_fwd_fused(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["S0"], mode=mode)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("mode", [1, 2])
def test_fused_packed_rows(gpu, mode):
    """The prologue on a packed batch (rows restart their state)."""
    lens = (70, 0, 1, 129, 64)
    T = sum(lens)
    d = _inputs(1, T, 2, 128, 128, torch.bfloat16, mode, 71, "norm+gates")
    N = len(lens)
    d["S0"] = 0.1 * torch.randn(N, 2, 128, 128, generator=torch.Generator().manual_seed(72))
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    o, S = _gpu_fwd(gpu, d, mode, "norm+gates", cu=cu)
    ro, rS = _oracle_fwd(d, mode, "norm+gates", cu=cu)
    eo = max(W.per_head_rel_err(o[:, a:b], ro[:, a:b], (0, 2))
             for a, b in zip(cu[:-1].tolist(), cu[1:].tolist()) if b > a)
    eS = W.per_head_rel_err(S, rS, (0, 1))
    assert eo <= 2e-2 and eS <= 2e-2, (eo, eS)


@pytest.mark.parametrize("mode", [1, 2])
def test_fused_packed_long_rows_split(gpu, mode):
    """The prologue on six packed rows over 16 heads, two of them (3000 and
    1800 tokens) longer than an even share of chunks per compute unit: their
    value slices run in two parts with a lead-in (from the history horizon
    under scalar decay).  Every (row, head) against the oracle."""
    lens = (3000, 100, 50, 1800, 0, 7)
    T, H, N = sum(lens), 16, len(lens)
    d = _inputs(1, T, H, 128, 128, torch.bfloat16, mode, 74, "norm+gates")
    d["S0"] = 0.1 * torch.randn(N, H, 128, 128, generator=torch.Generator().manual_seed(75))
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    print("fused packed long rows mode %d" % mode, flush=True)
    o, S = _gpu_fwd(gpu, d, mode, "norm+gates", cu=cu)
    ro, rS = _oracle_fwd(d, mode, "norm+gates", cu=cu)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    eo = max(W.per_head_rel_err(o[:, a:b], ro[:, a:b], (0, 2))
             for a, b in zip(cu[:-1].tolist(), cu[1:].tolist()) if b > a)
    eS = W.per_head_rel_err(S, rS, (0, 1))
    assert eo <= 2e-2 and eS <= 2e-2, (eo, eS)


def test_fused_prefill_workload_sampled(gpu):
    """B=8, H=16, T=4096, d=128, bf16 with raw q, k and logit gates: two heads
    checked against the oracle."""
    B, T, H = 8, 4096, 16
    d = W.make_prologue(B, T, H, 128, 128, torch.bfloat16, 1, seed=73)
    o, S = _gpu_fwd(gpu, d, 1, "norm+gates")
    heads = [(1, 3), (6, 12)]
    sub = {}
    for key, t in d.items():
        if t is None or key in ("A", "dt_bias"):
            sub[key] = t
        elif key == "S0":
            sub[key] = torch.stack([t[b, h] for b, h in heads])[:, None]
        else:
            sub[key] = torch.stack([t[b, :, h] for b, h in heads])[:, :, None]
    # each selected head keeps its own rate and bias
    A = np.array([d["A"][h].item() for _, h in heads])
    bias = np.array([d["dt_bias"][h].item() for _, h in heads])
    ro_list, rS_list = [], []
    for i, (b, h) in enumerate(heads):
        one = {k: (None if v is None else v[i:i + 1]) for k, v in sub.items()
               if k not in ("A", "dt_bias")}
        ro, rS = P.gdn_fwd(one["q"], one["k"], one["v"], one["alpha"], one["beta"], one["S0"],
                           mode=1, eps=EPS, l2norm_qk=True, beta_logits=True, alpha_logits=True,
                           A=A[i:i + 1], dt_bias=bias[i:i + 1])
        ro_list.append(ro)
        rS_list.append(rS)
    ro, rS = np.concatenate(ro_list), np.concatenate(rS_list)
    og = np.stack([o[b, :, h] for b, h in heads])[:, :, None]
    Sg = np.stack([S[b, h] for b, h in heads])[:, None]
    eo, eS = W.per_head_rel_err(og, ro, (0, 2)), W.per_head_rel_err(Sg, rS, (0, 1))
    print("fused gdn bf16 b8 h16 t4096: rel err o %.2e S %.2e" % (eo, eS), flush=True)
    assert eo <= 2e-2 and eS <= 2e-2


@pytest.mark.parametrize("which", ["norm+gates", "norm", "gates"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 128)])
def test_fused_decode(gpu, which, dtype, mode, dk, dv):
    B, H = 3, 4
    d = _inputs(B, 1, H, dk, dv, dtype, mode, 80 + dk, which)
    S = 0.1 * torch.randn(B, H, dv, dk, generator=torch.Generator().manual_seed(81))
    x = {k: (None if (v is None or k in ("A", "dt_bias", "S0")) else v[:, 0]) for k, v in d.items()}
    g = _dev(x)
    Sg = S.cuda()
    f = _flags(which)
    o = gpu.decode_step_fused(g["q"], g["k"], g["v"], g["alpha"], g["beta"], Sg, mode=mode,
                              eps=EPS, A=None if d["A"] is None else d["A"].cuda(),
                              dt_bias=None if d["dt_bias"] is None else d["dt_bias"].cuda(), **f)
    torch.cuda.synchronize()
    A = None if d["A"] is None else d["A"].numpy()
    bias = None if d["dt_bias"] is None else d["dt_bias"].numpy()
    ro, rS = P.gdn_decode(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S, mode=mode, eps=EPS,
                          A=A, dt_bias=bias, **f)
    eo = W.per_head_rel_err(o.float().cpu().numpy()[:, :, None], ro[:, :, None], (0, 1))
    eS = W.per_head_rel_err(Sg.cpu().numpy(), rS, (0, 1))
    assert eo <= TOL[dtype] and eS <= TOL[dtype], (eo, eS)
