"""GPU parity of Gated DeltaNet-2 (separate erase and write gates) against the
fp64 oracle's mode 3, per (b, h) slice max|x - ref| / max|ref|."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gdn_testlib import TOL

pytestmark = pytest.mark.gpu


def _dev(d):
    return {k: (None if v is None else v.cuda()) for k, v in d.items()}


def _gpu(gdn, d, cu=None):
    g = _dev(d)
    o, S = gdn.gdn2_chunk_fwd(g["q"], g["k"], g["v"], g["alpha"], g["erase"], g["write"], g["S0"],
                              cu_seqlens=None if cu is None else cu.cuda())
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy()


def _ref(d, cu=None):
    if cu is None:
        return oracle.gdn_fwd(d["q"], d["k"], d["v"], d["alpha"], None, d["S0"],
                              mode=oracle.MODE_GDN2, erase=d["erase"], write=d["write"])
    return oracle.gdn_fwd_varlen(d["q"], d["k"], d["v"], d["alpha"], None, cu, d["S0"],
                                 mode=oracle.MODE_GDN2, erase=d["erase"], write=d["write"])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 64), (64, 128)])
@pytest.mark.parametrize("T", [1, 63, 65, 130])
@pytest.mark.parametrize("gate", ["exp01_channel", "kda_literal"])
def test_gdn2_small(gpu, dtype, dk, dv, T, gate):
    w = W.Prefill("gdn2", 2, 3, T, dk, dv, dtype, gate, 0.2, seed=90 + T)
    d = W.make_gdn2(w)
    print("gdn2 %s dk %d dv %d T %d %s" % (dtype, dk, dv, T, gate), flush=True)
    o, S = _gpu(gpu, d)
    ro, rS = _ref(d)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    eo, eS = W.per_head_rel_err(o, ro, (0, 2)), W.per_head_rel_err(S, rS, (0, 1))
    assert eo <= TOL[dtype] and eS <= TOL[dtype], (eo, eS)


def test_gdn2_with_beta_gates_is_the_channel_rule(gpu):
    """erase = write = beta on every channel gives the per-channel (KDA) path's
    result (different kernels' arithmetic: compared to the bf16 tolerance)."""
    w = W.Prefill("kda", 2, 3, 200, 128, 128, torch.bfloat16, "exp01_channel", 0.1, seed=97)
    d = W.make_prefill(w)
    g = _dev(d)
    o1, S1 = gpu.chunk_fwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["S0"], mode=2)
    e = g["beta"][..., None].expand(-1, -1, -1, 128).contiguous().to(torch.bfloat16)
    o2, S2 = gpu.gdn2_chunk_fwd(g["q"], g["k"], g["v"], g["alpha"], e, e, g["S0"])
    torch.cuda.synchronize()
    # beta rounded to bf16 for the gates: compare with the oracle on those gates too
    eo = W.per_head_rel_err(o2.float().cpu().numpy(), o1.float().cpu().numpy(), (0, 2))
    eS = W.per_head_rel_err(S2.cpu().numpy(), S1.cpu().numpy(), (0, 1))
    assert eo <= 2e-2 and eS <= 2e-2, (eo, eS)


def test_gdn2_packed(gpu):
    lens = (100, 0, 1, 64, 129)
    T = sum(lens)
    w = W.Prefill("gdn2p", 1, 2, T, 128, 128, torch.bfloat16, "exp01_channel", 0.0, seed=98)
    d = W.make_gdn2(w)
    d["S0"] = 0.1 * torch.randn(len(lens), 2, 128, 128, generator=torch.Generator().manual_seed(99))
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    o, S = _gpu(gpu, d, cu)
    ro, rS = _ref(d, cu)
    eo = max(W.per_head_rel_err(o[:, a:b], ro[:, a:b], (0, 2))
             for a, b in zip(cu[:-1].tolist(), cu[1:].tolist()) if b > a)
    eS = W.per_head_rel_err(S, rS, (0, 1))
    assert eo <= 2e-2 and eS <= 2e-2, (eo, eS)


def test_gdn2_workload_sampled(gpu):
    """B=4, H=16, T=8192, d=128, bf16 with the clamped per-channel decay and
    sigmoid erase / write gates: two heads against the oracle."""
    w = W.KDA_BF16_PREFILL.with_(seed=100)
    d = W.make_gdn2(w)
    o, S = _gpu(gpu, d)
    heads = [(0, 5), (3, 14)]
    sub = {}
    for key, t in d.items():
        if t is None:
            sub[key] = None
        elif key == "S0":
            sub[key] = torch.stack([t[b, h] for b, h in heads])[:, None]
        else:
            sub[key] = torch.stack([t[b, :, h] for b, h in heads])[:, :, None]
    ro, rS = _ref(sub)
    og = np.stack([o[b, :, h] for b, h in heads])[:, :, None]
    Sg = np.stack([S[b, h] for b, h in heads])[:, None]
    eo, eS = W.per_head_rel_err(og, ro, (0, 2)), W.per_head_rel_err(Sg, rS, (0, 1))
    print("gdn2 bf16 b4 h16 t8192: rel err o %.2e S %.2e" % (eo, eS), flush=True)
    assert eo <= 2e-2 and eS <= 2e-2


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 128), (128, 64)])
def test_gdn2_decode(gpu, dtype, dk, dv):
    w = W.Prefill("gdn2d", 3, 4, 1, dk, dv, dtype, "exp01_channel", 0.0, seed=101)
    d = W.make_gdn2(w)
    x = {k: (None if v is None else v[:, 0]) for k, v in d.items() if k != "S0"}
    S = 0.1 * torch.randn(3, 4, dv, dk, generator=torch.Generator().manual_seed(102))
    g = _dev(x)
    Sg = S.cuda()
    o = gpu.gdn2_decode_step(g["q"], g["k"], g["v"], g["alpha"], g["erase"], g["write"], Sg)
    torch.cuda.synchronize()
    ro, rS = oracle.gdn_decode(x["q"], x["k"], x["v"], x["alpha"], None, S, mode=oracle.MODE_GDN2,
                               erase=x["erase"], write=x["write"])
    eo = W.per_head_rel_err(o.float().cpu().numpy()[:, :, None], ro[:, :, None], (0, 1))
    eS = W.per_head_rel_err(Sg.cpu().numpy(), rS, (0, 1))
    assert eo <= TOL[dtype] and eS <= TOL[dtype], (eo, eS)


def test_gdn2_prefill_matches_decode_steps(gpu):
    """T decode steps give the prefill's outputs and state."""
    w = W.Prefill("gdn2s", 2, 2, 20, 128, 128, torch.float32, "exp01_channel", 0.1, seed=103)
    d = W.make_gdn2(w)
    o, S = _gpu(gpu, d)
    g = _dev(d)
    St = g["S0"].clone()
    for t in range(w.T):
        ot = gpu.gdn2_decode_step(g["q"][:, t].contiguous(), g["k"][:, t].contiguous(),
                                  g["v"][:, t].contiguous(), g["alpha"][:, t].contiguous(),
                                  g["erase"][:, t].contiguous(), g["write"][:, t].contiguous(), St)
        torch.cuda.synchronize()
        assert W.per_head_rel_err(ot.cpu().numpy()[:, :, None], o[:, t][:, :, None], (0, 1)) < 1e-4
    assert W.per_head_rel_err(St.cpu().numpy(), S, (0, 1)) < 1e-4
