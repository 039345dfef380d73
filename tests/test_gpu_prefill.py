"""Chunked prefill on the GPU against the fp64 oracle (DeltaNet, Gated DeltaNet and
per-channel decay)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gdn_testlib import TOL, check_prefill, gpu_prefill, oracle_prefill, rel_o, rel_S, to_dev

pytestmark = pytest.mark.gpu

GATE_OF_MODE = {0: "none", 1: "exp01", 2: "kda_clamped"}


def _small(T, dk, dv, dtype, mode, s0, B=1, H=2, seed=5):
    return W.Prefill("small", B, H, T, dk, dv, dtype, GATE_OF_MODE[mode], 0.1 if s0 else 0.0, seed)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 130, 200])
def test_prefill_small(gpu, dtype, mode, dk, dv, T):
    w = _small(T, dk, dv, dtype, mode, s0=(T % 2 == 1), seed=T + dk)
    check_prefill(gpu, W.make_prefill(w), mode, dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("dk", [64, 128])
@pytest.mark.parametrize("mode", [1, 2])
def test_prefill_wide_slices(gpu, dtype, dk, mode):
    """Enough heads for 64-row value slices per workgroup."""
    w = _small(130, dk, 64, dtype, mode, s0=True, B=4, H=64, seed=9)
    check_prefill(gpu, W.make_prefill(w), mode, dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("gate", ["exp01_channel", "kda_literal"])
@pytest.mark.parametrize("dk,T", [(64, 200), (128, 130), (128, 256)])
def test_prefill_channel_gates(gpu, dtype, gate, dk, T):
    """Per-channel decay with mild gates and with the strong literal gate (typical
    alpha about 0.05: decay ratios span many orders of magnitude inside a chunk)."""
    w = W.Prefill("kda", 2, 3, T, dk, 128, dtype, gate, 0.1, seed=T + dk + 7)
    check_prefill(gpu, W.make_prefill(w), 2, dtype)


def test_prefill_channel_decay_equal_channels_is_scalar_decay(gpu):
    """A per-channel gate equal across channels is the scalar gate: the GPU's
    per-channel path against the oracle run in scalar mode."""
    w = _small(200, 128, 128, torch.float32, 2, s0=True, B=2, H=3, seed=31)
    inp = W.make_prefill(w)
    a1 = inp["alpha"][..., 0].contiguous()
    inp["alpha"] = a1[..., None].expand_as(inp["alpha"]).contiguous()
    o, S = gpu_prefill(gpu, inp, 2)
    ro, rS = oracle_prefill(dict(inp, alpha=a1), 1)
    assert rel_o(o, ro) <= 1e-4 and rel_S(S, rS) <= 1e-4


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("dk", [64, 128])
def test_prefill_channel_gates_at_boundary_values(gpu, dtype, dk):
    """Per-channel alpha in {0, 1} mixed across channels and tokens (hard resets of
    single channels), alpha = 0 everywhere, tiny alpha, then alpha = 1 with beta = 0."""
    w = _small(150, dk, 128, dtype, 2, s0=True, B=1, H=2, seed=32)
    inp = W.make_prefill(w)
    g = torch.Generator().manual_seed(33)
    inp["alpha"] = (torch.rand(inp["alpha"].shape, generator=g) < 0.7).to(dtype)
    check_prefill(gpu, inp, 2, dtype)
    inp["alpha"] = torch.zeros_like(inp["alpha"])
    check_prefill(gpu, inp, 2, dtype)
    inp["alpha"] = torch.where(torch.rand(inp["alpha"].shape, generator=g) < 0.9, 1.0, 1e-30).to(dtype)
    check_prefill(gpu, inp, 2, dtype)
    inp["alpha"] = torch.ones_like(inp["alpha"])
    inp["beta"] = torch.zeros_like(inp["beta"])
    _, S = gpu_prefill(gpu, inp, 2)
    assert rel_S(S, inp["S0"].numpy()) <= 1e-6


def test_prefill_kda_workload_sampled(gpu):
    """B=4, H=16, T=8192, d=128, bf16, per-channel decay: all heads on the GPU,
    eight checked (outputs and final states)."""
    w = W.KDA_BF16_PREFILL
    heads = [(0, 0), (0, 11), (1, 2), (1, 9), (2, 4), (2, 13), (3, 6), (3, 15)]
    eo, eS = check_prefill(gpu, W.make_prefill(w), w.mode, w.dtype, heads=heads)
    print("kda bf16 b4 h16 t8192: rel err o %.2e, S %.2e" % (eo, eS))


def test_prefill_gdn_fp32_workload(gpu):
    """B=1, H=2, T=256, d=64, fp32, S0=0: the whole output against the oracle."""
    w = W.GDN_FP32_SMALL
    eo, eS = check_prefill(gpu, W.make_prefill(w), w.mode, w.dtype)
    print("gdn fp32 b1 h2 t256 d64: rel err o %.2e, S %.2e" % (eo, eS))


def test_prefill_gdn_bf16_workload_sampled(gpu):
    """B=8, H=16, T=4096, d=128, bf16, random S0: all heads on the GPU, four checked."""
    w = W.GDN_BF16_PREFILL
    heads = [(0, 0), (3, 7), (5, 12), (7, 15)]
    eo, eS = check_prefill(gpu, W.make_prefill(w), w.mode, w.dtype, heads=heads)
    print("gdn bf16 b8 h16 t4096: rel err o %.2e, S %.2e" % (eo, eS))


def test_prefill_long_context_and_decode_handoff(gpu):
    """B=1, H=32, T=65536, d=128, bf16: eight heads checked (outputs and the
    final state itself), then one decode step from the GPU's final state against
    the oracle's decode from its own."""
    w = W.GDN_BF16_LONG
    inp = W.make_prefill(w)
    heads = [(0, h) for h in (0, 3, 7, 12, 17, 22, 27, 30)]
    dev = to_dev(inp)
    o, S = gpu.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["S0"])
    torch.cuda.synchronize()
    S_fin = S[0].cpu().numpy()   # the decode step below updates S in place
    tok = W.make_decode(W.Decode("next", 1, 32, 128, 128, 1, torch.bfloat16, "range095", 0.0, 55))
    o1 = gpu.decode_step(tok["q"][0].cuda(), tok["k"][0].cuda(), tok["v"][0].cuda(),
                         tok["alpha"][0].cuda(), tok["beta"][0].cuda(), S)
    torch.cuda.synchronize()
    from gdn_testlib import select_heads
    ro, rS = oracle_prefill(select_heads(inp, heads), w.mode)
    o_s = np.stack([o[0, :, h].float().cpu().numpy() for _, h in heads])[:, :, None]
    eo = rel_o(o_s, ro)
    hs = [h for _, h in heads]
    nh = len(hs)
    eSf = rel_S(S_fin[hs][:, None], rS)
    ro1, rS1 = oracle.gdn_decode(tok["q"][0][:, hs].reshape(nh, 1, 128), tok["k"][0][:, hs].reshape(nh, 1, 128),
                                 tok["v"][0][:, hs].reshape(nh, 1, 128), tok["alpha"][0][:, hs].reshape(nh, 1),
                                 tok["beta"][0][:, hs].reshape(nh, 1), rS, mode=1)
    S_s = S[0, hs].cpu().numpy()[:, None]
    eS = rel_S(S_s, rS1)
    e1 = W.per_head_rel_err(o1[0, hs].float().cpu().numpy()[:, None], ro1, (0, 1))
    print("gdn bf16 b1 h32 t65536: rel err o %.2e, S_final %.2e, S after decode %.2e, decode o %.2e"
          % (eo, eSf, eS, e1))
    tol = TOL[torch.bfloat16]
    assert eo <= tol and eSf <= tol and eS <= tol and e1 <= tol


def test_prefill_empty_sequence_copies_state(gpu):
    w = _small(0, 128, 64, torch.bfloat16, 1, s0=True, B=2, H=3)
    inp = W.make_prefill(w)
    _, S = gpu_prefill(gpu, inp, 1)
    assert np.array_equal(S, inp["S0"].numpy())
    inp["S0"] = None
    _, S = gpu_prefill(gpu, inp, 1)
    assert np.array_equal(S, np.zeros_like(S))


def test_prefill_in_place_state_and_no_final(gpu):
    w = _small(150, 128, 128, torch.bfloat16, 1, s0=True, B=2, H=2)
    inp = W.make_prefill(w)
    dev = to_dev(inp)
    o1, S1 = gpu.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["S0"])
    S_io = dev["S0"].clone()
    o2, S2 = gpu.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], S_io, S_final=S_io)
    o3, S3 = gpu.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["S0"],
                           need_final=False)
    torch.cuda.synchronize()
    assert S3 is None
    assert torch.equal(S1, S_io) and torch.equal(o1, o2) and torch.equal(o1, o3)


@pytest.mark.parametrize("mode", [1, 2])
def test_prefill_split_equals_whole(gpu, mode):
    """prefill(T1) then prefill(T2, S0 = S_final) against the oracle over T1 + T2."""
    w = _small(257, 128, 128, torch.bfloat16, mode, s0=True, B=1, H=4)
    inp = W.make_prefill(w)
    dev = to_dev(inp)
    t1 = 100
    part = lambda x, s: None if x is None else x[:, s].contiguous()
    oa, Sa = gpu.chunk_fwd(part(dev["q"], slice(0, t1)), part(dev["k"], slice(0, t1)),
                           part(dev["v"], slice(0, t1)), part(dev["alpha"], slice(0, t1)),
                           part(dev["beta"], slice(0, t1)), dev["S0"])
    ob, Sb = gpu.chunk_fwd(part(dev["q"], slice(t1, None)), part(dev["k"], slice(t1, None)),
                           part(dev["v"], slice(t1, None)), part(dev["alpha"], slice(t1, None)),
                           part(dev["beta"], slice(t1, None)), Sa)
    torch.cuda.synchronize()
    ro, rS = oracle_prefill(inp, mode)
    o = torch.cat([oa, ob], 1).float().cpu().numpy()
    assert rel_o(o, ro) <= 2e-2 and rel_S(Sb.cpu().numpy(), rS) <= 2e-2


def test_prefill_is_deterministic(gpu):
    w = _small(300, 128, 128, torch.bfloat16, 1, s0=True, B=2, H=8)
    inp = to_dev(W.make_prefill(w))
    runs = [gpu.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"])
            for _ in range(3)]
    torch.cuda.synchronize()
    for o, S in runs[1:]:
        assert torch.equal(o, runs[0][0]) and torch.equal(S, runs[0][1])


@pytest.mark.parametrize("mode", [1, 2])
def test_prefill_matches_decode_steps(gpu, mode):
    """T decode steps and one prefill over the same T tokens agree."""
    w = _small(70, 64, 128, torch.float32, mode, s0=True, B=2, H=3)
    inp = W.make_prefill(w)
    o_p, S_p = gpu_prefill(gpu, inp, mode)
    dev = to_dev(inp)
    S = dev["S0"].clone()
    outs = []
    for t in range(w.T):
        outs.append(gpu.decode_step(dev["q"][:, t].contiguous(), dev["k"][:, t].contiguous(),
                                    dev["v"][:, t].contiguous(), dev["alpha"][:, t].contiguous(),
                                    dev["beta"][:, t].contiguous(), S))
    o_d = torch.stack(outs, 1).cpu().numpy()
    torch.cuda.synchronize()
    assert rel_o(o_d, o_p) <= 1e-4 and rel_S(S.cpu().numpy(), S_p) <= 1e-4


def test_prefill_gates_at_boundary_values(gpu):
    """alpha = 1 and beta = 0 leave the state as S0; alpha = 0 resets it each token."""
    w = _small(96, 128, 128, torch.float32, 1, s0=True, B=1, H=2)
    inp = W.make_prefill(w)
    inp["alpha"] = torch.ones_like(inp["alpha"])
    inp["beta"] = torch.zeros_like(inp["beta"])
    _, S = gpu_prefill(gpu, inp, 1)
    assert rel_S(S, inp["S0"].numpy()) <= 1e-6
    inp = W.make_prefill(w)
    inp["alpha"] = torch.zeros_like(inp["alpha"])
    check_prefill(gpu, inp, 1, torch.float32)
