"""64-row value slices under per-channel decay and Gated DeltaNet-2.

The bf16 state kernel takes 64 value rows per workgroup for per-channel decay
once B * H * d_v / 64 reaches 128 (below 256 each slice runs in two parts along
the sequence, the second led in from chunk 0), and for Gated DeltaNet-2 once
it reaches 256; with 64-row slices its Q and phase-1 K rows have a single LDS
buffer.  These cases take that path on every head size and check sampled
heads against the oracle; every output is checked finite."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gdn_testlib import check_prefill, select_heads, to_dev

pytestmark = pytest.mark.gpu


def _heads(B, H):
    """Eight (b, h) heads spread over the batch."""
    return sorted({(i % B, (37 * i + 5) % H) for i in range(8)})


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
@pytest.mark.parametrize("slices,B,T", [(256, 2, 130), (128, 1, 700)], ids=["one_part", "two_parts"])
def test_kda_wide_slices(gpu, dk, dv, slices, B, T):
    H = slices * 64 // (B * dv)
    w = W.Prefill("kda_wide", B, H, T, dk, dv, torch.bfloat16, "exp01_channel", 0.1, seed=120 + T + dk)
    print("kda wide slices B %d H %d T %d dk %d dv %d" % (B, H, T, dk, dv), flush=True)
    eo, eS = check_prefill(gpu, W.make_prefill(w), 2, torch.bfloat16, heads=_heads(B, H))
    print("  rel err o %.2e, S_final %.2e" % (eo, eS))


def test_kda_wide_slices_literal_gate(gpu):
    """The literal gate (most channels decay by far more than e^64 within a
    chunk: the prep kernel's exact path) with 64-row slices in two parts."""
    w = W.Prefill("kda_wide_lit", 1, 64, 300, 128, 128, torch.bfloat16, "kda_literal", 0.1, seed=131)
    eo, eS = check_prefill(gpu, W.make_prefill(w), 2, torch.bfloat16, heads=_heads(1, 64))
    print("  rel err o %.2e, S_final %.2e" % (eo, eS))


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128)])
@pytest.mark.parametrize("T", [130, 300])
def test_gdn2_wide_slices(gpu, dk, dv, T):
    B, H = 2, 64   # 256 slices of 64 value rows
    w = W.Prefill("gdn2_wide", B, H, T, dk, dv, torch.bfloat16, "exp01_channel", 0.1, seed=140 + T)
    d = W.make_gdn2(w)
    g = to_dev(d)
    print("gdn2 wide slices T %d dk %d dv %d" % (T, dk, dv), flush=True)
    o, S = gpu.gdn2_chunk_fwd(g["q"], g["k"], g["v"], g["alpha"], g["erase"], g["write"], g["S0"])
    torch.cuda.synchronize()
    o, S = o.float().cpu().numpy(), S.cpu().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    heads = _heads(B, H)
    sub = select_heads({k: v for k, v in d.items() if k not in ("erase", "write")}, heads)
    for key in ("erase", "write"):
        sub[key] = torch.stack([d[key][b, :, h] for b, h in heads])[:, :, None]
    ro, rS = oracle.gdn_fwd(sub["q"], sub["k"], sub["v"], sub["alpha"], None, sub["S0"],
                            mode=oracle.MODE_GDN2, erase=sub["erase"], write=sub["write"])
    og = np.stack([o[b, :, h] for b, h in heads])[:, :, None]
    Sg = np.stack([S[b, h] for b, h in heads])[:, None]
    eo, eS = W.per_head_rel_err(og, ro, (0, 2)), W.per_head_rel_err(Sg, rS, (0, 1))
    print("  rel err o %.2e, S_final %.2e" % (eo, eS))
    assert eo <= 2e-2 and eS <= 2e-2, (eo, eS)


def test_kda_wide_slices_repeat_bitwise(gpu):
    """Two calls on the same inputs give the same bits (64-row slices in two
    parts: no races between the single-buffered rows and their readers)."""
    w = W.Prefill("kda_wide_rep", 1, 64, 700, 128, 128, torch.bfloat16, "exp01_channel", 0.1, seed=150)
    g = to_dev(W.make_prefill(w))
    outs = [gpu.chunk_fwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["S0"], mode=2) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
