"""The seeded generators: deterministic, and with the stated distributions."""
import numpy as np
import torch

import workloads as W


def _small(w, **kw):
    return w.with_(**kw)


def test_prefill_generator_is_deterministic():
    w = _small(W.GDN_BF16_PREFILL, B=1, H=2, T=70)
    a, b = W.make_prefill(w), W.make_prefill(w)
    for key in a:
        assert W.sha256(a[key]) == W.sha256(b[key])
    c = W.make_prefill(w.with_(seed=9))
    assert W.sha256(c["q"]) != W.sha256(a["q"])


def test_prefill_distributions():
    w = _small(W.GDN_BF16_PREFILL, B=2, H=4, T=512)
    d = W.make_prefill(w)
    n = torch.linalg.vector_norm(d["q"].float(), dim=-1)
    assert torch.all((n - 1).abs() < 1e-2)           # unit before the bf16 rounding
    assert d["q"].dtype == torch.bfloat16 and d["beta"].dtype == torch.float32
    assert torch.all((d["alpha"] > 0.9) & (d["alpha"] < 1.0))
    assert torch.all((d["beta"] > 0) & (d["beta"] < 1))
    assert abs(float(d["S0"].std()) - 0.1) < 0.01
    dl = W.make_prefill(_small(W.GDN_BF16_LONG, H=2, T=256))
    assert torch.all((dl["alpha"] > 0.95) & (dl["alpha"] < 1.0)) and dl["S0"] is None


def test_kda_gate_recipe():
    d = W.make_prefill(_small(W.KDA_BF16_PREFILL, B=1, H=2, T=256))
    a = d["alpha"].float()
    assert d["alpha"].dtype == torch.bfloat16 and a.shape == (1, 256, 2, 128)
    assert torch.all((a >= 0.8) & (a <= 1.0))
    assert 0.93 < float(a.median()) < 0.97
    lit = W.make_prefill(_small(W.KDA_BF16_PREFILL, B=1, H=1, T=64).with_(gate="kda_literal"))
    assert 0.03 < float(lit["alpha"].float().median()) < 0.07


def test_decode_generator_shapes():
    w = W.DECODE_DK64.with_(B=2, H=3, steps=5)
    d = W.make_decode(w)
    assert d["q"].shape == (5, 2, 3, 64) and d["v"].shape == (5, 2, 3, 128)
    assert d["S"].shape == (2, 3, 128, 64) and d["alpha"].shape == (5, 2, 3)


def test_rel_err_per_head():
    ref = np.ones((2, 3, 4, 5))
    x = ref.copy()
    x[1, :, 2] += 0.5
    assert W.per_head_rel_err(x, ref, (0, 2)) == 0.5
    x[0, 0, 0, 0] = np.nan
    assert W.per_head_rel_err(x, ref, (0, 2)) == float("inf")


def test_packed_lengths_and_offsets():
    """The packed split covers the token count exactly, every row has at least
    min_len tokens, the mix is broad, and the offsets are its prefix sums."""
    w = W.GDN_BF16_PACKED
    lens = W.packed_lengths(w)
    assert len(lens) == w.N and sum(lens) == w.T and min(lens) >= w.min_len
    assert max(lens) > 4 * min(lens)
    d = W.make_packed(w.with_(T=1000, N=7))
    cu = d["cu_seqlens"]
    assert cu.dtype == torch.int32 and int(cu[0]) == 0 and int(cu[-1]) == 1000
    assert torch.all(cu[1:] >= cu[:-1])
    assert d["q"].shape == (1, 1000, 16, 128) and d["S0"].shape == (7, 16, 128, 128)
    assert W.packed_lengths(w.with_(lengths=(3, 0, 5), N=3, T=8)) == [3, 0, 5]


def test_prologue_generator_recipe():
    """Raw q, k are not normalised; softplus(dt_bias) is the drawn dt in
    [1e-3, 1e-1]; the rates lie in [1, 16]."""
    d = W.make_prologue(2, 64, 3, 128, 64, torch.bfloat16, W.MODE_SCALAR, seed=9)
    n = torch.linalg.vector_norm(d["q"].float(), dim=-1)
    assert float(n.std()) > 1.0
    dt = torch.nn.functional.softplus(d["dt_bias"])
    assert torch.all((dt > 0.99e-3) & (dt < 1.01e-1))
    assert torch.all((d["A"] >= 1) & (d["A"] <= 16)) and d["A"].shape == (3,)
    dc = W.make_prologue(1, 8, 2, 64, 64, torch.float32, W.MODE_CHANNEL, seed=9)
    assert dc["alpha"].shape == (1, 8, 2, 64) and dc["dt_bias"].shape == (2, 64)
    assert W.make_prologue(1, 8, 2, 64, 64, torch.float32, W.MODE_NONE, seed=9)["A"] is None


def test_gdn2_generator_gates():
    w = W.KDA_BF16_PREFILL.with_(B=1, H=2, T=32)
    d = W.make_gdn2(w)
    assert d["beta"] is None and d["erase"].shape == (1, 32, 2, 128) and d["write"].shape == (1, 32, 2, 128)
    for g in (d["erase"].float(), d["write"].float()):
        assert torch.all((g > 0) & (g < 1))
