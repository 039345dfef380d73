"""The Python binding rejects tensors whose shapes disagree with the sizes the
kernels derive from q and v (the C-ABI sees only pointers, so a short tensor
would be read or written past its end).  CPU only: the shape checks run before
the device checks, so a well-shaped CPU call gets as far as "must be a GPU
tensor" and an ill-shaped one stops at the shape."""
import pytest
import torch

import gated_delta_rule_04_amd as gdn

B, T, H, DK, DV = 2, 70, 3, 64, 128
BF = torch.bfloat16


def _prefill(mode=gdn.DECAY_SCALAR):
    z = lambda *s, dt=BF: torch.zeros(*s, dtype=dt)
    alpha = {gdn.DECAY_NONE: None, gdn.DECAY_SCALAR: z(B, T, H, dt=torch.float32),
             gdn.DECAY_CHANNEL: z(B, T, H, DK)}[mode]
    return dict(q=z(B, T, H, DK), k=z(B, T, H, DK), v=z(B, T, H, DV), alpha=alpha,
                beta=z(B, T, H, dt=torch.float32), S0=z(B, H, DV, DK, dt=torch.float32))


def _shape_error(fn, *a, **kw):
    with pytest.raises(ValueError) as e:
        fn(*a, **kw)
    return str(e.value)


@pytest.mark.parametrize("mode", [gdn.DECAY_NONE, gdn.DECAY_SCALAR, gdn.DECAY_CHANNEL])
def test_well_shaped_prefill_reaches_device_check(mode):
    d = _prefill(mode)
    msg = _shape_error(gdn.chunk_fwd, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], mode=mode)
    assert "GPU tensor" in msg


@pytest.mark.parametrize("name,bad", [
    ("k", (B, T, H, 2 * DK)), ("k", (B, T - 1, H, DK)), ("v", (B, T, H + 1, DV)),
    ("beta", (B, T)), ("beta", (B, T, H, 1)), ("alpha", (B, T, H, DK)), ("S0", (B + 1, H, DV, DK)),
    ("S0", (B, H, DK, DV // 2)),
])
def test_prefill_rejects_mismatched_shapes(name, bad):
    d = _prefill()
    d[name] = torch.zeros(*bad, dtype=d[name].dtype)
    msg = _shape_error(gdn.chunk_fwd, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                       mode=gdn.DECAY_SCALAR)
    assert name in msg and "shape" in msg


def test_prefill_rejects_small_outputs_and_workspace():
    d = _prefill()
    args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    assert "o must" in _shape_error(gdn.chunk_fwd, *args, o=torch.zeros(B, T, H, DV // 2, dtype=BF))
    assert "S_final" in _shape_error(gdn.chunk_fwd, *args,
                                     S_final=torch.zeros(B, H, DV, DK - 1))
    assert "workspace" in _shape_error(gdn.chunk_fwd, *args, workspace=torch.zeros(4))


def test_per_channel_alpha_needs_key_axis():
    d = _prefill(gdn.DECAY_CHANNEL)
    d["alpha"] = torch.zeros(B, T, H, dtype=BF)
    msg = _shape_error(gdn.chunk_fwd, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                       mode=gdn.DECAY_CHANNEL)
    assert "alpha" in msg


def test_varlen_shapes():
    d = _prefill()
    q, k, v = d["q"][0], d["k"][0], d["v"][0]
    cu = torch.tensor([0, 30, T], dtype=torch.int32)
    a, b = d["alpha"][0], d["beta"][0]
    assert "GPU tensor" in _shape_error(gdn.chunk_fwd_varlen, q, k, v, a, b, cu,
                                        torch.zeros(2, H, DV, DK))
    assert "S0" in _shape_error(gdn.chunk_fwd_varlen, q, k, v, a, b, cu, torch.zeros(3, H, DV, DK))
    assert "beta" in _shape_error(gdn.chunk_fwd_varlen, q, k, v, a, b[:-1], cu)
    assert "leading axis" in _shape_error(gdn.chunk_fwd_varlen, d["q"], d["k"], d["v"], d["alpha"],
                                          d["beta"], cu)


def test_fused_prologue_shapes():
    d = _prefill()
    args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    assert "A must" in _shape_error(gdn.chunk_fwd_fused, *args, alpha_logits=True,
                                    A=torch.ones(H + 1))
    assert "dt_bias" in _shape_error(gdn.chunk_fwd_fused, *args, alpha_logits=True, A=torch.ones(H),
                                     dt_bias=torch.zeros(H, DK))
    assert "rates A" in _shape_error(gdn.chunk_fwd_fused, *args, alpha_logits=True)
    assert "GPU tensor" in _shape_error(gdn.chunk_fwd_fused, *args, alpha_logits=True,
                                        A=torch.ones(H), dt_bias=torch.zeros(H))


def test_gdn2_shapes():
    d = _prefill(gdn.DECAY_CHANNEL)
    er = torch.zeros(B, T, H, DK, dtype=BF)
    wr = torch.zeros(B, T, H, DV, dtype=BF)
    args = (d["q"], d["k"], d["v"], d["alpha"])
    assert "GPU tensor" in _shape_error(gdn.gdn2_chunk_fwd, *args, er, wr, d["S0"])
    assert "write" in _shape_error(gdn.gdn2_chunk_fwd, *args, er, wr[..., :DK], d["S0"])
    assert "erase" in _shape_error(gdn.gdn2_chunk_fwd, *args, er[..., :1], wr, d["S0"])


def test_decode_shapes():
    q = torch.zeros(B, H, DK, dtype=BF)
    v = torch.zeros(B, H, DV, dtype=BF)
    a, b = torch.zeros(B, H), torch.zeros(B, H)
    S = torch.zeros(B, H, DV, DK)
    assert "GPU tensor" in _shape_error(gdn.decode_step, q, q, v, a, b, S)
    assert "S must" in _shape_error(gdn.decode_step, q, q, v, a, b, S[:, :, :, :DK // 2])
    assert "k must" in _shape_error(gdn.decode_step, q, q[:1], v, a, b, S)
    assert "o must" in _shape_error(gdn.decode_step, q, q, v, a, b, S,
                                    o=torch.zeros(B, H, DK, dtype=BF))
    assert "alpha" in _shape_error(gdn.decode_step, q, q, v, torch.zeros(B, H, DK, dtype=BF), b, S,
                                   mode=gdn.DECAY_SCALAR)
    er, wr = torch.zeros(B, H, DK, dtype=BF), torch.zeros(B, H, DV, dtype=BF)
    assert "write" in _shape_error(gdn.gdn2_decode_step, q, q, v, er, er, er, S)
    assert "GPU tensor" in _shape_error(gdn.gdn2_decode_step, q, q, v, er, er, wr, S)


def test_backward_shapes():
    d = _prefill()
    dout = torch.zeros(B, T, H, DV, dtype=BF)
    args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    assert "GPU tensor" in _shape_error(gdn.chunk_bwd, *args, dout)
    assert "o must" in _shape_error(gdn.chunk_bwd, *args, dout[:, :-1])
    assert "S_final" in _shape_error(gdn.chunk_bwd, *args, dout, torch.zeros(B, H, DV, 1))
