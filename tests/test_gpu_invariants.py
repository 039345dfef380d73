"""Properties of the recurrence checked on the GPU path alone, at any size.

For fixed q, k, alpha and beta the delta rule is linear in (S0, V): every state
update is S <- S (alpha I - beta k k^T) + beta v k^T and every output is S q.
The rows of S (one per value channel) evolve independently of each other
("On State Reduction in Linear Attention" notes, section 2.5), so permuting
the value channels permutes the outputs and the state rows and nothing else.
With a scalar gate a rotation R of the key space (q -> R q, k -> R k,
S0 -> S0 R^T) leaves the outputs unchanged and turns S_final into
S_final R^T (the same section: orthogonal invariance); a per-channel gate
breaks rotations but not permutations of the key channels that move alpha's
channels with them.

Bitwise where the arithmetic is provably unchanged (power-of-two scaling,
value-channel permutation, splitting a slice's chunks over several
workgroups), otherwise to the path's tolerance (fp32 rounding of the rotated
operands)."""
import pytest
import torch

import workloads as W
from gdn_testlib import TOL, to_dev

pytestmark = pytest.mark.gpu

SEED = 71


def _inputs(mode, dtype, B=2, H=3, T=300, dk=128, dv=128, seed=SEED):
    gate = {0: "none", 1: "exp01", 2: "kda_clamped"}[mode]
    return W.make_prefill(W.Prefill("inv", B, H, T, dk, dv, dtype, gate, 0.1, seed))


def _run(gpu, inp, mode):
    d = to_dev(inp)
    o, S = gpu.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], mode=mode)
    torch.cuda.synchronize()
    return o.float().cpu(), S.cpu()


def _rel(x, ref):
    return ((x - ref).abs().max() / ref.abs().max().clamp_min(1e-30)).item()


@pytest.mark.parametrize("mode", [1, 2])
def test_linear_in_state_and_values_fp32(gpu, mode):
    """o(S0a + S0b, Va + Vb) = o(S0a, Va) + o(S0b, Vb), likewise S_final."""
    a = _inputs(mode, torch.float32, seed=SEED)
    b = _inputs(mode, torch.float32, seed=SEED + 1)
    s = dict(a, v=a["v"] + b["v"], S0=a["S0"] + b["S0"])
    b = dict(a, v=b["v"], S0=b["S0"])   # same q, k, gates as a
    oa, Sa = _run(gpu, a, mode)
    ob, Sb = _run(gpu, b, mode)
    os_, Ss = _run(gpu, s, mode)
    assert _rel(oa + ob, os_) <= TOL[torch.float32]
    assert _rel(Sa + Sb, Ss) <= TOL[torch.float32]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_power_of_two_scaling_is_exact(gpu, dtype, mode):
    """Scaling S0 and V by 4 scales every product, rounding and output by 4 exactly."""
    a = _inputs(mode, dtype)
    s = dict(a, v=a["v"] * 4, S0=a["S0"] * 4)
    oa, Sa = _run(gpu, a, mode)
    os_, Ss = _run(gpu, s, mode)
    assert torch.equal(oa * 4, os_) and torch.equal(Sa * 4, Ss)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("mode", [1, 2])
def test_value_channels_are_independent(gpu, dtype, mode):
    """Permuting the value channels (V columns, S0 rows) permutes o's columns and
    S_final's rows, bit for bit."""
    a = _inputs(mode, dtype)
    perm = torch.randperm(a["v"].shape[-1], generator=torch.Generator().manual_seed(3))
    p = dict(a, v=a["v"][..., perm].contiguous(), S0=a["S0"][:, :, perm].contiguous())
    oa, Sa = _run(gpu, a, mode)
    op, Sp = _run(gpu, p, mode)
    assert torch.equal(oa[..., perm], op) and torch.equal(Sa[:, :, perm], Sp)


@pytest.mark.parametrize("mode", [0, 1])
def test_key_rotation_invariance_gdn_fp32(gpu, mode):
    """Scalar or no gate: q, k rotated by an orthogonal R and S0 by R^T leave o
    unchanged and give S_final R^T."""
    a = _inputs(mode, torch.float32)
    dk = a["q"].shape[-1]
    g = torch.Generator().manual_seed(5)
    R, _ = torch.linalg.qr(torch.randn(dk, dk, generator=g, dtype=torch.float64))
    rot = lambda x: (x.double() @ R.T).float().contiguous()   # rows x -> R x
    r = dict(a, q=rot(a["q"]), k=rot(a["k"]), S0=(a["S0"].double() @ R.T).float().contiguous())
    oa, Sa = _run(gpu, a, mode)
    orr, Sr = _run(gpu, r, mode)
    assert _rel(orr, oa) <= TOL[torch.float32]
    assert _rel(Sr, (Sa.double() @ R.T).float()) <= TOL[torch.float32]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_key_channel_permutation_kda(gpu, dtype):
    """Per-channel gate: permuting the key channels of q, k, alpha and S0's
    columns leaves o unchanged and permutes S_final's columns (the sums are
    taken in another order, so to the path's tolerance)."""
    a = _inputs(2, dtype)
    dk = a["q"].shape[-1]
    perm = torch.randperm(dk, generator=torch.Generator().manual_seed(7))
    pk = lambda x: x[..., perm].contiguous()
    p = dict(a, q=pk(a["q"]), k=pk(a["k"]), alpha=pk(a["alpha"]), S0=pk(a["S0"]))
    oa, Sa = _run(gpu, a, 2)
    op, Sp = _run(gpu, p, 2)
    assert _rel(op, oa) <= TOL[dtype]
    assert _rel(Sp, Sa[..., perm]) <= TOL[dtype]


@pytest.mark.parametrize("mode", [1, 2])
def test_chunk_split_over_workgroups_is_bitwise(gpu, mode):
    """With few heads a value slice is split over several workgroups, each
    reaching its first chunk's state by the state recurrence alone.  One head
    alone (split) against the same head inside a batch large enough to need no
    split: identical bits."""
    big = _inputs(mode, torch.bfloat16, B=4, H=64, T=1000, dk=128, dv=128, seed=SEED + 2)
    one = {k: (None if v is None else (v[:1, :, :1] if k != "S0" else v[:1, :1]).contiguous())
           for k, v in big.items()}
    ob, Sb = _run(gpu, big, mode)
    o1, S1 = _run(gpu, one, mode)
    assert torch.equal(ob[:1, :, :1], o1) and torch.equal(Sb[:1, :1], S1)
