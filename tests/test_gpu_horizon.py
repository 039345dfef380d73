"""Split value slices with lead-ins from the history horizon (scalar decay).

With few heads each value slice is split into parts along the sequence; a part
reaches its starting state by a lead-in that runs the state recurrence alone.
Every token's transition S -> alpha S (I - beta k k^T) has norm at most alpha
for |k| = 1 and beta in [0, 1], so the state at chunk m depends on the state
at chunk s only through a factor of norm at most exp(sum of log alpha over
[s, m)).  Once that sum is below -40 the lead-in may start at s from a zero
state.  These cases take that path (few heads, long sequences, decaying
gates) and check it against the oracle and against the unsplit pass."""
import numpy as np
import pytest
import torch

import workloads as W
from gdn_testlib import TOL, check_prefill, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("gate", ["exp01", "exp1", "range090"])
def test_horizon_split_against_oracle(gpu, gate):
    """B=1, H=4, T=8192, bf16, S0 drawn (std 0.1): every head against the oracle.
    A part whose lead-in starts past chunk 0 ignores S0, which the decay has
    scaled far below fp32 resolution there."""
    w = W.Prefill("horizon", 1, 4, 8192, 128, 128, torch.bfloat16, gate, 0.1, seed=81)
    print("horizon split %s" % gate, flush=True)
    eo, eS = check_prefill(gpu, W.make_prefill(w), w.mode, w.dtype)
    print("  rel err o %.2e, S_final %.2e" % (eo, eS))


@pytest.mark.parametrize("dv", [128, 64])
def test_horizon_split_matches_unsplit(gpu, dv):
    """One head alone (split into parts with short lead-ins) against the same head
    inside a batch large enough to need no split: equal to far below the bf16
    tolerance (the neglected history is below e^-40 of the state)."""
    big = W.make_prefill(W.Prefill("hz", 2, 128, 2048, 128, dv, torch.bfloat16, "exp1", 0.1, seed=82))
    one = {k: (None if v is None else (v[:1, :, :1] if k != "S0" else v[:1, :1]).contiguous())
           for k, v in big.items()}
    print("horizon vs unsplit dv=%d" % dv, flush=True)
    d, d1 = to_dev(big), to_dev(one)
    ob, Sb = gpu.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], mode=1)
    o1, S1 = gpu.chunk_fwd(d1["q"], d1["k"], d1["v"], d1["alpha"], d1["beta"], d1["S0"], mode=1)
    torch.cuda.synchronize()
    ob, Sb = ob[:1, :, :1].float().cpu(), Sb[:1, :1].cpu()
    o1, S1 = o1.float().cpu(), S1.cpu()
    eo = ((o1 - ob).abs().max() / ob.abs().max()).item()
    eS = ((S1 - Sb).abs().max() / Sb.abs().max()).item()
    print("  rel diff o %.2e, S_final %.2e, bitwise %s" % (eo, eS, torch.equal(o1, ob) and torch.equal(S1, Sb)))
    assert eo <= 1e-5 and eS <= 1e-5


def test_horizon_split_packed_rows(gpu):
    """Packed rows (lengths 5000, 3000, 77, 1300) on four heads, strong decay:
    the per-row parts take their lead-ins from the row's own bounds."""
    import oracle
    from test_gpu_varlen import _check
    w = W.Packed("horizon_packed", 4, 9377, 4, 128, 128, torch.bfloat16, "exp01", 0.1, seed=83,
                 lengths=(5000, 3000, 77, 1300))
    eo, eS = _check(gpu, w)
    print("  rel err o %.2e, S_final %.2e" % (eo, eS))
