"""GPU parity of the packed (variable-length) prefill against the fp64 oracle.

Every case runs ``gdn_chunk_fwd_varlen`` through the binding and compares each
(sequence, head) slice of o and S_final with ``oracle.gdn_fwd_varlen`` on the
same inputs: max|x - ref| / max|ref| per slice, worst slice within the
tolerance of the dtype.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gdn_testlib import TOL

pytestmark = pytest.mark.gpu


def _run(gdn, inp, mode, **kw):
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    o, S = gdn.chunk_fwd_varlen(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu_seqlens"],
                                d["S0"], mode=mode, **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), None if S is None else S.cpu().numpy()


def _ref(inp, mode):
    return oracle.gdn_fwd_varlen(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                 inp["cu_seqlens"], inp["S0"], mode=mode)


def _rel_seq(o, ro, S, rS, cu):
    """Worst (sequence, head) slice error of o [1, T, H, dv] and S [N, H, dv, dk]."""
    eo = 0.0
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b > a:
            eo = max(eo, W.per_head_rel_err(o[:, a:b], ro[:, a:b], (0, 2)))
    eS = W.per_head_rel_err(S, rS, (0, 1))
    return eo, eS


def _check(gdn, w, tol=None):
    inp = W.make_packed(w)
    print("packed case %s lengths %s mode %d" % (w.name, W.packed_lengths(w), w.mode), flush=True)
    o, S = _run(gdn, inp, w.mode)
    ro, rS = _ref(inp, w.mode)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    eo, eS = _rel_seq(o, ro, S, rS, inp["cu_seqlens"].tolist())
    tol = TOL[w.dtype] if tol is None else tol
    assert eo <= tol, "o rel err %.3e > %.1e" % (eo, tol)
    assert eS <= tol, "S_final rel err %.3e > %.1e" % (eS, tol)
    return eo, eS


GATE_OF_MODE = {0: "none", 1: "exp01", 2: "exp01_channel"}
# empty rows, single tokens, exact chunks, one past a chunk, a long row
MIXES = [(5, 0, 1, 64, 63, 65, 130, 0, 7), (200,), (64, 64, 64), (1, 1, 1, 1, 300)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 64)])
@pytest.mark.parametrize("mix", range(len(MIXES)))
def test_varlen_small(gpu, dtype, mode, dk, dv, mix):
    lens = MIXES[mix]
    w = W.Packed("packed_small", len(lens), sum(lens), 2, dk, dv, dtype, GATE_OF_MODE[mode],
                 0.3 if mix % 2 == 0 else 0.0, seed=40 + mix, lengths=lens)
    _check(gpu, w)


@pytest.mark.parametrize("mode", [1, 2])
def test_varlen_random_split(gpu, mode):
    """Seeded random split of 3000 tokens into 9 rows, bf16, d = 128."""
    w = W.Packed("packed_split", 9, 3000, 3, 128, 128, torch.bfloat16, GATE_OF_MODE[mode], 0.1,
                 seed=47)
    _check(gpu, w)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_varlen_equal_rows_match_batched_call(gpu, mode):
    """Rows of equal length packed back to back give exactly (bitwise) what the
    batched entry point gives on the same rows: the same chunks run through the
    same kernels in the same order."""
    B, T, H = 3, 130, 4
    pw = W.Prefill("rows", B, H, T, 128, 128, torch.bfloat16, GATE_OF_MODE[mode], 0.1, seed=48)
    inp = {k: (None if v is None else v.cuda()) for k, v in W.make_prefill(pw).items()}
    o, S = gpu.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"],
                         mode=mode)
    flat = lambda x: None if x is None else x.reshape((1, B * T) + tuple(x.shape[2:]))
    cu = torch.arange(0, B * T + 1, T, dtype=torch.int32, device="cuda")
    ov, Sv = gpu.chunk_fwd_varlen(flat(inp["q"]), flat(inp["k"]), flat(inp["v"]),
                                  flat(inp["alpha"]), flat(inp["beta"]), cu, inp["S0"], mode=mode)
    torch.cuda.synchronize()
    assert torch.equal(ov, flat(o)) and torch.equal(Sv, S)


def test_varlen_all_rows_empty_copies_states(gpu):
    """T = 0 with N rows: S_final = S0 per row (zeros without S0), no o."""
    N, H, dv, dk = 3, 2, 64, 128
    S0 = torch.randn(N, H, dv, dk, device="cuda")
    z = torch.empty(1, 0, H, dk, dtype=torch.bfloat16, device="cuda")
    v = torch.empty(1, 0, H, dv, dtype=torch.bfloat16, device="cuda")
    b = torch.empty(1, 0, H, device="cuda")
    cu = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    o, S = gpu.chunk_fwd_varlen(z, z, v, b, b, cu, S0, mode=1)
    torch.cuda.synchronize()
    assert o.shape == (1, 0, H, dv) and torch.equal(S, S0)
    _, S = gpu.chunk_fwd_varlen(z, z, v, None, b, cu, None, mode=0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(S) == 0


def test_varlen_packed_workload_sampled(gpu):
    """The 16-row packed workload (32768 tokens, H=16, d=128, bf16): every row of
    two heads checked against the oracle."""
    w = W.GDN_BF16_PACKED
    inp = W.make_packed(w)
    print("packed workload %s lengths %s" % (w.name, W.packed_lengths(w)), flush=True)
    o, S = _run(gpu, inp, w.mode)
    heads = [3, 12]
    sub = {}
    for k, t in inp.items():
        if t is None or k == "cu_seqlens":
            sub[k] = t
        elif k == "S0":
            sub[k] = t[:, heads]
        else:
            sub[k] = t[:, :, heads]
    ro, rS = _ref(sub, w.mode)
    eo, eS = _rel_seq(o[:, :, heads], ro, S[:, heads], rS, inp["cu_seqlens"].tolist())
    print("packed workload: rel err o %.2e S %.2e" % (eo, eS), flush=True)
    assert eo <= TOL[w.dtype] and eS <= TOL[w.dtype]


@pytest.mark.parametrize("mode", [1, 2])
def test_varlen_many_rows_longest_first(gpu, mode):
    """Twelve rows of very different lengths on 32 heads: more value slices than
    compute units, so the state kernel takes the rows longest first.  Every
    (row, head) against the oracle."""
    lens = (1500, 64, 777, 1, 1203, 300, 65, 950, 0, 431, 1499, 130)
    w = W.Packed("packed_longest_first", len(lens), sum(lens), 32, 128, 128, torch.bfloat16,
                 GATE_OF_MODE[mode], 0.1, seed=49, lengths=lens)
    eo, eS = _check(gpu, w)
    print("  rel err o %.2e, S_final %.2e" % (eo, eS))


@pytest.mark.parametrize("mode,gate", [(0, "none"), (1, "exp01"), (1, "range090"), (2, "exp01_channel")])
def test_varlen_long_rows_split(gpu, mode, gate):
    """Eight rows on 16 heads, two of them (4000 and 2500 tokens) far longer than
    an even share of chunks per compute unit: their value slices run in two
    parts, the second reaching its start by a lead-in (from the history horizon
    under scalar decay, else from chunk 0).  Every (row, head) against the
    oracle, S0 drawn (std 0.1)."""
    lens = (4000, 300, 200, 100, 64, 1, 2500, 0)
    w = W.Packed("packed_long_rows", len(lens), sum(lens), 16, 128, 128, torch.bfloat16,
                 gate, 0.1, seed=50, lengths=lens)
    eo, eS = _check(gpu, w)
    print("  rel err o %.2e, S_final %.2e" % (eo, eS))
