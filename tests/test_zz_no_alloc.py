"""gdn_chunk_fwd_noalloc (the prefill entry point that allocates nothing: its
chunk records live in the library's per-GPU scratch array) against
gdn_chunk_fwd, the entry point whose kernels it shares, on two calls in a
row, the second with a smaller input, and against the fp64 oracle."""
import ctypes

import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu


def _run(gdn, w, inp):
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    ref_o, ref_S = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], mode=w.mode)
    o = torch.full_like(ref_o, float("nan"))
    S = torch.full_like(ref_S, float("nan"))
    gdn.chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], o, S, mode=w.mode)
    torch.cuda.synchronize()
    return o.cpu(), S.cpu(), ref_o.cpu(), ref_S.cpu()


@pytest.mark.parametrize("first,second", [
    (W.GDN_BF16_PREFILL.with_(B=2, H=16, T=4096 + 37),         # 2 x 16 x 65 = 2080 records
     W.GDN_BF16_PREFILL.with_(B=1, H=3, T=200)),               # then 12
    (W.KDA_BF16_PREFILL.with_(B=1, H=8, T=7990),               # 1000 per-channel records
     W.KDA_BF16_PREFILL.with_(B=1, H=2, T=130)),
    (W.GDN_FP32_SMALL, W.GDN_FP32_SMALL.with_(T=70, H=1)),
])
def test_noalloc_matches_chunk_fwd_twice(gpu, first, second):
    for w in (first, second):
        print("noalloc case %s B=%d H=%d T=%d" % (w.name, w.B, w.H, w.T), flush=True)
        inp = W.make_prefill(w)
        o, S, ro, rS = _run(gpu, w, inp)
        # the same kernels on the same inputs: identical results
        assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o,
                           ro.view(torch.int16) if ro.dtype == torch.bfloat16 else ro)
        assert torch.equal(S, rS)
        # and within the benchmark's tolerance of the fp64 oracle
        fo, fS = oracle.gdn_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"],
                                mode=w.mode)
        tol = 1e-4 if w.dtype == torch.float32 else 2e-2
        assert W.per_head_rel_err(o.float().numpy(), fo, (0, 2)) <= tol
        assert W.per_head_rel_err(S.numpy(), fS, (0, 1)) <= tol


def test_noalloc_rejects_oversized_call(gpu):
    w = W.GDN_BF16_PREFILL.with_(B=8, H=16, T=4096)   # 8192 records > the scratch array
    z = torch.zeros(1, dtype=torch.bfloat16, device="cuda")
    lib = gpu.load()
    st = lib.gdn_chunk_fwd_noalloc(*[ctypes.c_void_p(z.data_ptr())] * 8, w.B, w.T, w.H, 128, 128, 64,
                                   1, 1, None)
    assert st == -5   # GDN_ERR_WORKSPACE, before any launch
