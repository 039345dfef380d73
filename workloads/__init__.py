"""Seeded synthetic inputs for the gated delta-rule path.

This module is shared by the tests, the benchmark and the smoke check.  It holds
no arithmetic of the method itself: it only draws random numbers, shapes them
into the distributions listed below and rounds them to the storage dtype.  Both
the HIP path and the fp64 oracle consume exactly the tensors made here.

Distributions (all drawn in fp32 on the CPU with ``torch.Generator``):
  q, k    z ~ N(0, 1), then divided by its L2 norm per (b, t, h), as the layers
          on the pages normalise queries and keys per head; then cast.
  v       z ~ N(0, 1), cast.
  beta    sigmoid(z), fp32.
  alpha   per the workload's gate recipe (see ``GATES``), fp32 for a scalar
          gate, the input dtype for a per-channel gate.
  S0      zeros, or N(0, std^2) fp32.
Casting to bf16 is round-to-nearest-even (torch's ``.to``); the oracle is given
the rounded values, so parity measures GPU arithmetic only.

Seeds: a workload with seed ``s`` draws tensor number ``j`` (order q, k, v,
beta, alpha, S0) from ``torch.Generator().manual_seed(1000 * s + j)``.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import torch

MODE_NONE, MODE_SCALAR, MODE_CHANNEL = 0, 1, 2


def _gen(seed: int) -> torch.Generator:
    return torch.Generator().manual_seed(int(seed))


def _randn(shape, seed):
    return torch.randn(*shape, generator=_gen(seed), dtype=torch.float32)


def _unit(z: torch.Tensor) -> torch.Tensor:
    return z / torch.linalg.vector_norm(z, dim=-1, keepdim=True)


# Gate recipes: name -> (decay mode, function of z (fp32) giving alpha).
def _gate_exp01(z):        # alpha = exp(-0.1 softplus(z))
    return torch.exp(-0.1 * torch.nn.functional.softplus(z))


def _gate_exp1(z):         # alpha = exp(-softplus(z)): strong decay, median about 0.50
    return torch.exp(-torch.nn.functional.softplus(z))


def _gate_range(lo):       # alpha = lo + (1 - lo) sigmoid(z), inside (lo, 1)
    return lambda z: lo + (1.0 - lo) * torch.sigmoid(z)


def _gate_kda_clamped(z):  # alpha = max(0.8, exp(-softplus(z - 3))), mostly inside (0.8, 1)
    return torch.clamp(torch.exp(-torch.nn.functional.softplus(z - 3.0)), min=0.8)


def _gate_kda_literal(z):  # alpha = exp(-softplus(z + 3)): strong decay, median about 0.047
    return torch.exp(-torch.nn.functional.softplus(z + 3.0))


GATES = {
    "none": (MODE_NONE, None),
    "exp01": (MODE_SCALAR, _gate_exp01),
    "exp1": (MODE_SCALAR, _gate_exp1),
    "range090": (MODE_SCALAR, _gate_range(0.90)),
    "range095": (MODE_SCALAR, _gate_range(0.95)),
    "exp01_channel": (MODE_CHANNEL, _gate_exp01),
    "kda_clamped": (MODE_CHANNEL, _gate_kda_clamped),
    "kda_literal": (MODE_CHANNEL, _gate_kda_literal),
}


@dataclasses.dataclass(frozen=True)
class Prefill:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    dtype: torch.dtype
    gate: str
    s0_std: float          # 0 means S0 = zeros (passed as None)
    seed: int
    chunk: int = 64

    @property
    def mode(self) -> int:
        return GATES[self.gate][0]

    def with_(self, **kw) -> "Prefill":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class Decode:
    name: str
    B: int
    H: int
    dk: int
    dv: int
    steps: int
    dtype: torch.dtype
    gate: str
    s_std: float
    seed: int

    @property
    def mode(self) -> int:
        return GATES[self.gate][0]

    def with_(self, **kw) -> "Decode":
        return dataclasses.replace(self, **kw)


# The five workloads, named by what they are.
GDN_FP32_SMALL = Prefill("gdn_fp32_b1_h2_t256_d64", 1, 2, 256, 64, 64, torch.float32,
                         "exp01", 0.0, seed=1)
GDN_BF16_PREFILL = Prefill("gdn_bf16_b8_h16_t4096_d128", 8, 16, 4096, 128, 128, torch.bfloat16,
                           "range090", 0.1, seed=2)
KDA_BF16_PREFILL = Prefill("kda_bf16_b4_h16_t8192_d128", 4, 16, 8192, 128, 128, torch.bfloat16,
                           "kda_clamped", 0.0, seed=3)
DECODE_DK128 = Decode("decode_b64_h16_dv128_dk128_x1024", 64, 16, 128, 128, 1024, torch.bfloat16,
                      "exp01", 0.1, seed=4)
DECODE_DK64 = Decode("decode_b64_h16_dv128_dk64_x1024", 64, 16, 64, 128, 1024, torch.bfloat16,
                     "exp01", 0.1, seed=4)
GDN_BF16_LONG = Prefill("gdn_bf16_b1_h32_t65536_d128", 1, 32, 65536, 128, 128, torch.bfloat16,
                        "range095", 0.0, seed=5)

PREFILL_WORKLOADS = [GDN_FP32_SMALL, GDN_BF16_PREFILL, KDA_BF16_PREFILL, GDN_BF16_LONG]


@dataclasses.dataclass(frozen=True)
class Packed:
    """N sequences of varying length packed back to back on one token axis of
    T tokens (inputs [1, T, H, d], offsets cu_seqlens [N + 1]).  The lengths are
    a seeded uniform random split of T into N parts (normalised Exp(1) draws,
    rounded down, at least ``min_len`` each, the remainder spread one token at
    a time from the first sequence on): a broad mix of short and long rows with
    ragged tails.  ``lengths`` overrides the split."""
    name: str
    N: int
    T: int
    H: int
    dk: int
    dv: int
    dtype: torch.dtype
    gate: str
    s0_std: float
    seed: int
    min_len: int = 1
    lengths: Optional[tuple] = None

    @property
    def mode(self) -> int:
        return GATES[self.gate][0]

    def with_(self, **kw) -> "Packed":
        return dataclasses.replace(self, **kw)


# Same token count and head shape as the B=8 x T=4096 prefill, split into 16 rows.
GDN_BF16_PACKED = Packed("gdn_bf16_packed_n16_t32768_h16_d128", 16, 32768, 16, 128, 128,
                         torch.bfloat16, "range090", 0.1, seed=6)


def packed_lengths(w: Packed) -> list:
    """Sequence lengths of a packed workload (tensor number 6 of its seed)."""
    if w.lengths is not None:
        assert len(w.lengths) == w.N and sum(w.lengths) == w.T
        return list(w.lengths)
    assert w.T >= w.N * w.min_len
    u = -torch.log1p(-torch.rand(w.N, generator=_gen(1000 * w.seed + 6), dtype=torch.float64))
    spare = w.T - w.N * w.min_len
    lens = [w.min_len + int(x) for x in torch.floor(spare * u / u.sum()).tolist()]
    i = 0
    while sum(lens) < w.T:
        lens[i % w.N] += 1
        i += 1
    return lens


def make_packed(w: Packed) -> dict:
    """CPU tensors q, k [1, T, H, dk]; v [1, T, H, dv]; beta [1, T, H]; alpha
    [1, T, H] or [1, T, H, dk] or None; S0 [N, H, dv, dk] or None; cu_seqlens
    int32 [N + 1].  Same distributions and seeding as :func:`make_prefill`."""
    base = make_prefill(Prefill(w.name, 1, w.H, w.T, w.dk, w.dv, w.dtype, w.gate, 0.0, w.seed))
    if w.s0_std > 0:
        base["S0"] = w.s0_std * _randn((w.N, w.H, w.dv, w.dk), 1000 * w.seed + 5)
    lens = packed_lengths(w)
    cu = torch.zeros(w.N + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0).to(torch.int32)
    base["cu_seqlens"] = cu
    return base
DECODE_WORKLOADS = [DECODE_DK128, DECODE_DK64]


def make_prefill(w: Prefill) -> dict:
    """CPU tensors q, k, v, beta, alpha (None for DeltaNet), S0 (None for zeros)."""
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    s = 1000 * w.seed
    mode, fn = GATES[w.gate]
    q = _unit(_randn((B, T, H, dk), s + 0)).to(w.dtype)
    k = _unit(_randn((B, T, H, dk), s + 1)).to(w.dtype)
    v = _randn((B, T, H, dv), s + 2).to(w.dtype)
    beta = torch.sigmoid(_randn((B, T, H), s + 3))
    alpha = None
    if mode == MODE_SCALAR:
        alpha = fn(_randn((B, T, H), s + 4))
    elif mode == MODE_CHANNEL:
        alpha = fn(_randn((B, T, H, dk), s + 4)).to(w.dtype)
    S0 = None
    if w.s0_std > 0:
        S0 = w.s0_std * _randn((B, H, dv, dk), s + 5)
    return dict(q=q, k=k, v=v, beta=beta, alpha=alpha, S0=S0)


def make_decode(w: Decode) -> dict:
    """CPU tensors for ``steps`` decode tokens: q, k [steps, B, H, dk]; v [steps, B, H, dv];
    beta, alpha [steps, B, H] (per-channel alpha [steps, B, H, dk]); S [B, H, dv, dk]."""
    n, B, H, dk, dv = w.steps, w.B, w.H, w.dk, w.dv
    s = 1000 * w.seed
    mode, fn = GATES[w.gate]
    q = _unit(_randn((n, B, H, dk), s + 0)).to(w.dtype)
    k = _unit(_randn((n, B, H, dk), s + 1)).to(w.dtype)
    v = _randn((n, B, H, dv), s + 2).to(w.dtype)
    beta = torch.sigmoid(_randn((n, B, H), s + 3))
    alpha = None
    if mode == MODE_SCALAR:
        alpha = fn(_randn((n, B, H), s + 4))
    elif mode == MODE_CHANNEL:
        alpha = fn(_randn((n, B, H, dk), s + 4)).to(w.dtype)
    S = w.s_std * _randn((B, H, dv, dk), s + 5)
    return dict(q=q, k=k, v=v, beta=beta, alpha=alpha, S=S)


def sha256(t: Optional[torch.Tensor]) -> Optional[str]:
    """SHA-256 of a tensor's bytes (None for an absent tensor)."""
    if t is None:
        return None
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return hashlib.sha256(t.numpy().tobytes()).hexdigest()


def rel_err(x, ref) -> float:
    """Worst per-(b, h) slice of max|x - ref| / max|ref| (NaN/Inf -> inf).

    ``x`` and ``ref`` share a layout whose head axes are given by the caller
    through :func:`per_head_rel_err`; this helper treats the whole array as one
    slice."""
    import numpy as np
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        return float("inf")
    den = np.max(np.abs(ref))
    num = np.max(np.abs(x - ref)) if x.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


def per_head_rel_err(x, ref, head_axes) -> float:
    """Worst over (b, h) slices of max|x - ref| / max|ref|.  ``head_axes`` names the
    axes of b and h, e.g. (0, 2) for [B, T, H, d] and (0, 1) for [B, H, dv, dk]."""
    import numpy as np
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.size == 0:
        return 0.0
    if not np.all(np.isfinite(x)):
        return float("inf")
    axes = tuple(head_axes)
    other = tuple(i for i in range(x.ndim) if i not in axes)
    xs = np.transpose(x, axes + other).reshape(x.shape[axes[0]] * x.shape[axes[1]], -1)
    rs = np.transpose(ref, axes + other).reshape(xs.shape[0], -1)
    num = np.max(np.abs(xs - rs), axis=1)
    den = np.max(np.abs(rs), axis=1)
    r = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    return float(np.max(r))



def make_prologue(B: int, T: int, H: int, dk: int, dv: int, dtype: torch.dtype, mode: int,
                  seed: int, s0_std: float = 0.1) -> dict:
    """Raw inputs for the fused prologue (the values a mixer layer's projections
    produce before its normalisations and gates):
      q, k      z ~ N(0, 1) times a per-(b, t, h) scale exp(N(0, 0.5^2)), not
                normalised; cast to ``dtype``
      v         z, cast
      beta      logits z, fp32 [B, T, H]
      alpha     logits z, fp32 [B, T, H] (scalar decay) or ``dtype``
                [B, T, H, dk] (per channel); None without decay
      A         per-head rates U(1, 16), fp32 [H]
      dt_bias   inverse softplus of dt = exp(U(ln 0.001, ln 0.1)), fp32 [H]
                (scalar) or [H, dk] (per channel): a Mamba2-style initialisation
                of the decay, softplus(x + dt_bias) near dt
      S0        N(0, s0_std^2) fp32 [B, H, dv, dk], or None for s0_std = 0.
    Tensor j of the seed: q 0, k 1, v 2, beta 3, alpha 4, S0 5, scales 7, A 8,
    dt_bias 9."""
    s = 1000 * seed
    scale = torch.exp(0.5 * _randn((2, B, T, H, 1), s + 7))
    q = (_randn((B, T, H, dk), s + 0) * scale[0]).to(dtype)
    k = (_randn((B, T, H, dk), s + 1) * scale[1]).to(dtype)
    v = _randn((B, T, H, dv), s + 2).to(dtype)
    beta = _randn((B, T, H), s + 3)
    alpha = A = dt_bias = None
    if mode != MODE_NONE:
        A = 1.0 + 15.0 * torch.rand(H, generator=_gen(s + 8))
        bshape = (H,) if mode == MODE_SCALAR else (H, dk)
        dt = torch.exp(torch.empty(bshape).uniform_(float(torch.log(torch.tensor(1e-3))),
                                                    float(torch.log(torch.tensor(1e-1))),
                                                    generator=_gen(s + 9)))
        dt_bias = torch.log(torch.expm1(dt))
        if mode == MODE_SCALAR:
            alpha = _randn((B, T, H), s + 4)
        else:
            alpha = _randn((B, T, H, dk), s + 4).to(dtype)
    S0 = s0_std * _randn((B, H, dv, dk), s + 5) if s0_std > 0 else None
    return dict(q=q, k=k, v=v, beta=beta, alpha=alpha, S0=S0, A=A, dt_bias=dt_bias)



def make_gdn2(w: Prefill) -> dict:
    """Inputs of a Gated DeltaNet-2 run with the shape and per-channel decay of a
    workload ``w`` (gate recipe of ``w``): q, k, v, alpha, S0 as
    :func:`make_prefill`, and instead of beta an erase gate sigmoid(z) per key
    channel [B, T, H, dk] (tensor 10 of the seed) and a write gate sigmoid(z) per
    value channel [B, T, H, dv] (tensor 11), both in the input dtype."""
    d = make_prefill(w)
    s = 1000 * w.seed
    d["erase"] = torch.sigmoid(_randn((w.B, w.T, w.H, w.dk), s + 10)).to(w.dtype)
    d["write"] = torch.sigmoid(_randn((w.B, w.T, w.H, w.dv), s + 11)).to(w.dtype)
    d["beta"] = None
    return d
