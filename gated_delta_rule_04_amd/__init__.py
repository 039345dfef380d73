"""Python binding of libgdn.so, the MI355X gated delta-rule library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C-ABI declared in ``include/gdn.h``.  PyTorch supplies
device memory and the current HIP stream.  There is no CPU fallback: if the
library is missing or does not load, every call raises.

    o, S_final = chunk_fwd(q, k, v, alpha, beta, S0)      # prefill
    o, S_final = chunk_fwd_varlen(q, k, v, alpha, beta, cu_seqlens, S0)
                                                           # packed sequences
    o = decode_step(q, k, v, alpha, beta, S)               # one token, S in place
    o, S_final = chunk_fwd_fused(q, k, v, alpha, beta, S0, l2norm_qk=True,
                                 beta_logits=True, alpha_logits=True, A=A)
                                                           # prologue in the kernels
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = ["chunk_fwd", "chunk_fwd_noalloc", "chunk_fwd_varlen", "chunk_fwd_fused", "decode_step", "decode_step_fused",
           "gated_rmsnorm",
           "gdn2_chunk_fwd", "gdn2_decode_step", "chunk_bwd", "load", "lib_path", "GDNError",
           "DECAY_NONE", "DECAY_SCALAR", "DECAY_CHANNEL", "EXPORTED_SYMBOLS"]

DECAY_NONE, DECAY_SCALAR, DECAY_CHANNEL = 0, 1, 2
_DTYPES = {torch.float32: 0, torch.bfloat16: 1}
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")
EXPORTED_SYMBOLS = ("gdn_chunk_fwd_workspace_bytes", "gdn_chunk_fwd", "gdn_chunk_fwd_noalloc",
                    "gdn_chunk_fwd_varlen_workspace_bytes", "gdn_chunk_fwd_varlen",
                    "gdn_chunk_fwd_fused", "gdn_decode_step", "gdn_decode_step_fused",
                    "gdn2_chunk_fwd", "gdn2_decode_step", "gdn_chunk_bwd_workspace_bytes",
                    "gdn_chunk_bwd", "gdn_gated_rmsnorm", "gdn_status_string", "gdn_version")


class Prologue(ctypes.Structure):
    """``gdn_prologue`` of include/gdn.h."""
    _fields_ = [("l2norm_qk", ctypes.c_int), ("eps", ctypes.c_float),
                ("beta_logits", ctypes.c_int), ("alpha_logits", ctypes.c_int),
                ("A", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p)]

_lock = threading.Lock()
_lib = None


class GDNError(RuntimeError):
    """A non-zero gdn_status returned by the library."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libgdn.so (once).  Raises if it is missing: there is no fallback."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libgdn.so is not built (%s); run "
                               "`python -m gated_delta_rule_04_amd.build`" % _LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        lib.gdn_chunk_fwd_workspace_bytes.argtypes = [i] * 8
        lib.gdn_chunk_fwd_workspace_bytes.restype = sz
        lib.gdn_chunk_fwd.argtypes = [vp] * 8 + [vp, sz] + [i] * 8 + [vp]
        lib.gdn_chunk_fwd.restype = i
        lib.gdn_chunk_fwd_noalloc.argtypes = [vp] * 8 + [i] * 8 + [vp]
        lib.gdn_chunk_fwd_noalloc.restype = i
        lib.gdn_chunk_fwd_varlen_workspace_bytes.argtypes = [i] * 8
        lib.gdn_chunk_fwd_varlen_workspace_bytes.restype = sz
        lib.gdn_chunk_fwd_varlen.argtypes = [vp] * 9 + [vp, sz] + [i] * 8 + [vp]
        lib.gdn_chunk_fwd_varlen.restype = i
        lib.gdn_chunk_fwd_fused.argtypes = [vp] * 10 + [vp, sz] + [i] * 8 + [vp]
        lib.gdn_chunk_fwd_fused.restype = i
        lib.gdn_decode_step_fused.argtypes = [vp] * 8 + [i] * 6 + [vp]
        lib.gdn_decode_step_fused.restype = i
        lib.gdn2_chunk_fwd.argtypes = [vp] * 10 + [vp, sz] + [i] * 7 + [vp]
        lib.gdn2_chunk_fwd.restype = i
        lib.gdn2_decode_step.argtypes = [vp] * 8 + [i] * 5 + [vp]
        lib.gdn2_decode_step.restype = i
        lib.gdn_chunk_bwd_workspace_bytes.argtypes = [i] * 8
        lib.gdn_chunk_bwd_workspace_bytes.restype = sz
        lib.gdn_chunk_bwd.argtypes = [vp] * 14 + [vp, sz] + [i] * 8 + [vp]
        lib.gdn_chunk_bwd.restype = i
        lib.gdn_decode_step.argtypes = [vp] * 7 + [i] * 6 + [vp]
        lib.gdn_decode_step.restype = i
        lib.gdn_gated_rmsnorm.argtypes = [vp] * 4 + [ctypes.c_longlong, i, ctypes.c_float, i, vp]
        lib.gdn_gated_rmsnorm.restype = i
        lib.gdn_status_string.argtypes = [i]
        lib.gdn_status_string.restype = ctypes.c_char_p
        lib.gdn_version.argtypes = []
        lib.gdn_version.restype = i
        _lib = lib
        return lib


def _check(status: int):
    if status != 0:
        msg = load().gdn_status_string(status).decode()
        raise GDNError(status, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _infer_mode(alpha, q_dim):
    if alpha is None:
        return DECAY_NONE
    return DECAY_SCALAR if alpha.dim() == q_dim - 1 else DECAY_CHANNEL


def _require(t, name, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))



def _expect(t, name, shape):
    """Raise ValueError unless tensor ``t`` (if given) has exactly ``shape``."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _check_prefill_shapes(q, k, v, alpha, beta, S0, o, S_final, mode, lead, nseq, extra_h=None):
    """Shapes of a prefill call (batched: ``lead`` = (B, T, H); packed: (T, H)
    or (1, T, H)) against q's; ``nseq`` states per head (B, or N for a packed
    batch).  Every size the kernels derive from (B, T, H, dk, dv) must match,
    since the C-ABI sees only pointers: a short tensor would be read or written
    past its end."""
    dk = q.shape[-1]
    if v is None or v.dim() != q.dim():
        raise ValueError("v must have as many axes as q")
    dv = v.shape[-1]
    H = lead[-1]
    _expect(k, "k", tuple(lead) + (dk,))
    _expect(v, "v", tuple(lead) + (dv,))
    _expect(beta, "beta", tuple(lead))
    if mode == DECAY_SCALAR:
        _expect(alpha, "alpha", tuple(lead))
    elif mode == DECAY_CHANNEL:
        _expect(alpha, "alpha", tuple(lead) + (dk,))
    _expect(S0, "S0", (nseq, H, dv, dk))
    _expect(o, "o", tuple(lead) + (dv,))
    _expect(S_final, "S_final", (nseq, H, dv, dk))
    for t, n, last in (extra_h or ()):
        _expect(t, n, tuple(lead) + (last,))
    if mode not in (DECAY_NONE, DECAY_SCALAR, DECAY_CHANNEL):
        raise ValueError("mode must be DECAY_NONE, DECAY_SCALAR or DECAY_CHANNEL")
    if mode != DECAY_NONE and alpha is None:
        raise ValueError("alpha is required for a decay mode")
    return dk, dv


def _check_decode_shapes(q, k, v, alpha, beta, S, o, mode, extra=None):
    if q.dim() != 3:
        raise ValueError("q must be [B, H, dk]")
    B, H, dk = q.shape
    if v is None or v.dim() != 3:
        raise ValueError("v must be [B, H, dv]")
    dv = v.shape[-1]
    _expect(k, "k", (B, H, dk))
    _expect(v, "v", (B, H, dv))
    _expect(beta, "beta", (B, H))
    if mode == DECAY_SCALAR:
        _expect(alpha, "alpha", (B, H))
    elif mode == DECAY_CHANNEL:
        _expect(alpha, "alpha", (B, H, dk))
    if mode != DECAY_NONE and alpha is None:
        raise ValueError("alpha is required for a decay mode")
    if S is None:
        raise ValueError("S is required")
    _expect(S, "S", (B, H, dv, dk))
    _expect(o, "o", (B, H, dv))
    for t, n, last in (extra or ()):
        _expect(t, n, (B, H, last))
    return B, H, dk, dv


def _lead_of(q, cu_seqlens):
    """(B, T, H, dk) of a batched call, or (N, T, H, dk) of a packed one."""
    if cu_seqlens is None:
        if q.dim() != 4:
            raise ValueError("q must be [B, T, H, dk]")
        B, T, H, dk = q.shape
        return B, T, H, dk
    if q.dim() not in (3, 4) or (q.dim() == 4 and q.shape[0] != 1):
        raise ValueError("a packed q must be [T, H, dk] or [1, T, H, dk]")
    if cu_seqlens.dim() != 1 or cu_seqlens.shape[0] < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 GPU tensor of N + 1 offsets")
    T, H, dk = q.shape[-3:]
    return cu_seqlens.shape[0] - 1, T, H, dk


def _check_workspace(ws, nbytes):
    if ws is None:
        return None
    if ws.dtype != torch.uint8 or ws.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 tensor")
    if ws.numel() < nbytes:
        raise ValueError("workspace holds %d bytes, the call needs %d" % (ws.numel(), nbytes))
    return ws


def _check_prologue_shapes(mode, H, dk, alpha_logits, A, dt_bias):
    if A is not None:
        _expect(A, "A", (H,))
    if dt_bias is not None:
        _expect(dt_bias, "dt_bias", (H,) if mode == DECAY_SCALAR else (H, dk))
    if alpha_logits and mode != DECAY_NONE and A is None:
        raise ValueError("alpha_logits needs the per-head rates A")


def workspace_bytes(B, T, H, dk, dv, dtype=torch.bfloat16, mode=DECAY_SCALAR, chunk=64) -> int:
    return int(load().gdn_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk, _DTYPES[dtype], mode))


def chunk_fwd(q, k, v, alpha, beta, S0=None, *, mode=None, chunk=64, o=None, S_final=None,
              need_final=True, workspace=None, stream=None):
    """Chunked prefill through ``gdn_chunk_fwd``.

    q, k [B, T, H, dk]; v [B, T, H, dv] (fp32 or bf16, one dtype);
    alpha fp32 [B, T, H] (scalar decay), ``dtype`` [B, T, H, dk] (per-channel
    decay) or None (no decay); beta fp32 [B, T, H]; S0 fp32 [B, H, dv, dk] or None.
    ``workspace``: a uint8 GPU tensor of at least :func:`workspace_bytes` bytes
    (None: one is allocated per call).
    Returns (o, S_final); S_final is None when ``need_final`` is False."""
    lib = load()
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    B, T, H, dk = q.shape
    mode = _infer_mode(alpha, q.dim()) if mode is None else mode
    _, dv = _check_prefill_shapes(q, k, v, alpha, beta, S0, o, S_final, mode, (B, T, H), B)
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise ValueError("q must be float32 or bfloat16")
    ws_bytes = int(lib.gdn_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk, _DTYPES[dtype], mode))
    ws = _check_workspace(workspace, ws_bytes)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, n, dtype)
    _require(beta, "beta", torch.float32)
    _require(S0, "S0", torch.float32)
    if mode == DECAY_SCALAR:
        _require(alpha, "alpha", torch.float32)
    elif mode == DECAY_CHANNEL:
        _require(alpha, "alpha", dtype)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dtype, device=q.device)
    if S_final is None and need_final:
        S_final = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    _require(o, "o", dtype)
    _require(S_final, "S_final", torch.float32)
    _require(ws, "workspace")
    if ws is None and ws_bytes:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    if ws is not None:
        ws_bytes = ws.numel()
    st = lib.gdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha if mode else None), _ptr(beta),
                           _ptr(S0), _ptr(o), _ptr(S_final), _ptr(ws), ws_bytes,
                           B, T, H, dk, dv, chunk, _DTYPES[dtype], mode, _stream(stream))
    _check(st)
    return o, S_final


NOALLOC_SCRATCH_BYTES = 64 << 20   # GDN_NOALLOC_SCRATCH_BYTES of include/gdn.h


def chunk_fwd_noalloc(q, k, v, alpha, beta, S0, o, S_final, *, mode=None, chunk=64, stream=None):
    """Prefill through ``gdn_chunk_fwd_noalloc``: the library allocates nothing
    (its chunk records live in a per-GPU scratch array of NOALLOC_SCRATCH_BYTES),
    so the caller passes the outputs o [B, T, H, dv] and S_final [B, H, dv, dk]
    (S_final may be None).  Calls that overlap on one GPU race; calls in order
    on one stream do not."""
    lib = load()
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    if o is None:
        raise ValueError("o is required: this entry point allocates nothing")
    B, T, H, dk = q.shape
    mode = _infer_mode(alpha, q.dim()) if mode is None else mode
    _, dv = _check_prefill_shapes(q, k, v, alpha, beta, S0, o, S_final, mode, (B, T, H), B)
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise ValueError("q must be float32 or bfloat16")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _require(t, n, dtype)
    _require(beta, "beta", torch.float32)
    _require(S0, "S0", torch.float32)
    _require(S_final, "S_final", torch.float32)
    if mode == DECAY_SCALAR:
        _require(alpha, "alpha", torch.float32)
    elif mode == DECAY_CHANNEL:
        _require(alpha, "alpha", dtype)
    st = lib.gdn_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha if mode else None),
                                   _ptr(beta), _ptr(S0), _ptr(o), _ptr(S_final),
                                   B, T, H, dk, dv, chunk, _DTYPES[dtype], mode, _stream(stream))
    _check(st)
    return o, S_final


def chunk_fwd_varlen(q, k, v, alpha, beta, cu_seqlens, S0=None, *, mode=None, chunk=64, o=None,
                     S_final=None, need_final=True, stream=None):
    """Chunked prefill of a packed batch through ``gdn_chunk_fwd_varlen``.

    q, k [T, H, dk]; v [T, H, dv] (a leading axis of 1 is accepted and kept);
    alpha fp32 [T, H], ``dtype`` [T, H, dk] or None; beta fp32 [T, H];
    cu_seqlens int32 GPU tensor [N + 1] (0, ..., T, non-decreasing); S0 fp32
    [N, H, dv, dk] or None.  Returns (o, S_final [N, H, dv, dk])."""
    lib = load()
    if q.dim() not in (3, 4):
        raise ValueError("q must be [T, H, dk] or [1, T, H, dk]")
    lead = q.dim() == 4
    T, H, dk = q.shape[-3:]
    if lead and q.shape[0] != 1:
        raise ValueError("a packed batch has a leading axis of 1, got %d" % q.shape[0])
    if cu_seqlens is None or cu_seqlens.dim() != 1 or cu_seqlens.shape[0] < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 GPU tensor of N + 1 offsets")
    N = cu_seqlens.shape[0] - 1
    if mode is None:
        mode = DECAY_NONE if alpha is None else (
            DECAY_SCALAR if alpha.dim() == q.dim() - 1 else DECAY_CHANNEL)
    _, dv = _check_prefill_shapes(q, k, v, alpha, beta, S0, o, S_final, mode, tuple(q.shape[:-1]), N)
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise ValueError("q must be float32 or bfloat16")
    _require(cu_seqlens, "cu_seqlens", torch.int32)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, n, dtype)
    _require(beta, "beta", torch.float32)
    _require(S0, "S0", torch.float32)
    if mode == DECAY_SCALAR:
        _require(alpha, "alpha", torch.float32)
    elif mode == DECAY_CHANNEL:
        _require(alpha, "alpha", dtype)
    if o is None:
        o = torch.empty(tuple(q.shape[:-1]) + (dv,), dtype=dtype, device=q.device)
    if S_final is None and need_final:
        S_final = torch.empty((N, H, dv, dk), dtype=torch.float32, device=q.device)
    _require(o, "o", dtype)
    _require(S_final, "S_final", torch.float32)
    ws_bytes = int(lib.gdn_chunk_fwd_varlen_workspace_bytes(N, T, H, dk, dv, chunk,
                                                            _DTYPES[dtype], mode))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes else None
    st = lib.gdn_chunk_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha if mode else None),
                                  _ptr(beta), _ptr(S0), _ptr(o), _ptr(S_final), _ptr(cu_seqlens),
                                  _ptr(ws), ws_bytes, N, T, H, dk, dv, chunk, _DTYPES[dtype], mode,
                                  _stream(stream))
    _check(st)
    return o, S_final


def decode_step(q, k, v, alpha, beta, S, *, mode=None, o=None, stream=None):
    """One decode step through ``gdn_decode_step``; S is updated in place.

    q, k [B, H, dk]; v [B, H, dv]; alpha fp32 [B, H], ``dtype`` [B, H, dk] or
    None; beta fp32 [B, H]; S fp32 [B, H, dv, dk].  Returns o [B, H, dv]."""
    lib = load()
    mode = _infer_mode(alpha, q.dim()) if mode is None else mode
    B, H, dk, dv = _check_decode_shapes(q, k, v, alpha, beta, S, o, mode)
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise ValueError("q must be float32 or bfloat16")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, n, dtype)
    _require(beta, "beta", torch.float32)
    _require(S, "S", torch.float32)
    if mode == DECAY_SCALAR:
        _require(alpha, "alpha", torch.float32)
    elif mode == DECAY_CHANNEL:
        _require(alpha, "alpha", dtype)
    if o is None:
        o = torch.empty((B, H, dv), dtype=dtype, device=q.device)
    _require(o, "o", dtype)
    st = lib.gdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha if mode else None), _ptr(beta),
                             _ptr(S), _ptr(o), B, H, dk, dv, _DTYPES[dtype], mode, _stream(stream))
    _check(st)
    return o


def gated_rmsnorm(o, gate, weight, *, eps=1e-6, out=None, stream=None):
    """Output epilogue through ``gdn_gated_rmsnorm``: out = o / sqrt(mean(o^2)
    + eps) * weight * silu(gate) over the last axis of o (d_v values per row).

    o, gate: the same shape [..., dv] (a prefill's [B, T, H, dv] or a decode
    step's [B, H, dv]), float32 or bfloat16; weight fp32 [dv]; ``out`` may be
    o itself (in place).  Returns out."""
    lib = load()
    if o.dim() < 1:
        raise ValueError("o must have a value axis")
    dv = o.shape[-1]
    if tuple(gate.shape) != tuple(o.shape):
        raise ValueError("gate shape %s must equal o's %s" % (tuple(gate.shape), tuple(o.shape)))
    if tuple(weight.shape) != (dv,):
        raise ValueError("weight shape %s must be (%d,)" % (tuple(weight.shape), dv))
    dtype = o.dtype
    if dtype not in _DTYPES:
        raise ValueError("o must be float32 or bfloat16")
    if out is None:
        out = torch.empty_like(o)
    elif tuple(out.shape) != tuple(o.shape):
        raise ValueError("out shape %s must equal o's %s" % (tuple(out.shape), tuple(o.shape)))
    _require(o, "o", dtype)
    _require(gate, "gate", dtype)
    _require(weight, "weight", torch.float32)
    _require(out, "out", dtype)
    rows = o.numel() // dv if dv else 0
    st = lib.gdn_gated_rmsnorm(_ptr(o), _ptr(gate), _ptr(weight), _ptr(out), rows, dv, float(eps),
                               _DTYPES[dtype], _stream(stream))
    _check(st)
    return out


def _prologue(l2norm_qk, eps, beta_logits, alpha_logits, A, dt_bias):
    _require(A, "A", torch.float32)
    _require(dt_bias, "dt_bias", torch.float32)
    return Prologue(int(bool(l2norm_qk)), float(eps), int(bool(beta_logits)),
                    int(bool(alpha_logits)), None if A is None else A.data_ptr(),
                    None if dt_bias is None else dt_bias.data_ptr())


def chunk_fwd_fused(q, k, v, alpha, beta, S0=None, *, cu_seqlens=None, l2norm_qk=False,
                    eps=1e-6, beta_logits=False, alpha_logits=False, A=None, dt_bias=None,
                    mode=None, chunk=64, o=None, S_final=None, need_final=True, stream=None):
    """Prefill with the per-token prologue in the kernels (``gdn_chunk_fwd_fused``).

    The tensors are those of :func:`chunk_fwd` (``cu_seqlens`` None) or of
    :func:`chunk_fwd_varlen` (``cu_seqlens`` given); with ``alpha_logits`` the
    alpha tensor holds logits x and log alpha = -A[h] softplus(x + dt_bias),
    A fp32 [H], dt_bias fp32 [H] or [H, dk]; with ``beta_logits`` beta holds
    logits; ``l2norm_qk`` normalises q and k per (token, head) with ``eps``."""
    lib = load()
    packed = cu_seqlens is not None
    B, T, H, dk = _lead_of(q, cu_seqlens)
    if mode is None:
        mode = DECAY_NONE if alpha is None else (
            DECAY_SCALAR if alpha.dim() == q.dim() - 1 else DECAY_CHANNEL)
    _, dv = _check_prefill_shapes(q, k, v, alpha, beta, S0, o, S_final, mode, tuple(q.shape[:-1]), B)
    _check_prologue_shapes(mode, H, dk, alpha_logits, A, dt_bias)
    if packed:
        _require(cu_seqlens, "cu_seqlens", torch.int32)
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise ValueError("q must be float32 or bfloat16")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, n, dtype)
    _require(beta, "beta", torch.float32)
    _require(S0, "S0", torch.float32)
    if mode == DECAY_SCALAR:
        _require(alpha, "alpha", torch.float32)
    elif mode == DECAY_CHANNEL:
        _require(alpha, "alpha", dtype)
    pro = _prologue(l2norm_qk, eps, beta_logits, alpha_logits, A, dt_bias)
    if o is None:
        o = torch.empty(tuple(q.shape[:-1]) + (dv,), dtype=dtype, device=q.device)
    if S_final is None and need_final:
        S_final = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    _require(o, "o", dtype)
    _require(S_final, "S_final", torch.float32)
    wsf = lib.gdn_chunk_fwd_varlen_workspace_bytes if packed else lib.gdn_chunk_fwd_workspace_bytes
    ws_bytes = int(wsf(B, T, H, dk, dv, chunk, _DTYPES[dtype], mode))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes else None
    st = lib.gdn_chunk_fwd_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha if mode else None),
                                 _ptr(beta), _ptr(S0), _ptr(o), _ptr(S_final), _ptr(cu_seqlens),
                                 ctypes.byref(pro), _ptr(ws), ws_bytes, B, T, H, dk, dv, chunk,
                                 _DTYPES[dtype], mode, _stream(stream))
    _check(st)
    return o, S_final


def decode_step_fused(q, k, v, alpha, beta, S, *, l2norm_qk=False, eps=1e-6, beta_logits=False,
                      alpha_logits=False, A=None, dt_bias=None, mode=None, o=None, stream=None):
    """One decode step with the prologue in the kernel (``gdn_decode_step_fused``);
    tensors as in :func:`decode_step`, prologue as in :func:`chunk_fwd_fused`."""
    lib = load()
    mode = _infer_mode(alpha, q.dim()) if mode is None else mode
    B, H, dk, dv = _check_decode_shapes(q, k, v, alpha, beta, S, o, mode)
    _check_prologue_shapes(mode, H, dk, alpha_logits, A, dt_bias)
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise ValueError("q must be float32 or bfloat16")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, n, dtype)
    _require(beta, "beta", torch.float32)
    _require(S, "S", torch.float32)
    if mode == DECAY_SCALAR:
        _require(alpha, "alpha", torch.float32)
    elif mode == DECAY_CHANNEL:
        _require(alpha, "alpha", dtype)
    pro = _prologue(l2norm_qk, eps, beta_logits, alpha_logits, A, dt_bias)
    if o is None:
        o = torch.empty((B, H, dv), dtype=dtype, device=q.device)
    _require(o, "o", dtype)
    st = lib.gdn_decode_step_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha if mode else None),
                                   _ptr(beta), _ptr(S), _ptr(o), ctypes.byref(pro), B, H, dk, dv,
                                   _DTYPES[dtype], mode, _stream(stream))
    _check(st)
    return o


def gdn2_chunk_fwd(q, k, v, alpha, erase, write, S0=None, *, cu_seqlens=None, chunk=64, o=None,
                   S_final=None, need_final=True, stream=None):
    """Gated DeltaNet-2 prefill (``gdn2_chunk_fwd``): per-channel decay alpha and
    erase gate [.., T, H, dk], write gate [.., T, H, dv], all in q's dtype;
    batched ([B, T, H, d]) or packed (``cu_seqlens``, [1, T, H, d] or [T, H, d])."""
    lib = load()
    packed = cu_seqlens is not None
    B, T, H, dk = _lead_of(q, cu_seqlens)
    dv = v.shape[-1]
    lead = tuple(q.shape[:-1])
    if erase is None or write is None:
        raise ValueError("erase and write gates are required")
    _check_prefill_shapes(q, k, v, alpha, None, S0, o, S_final, DECAY_CHANNEL, lead, B,
                          extra_h=((erase, "erase", dk), (write, "write", dv)))
    if packed:
        _require(cu_seqlens, "cu_seqlens", torch.int32)
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise ValueError("q must be float32 or bfloat16")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (alpha, "alpha"), (erase, "erase"),
                 (write, "write")):
        _require(t, n, dtype)
    _require(S0, "S0", torch.float32)
    if o is None:
        o = torch.empty(tuple(q.shape[:-1]) + (dv,), dtype=dtype, device=q.device)
    if S_final is None and need_final:
        S_final = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    _require(o, "o", dtype)
    _require(S_final, "S_final", torch.float32)
    wsf = lib.gdn_chunk_fwd_varlen_workspace_bytes if packed else lib.gdn_chunk_fwd_workspace_bytes
    ws_bytes = int(wsf(B, T, H, dk, dv, chunk, _DTYPES[dtype], DECAY_CHANNEL))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes else None
    st = lib.gdn2_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(erase), _ptr(write),
                            _ptr(S0), _ptr(o), _ptr(S_final), _ptr(cu_seqlens), _ptr(ws), ws_bytes,
                            B, T, H, dk, dv, chunk, _DTYPES[dtype], _stream(stream))
    _check(st)
    return o, S_final


def gdn2_decode_step(q, k, v, alpha, erase, write, S, *, o=None, stream=None):
    """One Gated DeltaNet-2 decode step (``gdn2_decode_step``); S updated in place.
    q, k, alpha, erase [B, H, dk]; v, write [B, H, dv]; S fp32 [B, H, dv, dk]."""
    lib = load()
    if erase is None or write is None:
        raise ValueError("erase and write gates are required")
    if q.dim() != 3 or v is None or v.dim() != 3:
        raise ValueError("q must be [B, H, dk] and v [B, H, dv]")
    dk, dv = q.shape[-1], v.shape[-1]
    B, H, dk, dv = _check_decode_shapes(q, k, v, alpha, None, S, o, DECAY_CHANNEL,
                                        extra=((erase, "erase", dk), (write, "write", dv)))
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise ValueError("q must be float32 or bfloat16")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (alpha, "alpha"), (erase, "erase"),
                 (write, "write")):
        _require(t, n, dtype)
    _require(S, "S", torch.float32)
    if o is None:
        o = torch.empty((B, H, dv), dtype=dtype, device=q.device)
    _require(o, "o", dtype)
    st = lib.gdn2_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(erase), _ptr(write),
                              _ptr(S), _ptr(o), B, H, dk, dv, _DTYPES[dtype], _stream(stream))
    _check(st)
    return o


def chunk_bwd(q, k, v, alpha, beta, S0, dout, dS_final=None, *, mode=None, chunk=64,
              need_dS0=True, stream=None):
    """Gradients of L = sum(dout * o) + sum(dS_final * S_T) through ``gdn_chunk_bwd``.

    Inputs as :func:`chunk_fwd`; dout [B, T, H, dv] in q's dtype; dS_final fp32
    [B, H, dv, dk] or None.  Returns a dict: dq, dk, dv (q's dtype), dalpha (fp32,
    alpha's shape; None without decay), dbeta (fp32), dS0 (fp32, or None when
    ``need_dS0`` is False)."""
    lib = load()
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    B, T, H, dk = q.shape
    mode = _infer_mode(alpha, q.dim()) if mode is None else mode
    _, dv = _check_prefill_shapes(q, k, v, alpha, beta, S0, dout, dS_final, mode, (B, T, H), B)
    if beta is None or dout is None:
        raise ValueError("beta and dout are required")
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise ValueError("q must be float32 or bfloat16")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _require(t, n, dtype)
    _require(beta, "beta", torch.float32)
    _require(S0, "S0", torch.float32)
    _require(dS_final, "dS_final", torch.float32)
    if mode == DECAY_SCALAR:
        _require(alpha, "alpha", torch.float32)
    elif mode == DECAY_CHANNEL:
        _require(alpha, "alpha", dtype)
    dev = q.device
    dq, dk_, dv_ = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dalpha = None if mode == DECAY_NONE else torch.empty(alpha.shape, dtype=torch.float32, device=dev)
    dbeta = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    dS0 = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev) if need_dS0 else None
    ws_bytes = int(lib.gdn_chunk_bwd_workspace_bytes(B, T, H, dk, dv, chunk, _DTYPES[dtype], mode))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    st = lib.gdn_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha if mode else None), _ptr(beta),
                           _ptr(S0), _ptr(dout), _ptr(dS_final), _ptr(dq), _ptr(dk_), _ptr(dv_),
                           _ptr(dalpha), _ptr(dbeta), _ptr(dS0), _ptr(ws), ws_bytes,
                           B, T, H, dk, dv, chunk, _DTYPES[dtype], mode, _stream(stream))
    _check(st)
    return dict(dq=dq, dk=dk_, dv=dv_, dalpha=dalpha, dbeta=dbeta, dS0=dS0)
