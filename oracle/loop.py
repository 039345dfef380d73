"""ctypes loader for the fp64 C oracle (``gdn_oracle.c``).  Test infrastructure only.

The C file is compiled with gcc at ``-O2 -fopenmp`` with fp contraction off and
no fast-math, so every sum runs in index order in IEEE fp64.  Inputs of any
float dtype (fp32, bf16, as torch tensors or numpy arrays) are upcast exactly
to fp64 before the call.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

MODE_NONE, MODE_SCALAR, MODE_CHANNEL, MODE_GDN2 = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "_build", "libgdn_oracle.so")
_lock = threading.Lock()
_default = None


def compile_library(src: str, out: str) -> str:
    """gcc -O2, OpenMP, no fast-math, no fp contraction."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-o", tmp, src]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle library in-tree (``oracle/_build``)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(SOURCE):
        compile_library(SOURCE, _LIB)
    return _LIB


def _f64(x):
    """Exact upcast of a torch tensor or array to a C-contiguous fp64 ndarray."""
    if x is None:
        return None
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu")
        if x.dtype == torch.bfloat16:
            x = x.to(torch.float32)          # exact
        x = x.to(torch.float64).numpy()      # exact
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _check_gates(mode, alpha, beta, erase, write, lead, dk, dv):
    """Shapes of the gates of a decay mode (``lead`` = the token axes)."""
    if mode == MODE_SCALAR:
        assert alpha is not None and alpha.shape == lead
    elif mode in (MODE_CHANNEL, MODE_GDN2):
        assert alpha is not None and alpha.shape == lead + (dk,)
    if mode == MODE_GDN2:
        assert erase is not None and erase.shape == lead + (dk,)
        assert write is not None and write.shape == lead + (dv,)
    else:
        assert beta is not None and beta.shape == lead


class Oracle:
    """One loaded build of the oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_gdn_fwd_f64.argtypes = [dp] * 10 + [ctypes.c_int] * 6
        lib.oracle_gdn_fwd_f64.restype = ctypes.c_int
        lib.oracle_gdn_fwd_varlen_f64.argtypes = ([dp] * 10 + [ctypes.POINTER(ctypes.c_int)]
                                                  + [ctypes.c_int] * 6)
        lib.oracle_gdn_fwd_varlen_f64.restype = ctypes.c_int
        lib.oracle_gdn_decode_f64.argtypes = [dp] * 9 + [ctypes.c_int] * 5
        lib.oracle_gdn_decode_f64.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        self._lib = lib

    def num_threads(self) -> int:
        return int(self._lib.oracle_num_threads())

    def gdn_fwd(self, q, k, v, alpha, beta, S0=None, mode: int = MODE_SCALAR, erase=None,
                write=None):
        """Prefill: token loop over T for every (b, h).

        q, k [B, T, H, dk]; v [B, T, H, dv]; alpha [B, T, H] (mode 1) or
        [B, T, H, dk] (modes 2, 3) or None (mode 0); beta [B, T, H] (modes
        0-2); erase [B, T, H, dk] and write [B, T, H, dv] (mode 3, Gated
        DeltaNet-2); S0 [B, H, dv, dk] or None (= zeros).
        Returns (o [B, T, H, dv], S_final [B, H, dv, dk]) as fp64 ndarrays."""
        q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
        alpha, S0, erase, write = _f64(alpha), _f64(S0), _f64(erase), _f64(write)
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        assert k.shape == q.shape and v.shape == (B, T, H, dv)
        _check_gates(mode, alpha, beta, erase, write, (B, T, H), dk, dv)
        if mode == MODE_NONE:
            alpha = None
        if S0 is not None:
            assert S0.shape == (B, H, dv, dk)
        o = np.zeros((B, T, H, dv), dtype=np.float64)
        S = np.zeros((B, H, dv, dk), dtype=np.float64)
        rc = self._lib.oracle_gdn_fwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                          _ptr(erase), _ptr(write), _ptr(S0), _ptr(o), _ptr(S),
                                          B, T, H, dk, dv, mode)
        if rc != 0:
            raise RuntimeError("oracle_gdn_fwd_f64 failed (rc=%d)" % rc)
        return o, S

    def gdn_fwd_varlen(self, q, k, v, alpha, beta, cu_seqlens, S0=None, mode: int = MODE_SCALAR,
                       erase=None, write=None):
        """Prefill of a packed batch: sequence s holds tokens cu_seqlens[s] ..
        cu_seqlens[s + 1] - 1 of the token axis, and its state starts from S0[s]
        (zeros when S0 is None) at its first token.

        q, k [T, H, dk]; v [T, H, dv]; alpha [T, H] (mode 1), [T, H, dk] (mode 2)
        or None; beta [T, H]; cu_seqlens N + 1 integers; S0 [N, H, dv, dk] or None.
        A leading axis of size 1 on the token tensors is accepted and kept.
        Returns (o, S_final [N, H, dv, dk]) as fp64 ndarrays."""
        q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
        alpha, S0, erase, write = _f64(alpha), _f64(S0), _f64(erase), _f64(write)
        lead = q.ndim == 4
        if lead:
            assert q.shape[0] == 1
            first = lambda x: None if x is None else x[0]
            q, k, v, beta = q[0], k[0], v[0], first(beta)
            alpha, erase, write = first(alpha), first(erase), first(write)
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens, dtype=np.int32))
        N = cu.shape[0] - 1
        T, H, dk = q.shape
        dv = v.shape[-1]
        assert k.shape == q.shape and v.shape == (T, H, dv)
        _check_gates(mode, alpha, beta, erase, write, (T, H), dk, dv)
        if mode == MODE_NONE:
            alpha = None
        if S0 is not None:
            assert S0.shape == (N, H, dv, dk)
        o = np.zeros((T, H, dv), dtype=np.float64)
        S = np.zeros((N, H, dv, dk), dtype=np.float64)
        rc = self._lib.oracle_gdn_fwd_varlen_f64(
            _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(erase), _ptr(write),
            _ptr(S0), _ptr(o), _ptr(S),
            cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), N, T, H, dk, dv, mode)
        if rc != 0:
            raise RuntimeError("oracle_gdn_fwd_varlen_f64 failed (rc=%d)" % rc)
        return (o[None] if lead else o), S

    def gdn_decode(self, q, k, v, alpha, beta, S, mode: int = MODE_SCALAR, erase=None,
                   write=None):
        """One decode step.  q, k [B, H, dk]; v [B, H, dv]; alpha [B, H] or
        [B, H, dk] or None; beta [B, H] (modes 0-2); erase [B, H, dk] and write
        [B, H, dv] (mode 3); S [B, H, dv, dk].
        Returns (o [B, H, dv], S_new); the input S is not modified."""
        q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
        alpha, erase, write = _f64(alpha), _f64(erase), _f64(write)
        S = _f64(S).copy()
        B, H, dk = q.shape
        dv = v.shape[-1]
        assert k.shape == q.shape and v.shape == (B, H, dv)
        assert S.shape == (B, H, dv, dk)
        _check_gates(mode, alpha, beta, erase, write, (B, H), dk, dv)
        if mode == MODE_NONE:
            alpha = None
        o = np.zeros((B, H, dv), dtype=np.float64)
        rc = self._lib.oracle_gdn_decode_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                             _ptr(erase), _ptr(write), _ptr(S), _ptr(o),
                                             B, H, dk, dv, mode)
        if rc != 0:
            raise RuntimeError("oracle_gdn_decode_f64 failed (rc=%d)" % rc)
        return o, S


def default() -> Oracle:
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(SOURCE):
                build(force=True)
            _default = Oracle(_LIB)
    return _default


def gdn_fwd(*args, **kw):
    return default().gdn_fwd(*args, **kw)


def gdn_fwd_varlen(*args, **kw):
    return default().gdn_fwd_varlen(*args, **kw)


def gdn_decode(*args, **kw):
    return default().gdn_decode(*args, **kw)


def num_threads() -> int:
    return default().num_threads()
