"""The C-ABI library on the CPU: it loads, exports every symbol include/gdn.h
declares, and its host-side validation rejects bad arguments before any launch.

Only calls that validation must reject are made here (no compute call runs
without a GPU).  The pointers are fake addresses: validation never dereferences
them, and every call below fails validation before anything is enqueued.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "gated_delta_rule_04_amd", "libgdn.so")

OK, E_NULL, E_SHAPE, E_DTYPE, E_UNSUP, E_WS, E_LAUNCH, E_ALIAS, E_VALUE = 0, -1, -2, -3, -4, -5, -6, -7, -8


def _declared():
    text = open(os.path.join(ROOT, "include", "gdn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn2?_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libgdn.so is not built; run python -m gated_delta_rule_04_amd.build")
    lib = ctypes.CDLL(LIB)
    vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.gdn_chunk_fwd.argtypes = [vp] * 8 + [vp, sz] + [i] * 8 + [vp]
    lib.gdn_chunk_fwd.restype = i
    lib.gdn_decode_step.argtypes = [vp] * 7 + [i] * 6 + [vp]
    lib.gdn_decode_step.restype = i
    lib.gdn_status_string.argtypes = [i]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_chunk_fwd_workspace_bytes.argtypes = [i] * 8
    lib.gdn_chunk_fwd_workspace_bytes.restype = sz
    lib.gdn_chunk_fwd_varlen.argtypes = [vp] * 9 + [vp, sz] + [i] * 8 + [vp]
    lib.gdn_chunk_fwd_varlen.restype = i
    lib.gdn_chunk_fwd_varlen_workspace_bytes.argtypes = [i] * 8
    lib.gdn_chunk_fwd_varlen_workspace_bytes.restype = sz
    lib.gdn_chunk_fwd_fused.argtypes = [vp] * 10 + [vp, sz] + [i] * 8 + [vp]
    lib.gdn_chunk_fwd_fused.restype = i
    lib.gdn_decode_step_fused.argtypes = [vp] * 8 + [i] * 6 + [vp]
    lib.gdn_decode_step_fused.restype = i
    lib.gdn2_chunk_fwd.argtypes = [vp] * 10 + [vp, sz] + [i] * 7 + [vp]
    lib.gdn2_chunk_fwd.restype = i
    lib.gdn2_decode_step.argtypes = [vp] * 8 + [i] * 5 + [vp]
    lib.gdn2_decode_step.restype = i
    lib.gdn_chunk_bwd.argtypes = [vp] * 14 + [vp, sz] + [i] * 8 + [vp]
    lib.gdn_chunk_bwd.restype = i
    lib.gdn_chunk_bwd_workspace_bytes.argtypes = [i] * 8
    lib.gdn_chunk_bwd_workspace_bytes.restype = sz
    lib.gdn_gated_rmsnorm.argtypes = [vp] * 4 + [ctypes.c_longlong, i, ctypes.c_float, i, vp]
    lib.gdn_gated_rmsnorm.restype = i
    return lib


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert {"gdn_chunk_fwd", "gdn_decode_step", "gdn_chunk_fwd_workspace_bytes",
            "gdn_status_string", "gdn_version"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name
    import gated_delta_rule_04_amd as gdn
    assert set(gdn.EXPORTED_SYMBOLS) == set(names)


def test_status_strings(lib):
    for st in (OK, E_NULL, E_SHAPE, E_DTYPE, E_UNSUP, E_WS, E_LAUNCH, E_ALIAS, E_VALUE):
        s = lib.gdn_status_string(st)
        assert s and s.startswith(b"GDN_")
    assert lib.gdn_status_string(12345) == b"unknown gdn_status"
    assert lib.gdn_version() == 300


# fake, disjoint device addresses (never dereferenced: every call fails validation)
def _bufs(base=1 << 40, span=1 << 36):
    return [base + i * span for i in range(8)]


def _fwd(lib, B=2, T=100, H=3, dk=128, dv=128, chunk=64, dtype=1, mode=1, ptrs=None,
         ws=(1 << 40) + 9 * (1 << 36),
         ws_bytes=1 << 30):
    q, k, v, a, b, s0, o, sf = ptrs if ptrs is not None else _bufs()
    return lib.gdn_chunk_fwd(q, k, v, a, b, s0, o, sf, ws, ws_bytes, B, T, H, dk, dv, chunk,
                             dtype, mode, None)


def test_chunk_fwd_rejects_bad_sizes(lib):
    assert _fwd(lib, dk=96) == E_UNSUP
    assert _fwd(lib, dv=256) == E_UNSUP
    assert _fwd(lib, chunk=32) == E_UNSUP
    assert _fwd(lib, T=-1) == E_SHAPE
    assert _fwd(lib, B=-1) == E_SHAPE
    assert _fwd(lib, dk=0) == E_SHAPE
    assert _fwd(lib, dtype=7) == E_DTYPE
    assert _fwd(lib, mode=3) == E_DTYPE
    assert _fwd(lib, B=1 << 30, T=1 << 30, H=1 << 20) == E_SHAPE   # element count overflow


def test_chunk_fwd_rejects_null_and_alias(lib):
    q, k, v, a, b, s0, o, sf = _bufs()
    assert _fwd(lib, ptrs=[0, k, v, a, b, s0, o, sf]) == E_NULL
    assert _fwd(lib, ptrs=[q, k, v, a, 0, s0, o, sf]) == E_NULL
    assert _fwd(lib, ptrs=[q, k, v, a, b, s0, 0, sf]) == E_NULL
    assert _fwd(lib, ptrs=[q, k, v, 0, b, s0, o, sf], mode=1) == E_NULL
    assert _fwd(lib, ptrs=[q, k, v, 0, b, s0, o, sf], mode=2) == E_NULL
    assert _fwd(lib, ptrs=[q, k, v, a, b, s0, q + 64, sf]) == E_ALIAS      # o inside q
    assert _fwd(lib, ptrs=[q, k, v, a, b, s0, o, o + 2]) == E_ALIAS        # S_final inside o
    assert _fwd(lib, ptrs=[q, k, v, a, b, s0, o, s0 + 16]) == E_ALIAS      # partial overlap S0
    assert _fwd(lib, ptrs=[q, k, v, a, b, s0, o, v]) == E_ALIAS


def test_chunk_fwd_empty_batch_is_a_no_op(lib):
    # nothing to compute: returns OK without touching the (fake) pointers
    assert _fwd(lib, B=0) == OK
    assert _fwd(lib, H=0) == OK
    assert _fwd(lib, T=0, ptrs=[0, 0, 0, 0, 0, 0, 0, 0]) == OK   # no S_final requested


def _ws_bytes(B, T, H, es, dk=128, mode=1):
    chunks = B * H * ((T + 63) // 64)
    if mode == 2:   # T, P, three scaled copies of K / Q, per-channel decay
        return chunks * ((2 * 64 * 64 + 3 * 64 * dk) * es + 4 * dk)
    # T per chunk (and P in fp32: the bf16 state kernel forms P itself) + five fp32 gate rows;
    # scalar decay in bf16: one fp32 transition bound per chunk after the records, 256-byte aligned
    return chunks * ((2 if es == 4 else 1) * 64 * 64 * es + 5 * 64 * 4) + _bound_bytes(chunks, es, mode)


def _bound_bytes(chunks, es, mode):
    return (chunks * 4 + 255) // 256 * 256 if (es == 2 and mode == 1) else 0


def test_workspace_query(lib):
    assert lib.gdn_chunk_fwd_workspace_bytes(8, 4096, 16, 128, 128, 64, 1, 1) == _ws_bytes(8, 4096, 16, 2)
    assert lib.gdn_chunk_fwd_workspace_bytes(1, 256, 2, 64, 64, 64, 0, 1) == _ws_bytes(1, 256, 2, 4)
    assert lib.gdn_chunk_fwd_workspace_bytes(2, 65, 3, 128, 64, 64, 1, 0) == _ws_bytes(2, 65, 3, 2, mode=0)
    assert lib.gdn_chunk_fwd_workspace_bytes(4, 8192, 16, 128, 128, 64, 1, 2) == _ws_bytes(4, 8192, 16, 2, 128, 2)
    assert lib.gdn_chunk_fwd_workspace_bytes(1, 100, 2, 64, 128, 64, 0, 2) == _ws_bytes(1, 100, 2, 4, 64, 2)
    assert lib.gdn_chunk_fwd_workspace_bytes(2, 0, 3, 128, 64, 64, 1, 1) == 0
    assert lib.gdn_chunk_fwd_workspace_bytes(2, 10, 3, 96, 64, 64, 1, 1) == 0      # unsupported


def test_chunk_fwd_checks_workspace(lib):
    q, k, v, a, b, s0, o, sf = _bufs()
    need = _ws_bytes(2, 100, 3, 2)
    ws = (1 << 40) + 9 * (1 << 36)
    assert _fwd(lib, ws=ws, ws_bytes=need - 1) == E_WS
    assert _fwd(lib, ws=0, ws_bytes=need) == E_NULL
    assert _fwd(lib, ws=q + 128, ws_bytes=need) == E_ALIAS     # workspace over q
    need2 = _ws_bytes(2, 100, 3, 2, 128, 2)
    assert _fwd(lib, mode=2, ws=ws, ws_bytes=need2 - 1) == E_WS


def _varlen_ws_bytes(N, T, H, es, dk=128, mode=1):
    # one record per slot: T // 64 + N slots per head bound the chunks of any split
    if T == 0:
        return 0
    slots = H * (T // 64 + N)
    if mode == 2:
        return slots * ((2 * 64 * 64 + 3 * 64 * dk) * es + 4 * dk)
    return slots * ((2 if es == 4 else 1) * 64 * 64 * es + 5 * 64 * 4) + _bound_bytes(slots, es, mode)


def test_varlen_workspace_bounds_every_split():
    """T // 64 + N chunk slots hold the chunks of any split of T tokens into N
    sequences, and sequence s's chunk n at slot cu[s] // 64 + s + n never
    collides with another sequence's (checked over random splits)."""
    import numpy as np
    rng = np.random.default_rng(5)
    for _ in range(2000):
        N = int(rng.integers(1, 12))
        T = int(rng.integers(0, 700))
        cuts = np.sort(rng.integers(0, T + 1, N - 1))
        cu = np.concatenate([[0], cuts, [T]])
        used = set()
        for s in range(N):
            ln = cu[s + 1] - cu[s]
            for n in range((ln + 63) // 64):
                slot = cu[s] // 64 + s + n
                assert slot < T // 64 + N and slot not in used
                used.add(slot)


def test_varlen_workspace_query(lib):
    q = lib.gdn_chunk_fwd_varlen_workspace_bytes
    assert q(16, 32768, 16, 128, 128, 64, 1, 1) == _varlen_ws_bytes(16, 32768, 16, 2)
    assert q(3, 100, 2, 64, 64, 64, 0, 0) == _varlen_ws_bytes(3, 100, 2, 4, 64, 0)
    assert q(5, 1000, 4, 128, 128, 64, 1, 2) == _varlen_ws_bytes(5, 1000, 4, 2, 128, 2)
    assert q(4, 0, 2, 128, 128, 64, 1, 1) == 0
    assert q(4, 10, 2, 96, 128, 64, 1, 1) == 0          # unsupported d_k
    assert q(4, 10, 2, 128, 128, 32, 1, 1) == 0         # unsupported chunk


def test_varlen_rejects_bad_arguments(lib):
    q, k, v, a, b, s0, o, sf = _bufs()
    cu = (1 << 40) + 10 * (1 << 36)
    ws = (1 << 40) + 11 * (1 << 36)

    def fwd(ptrs=None, cu=cu, ws=ws, ws_bytes=1 << 30, N=4, T=300, H=2, dk=128, dv=128, chunk=64,
            dtype=1, mode=1):
        p = ptrs if ptrs is not None else (q, k, v, a, b, s0, o, sf)
        return lib.gdn_chunk_fwd_varlen(*p, cu, ws, ws_bytes, N, T, H, dk, dv, chunk, dtype, mode,
                                        None)

    assert fwd(dk=96) == E_UNSUP
    assert fwd(chunk=128) == E_UNSUP
    assert fwd(T=-1) == E_SHAPE
    assert fwd(N=-1) == E_SHAPE
    assert fwd(N=0, T=10) == E_SHAPE                    # tokens outside every sequence
    assert fwd(dtype=5) == E_DTYPE
    assert fwd(cu=0) == E_NULL
    assert fwd(ptrs=(q, k, v, 0, b, s0, o, sf)) == E_NULL
    assert fwd(ptrs=(q, k, v, a, b, s0, 0, sf)) == E_NULL
    assert fwd(ws=0) == E_NULL
    assert fwd(ws_bytes=_varlen_ws_bytes(4, 300, 2, 2) - 1) == E_WS
    assert fwd(ptrs=(q, k, v, a, b, s0, q + 64, sf)) == E_ALIAS     # o inside q
    assert fwd(cu=o + 64) == E_ALIAS                                # offsets inside o
    assert fwd(cu=sf + 64) == E_ALIAS                               # offsets inside S_final
    assert fwd(ws=cu - 64) == E_ALIAS                               # workspace over the offsets
    assert fwd(N=0, T=0, ptrs=(0, 0, 0, 0, 0, 0, 0, 0), cu=0, ws=0) == OK
    assert fwd(H=0) == OK


def test_decode_rejects_bad_arguments(lib):
    q, k, v, a, b, S, o, _ = _bufs()

    def dec(ptrs=(q, k, v, a, b, S, o), B=4, H=2, dk=128, dv=64, dtype=1, mode=1):
        return lib.gdn_decode_step(*ptrs, B, H, dk, dv, dtype, mode, None)

    assert dec(dk=32) == E_UNSUP
    assert dec(dtype=2) == E_DTYPE
    assert dec(B=-2) == E_SHAPE
    assert dec(ptrs=(q, k, v, a, b, 0, o)) == E_NULL
    assert dec(ptrs=(q, k, v, 0, b, S, o), mode=2) == E_NULL
    assert dec(ptrs=(q, k, v, a, b, S, S + 8)) == E_ALIAS
    assert dec(ptrs=(q, k, v, a, b, q, o)) == E_ALIAS
    assert dec(B=0) == OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import gated_delta_rule_04_amd as gdn
    monkeypatch.setattr(gdn, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(gdn, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        gdn.load()


def _pro(l2=1, eps=1e-6, bl=1, al=1, A=(1 << 40) + 12 * (1 << 36), bias=0):
    import gated_delta_rule_04_amd as gdn
    return gdn.Prologue(l2, eps, bl, al, A, bias or None)


def test_fused_prologue_validation(lib):
    q, k, v, a, b, s0, o, sf = _bufs()
    ws = (1 << 40) + 9 * (1 << 36)

    def fwd(pro, cu=None, mode=1, T=100, B=2, H=3):
        return lib.gdn_chunk_fwd_fused(q, k, v, a, b, s0, o, sf, cu,
                                       None if pro is None else ctypes.byref(pro), ws, 1 << 30,
                                       B, T, H, 128, 128, 64, 1, mode, None)

    assert fwd(_pro(eps=-1.0)) == E_VALUE
    assert fwd(_pro(eps=float("nan"))) == E_VALUE
    assert fwd(_pro(eps=float("inf"))) == E_VALUE
    assert fwd(_pro(A=0)) == E_NULL                        # alpha logits need A
    assert fwd(_pro(A=o + 4)) == E_ALIAS                   # A inside o
    assert fwd(_pro(bias=sf + 4)) == E_ALIAS               # dt_bias inside S_final
    assert fwd(_pro(bias=ws + 4)) == E_ALIAS               # dt_bias inside the workspace
    assert fwd(_pro(), mode=1, B=-1) == E_SHAPE
    assert fwd(_pro(), cu=None, B=0, T=10) == OK            # fixed rows: B = 0, nothing to do
    assert fwd(_pro(), cu=(1 << 40) + 13 * (1 << 36), B=0, T=10) == E_SHAPE   # packed: tokens, no rows
    assert fwd(None, B=0) == OK
    assert fwd(_pro(A=0, al=1), mode=0, B=0) == OK          # nothing to compute


def test_fused_decode_validation(lib):
    q, k, v, a, b, S, o, _ = _bufs()

    def dec(pro, mode=1, B=4, H=2):
        return lib.gdn_decode_step_fused(q, k, v, a, b, S, o,
                                         None if pro is None else ctypes.byref(pro),
                                         B, H, 128, 64, 1, mode, None)

    assert dec(_pro(eps=-0.5)) == E_VALUE
    assert dec(_pro(A=0)) == E_NULL
    assert dec(_pro(A=S + 8)) == E_ALIAS                   # A inside the state
    assert dec(_pro(A=o)) == E_ALIAS                       # A at o
    assert dec(_pro(), B=0) == OK


def test_gdn2_validation(lib):
    q, k, v, a, s0, o, sf, _ = _bufs()
    e, w = (1 << 40) + 14 * (1 << 36), (1 << 40) + 15 * (1 << 36)
    ws = (1 << 40) + 9 * (1 << 36)

    def fwd(ptrs=None, cu=None, B=2, T=100, H=3, dk=128, dv=128, ws_bytes=1 << 30):
        p = ptrs if ptrs is not None else (q, k, v, a, e, w, s0, o, sf)
        return lib.gdn2_chunk_fwd(*p, cu, ws, ws_bytes, B, T, H, dk, dv, 64, 1, None)

    assert fwd(ptrs=(q, k, v, a, 0, w, s0, o, sf)) == E_NULL     # no erase gate
    assert fwd(ptrs=(q, k, v, a, e, 0, s0, o, sf)) == E_NULL     # no write gate
    assert fwd(ptrs=(q, k, v, 0, e, w, s0, o, sf)) == E_NULL     # no decay
    assert fwd(ptrs=(q, k, v, a, e, o + 2, s0, o, sf)) == E_ALIAS
    assert fwd(ptrs=(q, k, v, a, sf, w, s0, o, sf)) == E_ALIAS
    assert fwd(dk=96) == E_UNSUP
    assert fwd(ws_bytes=_ws_bytes(2, 100, 3, 2, 128, 2) - 1) == E_WS
    assert fwd(B=0) == OK

    def dec(ptrs=None, B=4, H=2):
        p = ptrs if ptrs is not None else (q, k, v, a, e, w, s0, o)
        return lib.gdn2_decode_step(*p, B, H, 128, 64, 1, None)

    assert dec(ptrs=(q, k, v, a, 0, w, s0, o)) == E_NULL
    assert dec(ptrs=(q, k, v, a, e, w, s0, e)) == E_ALIAS           # o over the erase gate
    assert dec(ptrs=(q, k, v, a, e, s0 + 8, s0, o)) == E_ALIAS      # write gate inside S
    assert dec(B=0) == OK


def test_backward_validation(lib):
    base = 1 << 40
    p = [base + i * (1 << 36) for i in range(16)]
    q, k, v, a, b, s0, do, dst, dq, dk, dv, da, db, ds0, ws = p[:15]

    def bwd(ptrs=None, B=2, T=100, H=3, dk_=128, dv_=128, mode=1, ws_bytes=1 << 34, w=ws):
        args = ptrs if ptrs is not None else (q, k, v, a, b, s0, do, dst, dq, dk, dv, da, db, ds0)
        return lib.gdn_chunk_bwd(*args, w, ws_bytes, B, T, H, dk_, dv_, 64, 1, mode, None)

    assert bwd(dk_=96) == E_UNSUP
    assert bwd(T=-1) == E_SHAPE
    assert bwd(mode=4) == E_DTYPE
    assert bwd(ptrs=(q, k, v, a, b, s0, 0, dst, dq, dk, dv, da, db, ds0)) == E_NULL    # no dout
    assert bwd(ptrs=(q, k, v, a, b, s0, do, dst, dq, dk, dv, 0, db, ds0)) == E_NULL    # no dalpha
    assert bwd(ptrs=(q, k, v, a, b, s0, do, dst, q, dk, dv, da, db, ds0)) == E_ALIAS   # dq over q
    assert bwd(ptrs=(q, k, v, a, b, s0, do, dst, dq, dq + 64, dv, da, db, ds0)) == E_ALIAS   # dk in dq
    assert bwd(w=dq + 128) == E_ALIAS                                                 # ws in dq
    # fp32 (and per-channel decay): the token-level kernels, state checkpoints every 8 tokens
    need = lib.gdn_chunk_bwd_workspace_bytes(2, 100, 3, 128, 128, 64, 0, 1)
    chunks, nth = 13, 2 * 100 * 3
    assert need == 2 * 3 * chunks * 128 * 128 * 4 + 2 * 4 * nth * 128 * 4 + 2 * 4 * nth * 4
    # bf16, scalar or no decay: the chunk-level kernels; per chunk of every head the
    # forward's record (T bf16 + five fp32 gate rows), a bf16 state and a bf16 state gradient
    nch = 2 * 3 * 2
    need = lib.gdn_chunk_bwd_workspace_bytes(2, 100, 3, 128, 128, 64, 1, 1)
    assert need == nch * (64 * 64 * 2 + 5 * 64 * 4) + 2 * nch * 128 * 128 * 2
    assert lib.gdn_chunk_bwd_workspace_bytes(2, 100, 3, 128, 128, 64, 1, 0) == need
    assert bwd(ws_bytes=need - 1) == E_WS
    assert bwd(B=0) == OK


def test_noalloc_validation(lib):
    """gdn_chunk_fwd_noalloc validates exactly as gdn_chunk_fwd and rejects a
    call whose records exceed the scratch array before touching the device."""
    vp, i = ctypes.c_void_p, ctypes.c_int
    f = lib.gdn_chunk_fwd_noalloc
    f.argtypes = [vp] * 8 + [i] * 8 + [vp]
    f.restype = i
    q, k, v, a, b, s0, o, sf = _bufs()

    def call(B=2, T=100, H=3, dk=128, dv=128, chunk=64, dtype=1, mode=1, ptrs=None):
        p = ptrs if ptrs is not None else (q, k, v, a, b, s0, o, sf)
        return f(*p, B, T, H, dk, dv, chunk, dtype, mode, None)

    scratch = 64 << 20
    # bf16 scalar decay: the most chunk records (with their bounds) that fit the array
    nmax = max(n for n in range(7000, 7200) if _ws_bytes(1, 64 * n, 1, 2) <= scratch)
    assert nmax == 7081
    assert call(B=1, T=64 * (nmax + 1), H=1) == E_WS      # one record too many
    assert call(B=8, T=4096, H=16) == E_WS                 # 8192 records
    assert call(B=1, T=64 * 1017, H=1, mode=2) == E_WS     # per-channel records are larger
    assert call(dk=96) == E_UNSUP
    assert call(chunk=32) == E_UNSUP
    assert call(T=-1) == E_SHAPE
    assert call(dtype=5) == E_DTYPE
    assert call(ptrs=(0, k, v, a, b, s0, o, sf)) == E_NULL
    assert call(ptrs=(q, k, v, a, b, s0, q + 64, sf)) == E_ALIAS
    assert call(B=0) == OK and call(H=0) == OK
    assert call(T=0, ptrs=(0, 0, 0, 0, 0, 0, 0, 0)) == OK  # nothing to write


def test_gated_rmsnorm_validation(lib):
    o, g, w, y = _bufs()[:4]
    call = lambda o=o, g=g, w=w, y=y, rows=100, dv=128, eps=1e-6, dt=1: lib.gdn_gated_rmsnorm(
        o, g, w, y, rows, dv, eps, dt, None)
    assert call(dv=96) == E_UNSUP
    assert call(rows=-1) == E_SHAPE
    assert call(dv=0) == E_SHAPE
    assert call(dt=5) == E_DTYPE
    assert call(eps=-1.0) == E_VALUE
    assert call(eps=float("inf")) == E_VALUE
    assert call(eps=float("nan")) == E_VALUE
    assert call(o=0) == E_NULL and call(g=0) == E_NULL and call(w=0) == E_NULL and call(y=0) == E_NULL
    assert call(y=g) == E_ALIAS                  # out over the gate
    assert call(y=o + 64) == E_ALIAS             # out partly over o
    assert call(y=w - 16) == E_ALIAS             # out over the gain
    assert call(rows=0, o=0, g=0, w=0, y=0) == OK   # nothing to do
    assert call(rows=1 << 62) == E_SHAPE         # element count overflow
