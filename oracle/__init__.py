"""fp64 CPU oracle of the gated delta-rule recurrence.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import anything from this package.  The HIP
library never includes, links or calls it, and this package imports nothing
from the HIP library: the two share no code.

Contents
--------
``gdn_oracle.c``     plain fp64 token-by-token loop (prefill and decode), the
                     definition of what the path computes.
``loop.py``          ctypes loader for it: :func:`gdn_fwd`, :func:`gdn_fwd_varlen`
                     (packed sequences of varying length), :func:`gdn_decode`.
``prologue.py``      fp64 per-token prologue of the mixer layers (L2-normalised
                     q and k, beta from logits, alpha = exp(-a softplus(x + b)))
                     in front of the loop.
``epilogue.py``      fp64 gated RMSNorm of the output rows (RMSNorm, gain,
                     SiLU gate), the mixer's output epilogue.
``backward.py``      fp64 gradients of the loop (torch reverse mode on the same
                     recurrence), pinned to finite differences of the C loop.
``chunk_form.py``    fp64 NumPy chunkwise (UT/WY) rewrite of the same loop;
                     it is checked against the loop and documents the algebra
                     the GPU path follows, but never produces expected values
                     for the GPU path on its own.

Every function states the passage of the pages it follows.  Parity status:
all oracle functions are pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` (worked example, closed forms, exact rational
evaluation of the product form, invariants).
"""
from . import backward, epilogue, prologue  # noqa: F401
from .loop import (gdn_fwd, gdn_fwd_varlen, gdn_decode, build, num_threads, Oracle, compile_library,
                   SOURCE, MODE_NONE, MODE_SCALAR, MODE_CHANNEL, MODE_GDN2)

__all__ = ["gdn_fwd", "gdn_fwd_varlen", "gdn_decode", "build", "num_threads", "Oracle", "compile_library", "SOURCE",
           "MODE_NONE", "MODE_SCALAR", "MODE_CHANNEL", "MODE_GDN2"]
