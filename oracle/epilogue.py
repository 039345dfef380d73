"""fp64 reference of the output epilogue of the Gated DeltaNet mixer: a gated
RMSNorm of each (token, head) output row.  Test infrastructure only (see the
package docstring).

What the pages fix: the Gated DeltaNet baseline passes its output through an
RMSNorm, a learnable gain and a SiLU gate (NextTransformer "method sources"
page, baseline section, Gated DeltaNet entry), the output-gated RMSNorm of
the training backend (same page, backend and numerics section).  The pages
leave open the epsilon and the order of gain and gate; the plain reading
used here normalises first, then scales by the gain, then by the gate:

    y = o / sqrt(mean(o^2) + eps) * w * silu(g),   silu(g) = g sigmoid(g),

over the d_v values of each row, w a gain of d_v values shared by all heads.
"""
from __future__ import annotations

import numpy as np

from .loop import _f64


def silu(g):
    g = _f64(g)
    return g / (1.0 + np.exp(-g))


def gated_rmsnorm(o, gate, weight, eps: float):
    """o, gate [..., dv]; weight [dv].  Returns fp64 [..., dv]."""
    o = _f64(o)
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o * r * _f64(weight) * silu(gate)
