"""Virtual Head Attention (VHA) mixing step written out in NumPy float64.

TEST INFRASTRUCTURE ONLY: like the rest of this package, only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may use it, and it shares
no code with the HIP library.

ERNIE 5.5 Flash Base release blog, section 2.1: after attention, VHA adds a light low-rank
mixing step across heads with an identity skip connection, so that heads share information.
Read here, per token m and channel j of the head dimension, as
    out[m, h, j] = o[m, h, j] + sum_{h'} (U V^T)[h, h'] o[m, h', j]
with U, V of shape [H, r] (rank r; the pages give neither the rank nor the weights) and o the
gated attention output.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    """Stored values as float64 (uint16 arrays hold bfloat16 bits); widening is exact."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def vha_mix(o, u, v):
    """o [M, H, d], u and v [H, r] -> out [M, H, d] float64: z = V^T o per token (the rank-r
    mix of the heads), then out = o + U z."""
    O, U, V = _f64(o), _f64(u), _f64(v)
    Z = np.einsum("hr,mhj->mrj", V, O)
    return O + np.einsum("hr,mrj->mhj", U, Z)
