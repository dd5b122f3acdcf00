"""Oracle: grouped (MoE) W8A8 per-group-128 GEMM (test infrastructure only).

Follows [P3] sec. 1.3 / 4.4 (all experts resident, each token runs through a
few of them) with the rows already sorted by expert: expert e owns rows
[offsets[e], offsets[e+1]) of the quantised activations and multiplies them
with its own weights qw[e] / scales sw[e] by the dense rule of gemm.py.
Empty experts contribute nothing. [P2] "Loose ends" item 2 is the reason the
segment bounds (not any padded tile bound) decide which rows belong to an
expert.
"""
from __future__ import annotations

import numpy as np

from .gemm import gemm_ref, gemm_fp32_ordered_ref


def _segments(offsets, E):
    off = np.asarray(offsets, np.int64)
    if off.shape != (E + 1,) or off[0] != 0 or np.any(np.diff(off) < 0):
        raise ValueError("offsets must be [E+1], start at 0 and be non-decreasing")
    return off


def grouped_gemm_ref(q, sa, qw, sw, offsets):
    """float64 definition per expert segment. Returns (y64 [R,N], mag [R,N])."""
    E, N, _ = qw.shape
    off = _segments(offsets, E)
    R = int(off[-1])
    y = np.zeros((R, N), np.float64)
    mag = np.zeros((R, N), np.float64)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            y[lo:hi], mag[lo:hi] = gemm_ref(q[lo:hi], sa[lo:hi], qw[e], sw[e])
    return y, mag


def grouped_gemm_fp32_ordered_ref(q, sa, qw, sw, offsets):
    """float32 stated order per expert segment. Returns (y32 [R,N], y_bf16 [R,N])."""
    E, N, _ = qw.shape
    off = _segments(offsets, E)
    R = int(off[-1])
    y32 = np.zeros((R, N), np.float32)
    yb = np.zeros((R, N), np.uint16)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            y32[lo:hi], yb[lo:hi] = gemm_fp32_ordered_ref(q[lo:hi], sa[lo:hi], qw[e], sw[e])
    return y32, yb
