"""Oracle: W8A8 GEMM with per-channel or per-tensor weight scales (test infrastructure only).

[P3] sec. 3.1 names the three common weight-scale granularities: one scale for
the whole tensor, one per output channel (row n of the [N, K] weight), and one
per 128-element group (the path the rest of this package pins). Its
deployment checklist (sec. 6) runs per-tensor first and then moves to per-group
128. With per-token activation scales sa and the INT8 x INT8 -> INT32
multiply-accumulate of sec. 3.1, the two coarser forms read

    P[m,n] = sum_k q[m,k] * qw[n,k]                 (exact INT32, the whole of K)
    y[m,n] = sa[m] * sw[n] * P[m,n]                 (per-channel; per-tensor: sw[n] = s)

Reading (the pages give no order for the float steps): the INT32 total is
converted to float32 (round to nearest even), multiplied by the weight scale,
then by the activation scale ("FP32 scales last", the weight scale first as in
the per-group form), each product rounded to float32, and the BF16 store rounds
to nearest even. Per-tensor is the per-channel rule with every sw[n] equal.

Exactness: |q|, |qw| <= 127, so |P| <= 16129*K, which stays below 2^31 for
K <= 131072 (the INT32 accumulator's bound) and below 2^53, so the float64
matmul of the integer-valued operands is exact in any summation order.
"""
from __future__ import annotations

import numpy as np

from .gemm import f32_to_bf16_bits_ref

K_MAX = 131072   # 127 * 127 * 131072 = 2,114,060,288 < 2^31


def _check(q, qw, sw):
    if q.ndim != 2 or qw.ndim != 2 or q.shape[1] != qw.shape[1]:
        raise ValueError("q [M,K] and qw [N,K] required")
    if q.shape[1] > K_MAX:
        raise ValueError("K beyond the INT32 accumulator's bound")
    sw = np.asarray(sw, np.float32).reshape(-1)
    if sw.size not in (1, qw.shape[0]):
        raise ValueError("sw must hold one scale per row of qw, or one in all")
    return np.broadcast_to(sw, (qw.shape[0],))


def channel_total_ref(q: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """P [M,N] as int64 (exact)."""
    return (q.astype(np.float64) @ qw.astype(np.float64).T).astype(np.int64)


def gemm_channel_ref(q, sa, qw, sw):
    """Plain definition in float64. Returns (y64 [M,N], mag [M,N] = |y64|)."""
    swn = _check(q, qw, sw).astype(np.float64)
    P = channel_total_ref(q, qw).astype(np.float64)
    y = np.asarray(sa, np.float32).astype(np.float64)[:, None] * (P * swn[None, :])
    return y, np.abs(y)


def gemm_channel_fp32_ordered_ref(q, sa, qw, sw):
    """The float32 steps in order. Returns (y32 float32 [M,N], y_bf16 uint16 [M,N])."""
    swn = _check(q, qw, sw)
    p32 = channel_total_ref(q, qw).astype(np.float64).astype(np.float32)   # one rounding
    t = (p32 * swn[None, :]).astype(np.float32)
    y32 = (t * np.asarray(sa, np.float32)[:, None]).astype(np.float32)
    return y32, f32_to_bf16_bits_ref(y32)
