"""Oracle: GEMMs with BF16 activations (test infrastructure only).

[P1] sec. 1-2 describes the two routes the pages run besides W8A8: the dense
linears' FP8 weights are dequantised to BF16 when the model loads and run as
BF16 GEMMs, and the routed experts take a weight-only INT8 route ("WNA16":
INT8 weights, 16-bit activations). On this path's weights they read

    W8A16:  y[m,n] = sum_g sw[n,g] * sum_{k in group g} x[m,k] * qw[n,k]
    BF16:   y[m,n] = sum_k x[m,k] * w[n,k]

with x [M,K] BF16, qw [N,K] INT8 and sw [N,K/128] float32 as in the W8A8 form,
and w [N,K] BF16. The dequantisation that feeds the BF16 route is the exact
FP8 block value e4m3(w) * 2^(E-127) rounded to BF16 (to nearest even; exact
unless the value is a BF16 subnormal).

Reading (the pages fix no arithmetic for these routes): every product is exact
in float32 (BF16 x INT8 has at most 15 significant bits, BF16 x BF16 at most
16); the matrix core adds the 128 products of a group in float32 in an order
the hardware defines, and the group sums are combined in group order, by a
fused multiply-add with sw[n,g] (W8A16) or a float32 add (BF16). Only a bound
on the result is therefore fixed: any such order stays within
(127 + G) * 2^-24 * mag of the exact value, mag being the sum of the terms'
magnitudes returned here. The definitions below are exact in float64 (every
product is exact there, and the sums of at most 2^17 such terms lose less than
that bound by orders of magnitude).
"""
from __future__ import annotations

import numpy as np

from .decode import dequant_fp8_block_ref
from .gemm import GROUP, bf16_bits_to_f32_ref, f32_to_bf16_bits_ref


def _bf16(bits) -> np.ndarray:
    return bf16_bits_to_f32_ref(np.asarray(bits, np.uint16)).astype(np.float64)


def gemm_w8a16_ref(x_bits, qw, sw):
    """W8A16 in float64. Returns (y64 [M,N], mag [M,N] = sum_g |sw| * sum_k |x * qw|)."""
    x = _bf16(x_bits)
    M, K = x.shape
    N = qw.shape[0]
    if qw.shape != (N, K) or K % GROUP or np.shape(sw) != (N, K // GROUP):
        raise ValueError("x [M,K], qw [N,K], sw [N,K/128] with K a multiple of 128 required")
    sw64 = np.asarray(sw, np.float32).astype(np.float64)
    y = np.zeros((M, N))
    mag = np.zeros((M, N))
    for g in range(K // GROUP):
        sl = slice(GROUP * g, GROUP * (g + 1))
        xg, wg = x[:, sl], qw[:, sl].astype(np.float64)
        y += (xg @ wg.T) * sw64[:, g][None, :]
        mag += (np.abs(xg) @ np.abs(wg).T) * np.abs(sw64[:, g])[None, :]
    return y, mag


def gemm_bf16_ref(x_bits, w_bits):
    """BF16 GEMM in float64. Returns (y64 [M,N], mag [M,N] = sum_k |x * w|)."""
    x, w = _bf16(x_bits), _bf16(w_bits)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[1] or x.shape[1] % GROUP:
        raise ValueError("x [M,K] and w [N,K] with K a multiple of 128 required")
    return x @ w.T, np.abs(x) @ np.abs(w).T


def a16_tolerance(K: int) -> float:
    """The factor t with |y - y64| <= t * mag for any float32 order of the steps above."""
    return (127 + K // GROUP + 2) * 2.0 ** -24


def dequant_fp8_block_bf16_ref(w, bs, dialect) -> np.ndarray:
    """The load-time dequantisation to BF16: the exact FP8 block value, rounded to BF16."""
    return f32_to_bf16_bits_ref(dequant_fp8_block_ref(w, bs, dialect))
