"""Oracle: W8A8 per-group-128 GEMM (test infrastructure only).

Follows [P3] sec. 3.1: INT8 x INT8 multiply-accumulate into INT32 inside the
matmul, and the float32 scales multiplied in last. With per-(row n, 128-wide K
group g) weight scales sw and per-token activation scales sa that reads

    P[m,n,g] = sum_{k in group g} q[m,k] * qw[n,k]           (exact INT32)
    y[m,n]   = sa[m] * sum_g sw[n,g] * P[m,n,g]

Two forms are given:
  * ``gemm_ref``: the plain definition evaluated in float64 (group order
    ascending), plus the magnitude  mag = |sa| * sum_g |sw * P|  that the
    tolerance is stated against.
  * ``gemm_fp32_ordered_ref``: the same steps in float32 in the stated order
    (INT32 partial of group g, converted, fused multiply-add with sw[n,g] into
    a float32 accumulator, g ascending; then one float32 multiply by sa[m]),
    with the BF16 store rounding to nearest even. This is the reading of
    "INT32 accumulate, FP32 scale last" that the kernels follow; it is used
    for the strict (bit-for-bit) comparisons.

Exactness: |q|, |qw| <= 127, so every product is an integer of magnitude
<= 16129 and every group sum has magnitude <= 128*127^2 = 2,064,512 < 2^21.
A float64 matmul of the integer-valued operands is therefore exact in any
summation order, which is how P is formed here.
"""
from __future__ import annotations

import numpy as np

GROUP = 128


def _check(q, qw):
    if q.ndim != 2 or qw.ndim != 2 or q.shape[1] != qw.shape[1]:
        raise ValueError("q [M,K] and qw [N,K] required")
    if q.shape[1] % GROUP:
        raise ValueError("K must be a multiple of 128")


def group_partial_ref(q: np.ndarray, qw: np.ndarray, g: int) -> np.ndarray:
    """P[:, :, g] as float64 (exactly integer-valued)."""
    sl = slice(GROUP * g, GROUP * (g + 1))
    return q[:, sl].astype(np.float64) @ qw[:, sl].astype(np.float64).T


def group_partials_ref(q: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """All group partials P int32 [M, N, K/128]."""
    _check(q, qw)
    M, K = q.shape
    N = qw.shape[0]
    G = K // GROUP
    P = np.empty((M, N, G), np.int32)
    for g in range(G):
        P[:, :, g] = group_partial_ref(q, qw, g).astype(np.int32)
    return P


def gemm_ref(q, sa, qw, sw):
    """Plain definition in float64. Returns (y64 [M,N], mag [M,N])."""
    _check(q, qw)
    M, K = q.shape
    N = qw.shape[0]
    G = K // GROUP
    sw64 = np.asarray(sw, np.float32).astype(np.float64)
    acc = np.zeros((M, N), np.float64)
    mag = np.zeros((M, N), np.float64)
    for g in range(G):
        t = group_partial_ref(q, qw, g) * sw64[:, g][None, :]   # exact products
        acc += t
        mag += np.abs(t)
    sa64 = np.asarray(sa, np.float32).astype(np.float64)[:, None]
    return sa64 * acc, np.abs(sa64) * mag


def fmaf_ref(a, b, c) -> np.ndarray:
    """Correctly rounded float32 fused multiply-add  RN(a*b + c), elementwise.

    a*b of two float32 values is exact in float64. The float64 sum s = RN64(a*b + c)
    and its exact error e (TwoSum) give the exact result s + e; moving s one
    float64 ulp towards e whenever e != 0 and s has an even last bit yields the
    round-to-odd value of the exact sum, and rounding that to float32 is the
    correctly rounded result because 53 >= 24 + 2 (Boldo & Melquiond, "Emulation
    of FMA and correctly rounded sums: proved algorithms using rounding to odd",
    IEEE Trans. Computers 2008).
    """
    a64 = np.asarray(a, np.float32).astype(np.float64)
    b64 = np.asarray(b, np.float32).astype(np.float64)
    c64 = np.asarray(c, np.float32).astype(np.float64)
    p = a64 * b64
    p, c64 = np.broadcast_arrays(p, c64)
    s = p + c64
    bp = s - c64
    ap = s - bp
    e = (p - ap) + (c64 - bp)
    s = np.array(s, dtype=np.float64, copy=True)
    fix = (e != 0) & ((s.view(np.int64) & 1) == 0)
    if np.any(fix):
        s[fix] = np.nextafter(s[fix], np.where(e[fix] > 0, np.inf, -np.inf))
    return s.astype(np.float32)


def f32_to_bf16_bits_ref(y: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bit pattern, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(y, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32_ref(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def gemm_fp32_ordered_ref(q, sa, qw, sw):
    """The stated steps in float32 order. Returns (y32 float32 [M,N], y_bf16 uint16 [M,N])."""
    _check(q, qw)
    M, K = q.shape
    N = qw.shape[0]
    G = K // GROUP
    sw32 = np.asarray(sw, np.float32)
    acc = np.zeros((M, N), np.float32)
    for g in range(G):
        p = group_partial_ref(q, qw, g).astype(np.float32)   # exact: |P| < 2^24
        acc = fmaf_ref(p, sw32[:, g][None, :], acc)
    y32 = (acc * np.asarray(sa, np.float32)[:, None]).astype(np.float32)   # IEEE float32 multiply
    return y32, f32_to_bf16_bits_ref(y32)
