"""Oracle: INT8 weights repacked into the matrix cores' operand order (test infrastructure only).

[P1] sec. 2 has the quantised weights rearranged once, at load time, into the
layout of the kernel that consumes them; the pages leave that layout to the
kernel. The one used here cuts qw [N, K] into blocks of 16 rows x 64 columns
and stores each as 1024 contiguous bytes:

    packed[((n // 16) * (K // 64) + k // 64) * 1024 + 16 * l + k % 16] = qw[n, k]
        with l = n % 16 + 16 * ((k % 64) // 16)

(l is the lane that supplies those 16 bytes of one 16x16x64 INT8 matrix
instruction: lane l carries row l % 16 and K positions 16 * (l // 16) .. +15 of
the instruction's 64). The repack moves bytes only; the GEMM on the packed
weights computes what the row-major GEMM computes on qw, so its oracle is
``gemm_fp32_ordered_ref`` (and ``gemm_ref``) on the unpacked qw.
"""
from __future__ import annotations

import numpy as np


def _check(N: int, K: int) -> None:
    if N % 16 or K % 128 or N < 16:
        raise ValueError("N must be a multiple of 16 and K a multiple of 128")


def packed_position_ref(n, k, K: int):
    """Byte position of qw[n, k] in the packed form (n, k integer arrays or scalars)."""
    n = np.asarray(n, np.int64)
    k = np.asarray(k, np.int64)
    lane = n % 16 + 16 * ((k % 64) // 16)
    return ((n // 16) * (K // 64) + k // 64) * 1024 + 16 * lane + k % 16


def repack_mfma_ref(qw: np.ndarray) -> np.ndarray:
    """packed [N*K] int8: every qw[n, k] written at its position."""
    N, K = qw.shape
    _check(N, K)
    n, k = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    out = np.zeros(N * K, np.int8)
    out[packed_position_ref(n, k, K).ravel()] = qw.ravel()
    return out


def unpack_mfma_ref(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    """The inverse: qw [N, K] read back from the packed form."""
    _check(N, K)
    n, k = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    return np.asarray(packed)[packed_position_ref(n, k, K)]
