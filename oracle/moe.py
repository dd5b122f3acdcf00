"""Oracle: the MoE glue either side of the grouped GEMM (test infrastructure only).

[P3] sec. 1.3 / 4.4: all experts stay resident and each token runs through a
few of them; the tokens are dispatched to their experts and the experts'
outputs are combined back per token. On one GPU that is:

* quantise the T tokens once, then gather the INT8 rows and their scales
  into expert order (row r of the sorted batch is token token_of_row[r]).
  The quantisation rule works row by row, so quantising before or after the
  gather gives the same bits.
* after the grouped GEMM, combine: token t's output is the sum over its k
  selected experts of gate[t, k] times that expert's output row
  row_of_pair[t, k].

Readings (the pages give no precision for the combine): expert outputs are
BF16, the gate weights float32; the definition below is exact in float64,
and the ordered float32 replay is the order the kernel keeps: a fused
multiply-add per slot, k ascending, starting from 0, then one BF16 rounding
(round to nearest even).
"""
from __future__ import annotations

import numpy as np

from .gemm import fmaf_ref, f32_to_bf16_bits_ref, bf16_bits_to_f32_ref


def gather_rows_ref(q: np.ndarray, sa: np.ndarray, index: np.ndarray):
    """(q[index], sa[index]): the sorted batch's rows and scales."""
    index = np.asarray(index, np.int64)
    if index.size and (index.min() < 0 or index.max() >= q.shape[0]):
        raise ValueError("index out of range")
    return q[index], sa[index]


def _check_combine(y_bits, row_of_pair, gate):
    rp = np.asarray(row_of_pair, np.int64)
    if rp.shape != gate.shape:
        raise ValueError("row_of_pair and gate must both be [T, topk]")
    if rp.size and (rp.min() < 0 or rp.max() >= y_bits.shape[0]):
        raise ValueError("row_of_pair out of range")
    return rp


def moe_combine_ref(y_bits: np.ndarray, row_of_pair: np.ndarray, gate: np.ndarray):
    """float64 definition out[t] = sum_k gate[t,k] * y[row_of_pair[t,k]] and the
    magnitude sum_k |gate * y| (for the tolerance under cancellation)."""
    rp = _check_combine(y_bits, row_of_pair, gate)
    y = bf16_bits_to_f32_ref(y_bits).astype(np.float64)
    g = gate.astype(np.float64)
    T, topk = rp.shape
    out = np.zeros((T, y.shape[1]), np.float64)
    mag = np.zeros_like(out)
    for k in range(topk):
        term = g[:, k:k + 1] * y[rp[:, k]]
        out += term
        mag += np.abs(term)
    return out, mag


def moe_combine_fp32_ordered_ref(y_bits: np.ndarray, row_of_pair: np.ndarray,
                                 gate: np.ndarray):
    """The float32 steps in the kernel's order. Returns (out32, out_bf16_bits)."""
    rp = _check_combine(y_bits, row_of_pair, gate)
    y = bf16_bits_to_f32_ref(y_bits)
    T, topk = rp.shape
    acc = np.zeros((T, y.shape[1]), np.float32)
    for k in range(topk):
        w = np.broadcast_to(gate[:, k:k + 1].astype(np.float32), acc.shape)
        acc = fmaf_ref(w, y[rp[:, k]], acc)
    return acc, f32_to_bf16_bits_ref(acc)
