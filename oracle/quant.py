"""Oracle: dynamic per-token INT8 quantisation (test infrastructure only).

Follows [P3] sec. 3.1: activations are quantised per token at run time, the
scale derived from that token's own range. The rule written out here:

    amax  = max_k |x[k]|                        (exact)
    scale = fl32(amax / 127)                    (IEEE float32 divide, RN-even)
    q[k]  = clamp(rint(fl32(x[k] / scale)), -127, 127)   (rint = half-to-even)

Readings where the statement is silent:
  * amax == 0 (all-zero row): scale = 0 and q = 0 (no 0/0 is formed).
  * the divide is a true IEEE divide by the stored float32 scale, never a
    multiply by a reciprocal; subnormals are honoured (no flush to zero).
  * the same rule quantises a decoded weight group of 128 (see decode.py).
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns (uint16) -> float32 values; exact (zero-extend the mantissa)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def quantize_rows_ref(v: np.ndarray):
    """Absmax INT8 quantisation of each row of a float32 matrix.

    Returns (q int8 [R, L], scale float32 [R]).
    """
    v = np.ascontiguousarray(v, dtype=np.float32)
    if v.ndim != 2:
        raise ValueError("expected a 2-D array")
    amax = np.max(np.abs(v), axis=1) if v.shape[1] else np.zeros(v.shape[0], np.float32)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    q = np.zeros(v.shape, dtype=np.int8)
    nz = amax > 0
    if np.any(nz):
        t = v[nz] / scale[nz][:, None]          # float32 / float32: IEEE divide
        r = np.rint(t)                           # round half to even
        q[nz] = np.clip(r, -127.0, 127.0).astype(np.int8)
    return q, scale


def quantize_act_ref(x_bits: np.ndarray):
    """quantize_act: BF16 activations [M,K] (uint16 bits) -> (q int8 [M,K], sa float32 [M])."""
    return quantize_rows_ref(bf16_bits_to_f32(x_bits))
