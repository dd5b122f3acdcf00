"""Oracle: block-scaled weight formats -> INT8 per-group-128 (test infrastructure only).

Formats named by [P1] sec. 1 (ordinary linears: FP8 e4m3 with [128,128]
UE8M0 block scales; routed experts: packed MXFP4 E2M1 with UE8M0 scales) and
re-routed onto INT8 by dequantise-and-repack in [P1] sec. 2. [P2] "FP8
dialect clash": OCP and fnuz e4m3 share the bit layout but their exponent
biases differ by one, so the same byte read in the other dialect is off by
exactly a factor of two; the dialect is therefore an explicit argument.

Bit fields, written out from the format definitions:
  e4m3 byte b:  s = b>>7, e = (b>>3)&15, m = b&7
     OCP  (E4M3FN,  bias 7): e=0 -> m/8 * 2^-6 ; else (1+m/8) * 2^(e-7);
                             0x7F/0xFF are NaN, 0x80 is -0, max 448.
     fnuz (E4M3FNUZ, bias 8): e=0 -> m/8 * 2^-7 ; else (1+m/8) * 2^(e-8);
                             0x80 is NaN, no -0, no inf, max 240.
  E2M1 nibble c: s = c>>3, e = (c>>1)&3, m = c&1
                 e=0 -> m/2 ; else (1+m/2) * 2^(e-1)    (no NaN/inf; 8 is -0)
  UE8M0 byte E:  2^(E-127); E=255 is NaN.

Readings (the pages name the formats but not these details):
  * OCP carries bias 7 and fnuz bias 8, so OCP value = 2 x fnuz value.
  * the block-scale grid of an [N,K] weight is [N/128, K/128] (output rows x
    input columns); MXFP4 blocks are 1x32 along K.
  * nibble order: element 2j is the low nibble of byte j, 2j+1 the high one.
  * the repack rule is the same absmax rule as the activations (quant.py),
    applied to each (row n, 128-wide K group) of the decoded float32 weight.
    It is lossy in general (a group can span more than 127 distinct steps).
"""
from __future__ import annotations

import numpy as np

from .quant import quantize_rows_ref

GROUP = 128
OCP, FNUZ = 0, 1


def fp8_e4m3_table(dialect: int) -> np.ndarray:
    """float64 value of each of the 256 e4m3 bytes in the given dialect (NaN where undefined)."""
    if dialect not in (OCP, FNUZ):
        raise ValueError("dialect must be OCP (0) or FNUZ (1)")
    bias = 7 if dialect == OCP else 8
    t = np.empty(256, np.float64)
    for b in range(256):
        s, e, m = b >> 7, (b >> 3) & 15, b & 7
        if e == 0:
            mag = (m / 8.0) * 2.0 ** (1 - bias)
        else:
            mag = (1.0 + m / 8.0) * 2.0 ** (e - bias)
        t[b] = -mag if s else mag
    if dialect == OCP:
        t[0x7F] = np.nan
        t[0xFF] = np.nan
    else:
        t[0x80] = np.nan
    return t


def ue8m0_value(E) -> np.ndarray:
    """2^(E-127) as float64 (NaN for E == 255)."""
    E = np.asarray(E, np.int64)
    v = np.ldexp(1.0, E - 127)
    return np.where(E == 255, np.nan, v)


def e2m1_table() -> np.ndarray:
    """float64 value of each of the 16 E2M1 codes."""
    t = np.empty(16, np.float64)
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        mag = m / 2.0 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1)
        t[c] = -mag if s else mag
    return t


def dequant_fp8_block_ref(w: np.ndarray, bs: np.ndarray, dialect: int) -> np.ndarray:
    """Decoded float32 weight W[n,k] = e4m3(w[n,k]) * 2^(bs[n/128, k/128] - 127) (exact)."""
    N, K = w.shape
    if N % GROUP or K % GROUP or bs.shape != (N // GROUP, K // GROUP):
        raise ValueError("w [N,K] with N, K multiples of 128 and bs [N/128, K/128] required")
    vals = fp8_e4m3_table(dialect)[w]
    scale = np.repeat(np.repeat(ue8m0_value(bs), GROUP, axis=0), GROUP, axis=1)
    return (vals * scale).astype(np.float32)


def decode_fp8_block_ref(w, bs, dialect):
    """FP8 e4m3 [N,K] + [N/128,K/128] UE8M0 -> (qw int8 [N,K], sw float32 [N,K/128])."""
    W = dequant_fp8_block_ref(w, bs, dialect)
    N, K = W.shape
    q, s = quantize_rows_ref(W.reshape(N * (K // GROUP), GROUP))
    return q.reshape(N, K), s.reshape(N, K // GROUP)


def dequant_mxfp4_ref(packed: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Decoded float32 weight [E,N,K] from packed E2M1 [E,N,K/2] and UE8M0 [E,N,K/32] (exact)."""
    E, N, Kh = packed.shape
    K = 2 * Kh
    if K % GROUP or scale.shape != (E, N, K // 32):
        raise ValueError("packed [E,N,K/2] with K a multiple of 128 and scale [E,N,K/32] required")
    codes = np.empty((E, N, K), np.uint8)
    codes[..., 0::2] = packed & 0x0F
    codes[..., 1::2] = packed >> 4
    vals = e2m1_table()[codes]
    sc = np.repeat(ue8m0_value(scale), 32, axis=2)
    return (vals * sc).astype(np.float32)


def decode_mxfp4_ref(packed, scale):
    """MXFP4 -> (qw int8 [E,N,K], sw float32 [E,N,K/128])."""
    W = dequant_mxfp4_ref(packed, scale)
    E, N, K = W.shape
    q, s = quantize_rows_ref(W.reshape(E * N * (K // GROUP), GROUP))
    return q.reshape(E, N, K), s.reshape(E, N, K // GROUP)
