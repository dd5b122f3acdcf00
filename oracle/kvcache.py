"""Oracle: INT8 KV cache and decode attention over it (test infrastructure only).

[P3] sec. 2.2 counts the KV cache as a memory cost on the order of the
weights (2 x layers x KV heads x head dim x sequence x batch x bytes per
element; batch 32 at 4096 tokens in its example) and quantises it to INT8
too. Sec. 3.4 fixes the scheme: dynamic per-token scaling, one scale for
each key vector and each value vector, computed when the vector is written;
attention dequantises the INT8 keys and values before the products with the
query, and the dequantisation is fused into the attention kernel (a separate
pass would cost one more read and write of the cache). Sec. 4.1's operator
table lists the self-written blockwise attention with that fused
dequantisation; sec. 6's checklist repeats the requirement.

Written out (one key or value vector = the D = 128 values of one token and
one KV head):

    write:      (qk[t], sk[t]) = absmax rule of quant.py on k[t]   (same for v)
    dequantise: K[t,d] = sk[t] * qk[t,d],   V[t,d] = sv[t] * qv[t,d]
    attention:  z[t] = sum_d q[d] * K[t,d] / sqrt(D)      for t < L
                w[t] = exp(z[t]) / sum_u exp(z[u])
                o[d] = sum_t w[t] * V[t,d]

with grouped-query heads: query head h reads KV head h // G, G = Hq / Hkv.

Readings (the pages give no formula for the attention itself):
  * "per token" scale = one scale per (token, KV head) vector of D values,
    the plainest reading of "each key/value vector gets its own scale".
  * the softmax scale is 1/sqrt(D) (scaled dot-product attention).
  * L = 0 (no cached tokens): the empty sum, o = 0.
  * the kernel's floating-point steps are not fixed by the pages, so only a
    bound is: see ``attention_tolerance``.

``attention_int8kv_ref`` evaluates the definition in float64 on the
dequantised cache (every dequantised value is exact in float64) and returns
the magnitude mag[d] = sum_t w[t] * |V[t,d]| that the tolerance is stated
against.
"""
from __future__ import annotations

import numpy as np

from .quant import bf16_bits_to_f32, quantize_rows_ref

HEAD_DIM = 128


def kv_quantize_ref(x_bits: np.ndarray):
    """Quantise key or value vectors on write.

    x_bits: BF16 bits [..., D]. Returns (codes int8 [..., D], scales float32 [...]):
    each length-D vector by the absmax rule on its own.
    """
    x = bf16_bits_to_f32(x_bits)
    lead, D = x.shape[:-1], x.shape[-1]
    q, s = quantize_rows_ref(x.reshape(-1, D))
    return q.reshape(*lead, D), s.reshape(lead)


def dequant_kv_ref(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """K or V in float64: scale times code (exact)."""
    return np.asarray(scales, np.float32).astype(np.float64)[..., None] * codes.astype(np.float64)


def attention_int8kv_ref(q_bits, k_codes, k_scales, v_codes, v_scales, lens):
    """Decode attention of one query token per sequence over the INT8 cache.

    q_bits   BF16 bits [B, Hq, D]
    k_codes  int8 [B, Hkv, T, D],  k_scales float32 [B, Hkv, T]   (same for v)
    lens     int [B], 0 <= lens[b] <= T: tokens 0 .. lens[b]-1 are attended.
    Returns (o [B, Hq, D] float64, mag [B, Hq, D] float64).
    """
    q = bf16_bits_to_f32(q_bits).astype(np.float64)
    B, Hq, D = q.shape
    _, Hkv, T, Dk = k_codes.shape
    if Dk != D or v_codes.shape != k_codes.shape or Hq % Hkv:
        raise ValueError("q [B,Hq,D], k/v [B,Hkv,T,D] with Hq a multiple of Hkv required")
    G = Hq // Hkv
    o = np.zeros((B, Hq, D))
    mag = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(lens[b])
        if not 0 <= L <= T:
            raise ValueError("lens out of range")
        if L == 0:
            continue
        for kv in range(Hkv):       # only the attended slots are read
            K = dequant_kv_ref(k_codes[b, kv, :L], k_scales[b, kv, :L])
            V = dequant_kv_ref(v_codes[b, kv, :L], v_scales[b, kv, :L])
            for h in range(kv * G, (kv + 1) * G):
                z = K @ q[b, h] / np.sqrt(D)
                e = np.exp(z - z.max())
                w = e / e.sum()
                o[b, h] = w @ V
                mag[b, h] = w @ np.abs(V)
    return o, mag


def chunk_lengths_ref(lens, Qn: int) -> np.ndarray:
    """Tokens attended by each of the Qn newest tokens of every sequence: query i sits at
    position lens[b] - Qn + i and attends to tokens 0 .. that position. [B, Qn] int."""
    lens = np.asarray(lens, np.int64)
    L = lens[:, None] - Qn + np.arange(Qn)[None, :] + 1
    return np.clip(L, 0, lens[:, None])


def attention_int8kv_chunk_ref(q_bits, k_codes, k_scales, v_codes, v_scales, lens):
    """Attention of the Qn newest tokens of each sequence over the INT8 cache, causal.

    Reading (the pages name a blockwise attention that dequantises the INT8 cache, sec.
    4.1, and give no formula for several query tokens): the Qn query tokens of sequence
    b are its last Qn positions, lens[b] - Qn .. lens[b] - 1, whose keys and values are
    already in the cache (written before the attention, as a decode step writes its
    token first); query i attends to tokens 0 .. lens[b] - Qn + i (chunked prefill or
    verifying Qn drafted tokens). A query with no such token (lens[b] < Qn - i) gives 0.
    Each query is the decode attention above over its own prefix.

    q_bits BF16 bits [B, Qn, Hq, D]; cache and lens as attention_int8kv_ref.
    Returns (o [B, Qn, Hq, D], mag [B, Qn, Hq, D]) float64.
    """
    q_bits = np.asarray(q_bits)
    B, Qn, Hq, D = q_bits.shape
    Ls = chunk_lengths_ref(lens, Qn)
    o = np.zeros((B, Qn, Hq, D))
    mag = np.zeros((B, Qn, Hq, D))
    for i in range(Qn):
        o[:, i], mag[:, i] = attention_int8kv_ref(q_bits[:, i], k_codes, k_scales, v_codes,
                                                  v_scales, Ls[:, i])
    return o, mag


def attention_bf16kv_ref(q_bits, k_bits, v_bits, lens):
    """The same attention over a BF16 cache (the cache the INT8 one replaces): K and V
    are the cached BF16 values, exact in float64. Arguments as attention_int8kv_ref
    with k_bits, v_bits BF16 bits [B, Hkv, T, D]; returns (o, mag)."""
    q = bf16_bits_to_f32(q_bits).astype(np.float64)
    B, Hq, D = q.shape
    _, Hkv, T, Dk = k_bits.shape
    if Dk != D or v_bits.shape != k_bits.shape or Hq % Hkv:
        raise ValueError("q [B,Hq,D], k/v [B,Hkv,T,D] with Hq a multiple of Hkv required")
    G = Hq // Hkv
    o = np.zeros((B, Hq, D))
    mag = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(lens[b])
        if not 0 <= L <= T:
            raise ValueError("lens out of range")
        if L == 0:
            continue
        for kv in range(Hkv):
            K = bf16_bits_to_f32(k_bits[b, kv, :L]).astype(np.float64)
            V = bf16_bits_to_f32(v_bits[b, kv, :L]).astype(np.float64)
            for h in range(kv * G, (kv + 1) * G):
                z = K @ q[b, h] / np.sqrt(D)
                e = np.exp(z - z.max())
                w = e / e.sum()
                o[b, h] = w @ V
                mag[b, h] = w @ np.abs(V)
    return o, mag


def attention_tolerance(out_bf16: bool) -> float:
    """t with |o_kernel - o| <= t * mag elementwise (both caches).

    The matrix cores take the weights w[t] * sv[t] (w[t] for BF16 values) rounded to BF16 (relative
    error <= 2^-8 each, so <= 2^-8 * mag on the sum); the float32 scores,
    exponentials and normalisation add well under another 2^-8 * mag for
    score terms sum_d |q[d] K[t,d]| / sqrt(D) up to ~100; a BF16 output adds
    its own rounding, <= 2^-8 * |o| <= 2^-8 * mag.
    """
    return 2.0 ** -7 + (2.0 ** -8 if out_bf16 else 0.0)
