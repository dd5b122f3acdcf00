"""Seeded synthetic inputs for the block-scaled INT8 linear layer.

This module only draws random numbers and lays them out in the shapes the
method consumes. It holds none of the method's arithmetic: no quantisation,
no GEMM, no format decoding, no rescaling. Both sides of every parity check
(the CPU oracle and the HIP library) and the benchmark take their inputs from
here; the BF16 rounding of the drawn activations is done by torch's own
float32 -> bfloat16 cast.

Workloads (shapes and value distributions of the deployments the pages
describe; no checkpoint or dataset is available, so these seeded tensors
stand in for them):

* ``tiny``    M=16,   K=1024, N=1024   activations N(0,1), 1 % outliers x20
* ``decode``  M=32,   K=8192, N=28672  activations N(0,1), 0.5 % outliers x30
* ``prefill`` M=4096, K=8192, N=8192   same distributions as ``decode``
* ``moe``     4096 tokens routed top-8 over 64 experts (Zipf s=1.1 router with
              four zero-weight experts, so some experts are empty), K=4096,
              N=2048 per expert
* ``blockfmt`` dense FP8-e4m3 [4096, 7168] with [128,128] UE8M0 block scales,
              plus 8 MXFP4 experts [2048, 4096] with 1x32 UE8M0 scales.
* ``kv``      decode attention over a KV cache: 32 sequences of 4096 cached
              tokens, 64 query heads over 8 KV heads of dimension 128; queries,
              keys and values N(0,1) with 0.5 % outliers x30.

Weights are INT8 uniform over [-127, 127]; weight group scales are
lognormal(mu=-6, sigma=0.5) in float32, one per (output row, 128-wide K group).
"""
from __future__ import annotations

import numpy as np
import torch

GROUP = 128

LINEAR_CONFIGS = {
    "tiny": dict(M=16, K=1024, N=1024, outlier_p=0.01, outlier_f=20.0),
    "decode": dict(M=32, K=8192, N=28672, outlier_p=0.005, outlier_f=30.0),
    "prefill": dict(M=4096, K=8192, N=8192, outlier_p=0.005, outlier_f=30.0),
}

# FP8 byte codes that are finite in both the OCP (E4M3FN) and the fnuz (E4M3FNUZ)
# reading: every byte except 0x7F / 0xFF (NaN in OCP) and 0x80 (NaN in fnuz).
FP8_CODES_FINITE_BOTH = np.array(
    [b for b in range(256) if b not in (0x7F, 0xFF, 0x80)], dtype=np.uint8)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 BF16 bit patterns, via torch's (round-to-nearest-even) cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def activations(rng: np.random.Generator, rows: int, K: int, outlier_p: float,
                outlier_f: float) -> np.ndarray:
    """BF16 bits [rows, K]: N(0,1) with a Bernoulli(outlier_p) mask multiplied by outlier_f."""
    x = rng.standard_normal((rows, K), dtype=np.float32)
    if outlier_p > 0:
        mask = rng.random((rows, K)) < outlier_p
        x[mask] *= np.float32(outlier_f)
    return to_bf16_bits(x)


def int8_weights(rng: np.random.Generator, shape) -> np.ndarray:
    """INT8 uniform over the 255 values [-127, 127] (never -128)."""
    return rng.integers(-127, 128, size=shape, dtype=np.int8)


def group_scales(rng: np.random.Generator, shape) -> np.ndarray:
    """float32 lognormal(mu=-6, sigma=0.5) weight group scales."""
    return np.exp(rng.normal(-6.0, 0.5, size=shape)).astype(np.float32)


def channel_scales(n: int, seed: int = 0) -> np.ndarray:
    """float32 lognormal(mu=-6, sigma=0.5) weight scales, one per output row (n = N)
    or one for the whole weight (n = 1): the group-scale distribution, drawn from a
    stream of its own so that the other inputs of a seed do not change."""
    rng = np.random.Generator(np.random.PCG64([seed, 0xC4A]))
    return group_scales(rng, (n,))


def linear_inputs(M: int, K: int, N: int, outlier_p: float = 0.005,
                  outlier_f: float = 30.0, seed: int = 0) -> dict:
    """One dense linear layer: x BF16 bits [M,K], qw int8 [N,K], sw float32 [N,K/128]."""
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    rng = np.random.Generator(np.random.PCG64(seed))
    x = activations(rng, M, K, outlier_p, outlier_f)
    qw = int8_weights(rng, (N, K))
    sw = group_scales(rng, (N, K // GROUP))
    return dict(x=x, qw=qw, sw=sw, M=M, K=K, N=N)


def linear_config(name: str, seed: int = 0) -> dict:
    return linear_inputs(seed=seed, **LINEAR_CONFIGS[name])


def zipf_router(rng: np.random.Generator, T: int, E: int, topk: int, s: float,
                n_empty: int) -> np.ndarray:
    """topk_ids [T, topk]: each token draws `topk` distinct experts with
    probability proportional to rank^-s over a random rank permutation; the
    `n_empty` lowest-ranked experts get probability 0 (so they stay empty)."""
    perm = rng.permutation(E)
    ranks = np.arange(1, E + 1, dtype=np.float64)
    w_rank = ranks ** (-s)
    w_rank[E - n_empty:] = 0.0
    w = np.empty(E, np.float64)
    w[perm] = w_rank
    p = w / w.sum()
    ids = np.empty((T, topk), np.int64)
    for t in range(T):
        ids[t] = rng.choice(E, topk, replace=False, p=p)
    return ids


def sort_by_expert(topk_ids: np.ndarray, E: int):
    """Stable sort of the (token, slot) pairs by expert id.

    Returns (token_of_row [R], offsets int32 [E+1]); rows of expert e are
    [offsets[e], offsets[e+1]).
    """
    flat = topk_ids.reshape(-1)
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    token_of_row = order // topk_ids.shape[1]
    return token_of_row, offsets


def row_of_pair(topk_ids: np.ndarray) -> np.ndarray:
    """int32 [T, topk]: the sorted row that holds token t's k-th expert slot
    (the inverse of the stable sort of sort_by_expert)."""
    flat = topk_ids.reshape(-1)
    order = np.argsort(flat, kind="stable")
    inv = np.empty(flat.size, np.int64)
    inv[order] = np.arange(flat.size)
    return inv.reshape(topk_ids.shape).astype(np.int32)


def gate_weights(rng: np.random.Generator, T: int, topk: int) -> np.ndarray:
    """float32 [T, topk] router weights of the selected experts: positive,
    each token's weights normalised to sum to 1."""
    g = rng.random((T, topk)) + 0.05
    return (g / g.sum(axis=1, keepdims=True)).astype(np.float32)


def moe_inputs(T: int = 4096, K: int = 4096, N: int = 2048, E: int = 64,
               topk: int = 8, zipf_s: float = 1.1, n_empty: int = 4,
               outlier_p: float = 0.0, outlier_f: float = 1.0, seed: int = 0) -> dict:
    """Routed MoE expert layer.

    x_tokens BF16 bits [T,K] are the tokens; x_sorted [R,K] holds their rows
    gathered in expert order (token_of_row int32 [R]), offsets int32 [E+1]
    the per-expert row ranges, qw int8 [E,N,K], sw float32 [E,N,K/128];
    row_of_pair int32 [T,topk] is the inverse map and gate float32 [T,topk]
    the router weights of the combine.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    X = activations(rng, T, K, outlier_p, outlier_f)
    topk_ids = zipf_router(rng, T, E, topk, zipf_s, n_empty)
    token_of_row, offsets = sort_by_expert(topk_ids, E)
    qw = int8_weights(rng, (E, N, K))
    sw = group_scales(rng, (E, N, K // GROUP))
    gate = gate_weights(rng, T, topk)          # drawn last: earlier tensors unchanged
    return dict(x_tokens=X, topk_ids=topk_ids, token_of_row=token_of_row.astype(np.int32),
                row_of_pair=row_of_pair(topk_ids), gate=gate,
                x_sorted=X[token_of_row], offsets=offsets, qw=qw, sw=sw,
                T=T, K=K, N=N, E=E, R=int(offsets[-1]), topk=topk)


def fp8_block_weights(rng: np.random.Generator, N: int, K: int, exp_lo: int = -8,
                      exp_hi: int = 4):
    """FP8 e4m3 bytes [N,K] uniform over the codes finite in both dialects, and
    UE8M0 block-scale bytes [N/128, K/128] = 127 + U{exp_lo..exp_hi}."""
    w = rng.choice(FP8_CODES_FINITE_BOTH, size=(N, K))
    bs = (127 + rng.integers(exp_lo, exp_hi + 1, size=(N // GROUP, K // GROUP))).astype(np.uint8)
    return w, bs


def mxfp4_weights(rng: np.random.Generator, E: int, N: int, K: int, exp_lo: int = -8,
                  exp_hi: int = 4):
    """Packed E2M1 nibbles [E,N,K/2] (uniform over all 16 codes, element 2j in the
    low nibble of byte j) and UE8M0 scale bytes [E,N,K/32] = 127 + U{exp_lo..exp_hi}."""
    packed = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    sc = (127 + rng.integers(exp_lo, exp_hi + 1, size=(E, N, K // 32))).astype(np.uint8)
    return packed, sc


def blockfmt_inputs(M: int = 32, N_d: int = 4096, K_d: int = 7168, E: int = 8,
                    N_e: int = 2048, K_e: int = 4096, seed: int = 0) -> dict:
    """Block-format weights plus the activations that run against them.

    Dense: FP8 bytes w [N_d,K_d] + block scales bs [N_d/128,K_d/128]; the same
    bytes are read once as OCP and once as fnuz. Experts: MXFP4 packed
    [E,N_e,K_e/2] + scales [E,N_e,K_e/32]. Activations: x_d [M,K_d] and
    x_e [E*M,K_e] (each expert gets its own M rows, offsets e*M).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    w, bs = fp8_block_weights(rng, N_d, K_d)
    packed, sc = mxfp4_weights(rng, E, N_e, K_e)
    x_d = activations(rng, M, K_d, 0.005, 30.0)
    x_e = activations(rng, E * M, K_e, 0.005, 30.0)
    offsets = (np.arange(E + 1) * M).astype(np.int32)
    return dict(w_fp8=w, bs=bs, packed=packed, scale=sc, x_d=x_d, x_e=x_e,
                offsets=offsets, M=M, N_d=N_d, K_d=K_d, E=E, N_e=N_e, K_e=K_e)


KV_CONFIG = dict(B=32, Hq=64, Hkv=8, T=4096, D=128)


def kv_inputs(B: int, Hq: int, Hkv: int, T: int, lens=None, q_gain: float = 1.0,
              outlier_p: float = 0.005, outlier_f: float = 30.0, seed: int = 0) -> dict:
    """One decode step of attention over a cache of T token slots per sequence.

    q BF16 bits [B,Hq,128] (N(0,1) times q_gain, which sharpens the softmax),
    k and v BF16 bits [B,Hkv,T,128] (N(0,1) with outliers), lens int32 [B]
    (given, or uniform over 1..T when None): the cached tokens of each sequence.
    """
    D = 128
    rng = np.random.Generator(np.random.PCG64([seed, 0x4B56]))
    q = rng.standard_normal((B, Hq, D), dtype=np.float32) * np.float32(q_gain)
    k = activations(rng, B * Hkv * T, D, outlier_p, outlier_f).reshape(B, Hkv, T, D)
    v = activations(rng, B * Hkv * T, D, outlier_p, outlier_f).reshape(B, Hkv, T, D)
    if lens is None:
        lens = rng.integers(1, T + 1, size=B)
    return dict(q=to_bf16_bits(q), k=k, v=v, lens=np.asarray(lens, np.int32),
                B=B, Hq=Hq, Hkv=Hkv, T=T, D=D)
