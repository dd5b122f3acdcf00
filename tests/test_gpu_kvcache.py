"""GPU parity: the INT8 KV cache (quantisation on write) and decode attention over it.

The write is integer work: codes and scales are compared bit for bit with the
oracle's per-vector rule, and slots the call does not name must keep their
contents. The attention is compared with the oracle's float64 definition on the
same cache within the bound derived for the kernel's float32 / BF16 arithmetic,
|o - o64| <= t * sum_t w[t] |V[t,d]|. The cache layout is the one documented in
include/bsb.h; these tests encode and decode it on the host.
"""
import numpy as np
import pytest
import torch

import block_scaled_bit_amd as bsb
from block_scaled_bit_amd import synth
from oracle import (kv_quantize_ref, attention_int8kv_ref, attention_tolerance,
                    bf16_bits_to_f32_ref, attention_int8kv_chunk_ref, f32_to_bf16_bits_ref)
from tests.gpu_util import require_gpu, dev, dev_bf16, host, say

pytestmark = pytest.mark.gpu

D, KB, VB = 128, 16, 32
_d = np.arange(D)[None, :]
_kt = np.arange(KB)[:, None]
K_OFF = ((_d // 16) % 2) * 1024 + ((_d // 32) * 16 + _kt) * 16 + _d % 16
_tau = np.arange(VB)[:, None]
V_OFF = ((_d // 32) * 1024 + (((_tau % 16) // 4) * 16 + _d % 16) * 16 + ((_d // 16) % 2) * 8 +
         (_tau // 16) * 4 + _tau % 4)


CH = 64          # tokens per cache row


def _rows(blocks):
    """[B, H, T/blk, blk elements] -> the cache rows [T/64, B, H, 64*128]: row (c, b, h)
    holds the blocks of tokens 64c .. 64c+63 of (b, h) in token order."""
    B, H, N, W = blocks.shape
    per = CH * D // W
    return np.ascontiguousarray(blocks.reshape(B, H, N // per, per * W).transpose(2, 0, 1, 3))


def _blocks(rows, W):
    """Inverse of _rows for blocks of W elements."""
    C, B, H, R = rows.shape
    return rows.transpose(1, 2, 0, 3).reshape(B, H, C * R // W, W)


def k_encode(kc):
    """[B, H, T, 128] int8 -> k_cache [T/64, B, H, 8192] (16-token blocks of 2 KB)."""
    B, H, T, _ = kc.shape
    out = np.empty((B, H, T // KB, KB * D), np.int8)
    out[..., K_OFF] = kc.reshape(B, H, T // KB, KB, D)
    return _rows(out)


def k_decode(kb):
    kb = _blocks(np.asarray(kb), KB * D)
    B, H, NB, _ = kb.shape
    return kb[..., K_OFF].reshape(B, H, NB * KB, D)


def v_encode(vc):
    """[B, H, T, 128] int8 -> v_cache [T/64, B, H, 8192] (32-token blocks of 4 KB)."""
    B, H, T, _ = vc.shape
    out = np.empty((B, H, T // VB, VB * D), np.int8)
    out[..., V_OFF] = vc.reshape(B, H, T // VB, VB, D)
    return _rows(out)


def v_decode(vb):
    vb = _blocks(np.asarray(vb), VB * D)
    B, H, NB, _ = vb.shape
    return vb[..., V_OFF].reshape(B, H, NB * VB, D)


def test_kv_layouts_are_permutations():
    assert np.array_equal(np.sort(K_OFF.ravel()), np.arange(KB * D))
    assert np.array_equal(np.sort(V_OFF.ravel()), np.arange(VB * D))
    x = np.random.default_rng(0).integers(-127, 128, size=(2, 3, 64, D)).astype(np.int8)
    assert np.array_equal(k_decode(k_encode(x)), x)
    assert np.array_equal(v_decode(v_encode(x)), x)
    # rows are chunk-major: token 64 of (b, h) starts row (1, b, h)
    y = np.zeros((2, 3, 128, D), np.int8)
    y[1, 2, 64, 0] = 7
    assert k_encode(y)[1, 1, 2, 0] == 7 and v_encode(y)[1, 1, 2, 0] == 7


def _poisoned_cache(B, H, T, d):
    kc, ks, vc, vs = bsb.kv_cache_empty(B, H, T, d)
    kc.fill_(0x55)
    vc.fill_(0x55)
    ks.fill_(-1.0)
    vs.fill_(-2.0)
    return kc, ks, vc, vs


@pytest.mark.parametrize("B,H,T,frac", [(3, 2, 128, 1.0), (2, 8, 192, 0.4), (1, 1, 64, 0.1)])
def test_write_is_bit_exact_and_touches_only_named_slots(B, H, T, frac):
    d = require_gpu()
    rng = np.random.default_rng(B * 100 + H)
    inp = synth.kv_inputs(B, H, H, T, seed=B + H)
    k, v = inp["k"], inp["v"]
    # special vectors: all zero, tiny (subnormal scale), one huge outlier
    k[0, 0, 1] = 0
    v[0, 0, 2] = synth.to_bf16_bits(np.full(D, 1e-37, np.float32))
    k[-1, -1, 3, 5] = synth.to_bf16_bits(np.array([3e4], np.float32))[0]
    slots = [(b, t) for b in range(B) for t in range(T) if rng.random() < frac]
    seq = np.array([s[0] for s in slots] + [B, -1, 0], np.int32)      # last three: out of range
    pos = np.array([s[1] for s in slots] + [0, 0, T], np.int32)
    kn = np.stack([k[b, :, t] for b, t in slots] + [k[0, :, 0]] * 3)   # [n, H, D]
    vn = np.stack([v[b, :, t] for b, t in slots] + [v[0, :, 0]] * 3)
    kc, ks, vc, vs = _poisoned_cache(B, H, T, d)
    say(f"kv write B={B} H={H} T={T} n={len(seq)}")
    bsb.kv_cache_write(dev_bf16(kn, d), dev_bf16(vn, d), dev(seq, d), dev(pos, d), kc, ks, vc, vs)
    torch.cuda.synchronize()
    qk, sk = kv_quantize_ref(k)
    qv, sv = kv_quantize_ref(v)
    gk, gks, gv, gvs = k_decode(host(kc)), host(ks), v_decode(host(vc)), host(vs)
    written = np.zeros((B, T), bool)
    for b, t in slots:
        written[b, t] = True
    for b in range(B):
        for t in range(T):
            if written[b, t]:
                assert np.array_equal(gk[b, :, t], qk[b, :, t]), (b, t)
                assert np.array_equal(gv[b, :, t], qv[b, :, t]), (b, t)
                assert np.array_equal(gks[b, :, t].view(np.uint32), sk[b, :, t].view(np.uint32))
                assert np.array_equal(gvs[b, :, t].view(np.uint32), sv[b, :, t].view(np.uint32))
            else:
                assert (gk[b, :, t] == 0x55).all() and (gv[b, :, t] == 0x55).all(), (b, t)
                assert (gks[b, :, t] == -1.0).all() and (gvs[b, :, t] == -2.0).all()


def test_decode_step_appends_one_token_per_sequence():
    d = require_gpu()
    B, H, T = 4, 2, 128
    lens = np.array([5, 0, 127, 64], np.int32)
    inp = synth.kv_inputs(B, H, H, T, seed=7)
    kc, ks, vc, vs = _poisoned_cache(B, H, T, d)
    seq = np.arange(B, dtype=np.int32)
    kn = inp["k"][np.arange(B), :, lens]
    vn = inp["v"][np.arange(B), :, lens]
    bsb.kv_cache_write(dev_bf16(kn, d), dev_bf16(vn, d), dev(seq, d), dev(lens, d), kc, ks, vc, vs)
    torch.cuda.synchronize()
    qk, sk = kv_quantize_ref(kn)
    qv, sv = kv_quantize_ref(vn)
    gk, gv, gks = k_decode(host(kc)), v_decode(host(vc)), host(ks)
    for b in range(B):
        assert np.array_equal(gk[b, :, lens[b]], qk[b])
        assert np.array_equal(gv[b, :, lens[b]], qv[b])
        assert np.array_equal(gks[b, :, lens[b]], sk[b])


def _upload_cache(kc, ks, vc, vs, d):
    return dev(k_encode(kc), d), dev(ks, d), dev(v_encode(vc), d), dev(vs, d)


def _attn_case(B, Hq, Hkv, T, lens, max_len, seed, q_gain=1.0):
    lens = np.asarray(lens, np.int32)
    inp = synth.kv_inputs(B, Hq, Hkv, T, lens=lens, q_gain=q_gain, seed=seed)
    kc, ks = kv_quantize_ref(inp["k"])
    vc, vs = kv_quantize_ref(inp["v"])
    rng = np.random.default_rng(seed + 1)
    for b in range(B):           # slots past each sequence hold garbage, NaN / inf scales
        L = lens[b]
        kc[b, :, L:] = rng.integers(-128, 128, size=kc[b, :, L:].shape)
        vc[b, :, L:] = rng.integers(-128, 128, size=vc[b, :, L:].shape)
        ks[b, :, L:] = np.nan
        vs[b, :, L:] = np.inf
    eff = np.minimum(lens, max_len)
    o64, mag = attention_int8kv_ref(inp["q"], kc, ks, vc, vs, eff)
    return inp["q"], kc, ks, vc, vs, lens, o64, mag


def _run_attn(qb, kc, ks, vc, vs, lens, max_len, dtype, d):
    out = bsb.attention_decode_int8kv(dev_bf16(qb, d), *_upload_cache(kc, ks, vc, vs, d),
                                      dev(lens, d), max_len, out_dtype=dtype)
    torch.cuda.synchronize()
    y = host(out)
    if dtype == torch.bfloat16:
        return bf16_bits_to_f32_ref(y).astype(np.float64)
    return y.astype(np.float64)


def _check(y, o64, mag, bf16):
    t = attention_tolerance(bf16)
    err = np.abs(y - o64)
    bad = err > t * mag
    assert not bad.any(), f"{bad.sum()} outputs beyond the bound (max err/mag {(err / np.maximum(mag, 1e-300)).max():.3g})"
    assert np.all(y[mag == 0] == 0)


CASES = [
    # B, Hq, Hkv, T, lens, max_len
    (2, 8, 1, 128, [128, 77], 128),
    (3, 16, 2, 576, [576, 1, 300], 576),          # two splits, one-token sequence
    (2, 32, 2, 1088, [1088, 513], 1088),         # G = 16, three splits
    (2, 4, 4, 256, [200, 64], 256),              # G = 1
    (2, 6, 2, 192, [191, 65], 192),              # G = 3
    (3, 8, 2, 1024, [700, 0, 599], 600),         # max_len below T and below lens[0]; an empty sequence
    (2, 8, 8, 640, [640, 640], 640),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_attention_matches_oracle(case, dtype):
    d = require_gpu()
    B, Hq, Hkv, T, lens, max_len = case
    say(f"attention B={B} Hq={Hq} Hkv={Hkv} T={T} lens={lens} max_len={max_len} {dtype}")
    qb, kc, ks, vc, vs, lens, o64, mag = _attn_case(B, Hq, Hkv, T, lens, max_len, seed=B + Hq + T)
    y = _run_attn(qb, kc, ks, vc, vs, lens, max_len, dtype, d)
    _check(y, o64, mag, dtype == torch.bfloat16)


@pytest.mark.parametrize("q_gain", [0.05, 6.0])
def test_attention_flat_and_peaked_softmax(q_gain):
    d = require_gpu()
    say(f"attention q_gain={q_gain}")
    qb, kc, ks, vc, vs, lens, o64, mag = _attn_case(2, 16, 2, 1024, [1024, 700], 1024, seed=31,
                                                    q_gain=q_gain)
    y = _run_attn(qb, kc, ks, vc, vs, lens, 1024, torch.float32, d)
    _check(y, o64, mag, False)


def test_attention_no_tokens_gives_zeros_and_is_deterministic():
    d = require_gpu()
    qb, kc, ks, vc, vs, lens, o64, mag = _attn_case(2, 8, 1, 128, [0, 0], 128, seed=5)
    y = _run_attn(qb, kc, ks, vc, vs, lens, 128, torch.float32, d)
    assert not y.any()
    # a negative length is clamped to no tokens; the other sequence is unaffected
    qb, kc, ks, vc, vs, _, _, _ = _attn_case(2, 8, 1, 128, [128, 128], 128, seed=8)
    neg = np.array([-5, 128], np.int32)
    y = _run_attn(qb, kc, ks, vc, vs, neg, 128, torch.float32, d)
    assert not y[0].any()
    o64, mag = attention_int8kv_ref(qb[1:], kc[1:], ks[1:], vc[1:], vs[1:], neg[1:])
    _check(y[1:], o64, mag, False)
    y0 = _run_attn(qb, kc, ks, vc, vs, lens, 0, torch.bfloat16, d)     # max_len 0: no split runs
    assert not y0.any()
    qb, kc, ks, vc, vs, lens, o64, mag = _attn_case(2, 8, 1, 256, [256, 100], 256, seed=6)
    a = _run_attn(qb, kc, ks, vc, vs, lens, 256, torch.float32, d)
    b = _run_attn(qb, kc, ks, vc, vs, lens, 256, torch.float32, d)
    assert np.array_equal(a, b)


def test_full_size_decode_attention_sampled():
    """The benchmark's workload: 32 sequences x 4096 cached tokens, 64 query heads over
    8 KV heads, written through the GPU write kernel and attended in the launch the
    benchmark times; three sequences are checked against the oracle (cache bytes bit
    for bit, outputs within the bound)."""
    d = require_gpu()
    c = synth.KV_CONFIG
    B, Hq, Hkv, T = c["B"], c["Hq"], c["Hkv"], c["T"]
    inp = synth.kv_inputs(B, Hq, Hkv, T, lens=np.full(B, T), seed=0)
    say("full-size kv write + attention")
    kc, ks, vc, vs = bsb.kv_cache_empty(B, Hkv, T, d)
    kt = dev_bf16(inp["k"], d).permute(0, 2, 1, 3).reshape(B * T, Hkv, D).contiguous()
    vt = dev_bf16(inp["v"], d).permute(0, 2, 1, 3).reshape(B * T, Hkv, D).contiguous()
    seq = torch.arange(B, dtype=torch.int32, device=d).repeat_interleave(T)
    pos = torch.arange(T, dtype=torch.int32, device=d).repeat(B)
    bsb.kv_cache_write(kt, vt, seq, pos, kc, ks, vc, vs)
    lens = dev(inp["lens"], d)
    out = bsb.attention_decode_int8kv(dev_bf16(inp["q"], d), kc, ks, vc, vs, lens, T)
    torch.cuda.synchronize()
    y = bf16_bits_to_f32_ref(host(out)).astype(np.float64)
    for b in (0, 17, 31):
        qk, sk = kv_quantize_ref(inp["k"][b:b + 1])
        qv, sv = kv_quantize_ref(inp["v"][b:b + 1])
        assert np.array_equal(k_decode(host(kc[:, b:b + 1])), qk)
        assert np.array_equal(v_decode(host(vc[:, b:b + 1])), qv)
        assert np.array_equal(host(ks[b:b + 1]), sk) and np.array_equal(host(vs[b:b + 1]), sv)
        o64, mag = attention_int8kv_ref(inp["q"][b:b + 1], qk, sk, qv, sv, inp["lens"][b:b + 1])
        _check(y[b:b + 1], o64, mag, True)


@pytest.mark.parametrize("B,Hq,Hkv,T,max_len", [
    (64, 8, 8, 512, 512),       # 512 (sequence, KV head) pairs: two chunks per wave, one split
    (32, 64, 8, 2048, 2000),    # 1024 split units: four chunks per wave, one split
    (32, 8, 8, 1280, 1280),     # two chunks per wave over two splits (merged by the second kernel)
])
def test_attention_multi_chunk_waves(B, Hq, Hkv, T, max_len):
    """Grids large enough that each wave walks several 64-token chunks (running
    maximum and sums across chunks), ragged lengths including 0, 1, 63, 64, 65 and
    lengths above max_len; a sample of sequences checked against the oracle."""
    d = require_gpu()
    rng = np.random.default_rng(B + T)
    lens = rng.integers(1, T + 1, size=B).astype(np.int32)
    lens[:6] = [0, 1, 63, 64, 65, T]
    say(f"attention multi-chunk B={B} Hq={Hq} Hkv={Hkv} T={T} max_len={max_len}")
    inp = synth.kv_inputs(B, Hq, Hkv, T, lens=lens, seed=B + Hkv)
    kc, ks = kv_quantize_ref(inp["k"])
    vc, vs = kv_quantize_ref(inp["v"])
    for b in range(B):
        ks[b, :, lens[b]:] = np.nan
        vs[b, :, lens[b]:] = np.inf
    for dtype in (torch.float32, torch.bfloat16):
        y = _run_attn(inp["q"], kc, ks, vc, vs, lens, max_len, dtype, d)
        for b in list(range(6)) + list(rng.choice(np.arange(6, B), 6, replace=False)):
            eff = np.minimum(lens[b:b + 1], max_len)
            o64, mag = attention_int8kv_ref(inp["q"][b:b + 1], kc[b:b + 1], ks[b:b + 1],
                                            vc[b:b + 1], vs[b:b + 1], eff)
            _check(y[b:b + 1], o64, mag, dtype == torch.bfloat16)


# ---- the BF16 cache of the comparison route ----------------------------------

K16_OFF = ((_d // 8) % 4) * 512 + ((_d // 32) * 16 + _kt) * 8 + _d % 8
V16_OFF = (_d // 16) * 512 + (((_tau % 16) // 4) * 16 + _d % 16) * 8 + (_tau // 16) * 4 + _tau % 4


def k16_encode(k):
    B, H, T, _ = k.shape
    out = np.empty((B, H, T // KB, KB * D), np.uint16)
    out[..., K16_OFF] = k.reshape(B, H, T // KB, KB, D)
    return _rows(out)


def v16_encode(v):
    B, H, T, _ = v.shape
    out = np.empty((B, H, T // VB, VB * D), np.uint16)
    out[..., V16_OFF] = v.reshape(B, H, T // VB, VB, D)
    return _rows(out)


def test_bf16_layouts_are_permutations():
    assert np.array_equal(np.sort(K16_OFF.ravel()), np.arange(KB * D))
    assert np.array_equal(np.sort(V16_OFF.ravel()), np.arange(VB * D))
    x = np.random.default_rng(1).integers(0, 1 << 16, size=(2, 3, 128, D)).astype(np.uint16)
    assert np.array_equal(_blocks(k16_encode(x), KB * D)[..., K16_OFF].reshape(x.shape), x)
    assert np.array_equal(_blocks(v16_encode(x), VB * D)[..., V16_OFF].reshape(x.shape), x)


def test_bf16_write_copies_into_the_layout():
    d = require_gpu()
    B, H, T = 2, 4, 128
    inp = synth.kv_inputs(B, H, H, T, seed=50)
    kc, vc = bsb.kv_cache_empty_bf16(B, H, T, d)
    kc.view(torch.int16).fill_(0x5555)
    vc.view(torch.int16).fill_(0x5555)
    slots = [(b, t) for b in range(B) for t in range(T) if (b + t) % 3]
    seq = np.array([s[0] for s in slots] + [B], np.int32)
    pos = np.array([s[1] for s in slots] + [0], np.int32)
    kn = np.stack([inp["k"][b, :, t] for b, t in slots] + [inp["k"][0, :, 0]])
    vn = np.stack([inp["v"][b, :, t] for b, t in slots] + [inp["v"][0, :, 0]])
    bsb.kv_cache_write_bf16(dev_bf16(kn, d), dev_bf16(vn, d), dev(seq, d), dev(pos, d), kc, vc)
    torch.cuda.synchronize()
    gk = _blocks(host(kc), KB * D)[..., K16_OFF].reshape(B, H, T, D)
    gv = _blocks(host(vc), VB * D)[..., V16_OFF].reshape(B, H, T, D)
    for b in range(B):
        for t in range(T):
            if (b + t) % 3:
                assert np.array_equal(gk[b, :, t], inp["k"][b, :, t])
                assert np.array_equal(gv[b, :, t], inp["v"][b, :, t])
            else:
                assert (gk[b, :, t] == 0x5555).all() and (gv[b, :, t] == 0x5555).all()


@pytest.mark.parametrize("B,Hq,Hkv,T,lens,max_len", [
    (2, 8, 1, 128, [128, 77], 128),
    (3, 32, 2, 1088, [1088, 1, 600], 1088),     # G = 16, three splits
    (32, 8, 8, 1280, None, 1280),               # two chunks per wave over two splits
])
def test_bf16_attention_matches_oracle(B, Hq, Hkv, T, lens, max_len):
    from oracle import attention_bf16kv_ref
    d = require_gpu()
    say(f"bf16 attention B={B} Hq={Hq} Hkv={Hkv} T={T}")
    inp = synth.kv_inputs(B, Hq, Hkv, T, lens=lens, seed=B + T)
    lens = inp["lens"]
    for dtype in (torch.float32, torch.bfloat16):
        out = bsb.attention_decode_bf16kv(dev_bf16(inp["q"], d), dev_bf16(k16_encode(inp["k"]), d),
                                          dev_bf16(v16_encode(inp["v"]), d), dev(lens, d),
                                          max_len, out_dtype=dtype)
        torch.cuda.synchronize()
        y = host(out)
        y = (bf16_bits_to_f32_ref(y) if dtype == torch.bfloat16 else y).astype(np.float64)
        for b in range(min(B, 6)):
            o64, mag = attention_bf16kv_ref(inp["q"][b:b + 1], inp["k"][b:b + 1], inp["v"][b:b + 1],
                                            np.minimum(lens[b:b + 1], max_len))
            _check(y[b:b + 1], o64, mag, dtype == torch.bfloat16)


@pytest.mark.parametrize("route", ["int8", "bf16"])
def test_attention_more_than_eight_splits(route):
    """One sequence of 5120 tokens: ten 512-token splits, which the merge kernel reads
    in two batches of eight (running maximum across batches)."""
    from oracle import attention_bf16kv_ref
    d = require_gpu()
    B, Hq, Hkv, T = 2, 8, 1, 5120
    lens = np.array([5120, 4700], np.int32)
    say(f"attention {route}, ten splits")
    inp = synth.kv_inputs(B, Hq, Hkv, T, lens=lens, q_gain=3.0, seed=77)
    if route == "int8":
        kc, ks = kv_quantize_ref(inp["k"])
        vc, vs = kv_quantize_ref(inp["v"])
        y = _run_attn(inp["q"], kc, ks, vc, vs, lens, T, torch.float32, d)
        o64, mag = attention_int8kv_ref(inp["q"], kc, ks, vc, vs, lens)
    else:
        out = bsb.attention_decode_bf16kv(dev_bf16(inp["q"], d), dev_bf16(k16_encode(inp["k"]), d),
                                          dev_bf16(v16_encode(inp["v"]), d), dev(lens, d), T,
                                          out_dtype=torch.float32)
        torch.cuda.synchronize()
        y = host(out).astype(np.float64)
        o64, mag = attention_bf16kv_ref(inp["q"], inp["k"], inp["v"], lens)
    _check(y, o64, mag, False)


# several query tokens per sequence: B, Qn, Hq, Hkv, T, lens, max_len
CHUNK_CASES = [
    (2, 2, 16, 2, 128, [128, 77], 128),          # 2 tokens x 8 heads: all 16 columns
    (3, 4, 8, 2, 576, [576, 2, 300], 576),       # two splits; a sequence shorter than the chunk
    (2, 16, 2, 2, 1088, [1088, 513], 1088),      # 16 tokens x 1 head; three splits
    (3, 3, 12, 3, 640, [640, 0, 601], 600),      # G = 4, 12 columns; max_len below T; empty
    (1, 5, 3, 1, 192, [191], 192),               # G = 3, 15 columns
    (32, 2, 64, 8, 512, [512] * 32, 512),        # many (sequence, KV head) pairs: several chunks per wave
]


@pytest.mark.parametrize("case", CHUNK_CASES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_chunk_attention_matches_oracle(case, dtype):
    """Causal attention of the newest Qn tokens over the INT8 cache: every query against
    the oracle's per-query prefix within the attention bound; queries with no token give 0."""
    d = require_gpu()
    B, Qn, Hq, Hkv, T, lens, max_len = case
    say(f"chunk attention B={B} Qn={Qn} Hq={Hq} Hkv={Hkv} T={T} lens={lens} max_len={max_len} {dtype}")
    _, kc, ks, vc, vs, lens, _, _ = _attn_case(B, Hq, Hkv, T, lens, max_len, seed=B + Qn + Hq + T)
    rng = np.random.default_rng(B * Qn + T)
    qb = f32_to_bf16_bits_ref(rng.standard_normal((B, Qn, Hq, D)).astype(np.float32) * 2)
    eff = np.minimum(lens, max_len)
    o64, mag = attention_int8kv_chunk_ref(qb, kc, ks, vc, vs, eff)
    out = bsb.attention_chunk_int8kv(dev_bf16(qb, d), *_upload_cache(kc, ks, vc, vs, d),
                                     dev(lens, d), max_len, out_dtype=dtype)
    torch.cuda.synchronize()
    y = host(out)
    y = (bf16_bits_to_f32_ref(y) if dtype == torch.bfloat16 else y).astype(np.float64)
    _check(y, o64, mag, dtype == torch.bfloat16)


def test_chunk_attention_of_one_token_is_the_decode_attention():
    """Qn = 1 runs the decode kernel's arithmetic: bit-identical outputs."""
    d = require_gpu()
    qb, kc, ks, vc, vs, lens, _, _ = _attn_case(3, 16, 2, 1088, [1088, 1, 500], 1088, seed=77)
    cache = _upload_cache(kc, ks, vc, vs, d)
    q = dev_bf16(qb, d)
    a = bsb.attention_decode_int8kv(q, *cache, dev(lens, d), 1088, out_dtype=torch.float32)
    c = bsb.attention_chunk_int8kv(q[:, None], *cache, dev(lens, d), 1088, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, c[:, 0])


def test_full_size_chunk_attention_sampled():
    """Two query tokens per sequence over the benchmark's cache (32 sequences x 4096
    tokens, 64 / 8 heads, written by the GPU write kernel), in the launch the benchmark
    times (2 x 8 = 16 query columns); three sequences against the oracle."""
    d = require_gpu()
    c = synth.KV_CONFIG
    B, Hq, Hkv, T, Qn = c["B"], c["Hq"], c["Hkv"], c["T"], 2
    inp = synth.kv_inputs(B, Hq, Hkv, T, lens=np.full(B, T), seed=3)
    say("full-size kv write + chunk attention (2 query tokens)")
    kc, ks, vc, vs = bsb.kv_cache_empty(B, Hkv, T, d)
    kt = dev_bf16(inp["k"], d).permute(0, 2, 1, 3).reshape(B * T, Hkv, D).contiguous()
    vt = dev_bf16(inp["v"], d).permute(0, 2, 1, 3).reshape(B * T, Hkv, D).contiguous()
    seq = torch.arange(B, dtype=torch.int32, device=d).repeat_interleave(T)
    pos = torch.arange(T, dtype=torch.int32, device=d).repeat(B)
    bsb.kv_cache_write(kt, vt, seq, pos, kc, ks, vc, vs)
    rng = np.random.default_rng(11)
    qb = f32_to_bf16_bits_ref(rng.standard_normal((B, Qn, Hq, D)).astype(np.float32))
    lens = inp["lens"].copy()
    lens[5] = 4000                                  # a shorter sequence among the full ones
    out = bsb.attention_chunk_int8kv(dev_bf16(qb, d), kc, ks, vc, vs, dev(lens, d), T)
    torch.cuda.synchronize()
    y = bf16_bits_to_f32_ref(host(out)).astype(np.float64)
    for b in (0, 5, 31):
        qk, sk = kv_quantize_ref(inp["k"][b:b + 1])
        qv, sv = kv_quantize_ref(inp["v"][b:b + 1])
        o64, mag = attention_int8kv_chunk_ref(qb[b:b + 1], qk, sk, qv, sv, lens[b:b + 1])
        _check(y[b:b + 1], o64, mag, True)
