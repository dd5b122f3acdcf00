"""GPU parity: the grouped (MoE) W8A8 per-group-128 GEMM vs the oracle."""
import numpy as np
import pytest
import torch

import block_scaled_bit_amd as bsb
from block_scaled_bit_amd import synth
from oracle import (quantize_act_ref, gemm_fp32_ordered_ref, gemm_ref, grouped_gemm_ref,
                    grouped_gemm_fp32_ordered_ref, decode_mxfp4_ref)
from tests.gpu_util import (require_gpu, dev, dev_bf16, host, say, Guarded, check_fp32,
                            check_bf16)

pytestmark = pytest.mark.gpu


def _case(lengths, N, K, seed):
    rng = np.random.default_rng(seed)
    E = len(lengths)
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(lengths)
    R = int(off[-1])
    x = synth.activations(rng, R, K, 0.01, 20.0)
    qw = synth.int8_weights(rng, (E, N, K))
    sw = synth.group_scales(rng, (E, N, K // 128))
    return x, qw, sw, off


def _gpu_grouped(q, sa, qw, sw, off, dtype, d):
    R, N = q.shape[0], qw.shape[1]
    g = Guarded((R, N), dtype, d)
    bsb.grouped_gemm_w8a8_g128(dev(q, d), dev(sa, d), dev(qw, d), dev(sw, d), dev(off, d),
                               out_dtype=dtype, out=g.view)
    torch.cuda.synchronize()
    return g.check()


@pytest.mark.parametrize("lengths,N,K", [
    # at most 32 rows per expert on average: weights streamed per expert, rows
    # in passes of 32 (segments of 1, 2, 31, 33, 64, 70 rows)
    ([0, 0, 0, 64], 64, 128),
    ([17] * 9, 257, 512),
    ([0, 70, 1, 33, 0, 31, 2], 200, 384),
    ([31, 0, 33, 1, 32, 5, 64, 2], 2048, 4224),    # >= 4 waves per workgroup, 33 groups
    ([5, 40, 0, 64, 3, 20, 31, 1], 2048, 2560),     # 20 groups: 16-row scale pieces
    # up to 128 rows per expert on average: 128x128 tiles
    ([0, 1, 127, 128, 129, 0, 5], 96, 256),     # segment ends at 0, 1, BM-1, BM, BM+1
    ([300, 0, 0, 2], 130, 384),
    # at least 128 rows per expert on average but too few tiles for the 256x256
    # kernel (at most 15): 128x128 tiles, segments ending at 1, 63/64/65,
    # 255/256/257
    ([0, 1, 255, 256, 257, 0, 64, 65, 300], 96, 256),
    ([700, 0, 129, 513, 63], 300, 384),
    ([1, 1100], 520, 128),
    # enough tiles for the 256x256 kernel (19 tile rows x 8 columns, more than
    # 128): segments ending at 1, 63/64/65 (one wave's rows), 255/256/257 (one
    # tile) inside it
    ([0, 1, 255, 256, 257, 0, 64, 65, 300, 63, 2300, 600, 513], 2048, 256),
    # the same with a ragged last tile column: N not a multiple of 8 (outputs stored
    # one by one at the end of each row) and a multiple of 8 that is not one of 256
    ([0, 1, 255, 256, 257, 0, 64, 65, 300, 63, 2300, 600, 513], 2053, 256),
    ([0, 1, 255, 256, 257, 0, 64, 65, 300, 63, 2300, 600, 513], 2056, 256),
])
def test_segments_and_tails(lengths, N, K):
    d = require_gpu()
    say(f"grouped lengths={lengths} N={N} K={K}")
    x, qw, sw, off = _case(lengths, N, K, sum(lengths) + N)
    q, sa = quantize_act_ref(x)
    y64, mag = grouped_gemm_ref(q, sa, qw, sw, off)
    c32, cb = grouped_gemm_fp32_ordered_ref(q, sa, qw, sw, off)
    check_fp32(_gpu_grouped(q, sa, qw, sw, off, torch.float32, d), y64, mag, c32)
    check_bf16(_gpu_grouped(q, sa, qw, sw, off, torch.bfloat16, d), y64, mag, cb)


def test_single_expert_equals_dense_bit_for_bit():
    d = require_gpu()
    x, qw, sw, off = _case([200], 160, 512, 3)
    q, sa = quantize_act_ref(x)
    say("grouped E=1 vs dense")
    yg = _gpu_grouped(q, sa, qw, sw, off, torch.float32, d)
    yd = host(bsb.gemm_w8a8_g128(dev(q, d), dev(sa, d), dev(qw[0], d), dev(sw[0], d),
                                 out_dtype=torch.float32))
    assert np.array_equal(yg.view(np.uint32), yd.view(np.uint32))


def test_empty_batch():
    d = require_gpu()
    y = bsb.grouped_gemm_w8a8_g128(torch.empty((0, 128), dtype=torch.int8, device=d),
                                   torch.empty((0,), dtype=torch.float32, device=d),
                                   torch.zeros((3, 8, 128), dtype=torch.int8, device=d),
                                   torch.ones((3, 8, 1), dtype=torch.float32, device=d),
                                   torch.zeros((4,), dtype=torch.int32, device=d))
    assert y.shape == (0, 8)


def test_moe_config_sampled_rows():
    """The routed MoE layer at full size (4096 tokens x top-8 over 64 experts, Zipf-skewed,
    some experts empty). Every expert's first and last rows plus a random sample are
    checked against the oracle; the whole output is checked for determinism."""
    d = require_gpu()
    say("grouped moe T=4096 E=64 K=4096 N=2048 (full, sampled rows)")
    m = synth.moe_inputs()
    off, qw, sw = m["offsets"], m["qw"], m["sw"]
    xd = dev_bf16(m["x_sorted"], d)
    qd, sd = bsb.quantize_act(xd)
    q, sa = quantize_act_ref(m["x_sorted"])
    assert np.array_equal(host(qd), q) and np.array_equal(host(sd), sa)
    qwd, swd, offd = dev(qw, d), dev(sw, d), dev(off, d)
    yb = host(bsb.grouped_gemm_w8a8_g128(qd, sd, qwd, swd, offd))
    yb2 = host(bsb.grouped_gemm_w8a8_g128(qd, sd, qwd, swd, offd))
    assert np.array_equal(yb, yb2)
    y32 = host(bsb.grouped_gemm_w8a8_g128(qd, sd, qwd, swd, offd, out_dtype=torch.float32))
    rng = np.random.default_rng(1)
    for e in range(64):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        # segment ends, random rows, and the rows either side of every 64-row wave
        # boundary and 256-row tile boundary inside the segment
        edges = [lo + b + d for b in range(64, hi - lo, 64) for d in (-1, 0)]
        rows = sorted(set([lo, hi - 1] + rng.integers(lo, hi, 3).tolist() +
                          [r for r in edges if lo <= r < hi]))
        y64, mag = gemm_ref(q[rows], sa[rows], qw[e], sw[e])
        c32, cb = gemm_fp32_ordered_ref(q[rows], sa[rows], qw[e], sw[e])
        check_bf16(yb[rows], y64, mag, cb)
        check_fp32(y32[rows], y64, mag, c32)


@pytest.mark.parametrize("M", [32, 1024])
def test_blockfmt_experts_decode_then_grouped(M):
    """MXFP4 experts decoded on the GPU, then the grouped GEMM with M rows per expert."""
    d = require_gpu()
    say(f"blockfmt experts decode+grouped M={M}")
    b = synth.blockfmt_inputs(M=M)
    qwd, swd = bsb.decode_mxfp4(dev(b["packed"], d), dev(b["scale"], d))
    qd, sd = bsb.quantize_act(dev_bf16(b["x_e"], d))
    yb = host(bsb.grouped_gemm_w8a8_g128(qd, sd, qwd, swd, dev(b["offsets"], d)))
    qw, sw = decode_mxfp4_ref(b["packed"], b["scale"])
    assert np.array_equal(host(qwd), qw)
    q, sa = quantize_act_ref(b["x_e"])
    off = b["offsets"]
    cols = np.r_[0:64, 2048 - 64:2048]
    for e in (0, 3, 7):
        rows = np.r_[off[e]:off[e] + min(M, 40)]
        y64, mag = gemm_ref(q[rows], sa[rows], qw[e][cols], sw[e][cols])
        _, cb = gemm_fp32_ordered_ref(q[rows], sa[rows], qw[e][cols], sw[e][cols])
        check_bf16(yb[rows][:, cols], y64, mag, cb)


@pytest.mark.parametrize("lengths,N,K,T", [
    ([3, 0, 17, 32, 1, 0, 31], 200, 384, 40),         # <= 32 rows per expert: passes of 32 rows
    ([0, 1, 127, 128, 129, 0, 5], 96, 256, 100),       # 128x128 tiles
    ([0, 1, 255, 256, 257, 0, 64, 65, 300, 63, 2300, 600, 513], 2048, 256, 1000),   # 256x256
    ([0, 1, 255, 256, 257, 0, 64, 65, 300, 63, 2300, 600, 513], 2053, 256, 1000),   # ragged N
    ([0, 1, 127, 128, 129, 0, 5], 99, 256, 100),       # 128x128 tiles, ragged N
])
def test_rows_gathered_by_the_kernel(lengths, N, K, T):
    """The grouped GEMM reading its rows through the token index: bit-identical to
    gathering the rows first and running the grouped GEMM, and held to the same bar
    against the oracle on the gathered rows; indices outside [0, T) read a zero row with
    scale 0 (the gather's rule)."""
    d = require_gpu()
    R = sum(lengths)
    say(f"grouped gather lengths={lengths} N={N} K={K} T={T}")
    _, qw, sw, off = _case(lengths, N, K, R + N)
    rng = np.random.default_rng(T + R)
    q, sa = quantize_act_ref(synth.activations(rng, T, K, 0.01, 20.0))
    index = rng.integers(0, T, size=R).astype(np.int32)
    index[::97] = -1
    index[5::101] = T
    ok = (index >= 0) & (index < T)
    qg = np.zeros((R, K), np.int8)
    sg = np.zeros(R, np.float32)
    qg[ok], sg[ok] = q[index[ok]], sa[index[ok]]
    y64, mag = grouped_gemm_ref(qg, sg, qw, sw, off)
    c32, cb = grouped_gemm_fp32_ordered_ref(qg, sg, qw, sw, off)
    qd, sd, idd = dev(q, d), dev(sa, d), dev(index, d)
    qwd, swd, offd = dev(qw, d), dev(sw, d), dev(off, d)
    qs, ss = bsb.gather_rows(qd, sd, idd)
    for dtype in (torch.float32, torch.bfloat16):
        g = Guarded((R, N), dtype, d)
        bsb.grouped_gemm_w8a8_g128_gather(qd, sd, idd, qwd, swd, offd, out_dtype=dtype,
                                          out=g.view)
        y2 = bsb.grouped_gemm_w8a8_g128(qs, ss, qwd, swd, offd, out_dtype=dtype)
        torch.cuda.synchronize()
        y = g.check()
        assert np.array_equal(y.view(np.uint8), host(y2).view(np.uint8))
        if dtype == torch.float32:
            check_fp32(y, y64, mag, c32)
        else:
            check_bf16(y, y64, mag, cb)


def test_moe_config_rows_gathered_by_the_kernel():
    """The MoE layer's grouped GEMM (4096 tokens, top-8 of 64 experts) reading its 32768
    rows through the token index, as the routed layer runs it: bit-identical to the
    gather followed by the grouped GEMM."""
    d = require_gpu()
    say("moe config, rows gathered by the kernel")
    m = synth.moe_inputs()
    x = dev_bf16(m["x_tokens"], d)
    qt, st = bsb.quantize_act(x)
    idx, qw, sw, off = dev(m["token_of_row"], d), dev(m["qw"], d), dev(m["sw"], d), dev(m["offsets"], d)
    qs, ss = bsb.gather_rows(qt, st, idx)
    a = bsb.grouped_gemm_w8a8_g128(qs, ss, qw, sw, off)
    b = bsb.grouped_gemm_w8a8_g128_gather(qt, st, idx, qw, sw, off)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
