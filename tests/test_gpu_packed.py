"""GPU parity: weights repacked into the matrix cores' operand order, and the W8A8
per-group-128 GEMM that reads them.

The repack moves bytes, so it must match the oracle's layout bit for bit. The
GEMM on packed weights keeps the stated float32 group order, so its FP32 and
BF16 outputs must equal the oracle's float32 replay on the unpacked weights bit
for bit (and lie within the float64 definition's tolerances).
"""
import numpy as np
import pytest
import torch

import block_scaled_bit_amd as bsb
from block_scaled_bit_amd import synth
from oracle import (quantize_act_ref, gemm_ref, gemm_fp32_ordered_ref, repack_mfma_ref,
                    packed_position_ref)
from tests.gpu_util import require_gpu, dev, dev_bf16, host, say, Guarded, check_fp32, check_bf16

pytestmark = pytest.mark.gpu


def _inputs(M, K, N, seed):
    d = synth.linear_inputs(M, K, N, outlier_p=0.01, outlier_f=20.0, seed=seed)
    q, sa = quantize_act_ref(d["x"])
    return d, q, sa


def _gpu_repack(qw, d):
    N, K = qw.shape
    g = Guarded((N * K,), torch.int8, d)
    bsb.repack_weights_mfma(dev(qw, d), out=g.view)
    torch.cuda.synchronize()
    return g.check()


def _gpu_packed_gemm(q, sa, packed_d, sw, dtype, d):
    M, N = q.shape[0], sw.shape[0]
    g = Guarded((M, N), dtype, d)
    bsb.gemm_w8a8_g128_packed(dev(q, d), dev(sa, d), packed_d, dev(sw, d), out_dtype=dtype,
                              out=g.view)
    torch.cuda.synchronize()
    return g.check()


@pytest.mark.parametrize("N,K", [(16, 128), (48, 1152), (1024, 7168), (144, 3584)])
def test_repack_matches_the_layout(N, K):
    d = require_gpu()
    say(f"repack N={N} K={K}")
    qw = np.random.default_rng(N + K).integers(-127, 128, (N, K), dtype=np.int8)
    assert np.array_equal(_gpu_repack(qw, d), repack_mfma_ref(qw))


# M spans one, two and four 16-row token blocks with ragged tails; K gives group
# counts that do and do not fill the last chunk of the weight ring (12, 8 or 4
# groups by token blocks) or of the activation chunk (one or two rings). N up to
# 4096 (at most one 16-row block per CU) runs the narrow one-wave kernel; wider N
# the workgroup kernel with 2 to 8 waves.
@pytest.mark.parametrize("M,N,K", [
    (1, 16, 128), (5, 48, 3584), (16, 2048, 4096), (17, 1024, 1024), (32, 4096, 1536),
    (33, 3584, 1152), (48, 272, 1152), (64, 4096, 7168),
    (7, 8192, 896), (16, 8192, 1024), (1, 32768, 256), (64, 8192, 1152), (48, 16384, 768),
    (33, 12288, 2176), (32, 20480, 3200),
])
def test_packed_gemm_matches_the_oracle(M, N, K):
    d = require_gpu()
    say(f"packed gemm M={M} N={N} K={K}")
    cfg, q, sa = _inputs(M, K, N, M * 7 + N)
    qw, sw = cfg["qw"], cfg["sw"]
    packed = _gpu_repack(qw, d)
    pd = dev(packed, d)
    y64, mag = gemm_ref(q, sa, qw, sw)
    c32, cb = gemm_fp32_ordered_ref(q, sa, qw, sw)
    check_fp32(_gpu_packed_gemm(q, sa, pd, sw, torch.float32, d), y64, mag, c32)
    check_bf16(_gpu_packed_gemm(q, sa, pd, sw, torch.bfloat16, d), y64, mag, cb)


def test_tp8_share_of_the_decode_linear():
    """One GPU's column share of the decode linear under 8-way tensor parallelism
    (32 x 8192 x 3584, the narrow kernel) at full size against the oracle."""
    d = require_gpu()
    M, N, K = 32, 3584, 8192
    say(f"packed gemm tp8 share M={M} N={N} K={K}")
    cfg, q, sa = _inputs(M, K, N, 11)
    qw, sw = cfg["qw"], cfg["sw"]
    pd = bsb.repack_weights_mfma(dev(qw, d))
    y64, mag = gemm_ref(q, sa, qw, sw)
    c32, cb = gemm_fp32_ordered_ref(q, sa, qw, sw)
    check_bf16(_gpu_packed_gemm(q, sa, pd, sw, torch.bfloat16, d), y64, mag, cb)
    check_fp32(_gpu_packed_gemm(q, sa, pd, sw, torch.float32, d), y64, mag, c32)


def test_waves_past_the_last_row_block():
    """1795 row blocks over 8-wave workgroups: the last workgroup has five waves
    with no weight rows; they still take part in every barrier and store nothing."""
    d = require_gpu()
    M, N, K = 32, 16 * 1795, 256
    say(f"packed gemm dead waves M={M} N={N} K={K}")
    cfg, q, sa = _inputs(M, K, N, 5)
    qw, sw = cfg["qw"], cfg["sw"]
    pd = bsb.repack_weights_mfma(dev(qw, d))
    y64, mag = gemm_ref(q, sa, qw, sw)
    c32, cb = gemm_fp32_ordered_ref(q, sa, qw, sw)
    check_bf16(_gpu_packed_gemm(q, sa, pd, sw, torch.bfloat16, d), y64, mag, cb)


def test_decode_config_full():
    """The decode-shaped linear (32 x 8192 x 28672) at full size, in the launch
    configuration the benchmark times: repack sampled against the layout, GEMM
    bit-identical to the oracle's float32 replay and to the row-major kernel,
    repeated launches identical."""
    d = require_gpu()
    say("packed gemm decode M=32 K=8192 N=28672 (full)")
    cfg = synth.linear_config("decode")
    qw, sw = cfg["qw"], cfg["sw"]
    N, K = qw.shape
    qd, sd = bsb.quantize_act(dev_bf16(cfg["x"], d))
    q, sa = quantize_act_ref(cfg["x"])
    assert np.array_equal(host(qd), q) and np.array_equal(host(sd), sa)
    qwd, swd = dev(qw, d), dev(sw, d)
    pd = bsb.repack_weights_mfma(qwd)
    rng = np.random.default_rng(1)
    n = rng.integers(0, N, 200000)
    k = rng.integers(0, K, 200000)
    pos = torch.from_numpy(packed_position_ref(n, k, K)).to(d)
    assert np.array_equal(host(pd[pos]), qw[n, k])
    y64, mag = gemm_ref(q, sa, qw, sw)
    c32, cb = gemm_fp32_ordered_ref(q, sa, qw, sw)
    yb = host(bsb.gemm_w8a8_g128_packed(qd, sd, pd, swd))
    check_bf16(yb, y64, mag, cb)
    y32 = host(bsb.gemm_w8a8_g128_packed(qd, sd, pd, swd, out_dtype=torch.float32))
    check_fp32(y32, y64, mag, c32)
    assert np.array_equal(host(bsb.gemm_w8a8_g128(qd, sd, qwd, swd)), yb)
    for _ in range(2):
        assert np.array_equal(host(bsb.gemm_w8a8_g128_packed(qd, sd, pd, swd)), yb)


def test_empty_rows_and_limits():
    d = require_gpu()
    say("packed gemm M=0 and M=65")
    qw = np.ones((16, 128), np.int8)
    pd = bsb.repack_weights_mfma(dev(qw, d))
    sw = dev(np.ones((16, 1), np.float32), d)
    g = Guarded((0, 16), torch.bfloat16, d)
    bsb.gemm_w8a8_g128_packed(torch.empty((0, 128), dtype=torch.int8, device=d),
                              torch.empty((0,), dtype=torch.float32, device=d), pd, sw,
                              out=g.view)
    torch.cuda.synchronize()
    g.check()
    with pytest.raises(bsb.BsbError):
        bsb.gemm_w8a8_g128_packed(torch.zeros((65, 128), dtype=torch.int8, device=d),
                                  torch.ones((65,), dtype=torch.float32, device=d), pd, sw)


@pytest.mark.parametrize("N,K", [(128, 128), (256, 7168), (4096, 1152)])
@pytest.mark.parametrize("dialect", [bsb.BSB_FP8_OCP, bsb.BSB_FP8_FNUZ])
def test_fp8_decode_straight_into_the_packed_layout(N, K, dialect):
    """The FP8 [128,128] UE8M0 decoder writing the operand order: the oracle's
    decode, repacked by the oracle's layout, bit for bit; the scales as the
    row-major decoder writes them."""
    d = require_gpu()
    say(f"decode fp8 packed N={N} K={K} dialect={dialect}")
    from oracle import decode_fp8_block_ref
    w, bs = synth.fp8_block_weights(np.random.default_rng(N + K + dialect), N, K)
    pk = Guarded((N * K,), torch.int8, d)
    sg = Guarded((N, K // 128), torch.float32, d)
    bsb.decode_fp8_block_packed(dev(w, d), dev(bs, d), dialect, packed=pk.view, sw=sg.view)
    torch.cuda.synchronize()
    qr, sr = decode_fp8_block_ref(w, bs, dialect)
    assert np.array_equal(pk.check(), repack_mfma_ref(qr))
    assert np.array_equal(sg.check(), sr)


# one expert of one 16-row block (one partly filled workgroup); K/32 = 12 and 4
# input chunks per row (64-byte row segments), 8 and 128 (128-byte ones); the
# MXFP4 expert shape
@pytest.mark.parametrize("E,N,K", [(1, 16, 128), (3, 48, 384), (2, 32, 256), (5, 80, 1152),
                                   (8, 2048, 4096)])
def test_mxfp4_decode_straight_into_the_packed_layout(E, N, K):
    """The MXFP4 decoder writing the operand order: the oracle's decode of the
    stacked [E*N, K] experts, repacked by the oracle's layout, bit for bit; the
    scales as the row-major decoder writes them. Every UE8M0 exponent with a
    finite scale occurs at the small shapes."""
    d = require_gpu()
    say(f"decode mxfp4 packed E={E} N={N} K={K}")
    from oracle import decode_mxfp4_ref
    rng = np.random.default_rng(E * 1000 + N + K)
    if E * N * K <= 1 << 20:
        packed = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
        sc = rng.integers(0, 251, size=(E, N, K // 32)).astype(np.uint8)
    else:
        packed, sc = synth.mxfp4_weights(rng, E, N, K)
    pk = Guarded((E * N * K,), torch.int8, d)
    sg = Guarded((E, N, K // 128), torch.float32, d)
    bsb.decode_mxfp4_packed(dev(packed, d), dev(sc, d), packed_qw=pk.view, sw=sg.view)
    torch.cuda.synchronize()
    qr, sr = decode_mxfp4_ref(packed, sc)
    assert np.array_equal(pk.check(), repack_mfma_ref(qr.reshape(E * N, K)))
    assert np.array_equal(sg.check().view(np.uint32), sr.view(np.uint32))


def _grouped_case(lengths, N, K, seed):
    rng = np.random.default_rng(seed)
    E = len(lengths)
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(lengths)
    x = synth.activations(rng, int(off[-1]), K, 0.01, 20.0)
    qw = synth.int8_weights(rng, (E, N, K))
    sw = synth.group_scales(rng, (E, N, K // 128))
    return x, qw, sw, off


# experts empty, of 1, 2, 31, 33, 64, 70 and 300 rows (passes of 32 rows); group
# counts that do and do not fill the activation chunk; the MXFP4 expert shape
@pytest.mark.parametrize("lengths,N,K", [
    ([0, 0, 0, 64], 64, 128),
    ([17] * 9, 256, 512),
    ([0, 70, 1, 33, 0, 31, 2], 208, 384),
    ([31, 0, 33, 1, 32, 5, 64, 2], 2048, 4224),
    ([300, 0, 0, 2], 144, 1152),
    ([32] * 8, 2048, 4096),
])
def test_grouped_packed_matches_the_oracle(lengths, N, K):
    from oracle import grouped_gemm_ref, grouped_gemm_fp32_ordered_ref
    d = require_gpu()
    say(f"grouped packed lengths={lengths} N={N} K={K}")
    x, qw, sw, off = _grouped_case(lengths, N, K, len(lengths) + N)
    q, sa = quantize_act_ref(x)
    E, R = len(lengths), q.shape[0]
    pd = bsb.repack_weights_mfma(dev(qw.reshape(E * N, K), d))
    y64, mag = grouped_gemm_ref(q, sa, qw, sw, off)
    c32, cb = grouped_gemm_fp32_ordered_ref(q, sa, qw, sw, off)
    for dtype in (torch.float32, torch.bfloat16):
        g = Guarded((R, N), dtype, d)
        bsb.grouped_gemm_w8a8_g128_packed(dev(q, d), dev(sa, d), pd, dev(sw, d), dev(off, d),
                                          out_dtype=dtype, out=g.view)
        torch.cuda.synchronize()
        if dtype == torch.float32:
            check_fp32(g.check(), y64, mag, c32)
        else:
            check_bf16(g.check(), y64, mag, cb)
