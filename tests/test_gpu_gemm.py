"""GPU parity: the W8A8 per-group-128 GEMM (dense) and its INT32 partials vs the oracle.

INT32 partials and quantised inputs must match bit for bit. FP32/BF16 outputs
are checked against the float64 definition with the stated tolerances
(gpu_util.check_fp32 / check_bf16) and, because the kernels keep the stated
float32 group order, also bit for bit against the oracle's float32 replay.
"""
import numpy as np
import pytest
import torch

import block_scaled_bit_amd as bsb
from block_scaled_bit_amd import synth
from block_scaled_bit_amd import _lib as bsb_lib
from oracle import (quantize_act_ref, group_partials_ref, gemm_ref, gemm_fp32_ordered_ref,
                    decode_fp8_block_ref)
from oracle.decode import OCP, FNUZ
from tests.gpu_util import (require_gpu, dev, dev_bf16, host, say, Guarded, check_fp32,
                            check_bf16)

pytestmark = pytest.mark.gpu


def _inputs(M, K, N, seed, p=0.01, f=20.0):
    d = synth.linear_inputs(M, K, N, outlier_p=p, outlier_f=f, seed=seed)
    q, sa = quantize_act_ref(d["x"])
    return d, q, sa


def _gpu_gemm(q, sa, qw, sw, dtype, d):
    M, N = q.shape[0], qw.shape[0]
    g = Guarded((M, N), dtype, d)
    bsb.gemm_w8a8_g128(dev(q, d), dev(sa, d), dev(qw, d), dev(sw, d), out_dtype=dtype, out=g.view)
    torch.cuda.synchronize()
    return g.check()


def _gpu_partials(q, qw, d):
    M, K = q.shape
    g = Guarded((M, qw.shape[0], K // 128), torch.int32, d)
    bsb.gemm_w8a8_g128_partials(dev(q, d), dev(qw, d), out=g.view)
    torch.cuda.synchronize()
    return g.check()


def _full_check(q, sa, qw, sw, d):
    P = _gpu_partials(q, qw, d)
    Pr = group_partials_ref(q, qw)
    assert np.array_equal(P, Pr), f"{np.sum(P != Pr)} INT32 partials differ"
    y64, mag = gemm_ref(q, sa, qw, sw)
    c32, cb = gemm_fp32_ordered_ref(q, sa, qw, sw)
    y32 = _gpu_gemm(q, sa, qw, sw, torch.float32, d)
    check_fp32(y32, y64, mag, c32)
    yb = _gpu_gemm(q, sa, qw, sw, torch.bfloat16, d)
    check_bf16(yb, y64, mag, cb)


def test_tiny_config():
    d = require_gpu()
    cfg, q, sa = _inputs(16, 1024, 1024, 0)
    say("gemm tiny M=16 K=1024 N=1024")
    # the GPU quantisation is the input of the GPU GEMM in the real path
    qg, sg = bsb.quantize_act(dev_bf16(cfg["x"], d))
    assert np.array_equal(host(qg), q) and np.array_equal(host(sg), sa)
    _full_check(q, sa, cfg["qw"], cfg["sw"], d)


@pytest.mark.parametrize("M,N,K", [
    (1, 1, 128), (3, 65, 256), (16, 64, 384), (17, 100, 128), (32, 257, 512),
    (33, 64, 256), (64, 130, 640), (65, 129, 256), (100, 300, 384), (128, 128, 128),
    (130, 257, 512), (257, 1, 256), (300, 96, 1024),
    (512, 256, 256), (600, 300, 384), (777, 1000, 256), (1024, 520, 128), (513, 7, 1152),
    (2049, 7425, 256), (2305, 7000, 384), (1537, 5000, 256),
    # M <= 64 with at least 4 waves per workgroup (scales staged in 16-group
    # chunks): a ragged last chunk, less than one chunk, odd N
    (33, 12400, 2176), (1, 20000, 1152), (64, 13001, 4224),
    (17, 12900, 2560)])     # G a multiple of 4: 16-row scale pieces, partial last chunk
def test_ragged_shapes(M, N, K):
    """Every kernel (M <= 64; 128x128 tiles; 256x256 tiles from 512 rows when there are
    more than 128 such tiles: 2049 x 7425, 2305 x 7000 and 1537 x 5000, the last 140 tiles),
    partial tiles in M and N, several groups."""
    d = require_gpu()
    say(f"gemm ragged M={M} N={N} K={K}")
    cfg, q, sa = _inputs(M, K, N, M * 1000 + N + K)
    _full_check(q, sa, cfg["qw"], cfg["sw"], d)


def test_integer_identity_on_gpu():
    """Integer activations with unit scales: the GPU output is the exact integer matmul."""
    d = require_gpu()
    rng = np.random.default_rng(21)
    for M in (8, 80):
        K, N = 1024, 200
        xi = rng.integers(-127, 128, size=(M, K)).astype(np.float32)
        xi[:, 7] = 127.0
        qg, sg = bsb.quantize_act(dev_bf16(synth.to_bf16_bits(xi), d))
        assert bool((sg == 1.0).all())
        qw = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
        sw = np.ones((N, K // 128), np.float32)
        y = bsb.gemm_w8a8_g128(qg, sg, dev(qw, d), dev(sw, d), out_dtype=torch.float32)
        want = xi.astype(np.int64) @ qw.astype(np.int64).T
        assert np.array_equal(host(y).astype(np.int64), want)


def test_decode_config_full():
    """The decode-shaped linear at full size, in the launch configuration the benchmark times."""
    d = require_gpu()
    say("gemm decode M=32 K=8192 N=28672 (full)")
    cfg = synth.linear_config("decode")
    xd = dev_bf16(cfg["x"], d)
    qd, sd = bsb.quantize_act(xd)
    q, sa = quantize_act_ref(cfg["x"])
    assert np.array_equal(host(qd), q) and np.array_equal(host(sd), sa)
    qw, sw = cfg["qw"], cfg["sw"]
    qwd, swd = dev(qw, d), dev(sw, d)
    P = host(bsb.gemm_w8a8_g128_partials(qd, qwd))
    assert np.array_equal(P, group_partials_ref(q, qw))
    del P
    y64, mag = gemm_ref(q, sa, qw, sw)
    c32, cb = gemm_fp32_ordered_ref(q, sa, qw, sw)
    yb = host(bsb.gemm_w8a8_g128(qd, sd, qwd, swd))
    check_bf16(yb, y64, mag, cb)
    y32 = host(bsb.gemm_w8a8_g128(qd, sd, qwd, swd, out_dtype=torch.float32))
    check_fp32(y32, y64, mag, c32)
    # determinism: repeated launches are bit-identical
    for _ in range(2):
        assert np.array_equal(host(bsb.gemm_w8a8_g128(qd, sd, qwd, swd)), yb)


def test_tp8_share_of_the_decode_linear():
    """One GPU's column share of the decode linear under 8-way tensor parallelism
    (N = 3584), as the benchmark times it: full output against the oracle."""
    d = require_gpu()
    say("gemm decode share M=32 K=8192 N=3584")
    cfg = synth.linear_inputs(32, 8192, 3584, outlier_p=0.005, outlier_f=30.0, seed=0)
    q, sa = quantize_act_ref(cfg["x"])
    qd, sd = bsb.quantize_act(dev_bf16(cfg["x"], d))
    assert np.array_equal(host(qd), q) and np.array_equal(host(sd), sa)
    y64, mag = gemm_ref(q, sa, cfg["qw"], cfg["sw"])
    _, cb = gemm_fp32_ordered_ref(q, sa, cfg["qw"], cfg["sw"])
    check_bf16(host(bsb.gemm_w8a8_g128(qd, sd, dev(cfg["qw"], d), dev(cfg["sw"], d))), y64, mag, cb)


def test_prefill_config_sampled():
    """Prefill-shaped linear at full size; eight 128x128 output tiles checked against the oracle."""
    d = require_gpu()
    say("gemm prefill M=4096 K=8192 N=8192 (full, sampled tiles)")
    cfg = synth.linear_config("prefill")
    q, sa = quantize_act_ref(cfg["x"])
    qd, sd = bsb.quantize_act(dev_bf16(cfg["x"], d))
    assert np.array_equal(host(qd), q) and np.array_equal(host(sd), sa)
    qw, sw = cfg["qw"], cfg["sw"]
    qwd, swd = dev(qw, d), dev(sw, d)
    yb = host(bsb.gemm_w8a8_g128(qd, sd, qwd, swd))
    P = bsb.gemm_w8a8_g128_partials(qd, qwd)
    rng = np.random.default_rng(0)
    tiles = [(0, 0), (31, 63)] + [tuple(rng.integers(0, [32, 64])) for _ in range(6)]
    for tm, tn in tiles:
        rs, cs = slice(128 * tm, 128 * tm + 128), slice(128 * tn, 128 * tn + 128)
        y64, mag = gemm_ref(q[rs], sa[rs], qw[cs], sw[cs])
        _, cb = gemm_fp32_ordered_ref(q[rs], sa[rs], qw[cs], sw[cs])
        check_bf16(yb[rs, cs], y64, mag, cb)
        assert np.array_equal(host(P[rs, cs]), group_partials_ref(q[rs], qw[cs]))


def test_prefill_config_every_tile_row_and_column():
    """Prefill-shaped linear at full size: one whole output row in every 256-row tile
    row (16 rows x 8192 columns) and one whole output column in every 256-column tile
    (32 columns x 4096 rows), so every workgroup of the 256x256 kernel is checked, in
    BF16 and FP32, strictly against the stated float32 order. The row and column
    inside each tile move from tile to tile so that every wave position is hit."""
    d = require_gpu()
    say("gemm prefill M=4096 K=8192 N=8192 (full, a row per tile row, a column per tile)")
    cfg = synth.linear_config("prefill")
    q, sa = quantize_act_ref(cfg["x"])
    qd, sd = bsb.quantize_act(dev_bf16(cfg["x"], d))
    qw, sw = cfg["qw"], cfg["sw"]
    qwd, swd = dev(qw, d), dev(sw, d)
    yb = host(bsb.gemm_w8a8_g128(qd, sd, qwd, swd))
    y32 = host(bsb.gemm_w8a8_g128(qd, sd, qwd, swd, out_dtype=torch.float32))
    rows = np.array([256 * t + (t * 37 + 5) % 256 for t in range(16)])
    cols = np.array([256 * t + (t * 53 + 11) % 256 for t in range(32)])
    y64, mag = gemm_ref(q[rows], sa[rows], qw, sw)
    c32, cb = gemm_fp32_ordered_ref(q[rows], sa[rows], qw, sw)
    check_bf16(yb[rows], y64, mag, cb)
    check_fp32(y32[rows], y64, mag, c32)
    y64, mag = gemm_ref(q, sa, qw[cols], sw[cols])
    c32, cb = gemm_fp32_ordered_ref(q, sa, qw[cols], sw[cols])
    check_bf16(yb[:, cols], y64, mag, cb)
    check_fp32(y32[:, cols], y64, mag, c32)


@pytest.mark.parametrize("M", [32, 1024])
def test_blockfmt_dense_decode_then_gemm(M):
    """FP8 [128,128]-block weights decoded on the GPU, then the GEMM at M tokens. The
    same bytes read as OCP give exactly twice the fnuz outputs, bit for bit."""
    d = require_gpu()
    say(f"blockfmt dense decode+gemm M={M}")
    b = synth.blockfmt_inputs(M=M)
    w, bs, x = b["w_fp8"], b["bs"], b["x_d"]
    qd, sd = bsb.quantize_act(dev_bf16(x, d))
    q, sa = quantize_act_ref(x)
    outs = {}
    for dialect in (OCP, FNUZ):
        qwd, swd = bsb.decode_fp8_block(dev(w, d), dev(bs, d), dialect)
        outs[dialect] = (host(bsb.gemm_w8a8_g128(qd, sd, qwd, swd)),
                         host(bsb.gemm_w8a8_g128(qd, sd, qwd, swd, out_dtype=torch.float32)))
    assert np.array_equal(outs[OCP][1], (2 * outs[FNUZ][1]).astype(np.float32))
    from oracle import bf16_bits_to_f32_ref
    assert np.array_equal(bf16_bits_to_f32_ref(outs[OCP][0]), 2 * bf16_bits_to_f32_ref(outs[FNUZ][0]))
    qw, sw = decode_fp8_block_ref(w, bs, OCP)
    rows = slice(0, min(M, 64))
    cols = np.r_[0:128, 4096 - 128:4096]
    y64, mag = gemm_ref(q[rows], sa[rows], qw[cols], sw[cols])
    c32, cb = gemm_fp32_ordered_ref(q[rows], sa[rows], qw[cols], sw[cols])
    check_fp32(outs[OCP][1][rows][:, cols], y64, mag, c32)
    check_bf16(outs[OCP][0][rows][:, cols], y64, mag, cb)


@pytest.mark.gpu
def test_mfma_probes_run_and_repeat():
    """The MFMA rate probes (plain, and with the per-group epilogue beside the MFMAs)
    launch, write every thread's value, and give the same values on a second call
    (the work is a fixed function of the operand bytes)."""
    d = require_gpu()
    say("mfma probes")
    L = bsb_lib.lib()
    g = torch.Generator(device="cpu").manual_seed(5)
    a = torch.randint(-127, 128, (1 << 16,), dtype=torch.int8, generator=g).to(d)
    b = torch.randint(-127, 128, (1 << 16,), dtype=torch.int8, generator=g).to(d)
    st = torch.cuda.current_stream(d).cuda_stream
    outs = []
    for probe in (L.bsb_probe_mfma_i8, L.bsb_probe_mfma_i8_epilogue):
        res = []
        for _ in range(2):
            o = torch.full((131072,), 0x5A5A5A5A, dtype=torch.int32, device=d)
            assert probe(a.data_ptr(), b.data_ptr(), a.numel(), 2, o.data_ptr(), st) == 0
            torch.cuda.synchronize(d)
            res.append(o.cpu())
        assert torch.equal(res[0], res[1])
        assert (res[0] != 0x5A5A5A5A).float().mean() > 0.99
        outs.append(res[0])
    assert not torch.equal(outs[0], outs[1])
