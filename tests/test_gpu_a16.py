"""GPU parity: the BF16-activation routes (weight-only INT8 W8A16, BF16 weights) and
the FP8 -> BF16 load-time dequantisation vs the oracle.

The matrix core sums a group's products in float32 in its own order, so the GEMMs
are checked against the float64 definition with the bound derived for any such
order, |y - y64| <= (127 + G + 2) * 2^-24 * mag (plus half a BF16 ulp for BF16
output); the dequantisation is exact and compared bit for bit.
"""
import numpy as np
import pytest
import torch

import block_scaled_bit_amd as bsb
from block_scaled_bit_amd import synth
from oracle import (gemm_w8a16_ref, gemm_bf16_ref, a16_tolerance, dequant_fp8_block_bf16_ref,
                    bf16_bits_to_f32_ref, f32_to_bf16_bits_ref)
from oracle.decode import OCP, FNUZ
from tests.gpu_util import require_gpu, dev, dev_bf16, host, say, Guarded

pytestmark = pytest.mark.gpu


def _check(y, y64, mag, K, bf16):
    t = a16_tolerance(K)
    if bf16:
        v = bf16_bits_to_f32_ref(np.asarray(y, np.uint16)).astype(np.float64)
        half_ulp = np.abs(v) * 2.0 ** -8
    else:
        v = np.asarray(y, np.float32).astype(np.float64)
        half_ulp = 0.0
    err = np.abs(v - y64)
    bad = err > t * mag + half_ulp
    assert not bad.any(), f"{bad.sum()} outputs beyond the bound (max err/mag {(err / mag).max():.3g})"


def _w8a16(xb, qw, sw, dtype, d):
    g = Guarded((xb.shape[0], qw.shape[0]), dtype, d)
    bsb.gemm_w8a16_g128(dev_bf16(xb, d), dev(qw, d), dev(sw, d), out_dtype=dtype, out=g.view)
    torch.cuda.synchronize()
    return g.check()


def _bf16(xb, wb, dtype, d):
    g = Guarded((xb.shape[0], wb.shape[0]), dtype, d)
    bsb.gemm_bf16(dev_bf16(xb, d), dev_bf16(wb, d), out_dtype=dtype, out=g.view)
    torch.cuda.synchronize()
    return g.check()


SHAPES = [(1, 1, 128), (17, 100, 384), (33, 64, 256), (64, 130, 640),   # 2-wave groups
          (32, 13000, 1152), (64, 13001, 2176)]                         # wider groups


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_w8a16_ragged(M, N, K):
    d = require_gpu()
    say(f"w8a16 M={M} N={N} K={K}")
    cfg = synth.linear_inputs(M, K, N, outlier_p=0.01, outlier_f=20.0, seed=M + N + K)
    y64, mag = gemm_w8a16_ref(cfg["x"], cfg["qw"], cfg["sw"])
    _check(_w8a16(cfg["x"], cfg["qw"], cfg["sw"], torch.float32, d), y64, mag, K, False)
    _check(_w8a16(cfg["x"], cfg["qw"], cfg["sw"], torch.bfloat16, d), y64, mag, K, True)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_bf16_ragged(M, N, K):
    d = require_gpu()
    say(f"bf16 gemm M={M} N={N} K={K}")
    cfg = synth.linear_inputs(M, K, N, outlier_p=0.01, outlier_f=20.0, seed=M + N + K)
    rng = np.random.default_rng(M + N + K)
    wb = synth.to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02))
    y64, mag = gemm_bf16_ref(cfg["x"], wb)
    _check(_bf16(cfg["x"], wb, torch.float32, d), y64, mag, K, False)
    _check(_bf16(cfg["x"], wb, torch.bfloat16, d), y64, mag, K, True)


# beyond 64 rows: 128x128 tiles; partial tiles in M and N, group counts 1 to 17
# (the stage loop's unrolled body and its two-stage remainder)
TILED = [(65, 1, 128), (100, 257, 384), (130, 128, 256), (257, 100, 1152), (600, 300, 640),
         (1000, 520, 2176)]


@pytest.mark.parametrize("M,N,K", TILED)
def test_w8a16_tiled_ragged(M, N, K):
    test_w8a16_ragged(M, N, K)


@pytest.mark.parametrize("M,N,K", TILED)
def test_bf16_tiled_ragged(M, N, K):
    test_bf16_ragged(M, N, K)


@pytest.mark.parametrize("route", ["w8a16", "bf16"])
def test_prefill_config_every_tile_row_and_column(route):
    """The prefill-shaped linear (4096 x 8192 x 8192) on both BF16-activation routes: one
    whole output row in every 128-row tile row and one whole column in every 128-column
    tile, against the float64 definition with the order-independent bound."""
    d = require_gpu()
    say(f"{route} prefill M=4096 K=8192 N=8192 (a row per tile row, a column per tile)")
    cfg = synth.linear_config("prefill")
    x = cfg["x"]
    xd = dev_bf16(x, d)
    rows = np.array([128 * t + (t * 37 + 5) % 128 for t in range(32)])
    cols = np.array([128 * t + (t * 53 + 11) % 128 for t in range(64)])
    if route == "w8a16":
        qw, sw = cfg["qw"], cfg["sw"]
        y32 = host(bsb.gemm_w8a16_g128(xd, dev(qw, d), dev(sw, d), out_dtype=torch.float32))
        yb = host(bsb.gemm_w8a16_g128(xd, dev(qw, d), dev(sw, d)))
        ref_rows = gemm_w8a16_ref(x[rows], qw, sw)
        ref_cols = gemm_w8a16_ref(x, qw[cols], sw[cols])
    else:
        rng = np.random.default_rng(4)
        wb = synth.to_bf16_bits(rng.standard_normal((8192, 8192), dtype=np.float32) *
                                np.float32(0.02))
        wd = dev_bf16(wb, d)
        y32 = host(bsb.gemm_bf16(xd, wd, out_dtype=torch.float32))
        yb = host(bsb.gemm_bf16(xd, wd))
        ref_rows = gemm_bf16_ref(x[rows], wb)
        ref_cols = gemm_bf16_ref(x, wb[cols])
    _check(y32[rows], *ref_rows, 8192, False)
    _check(yb[rows], *ref_rows, 8192, True)
    _check(y32[:, cols], *ref_cols, 8192, False)
    _check(yb[:, cols], *ref_cols, 8192, True)


def test_w8a16_decode_config():
    """The decode-shaped linear (32 x 8192 x 28672) on its INT8 weights, BF16 activations
    as they are; every output checked."""
    d = require_gpu()
    say("w8a16 decode M=32 K=8192 N=28672")
    cfg = synth.linear_config("decode")
    y64, mag = gemm_w8a16_ref(cfg["x"], cfg["qw"], cfg["sw"])
    y = host(bsb.gemm_w8a16_g128(dev_bf16(cfg["x"], d), dev(cfg["qw"], d), dev(cfg["sw"], d)))
    _check(y, y64, mag, 8192, True)


def test_dequant_fp8_to_bf16_bit_exact_both_dialects():
    d = require_gpu()
    say("dequant fp8 -> bf16 4096 x 7168, OCP and fnuz")
    b = synth.blockfmt_inputs(M=32)
    w, bs = b["w_fp8"], b["bs"]
    outs = {}
    for dialect in (OCP, FNUZ):
        g = Guarded(w.shape, torch.int16, d)
        bsb.dequant_fp8_block_bf16(dev(w, d), dev(bs, d), dialect, out=g.view)
        torch.cuda.synchronize()
        got = np.asarray(g.check()).view(np.uint16)
        assert np.array_equal(got, dequant_fp8_block_bf16_ref(w, bs, dialect))
        outs[dialect] = bf16_bits_to_f32_ref(got)
    assert np.array_equal(outs[OCP], 2 * outs[FNUZ])


def test_dequant_fp8_to_bf16_every_code_and_low_exponents():
    """Every byte under block exponents 0 .. 8 (values down among the BF16 subnormals,
    rounded to nearest even) and a high one, both dialects, bit for bit."""
    d = require_gpu()
    say("dequant fp8 -> bf16 code sweep")
    w = np.resize(np.arange(256, dtype=np.uint8), (256, 1024)).astype(np.uint8)
    bs = np.array([[0, 1, 2, 4, 8, 100, 127, 150]] * 2, np.uint8)
    for dialect in (OCP, FNUZ):
        nan = {OCP: (0x7F, 0xFF), FNUZ: (0x80,)}[dialect]
        ww = w.copy()
        ww[np.isin(ww, nan)] = 0                   # NaN codes are outside the domain
        got = host(bsb.dequant_fp8_block_bf16(dev(ww, d), dev(bs, d), dialect)).view(np.uint16)
        assert np.array_equal(got, dequant_fp8_block_bf16_ref(ww, bs, dialect)), dialect


def test_bf16_route_end_to_end_on_fp8_weights():
    """The BF16 route: FP8 dense weights (4096 x 7168) dequantised on the GPU, then the
    BF16 GEMM at 32 tokens, against the float64 definition on the exact weights."""
    d = require_gpu()
    say("bf16 route: dequant + gemm_bf16, 32 x 7168 x 4096")
    b = synth.blockfmt_inputs(M=32)
    wb = bsb.dequant_fp8_block_bf16(dev(b["w_fp8"], d), dev(b["bs"], d), OCP)
    y = host(bsb.gemm_bf16(dev_bf16(b["x_d"], d), wb, out_dtype=torch.float32))
    y64, mag = gemm_bf16_ref(b["x_d"], dequant_fp8_block_bf16_ref(b["w_fp8"], b["bs"], OCP))
    _check(y, y64, mag, 7168, False)
