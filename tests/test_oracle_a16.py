"""Pins for the oracle's BF16-activation GEMMs (W8A16, BF16) and the FP8 -> BF16
dequantisation (CPU only)."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

from block_scaled_bit_amd import synth
from oracle import (gemm_w8a16_ref, gemm_bf16_ref, a16_tolerance, dequant_fp8_block_bf16_ref,
                    dequant_fp8_block_ref, gemm_ref, f32_to_bf16_bits_ref, bf16_bits_to_f32_ref)
from oracle.decode import OCP, FNUZ
from tests import exact


def _x_bits(rng, M, K):
    return synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))


def _qw(rng, N, K):
    return rng.integers(-127, 128, size=(N, K)).astype(np.int8)


def _sw(rng, N, G):
    return np.exp(rng.normal(-6.0, 0.5, size=(N, G))).astype(np.float32)


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (2, 3, 256), (3, 2, 384)])
def test_w8a16_against_fractions(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    xb, qw, sw = _x_bits(rng, M, K), _qw(rng, N, K), _sw(rng, N, K // 128)
    y, mag = gemm_w8a16_ref(xb, qw, sw)
    x = bf16_bits_to_f32_ref(xb)
    for m, n in itertools.product(range(M), range(N)):
        ex, em = Fraction(0), Fraction(0)
        for g in range(K // 128):
            s = sum(exact.F(x[m, k]) * int(qw[n, k]) for k in range(128 * g, 128 * g + 128))
            a = sum(abs(exact.F(x[m, k]) * int(qw[n, k])) for k in range(128 * g, 128 * g + 128))
            ex += s * exact.F(sw[n, g])
            em += a * exact.F(sw[n, g])
        assert abs(exact.F(y[m, n]) - ex) <= em * Fraction(1, 2 ** 48)
        assert abs(exact.F(mag[m, n]) - em) <= em * Fraction(1, 2 ** 48)


def test_w8a16_reduces_to_w8a8_when_x_is_q_times_a_power_of_two():
    """x[m,k] = q[m,k] * 2^-j is exact in BF16; then W8A16 is the W8A8 definition."""
    rng = np.random.default_rng(3)
    M, N, K = 4, 5, 512
    q = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    sa = (2.0 ** -rng.integers(3, 12, size=M)).astype(np.float32)
    xb = f32_to_bf16_bits_ref(q.astype(np.float32) * sa[:, None])
    assert np.array_equal(bf16_bits_to_f32_ref(xb), q.astype(np.float32) * sa[:, None])
    qw, sw = _qw(rng, N, K), _sw(rng, N, K // 128)
    y16, mag = gemm_w8a16_ref(xb, qw, sw)
    y8, mag8 = gemm_ref(q, sa, qw, sw)
    assert np.all(np.abs(y16 - y8) <= 1e-14 * mag)
    # W8A8's magnitude sums exact group totals, W8A16's every product: never smaller
    assert np.all(mag >= mag8 * (1 - 1e-14))


def test_bf16_reduces_to_w8a16_with_unit_scales():
    """INT8 values are exact in BF16: the BF16 GEMM of bf16(qw) is W8A16 with sw = 1."""
    rng = np.random.default_rng(4)
    M, N, K = 3, 6, 384
    xb, qw = _x_bits(rng, M, K), _qw(rng, N, K)
    wb = f32_to_bf16_bits_ref(qw.astype(np.float32))
    assert np.array_equal(bf16_bits_to_f32_ref(wb), qw.astype(np.float32))
    yb, mb = gemm_bf16_ref(xb, wb)
    yw, mw = gemm_w8a16_ref(xb, qw, np.ones((N, K // 128), np.float32))
    assert np.all(np.abs(yb - yw) <= 1e-14 * mb) and np.allclose(mb, mw, rtol=1e-14)


def test_integer_identity():
    rng = np.random.default_rng(5)
    M, N, K = 3, 4, 1024
    xi = rng.integers(-127, 128, size=(M, K))
    xb = f32_to_bf16_bits_ref(xi.astype(np.float32))
    qw = _qw(rng, N, K)
    y, _ = gemm_w8a16_ref(xb, qw, np.ones((N, K // 128), np.float32))
    assert np.array_equal(y, (xi @ qw.astype(np.int64).T).astype(np.float64))


@pytest.mark.parametrize("K", [128, 1024, 8192])
def test_tolerance_holds_for_float32_orders(K):
    """The stated bound covers float32 evaluation in different orders: products
    exact, group sums left to right or pairwise, then the group combine."""
    rng = np.random.default_rng(K)
    M, N = 4, 8
    xb, qw, sw = _x_bits(rng, M, K), _qw(rng, N, K), _sw(rng, N, K // 128)
    y64, mag = gemm_w8a16_ref(xb, qw, sw)
    x = bf16_bits_to_f32_ref(xb)
    t = a16_tolerance(K)
    for order in ("sequential", "pairwise"):
        acc = np.zeros((M, N), np.float32)
        for g in range(K // 128):
            prods = (x[:, None, 128 * g:128 * g + 128] *
                     qw[None, :, 128 * g:128 * g + 128].astype(np.float32))   # exact
            if order == "sequential":
                p = np.zeros((M, N), np.float32)
                for k in range(128):
                    p = (p + prods[:, :, k]).astype(np.float32)
            else:
                p = prods
                while p.shape[2] > 1:
                    p = (p[:, :, 0::2] + p[:, :, 1::2]).astype(np.float32)
                p = p[:, :, 0]
            from oracle import fmaf_ref
            acc = fmaf_ref(p, sw[:, g][None, :], acc)
        err = np.abs(acc.astype(np.float64) - y64)
        assert np.all(err <= t * mag), (order, float((err / mag).max()))


def test_mag_bounds_the_result():
    rng = np.random.default_rng(6)
    xb, qw, sw = _x_bits(rng, 5, 640), _qw(rng, 7, 640), _sw(rng, 7, 5)
    y, mag = gemm_w8a16_ref(xb, qw, sw)
    assert np.all(np.abs(y) <= mag * (1 + 1e-15))
    wb = f32_to_bf16_bits_ref(rng.standard_normal((7, 640)).astype(np.float32))
    y, mag = gemm_bf16_ref(xb, wb)
    assert np.all(np.abs(y) <= mag * (1 + 1e-15))


def test_fp8_to_bf16_dequant_is_exact_and_dialects_differ_by_two():
    """Normal-range block values have at most 4 significant bits: exact in BF16. The
    same bytes read as OCP are twice the fnuz values, bit for bit after rounding."""
    rng = np.random.default_rng(7)
    b = synth.blockfmt_inputs(M=1, N_d=256, K_d=384, E=1, N_e=128, K_e=128)
    w, bs = b["w_fp8"], b["bs"]
    for d in (OCP, FNUZ):
        wb = dequant_fp8_block_bf16_ref(w, bs, d)
        assert np.array_equal(bf16_bits_to_f32_ref(wb), dequant_fp8_block_ref(w, bs, d))
    ocp = bf16_bits_to_f32_ref(dequant_fp8_block_bf16_ref(w, bs, OCP))
    fnuz = bf16_bits_to_f32_ref(dequant_fp8_block_bf16_ref(w, bs, FNUZ))
    assert np.array_equal(ocp, 2 * fnuz)


def test_fp8_to_bf16_rounds_subnormal_values_to_nearest_even():
    """A block exponent low enough to make the value a BF16 subnormal rounds it to
    nearest even, as the exact rational rounding does."""
    w = np.full((128, 128), 0x3F, np.uint8)            # OCP e4m3 1.875
    w[0, 1] = 0x39                                      # 1.125
    bs = np.array([[1]], np.uint8)                      # 2^-126: 1.875 * 2^-126 normal
    f = dequant_fp8_block_ref(w, bs, OCP)
    bs0 = np.array([[0]], np.uint8)                     # 2^-127: subnormal
    f0 = dequant_fp8_block_ref(w, bs0, OCP)
    wb0 = dequant_fp8_block_bf16_ref(w, bs0, OCP)
    for v, bits in ((f0[0, 0], wb0[0, 0]), (f0[0, 1], wb0[0, 1])):
        r = exact.round_f32(exact.F(v))                 # exact in float32 (subnormal range)
        assert float(r) == float(v)
        # BF16 subnormal quantum 2^-133: round the exact value to a multiple of it
        q = Fraction(2) ** -133
        n = exact.rint_half_even(exact.F(v) / q)
        assert float(bf16_bits_to_f32_ref(np.array([bits], np.uint16))[0]) == float(n * q)
    assert np.array_equal(bf16_bits_to_f32_ref(dequant_fp8_block_bf16_ref(w, bs, OCP)), f)


def test_tolerance_covers_a_worst_case_sum():
    """127 terms just under half an ulp of 1 after a leading 1: left-to-right float32
    addition drops every one of them, an error of ~127 * 2^-24 * mag, which the
    bound must (and does) cover."""
    K = 128
    d = np.float32(2.0 ** -24 * (1 - 2.0 ** -8))          # exact in BF16
    x = np.full((1, K), d, np.float32)
    x[0, 0] = 1.0
    xb = f32_to_bf16_bits_ref(x)
    assert np.array_equal(bf16_bits_to_f32_ref(xb), x)
    qw = np.ones((1, K), np.int8)
    y64, mag = gemm_w8a16_ref(xb, qw, np.ones((1, 1), np.float32))
    p = np.float32(0)
    for k in range(K):
        p = np.float32(p + x[0, k])
    err = abs(float(p) - y64[0, 0])
    assert err > 120 * 2.0 ** -24 * mag[0, 0]
    assert err <= a16_tolerance(K) * mag[0, 0]


def test_fp8_to_bf16_rounds_below_the_bf16_subnormal_quantum():
    """Block exponent 0 on small FP8 codes: values between BF16 subnormals (2^-133
    apart) round to nearest even, ties included; below 2^-134 they go to zero."""
    w = np.zeros((128, 128), np.uint8)
    codes = [0x1F, 0x1B, 0x19, 0x0F, 0x01, 0x02, 0x03]
    w[0, :len(codes)] = codes
    bs = np.zeros((1, 1), np.uint8)
    f = dequant_fp8_block_ref(w, bs, OCP)
    wb = dequant_fp8_block_bf16_ref(w, bs, OCP)
    got = bf16_bits_to_f32_ref(wb)
    q = Fraction(2) ** -133
    for j in range(len(codes)):
        v = exact.F(f[0, j])
        assert float(exact.round_f32(v)) == float(f[0, j])          # exact in float32
        assert float(got[0, j]) == float(exact.rint_half_even(v / q) * q), hex(codes[j])
