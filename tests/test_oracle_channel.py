"""Pins for the oracle's per-channel / per-tensor W8A8 GEMM (CPU only)."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle import (channel_total_ref, gemm_channel_ref, gemm_channel_fp32_ordered_ref,
                    gemm_ref, f32_to_bf16_bits_ref)
from tests import exact


def _rand_q(rng, shape):
    return rng.integers(-127, 128, size=shape).astype(np.int8)


def _scales(rng, n):
    return rng.lognormal(-6.0, 0.5, size=n).astype(np.float32)


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (3, 5, 256), (4, 3, 384), (2, 7, 1024)])
def test_brute_force_against_fractions(M, N, K):
    """The INT32 total by Python integers, each float32 step by an exact rational
    rounded to nearest even: bit-identical to the ordered form; the float64
    definition within float64 rounding of the exact product."""
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    q, qw = _rand_q(rng, (M, K)), _rand_q(rng, (N, K))
    q[0, :7] = 127
    qw[0, :7] = -127
    sa = (rng.random(M).astype(np.float32) + np.float32(0.5)) / np.float32(127)
    sw = _scales(rng, N)
    y32, yb = gemm_channel_fp32_ordered_ref(q, sa, qw, sw)
    y64, _ = gemm_channel_ref(q, sa, qw, sw)
    P = channel_total_ref(q, qw)
    for m, n in itertools.product(range(M), range(N)):
        p = sum(int(q[m, k]) * int(qw[n, k]) for k in range(K))
        assert int(P[m, n]) == p
        pf = exact.round_f32(Fraction(p))
        t = exact.round_f32(exact.F(pf) * exact.F(sw[n]))
        y = exact.round_f32(exact.F(t) * exact.F(sa[m]))
        assert exact.f32_bits(y32[m, n]) == exact.f32_bits(y)
        ex = Fraction(p) * exact.F(sw[n]) * exact.F(sa[m])
        assert abs(exact.F(y64[m, n]) - ex) <= abs(ex) * Fraction(1, 2 ** 51)
    assert np.array_equal(yb, f32_to_bf16_bits_ref(y32))


def test_integer_identity_and_total_rounding():
    """Unit scales: y is the integer matmul, rounded once to float32 where the
    total needs more than 24 bits (|P| up to 127^2 * 4096 > 2^24 here)."""
    rng = np.random.default_rng(5)
    K = 4096
    q, qw = _rand_q(rng, (6, K)), _rand_q(rng, (5, K))
    q[0], qw[0] = 127, 127                      # P[0,0] = 127^2 * 4096, > 2^24
    q[1], qw[1] = 127, -127
    ones = np.ones(6, np.float32)
    y32, _ = gemm_channel_fp32_ordered_ref(q, ones, qw, np.ones(5, np.float32))
    P = q.astype(np.int64) @ qw.astype(np.int64).T
    assert abs(int(P[0, 0])) > 2 ** 24
    for m, n in itertools.product(range(6), range(5)):
        assert exact.f32_bits(y32[m, n]) == exact.f32_bits(exact.round_f32(Fraction(int(P[m, n]))))
    y64, _ = gemm_channel_ref(q, ones, qw, np.ones(5, np.float32))
    assert np.array_equal(y64, P.astype(np.float64))


def test_accumulator_bound_at_k_max():
    """K = 131072, every product 127^2 of one sign: the total 2,114,060,288 still
    fits INT32; one more group would not, and the oracle refuses it."""
    K = 131072
    q = np.full((1, K), 127, np.int8)
    qw = np.full((2, K), 127, np.int8)
    qw[1] = -127
    P = channel_total_ref(q, qw)
    assert int(P[0, 0]) == 127 * 127 * K == 2114060288 < 2 ** 31
    assert int(P[0, 1]) == -2114060288
    with pytest.raises(ValueError):
        gemm_channel_ref(np.zeros((1, K + 128), np.int8), np.ones(1, np.float32),
                         np.zeros((1, K + 128), np.int8), np.ones(1, np.float32))


def test_per_group_form_with_equal_group_scales():
    """Special case: per-group scales that are equal along a row give the
    per-channel value (float64 definitions of the two forms agree)."""
    rng = np.random.default_rng(9)
    M, N, K = 5, 6, 1024
    q, qw = _rand_q(rng, (M, K)), _rand_q(rng, (N, K))
    sa = _scales(rng, M)
    swn = _scales(rng, N)
    y_ch, _ = gemm_channel_ref(q, sa, qw, swn)
    y_pg, mag = gemm_ref(q, sa, qw, np.repeat(swn[:, None], K // 128, axis=1))
    assert np.all(np.abs(y_ch - y_pg) <= 1e-13 * mag)


def test_per_tensor_is_per_channel_with_one_scale():
    rng = np.random.default_rng(11)
    q, qw = _rand_q(rng, (3, 256)), _rand_q(rng, (4, 256))
    sa = _scales(rng, 3)
    s = np.float32(0.0123)
    a = gemm_channel_fp32_ordered_ref(q, sa, qw, np.array([s], np.float32))
    b = gemm_channel_fp32_ordered_ref(q, sa, qw, np.full(4, s, np.float32))
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))


@pytest.mark.parametrize("j", [-3, 1, 4])
def test_power_of_two_scaling_is_exact(j):
    """Scaling sw or sa by 2^j scales every float32 step by 2^j exactly."""
    rng = np.random.default_rng(13 + j)
    q, qw = _rand_q(rng, (4, 512)), _rand_q(rng, (5, 512))
    sa, sw = _scales(rng, 4), _scales(rng, 5)
    y, _ = gemm_channel_fp32_ordered_ref(q, sa, qw, sw)
    f = np.float32(2.0 ** j)
    y_w, _ = gemm_channel_fp32_ordered_ref(q, sa, qw, sw * f)
    y_a, _ = gemm_channel_fp32_ordered_ref(q, sa * f, qw, sw)
    assert np.array_equal(y_w, y * f) and np.array_equal(y_a, y * f)


def test_operands_not_transposed():
    """A row of q meets a row of qw: a one-hot q row picks one column of qw."""
    K = 256
    q = np.zeros((2, K), np.int8)
    q[0, 3], q[1, 200] = 1, 1
    qw = np.arange(3 * K, dtype=np.int64).reshape(3, K) % 255 - 127
    qw = qw.astype(np.int8)
    P = channel_total_ref(q, qw)
    assert np.array_equal(P[0], qw[:, 3].astype(np.int64))
    assert np.array_equal(P[1], qw[:, 200].astype(np.int64))
