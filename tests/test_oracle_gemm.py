"""Pins for the oracle's W8A8 per-group-128 GEMM (CPU only)."""
import itertools

import numpy as np
import pytest

from block_scaled_bit_amd import synth
from oracle import (quantize_act_ref, group_partials_ref, gemm_ref, gemm_fp32_ordered_ref,
                    fmaf_ref, f32_to_bf16_bits_ref, bf16_bits_to_f32_ref)
from tests import exact
from tests.golden_io import keyed_blocks, sparse_row

G128 = 128


def _rand_q(rng, shape):
    return rng.integers(-127, 128, size=shape).astype(np.int8)


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (3, 5, 128), (7, 2, 256), (8, 8, 256), (2, 6, 384)])
def test_partials_brute_force(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    q, qw = _rand_q(rng, (M, K)), _rand_q(rng, (N, K))
    q[0, :5] = 127
    qw[0, :5] = -127                                  # extreme products
    P = group_partials_ref(q, qw)
    assert P.shape == (M, N, K // G128)
    for m, n, g in itertools.product(range(M), range(N), range(K // G128)):
        s = 0
        for k in range(G128 * g, G128 * (g + 1)):
            s += int(q[m, k]) * int(qw[n, k])
        assert int(P[m, n, g]) == s


def test_partials_bound_and_extremes():
    q = np.full((2, 256), 127, np.int8)
    qw = np.full((3, 256), -127, np.int8)
    P = group_partials_ref(q, qw)
    assert np.all(P == -128 * 127 * 127)


def test_integer_identity():
    """Integer activations with a +-127 per row and unit scales: y is the exact integer matmul."""
    import torch
    rng = np.random.default_rng(5)
    M, N, K = 6, 40, 1024
    xi = rng.integers(-127, 128, size=(M, K)).astype(np.float32)
    xi[np.arange(M), rng.integers(0, K, M)] = np.where(rng.random(M) < 0.5, 127.0, -127.0)
    bits = synth.to_bf16_bits(xi)
    assert np.array_equal(bf16_bits_to_f32_ref(bits), xi)
    q, sa = quantize_act_ref(bits)
    assert np.all(sa == 1.0) and np.array_equal(q.astype(np.float32), xi)
    qw = _rand_q(rng, (N, K))
    sw = np.ones((N, K // G128), np.float32)
    exact_int = q.astype(np.int64) @ qw.astype(np.int64).T
    y64, mag = gemm_ref(q, sa, qw, sw)
    y32, yb = gemm_fp32_ordered_ref(q, sa, qw, sw)
    assert np.array_equal(y64, exact_int.astype(np.float64))
    assert np.array_equal(y32.astype(np.int64), exact_int)
    ref_b = torch.from_numpy(exact_int.astype(np.float32)).to(torch.bfloat16).view(torch.int16)
    assert np.array_equal(yb, ref_b.numpy().view(np.uint16))


def test_golden_small_gemm():
    n = 0
    for blk in keyed_blocks("gemm_small.txt", ["K", "x", "qw", "sw", "y32", "ybf16"]):
        K = int(blk["K"][0])
        x = sparse_row(blk["x"], K, np.float32)[None, :]
        qw = sparse_row(blk["qw"], K).astype(np.int8)[None, :]
        sw = np.array([float(v) for v in blk["sw"]], np.float32)[None, :]
        q, sa = quantize_act_ref(synth.to_bf16_bits(x))
        y64, _ = gemm_ref(q, sa, qw, sw)
        y32, yb = gemm_fp32_ordered_ref(q, sa, qw, sw)
        assert y64[0, 0] == float(blk["y32"][0])
        assert y32[0, 0] == np.float32(float(blk["y32"][0]))
        assert bf16_bits_to_f32_ref(yb)[0, 0] == np.float32(float(blk["ybf16"][0]))
        n += 1
    assert n == 3


@pytest.mark.parametrize("M,N,K", [(2, 3, 128), (4, 3, 384), (3, 5, 256)])
def test_reference_and_ordered_against_fractions(M, N, K):
    """Exact y with Fractions; sequential float32 replay with explicit rounding."""
    d = synth.linear_inputs(M, K, N, outlier_p=0.05, outlier_f=20.0, seed=M + N + K)
    q, sa = quantize_act_ref(d["x"])
    qw, sw = d["qw"], d["sw"]
    y64, mag = gemm_ref(q, sa, qw, sw)
    y32, yb = gemm_fp32_ordered_ref(q, sa, qw, sw)
    G = K // G128
    for m in range(M):
        for n in range(N):
            P = [sum(int(q[m, k]) * int(qw[n, k]) for k in range(G128 * g, G128 * (g + 1)))
                 for g in range(G)]
            yex = exact.F(sa[m]) * sum(exact.F(sw[n, g]) * P[g] for g in range(G))
            assert abs(exact.F(y64[m, n]) - yex) <= exact.F(mag[m, n]) * exact.F(2.0 ** -50)
            acc = np.float32(0)
            for g in range(G):
                acc = exact.fma_f32(np.float32(P[g]), sw[n, g], acc)
            want = exact.round_f32(exact.F(acc) * exact.F(sa[m]))
            assert exact.f32_bits(want) == exact.f32_bits(y32[m, n])


def test_fmaf_against_fractions():
    rng = np.random.default_rng(1)
    a = rng.standard_normal(4000).astype(np.float32) * np.float32(1000)
    b = np.exp(rng.normal(-6, 3, 4000)).astype(np.float32)
    c = (rng.standard_normal(4000) * 10).astype(np.float32)
    # adversarial: a*b exactly half an ulp of c away, and tiny a*b next to large c
    c[:500] = np.float32(1.0)
    a[:500] = np.float32(1.0)
    b[:500] = np.float32(2.0 ** -24) * np.where(np.arange(500) % 2 == 0, 1, 3).astype(np.float32)
    a[500:1000] = np.float32(1.0) + np.float32(2.0 ** -23)
    b[500:1000] = np.float32(2.0 ** -25)
    got = fmaf_ref(a, b, c)
    for i in range(len(a)):
        assert exact.f32_bits(got[i]) == exact.f32_bits(exact.fma_f32(a[i], b[i], c[i])), i


def test_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(2)
    y = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(1e3),
        # exact ties: low 16 bits == 0x8000, both parities of bit 16
        (np.arange(2000, dtype=np.uint32) << np.uint32(16) | np.uint32(0x3F808000)).view(np.float32),
        np.array([0.0, -0.0, 1e-40, -3e-39, 3.0e38], np.float32),
    ])
    ours = f32_to_bf16_bits_ref(y)
    ref = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("j", [-7, 1, 5])
def test_power_of_two_weight_scaling(j):
    d = synth.linear_inputs(5, 512, 33, seed=9)
    q, sa = quantize_act_ref(d["x"])
    y32, yb = gemm_fp32_ordered_ref(q, sa, d["qw"], d["sw"])
    y32j, ybj = gemm_fp32_ordered_ref(q, sa, d["qw"], (d["sw"] * np.float32(2.0 ** j)).astype(np.float32))
    assert np.array_equal(y32j, (y32 * np.float32(2.0 ** j)).astype(np.float32))
    assert np.array_equal(bf16_bits_to_f32_ref(ybj), bf16_bits_to_f32_ref(yb) * np.float32(2.0 ** j))


def test_ordered_within_float32_bound_of_reference():
    d = synth.linear_inputs(16, 2048, 96, outlier_p=0.01, outlier_f=20.0, seed=4)
    q, sa = quantize_act_ref(d["x"])
    y64, mag = gemm_ref(q, sa, d["qw"], d["sw"])
    y32, _ = gemm_fp32_ordered_ref(q, sa, d["qw"], d["sw"])
    G = 2048 // G128
    assert np.all(np.abs(y32.astype(np.float64) - y64) <= (G + 1) * 2.0 ** -24 * mag + 1e-300)


def test_operands_not_transposed():
    """Distinct M, N, K so a swapped operand or a wrong group index changes the answer."""
    rng = np.random.default_rng(12)
    q, qw = _rand_q(rng, (3, 256)), _rand_q(rng, (5, 256))
    sa = np.array([1.0, 2.0, 4.0], np.float32)
    sw = np.array([[1.0, 0.0]] * 5, np.float32)          # only group 0 counts
    y64, _ = gemm_ref(q, sa, qw, sw)
    want = (q[:, :128].astype(np.int64) @ qw[:, :128].astype(np.int64).T) * sa[:, None]
    assert np.array_equal(y64, want.astype(np.float64))
