"""Pins for the oracle's grouped (MoE) GEMM (CPU only)."""
import numpy as np
import pytest

from block_scaled_bit_amd import synth
from oracle import (quantize_act_ref, gemm_ref, gemm_fp32_ordered_ref, grouped_gemm_ref,
                    grouped_gemm_fp32_ordered_ref)


def _grouped_case(lengths, N=24, K=256, seed=0):
    rng = np.random.default_rng(seed)
    E = len(lengths)
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(lengths)
    R = int(off[-1])
    x = synth.activations(rng, R, K, 0.01, 20.0)
    q, sa = quantize_act_ref(x)
    qw = rng.integers(-127, 128, size=(E, N, K)).astype(np.int8)
    sw = np.exp(rng.normal(-6, 0.5, size=(E, N, K // 128))).astype(np.float32)
    return q, sa, qw, sw, off


def test_single_expert_equals_dense():
    q, sa, qw, sw, off = _grouped_case([37])
    y64, mag = grouped_gemm_ref(q, sa, qw, sw, off)
    y32, yb = grouped_gemm_fp32_ordered_ref(q, sa, qw, sw, off)
    d64, dmag = gemm_ref(q, sa, qw[0], sw[0])
    d32, db = gemm_fp32_ordered_ref(q, sa, qw[0], sw[0])
    assert np.array_equal(y64, d64) and np.array_equal(mag, dmag)
    assert np.array_equal(y32, d32) and np.array_equal(yb, db)


@pytest.mark.parametrize("lengths", [[0, 1, 127, 128, 129, 0], [5, 0, 0, 3], [0, 0, 64]])
def test_concatenation_of_dense_calls(lengths):
    q, sa, qw, sw, off = _grouped_case(lengths, seed=len(lengths))
    y32, yb = grouped_gemm_fp32_ordered_ref(q, sa, qw, sw, off)
    assert y32.shape[0] == sum(lengths)
    for e in range(len(lengths)):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        d32, db = gemm_fp32_ordered_ref(q[lo:hi], sa[lo:hi], qw[e], sw[e])
        assert np.array_equal(y32[lo:hi], d32) and np.array_equal(yb[lo:hi], db)


def test_brute_force_segments():
    q, sa, qw, sw, off = _grouped_case([2, 0, 3], N=3, K=128, seed=3)
    y64, _ = grouped_gemm_ref(q, sa, qw, sw, off)
    for e in range(3):
        for r in range(off[e], off[e + 1]):
            for n in range(3):
                P = sum(int(q[r, k]) * int(qw[e, n, k]) for k in range(128))
                assert y64[r, n] == float(sa[r]) * (float(sw[e, n, 0]) * P)


def test_row_permutation_within_segment():
    q, sa, qw, sw, off = _grouped_case([9, 14], seed=4)
    perm = np.concatenate([np.random.default_rng(0).permutation(9),
                           9 + np.random.default_rng(1).permutation(14)])
    y32, yb = grouped_gemm_fp32_ordered_ref(q, sa, qw, sw, off)
    yp32, ypb = grouped_gemm_fp32_ordered_ref(q[perm], sa[perm], qw, sw, off)
    assert np.array_equal(yp32, y32[perm]) and np.array_equal(ypb, yb[perm])


def test_expert_weights_are_not_mixed():
    """Swapping two experts' weights changes exactly their segments."""
    q, sa, qw, sw, off = _grouped_case([6, 7, 8], seed=5)
    y64, _ = grouped_gemm_ref(q, sa, qw, sw, off)
    qw2, sw2 = qw[[1, 0, 2]], sw[[1, 0, 2]]
    z64, _ = grouped_gemm_ref(q, sa, qw2, sw2, off)
    assert np.array_equal(y64[13:], z64[13:])
    assert not np.array_equal(y64[:6], z64[:6]) and not np.array_equal(y64[6:13], z64[6:13])


def test_moe_router_structure():
    d = synth.moe_inputs(T=512, K=256, N=16, E=64, seed=0)
    off = d["offsets"]
    counts = np.diff(off)
    assert off[0] == 0 and off[-1] == 512 * 8 and np.all(counts >= 0)
    assert np.sum(counts == 0) >= 4                     # zero-weight experts stay empty
    # each token appears in exactly 8 distinct experts
    for t in range(0, 512, 37):
        ex = np.searchsorted(off, np.nonzero(d["token_of_row"] == t)[0], side="right") - 1
        assert len(set(ex.tolist())) == 8
    with pytest.raises(ValueError):
        grouped_gemm_ref(np.zeros((2, 128), np.int8), np.ones(2, np.float32),
                         np.zeros((2, 4, 128), np.int8), np.ones((2, 4, 1), np.float32),
                         np.array([0, 2, 1], np.int32))
