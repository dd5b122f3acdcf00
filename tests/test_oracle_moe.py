"""Pins of the MoE glue oracle (quantise-then-gather, top-k weighted combine).

The combine is pinned against step-by-step exact rational arithmetic on small
random cases (a fused multiply-add is one rounding of the exact a*b + c; the
BF16 rounding is round-to-nearest-even at 8 significant bits), against the
single-slot identity and power-of-two scaling; the gather against the
per-row independence of the quantisation rule on the routed workload, and the
routing maps against the sort they invert.
"""
from fractions import Fraction

import numpy as np
import pytest

from block_scaled_bit_amd import synth
from oracle import (quantize_act_ref, gather_rows_ref, moe_combine_ref,
                    moe_combine_fp32_ordered_ref, bf16_bits_to_f32_ref)
from tests.exact import F, fma_f32, rint_half_even, _floor_log2


def round_bf16_bits(fr: Fraction) -> int:
    """Exact RN-even of a rational to BF16 (normal range), as 16-bit pattern."""
    if fr == 0:
        return 0
    sign = 0x8000 if fr < 0 else 0
    a = abs(fr)
    e = _floor_log2(a)
    quantum = Fraction(2) ** (max(e, -126) - 7)
    val = float(rint_half_even(a / quantum) * quantum)
    return sign | int(np.array([val], np.float32).view(np.uint32)[0] >> 16)


@pytest.fixture(scope="module")
def small_moe():
    return synth.moe_inputs(T=256, K=256, N=16, E=16, topk=4, seed=3)


def test_routing_maps_invert_the_sort(small_moe):
    m = small_moe
    rp, tor, ids, off = m["row_of_pair"], m["token_of_row"], m["topk_ids"], m["offsets"]
    T, topk = rp.shape
    assert sorted(rp.reshape(-1).tolist()) == list(range(m["R"]))
    for t in range(T):
        for k in range(topk):
            r = int(rp[t, k])
            assert tor[r] == t
            e = int(ids[t, k])
            assert off[e] <= r < off[e + 1]


def test_quantise_before_gather_is_bit_identical(small_moe):
    m = small_moe
    q_tok, sa_tok = quantize_act_ref(m["x_tokens"])
    q_g, sa_g = gather_rows_ref(q_tok, sa_tok, m["token_of_row"])
    q_s, sa_s = quantize_act_ref(m["x_sorted"])
    assert np.array_equal(q_g, q_s)
    assert np.array_equal(sa_g.view(np.uint32), sa_s.view(np.uint32))


def test_gate_weights_sum_to_one(small_moe):
    g = small_moe["gate"].astype(np.float64)
    assert np.all(g > 0) and np.allclose(g.sum(axis=1), 1.0, atol=1e-6)


def _random_case(rng, T, topk, R, N):
    y = synth.to_bf16_bits(rng.standard_normal((R, N)).astype(np.float32) * 3)
    rp = np.stack([rng.permutation(R)[:topk] for _ in range(T)]).astype(np.int32)
    gate = synth.gate_weights(rng, T, topk)
    return y, rp, gate


def test_combine_against_exact_steps():
    rng = np.random.default_rng(5)
    y, rp, gate = _random_case(rng, 6, 3, 9, 7)
    out64, mag = moe_combine_ref(y, rp, gate)
    out32, outb = moe_combine_fp32_ordered_ref(y, rp, gate)
    yf = bf16_bits_to_f32_ref(y)
    for t in range(6):
        for n in range(7):
            exact = sum(F(gate[t, k]) * F(yf[rp[t, k], n]) for k in range(3))
            assert abs(F(out64[t, n]) - exact) <= Fraction(1, 2 ** 50) * F(mag[t, n])
            acc = np.float32(0.0)
            for k in range(3):                  # k ascending, one rounding per step
                acc = fma_f32(gate[t, k], yf[rp[t, k], n], acc)
            assert out32[t, n].view(np.uint32) == np.float32(acc).view(np.uint32)
            assert int(outb[t, n]) == round_bf16_bits(F(acc))


def test_single_slot_unit_gate_returns_the_row():
    rng = np.random.default_rng(6)
    y, rp, _ = _random_case(rng, 10, 1, 12, 9)
    gate = np.ones((10, 1), np.float32)
    out32, outb = moe_combine_fp32_ordered_ref(y, rp, gate)
    assert np.array_equal(outb, y[rp[:, 0]])
    out64, _ = moe_combine_ref(y, rp, gate)
    assert np.array_equal(out64, bf16_bits_to_f32_ref(y[rp[:, 0]]).astype(np.float64))


def test_power_of_two_gate_scaling_is_exact():
    rng = np.random.default_rng(7)
    y, rp, gate = _random_case(rng, 8, 4, 20, 11)
    a32, _ = moe_combine_fp32_ordered_ref(y, rp, gate)
    b32, _ = moe_combine_fp32_ordered_ref(y, rp, (gate * 4).astype(np.float32))
    assert np.array_equal(b32, a32 * 4)
