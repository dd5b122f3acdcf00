"""Pins for the oracle's per-token INT8 quantisation (CPU only).

Each check rests on something other than the oracle's own NumPy code: hand
fixtures, an exact-rational re-computation with explicit rounding, and
invariants that follow from the rule's mathematics.
"""
import numpy as np
import pytest

from block_scaled_bit_amd import synth
from oracle import quantize_act_ref, quantize_rows_ref, bf16_bits_to_f32
from tests import exact
from tests.golden_io import keyed_blocks


def test_bf16_widening_matches_torch():
    import torch
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]            # finite codes
    ours = bf16_bits_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_golden_cases():
    n = 0
    for blk in keyed_blocks("quant_cases.txt", ["x", "scale", "q"]):
        x = np.array([float(v) for v in blk["x"]], np.float32)[None, :]
        bits = synth.to_bf16_bits(x)
        assert np.array_equal(bf16_bits_to_f32(bits), x)        # fixture exact in BF16
        q, s = quantize_act_ref(bits)
        assert s[0] == np.float32(float(blk["scale"][0]))
        assert q[0].tolist() == [int(v) for v in blk["q"]]
        n += 1
    assert n == 5


def test_tiny_config_against_exact_rationals():
    """Every element of the tiny workload, recomputed with Fractions + explicit RN-even."""
    d = synth.linear_config("tiny")
    q, s = quantize_act_ref(d["x"])
    x = bf16_bits_to_f32(d["x"])
    for m in range(x.shape[0]):
        qe, se = exact.quant_rule_exact(x[m].tolist())
        assert exact.f32_bits(se) == exact.f32_bits(s[m])
        assert q[m].tolist() == qe


def test_near_ties_against_exact_rationals():
    """Rows built so that many x/scale land within a few ulps of a .5 tie."""
    rng = np.random.default_rng(7)
    rows = []
    for amax_mant in range(128, 256, 3):                  # every 3rd BF16 mantissa of amax
        amax = np.float32(amax_mant) / 128.0
        scale = np.float32(amax / np.float32(127.0))
        k = rng.integers(0, 127, 60)
        cand = ((k + 0.5) * scale).astype(np.float32)     # near-ties before BF16 rounding
        row = np.concatenate([[amax], cand, -cand[:20], rng.standard_normal(47).astype(np.float32)])
        rows.append(row.astype(np.float32))
    bits = synth.to_bf16_bits(np.stack(rows))
    q, s = quantize_act_ref(bits)
    x = bf16_bits_to_f32(bits)
    for m in range(x.shape[0]):
        qe, se = exact.quant_rule_exact(x[m].tolist())
        assert exact.f32_bits(se) == exact.f32_bits(s[m])
        assert q[m].tolist() == qe


def test_subnormal_scale_row():
    """amax ~ 1e-37 gives a subnormal float32 scale; no flush to zero anywhere."""
    x = np.array([[1e-37, -3e-38, 5e-38, 2.5e-39, 0.0, -1e-37]], np.float32)
    bits = synth.to_bf16_bits(x)
    q, s = quantize_act_ref(bits)
    xb = bf16_bits_to_f32(bits)
    assert 0 < s[0] < np.finfo(np.float32).tiny                 # subnormal
    qe, se = exact.quant_rule_exact(xb[0].tolist())
    assert exact.f32_bits(se) == exact.f32_bits(s[0])
    assert q[0].tolist() == qe


def test_invariants_decode_shaped_rows():
    d = synth.linear_inputs(8, 8192, 1, outlier_p=0.005, outlier_f=30.0, seed=3)
    x = bf16_bits_to_f32(d["x"])
    q, s = quantize_act_ref(d["x"])
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    for m in range(x.shape[0]):
        i = int(np.argmax(np.abs(x[m])))
        assert abs(int(q[m, i])) == 127 and np.sign(q[m, i]) == np.sign(x[m, i])
        # half a step from rounding plus the float32 rounding of x/scale
        err = np.abs(x[m].astype(np.float64) - q[m].astype(np.float64) * np.float64(s[m]))
        assert np.all(err <= np.float64(s[m]) * (0.5 + 127 * 2.0 ** -24))


@pytest.mark.parametrize("j", [-20, -3, 1, 9])
def test_power_of_two_scaling(j):
    d = synth.linear_inputs(4, 1024, 1, outlier_p=0.01, outlier_f=20.0, seed=11)
    x = bf16_bits_to_f32(d["x"])
    q0, s0 = quantize_rows_ref(x)
    q1, s1 = quantize_rows_ref((x * np.float32(2.0 ** j)).astype(np.float32))
    assert np.array_equal(q0, q1)
    assert np.array_equal(s1, (s0 * np.float32(2.0 ** j)).astype(np.float32))


def test_rounding_is_half_even_not_half_away():
    # a rule that rounds half away from zero, or multiplies by a reciprocal, fails here
    x = np.array([[127.0, 2.5, 0.5, -2.5, 1.5]], np.float32)
    q, _ = quantize_act_ref(synth.to_bf16_bits(x))
    assert q[0].tolist() == [127, 2, 0, -2, 2]
