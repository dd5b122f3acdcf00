"""Pins for the oracle's FP8-block and MXFP4 decoders (CPU only).

Independent references: torch's float8_e4m3fn / float8_e4m3fnuz /
float8_e8m0fnu casts, transformers' MXFP4 dequantiser (value table, nibble
order and UE8M0 scaling of the MXFP4 checkpoints it loads), hand fixtures, and
exact-rational re-computation of the requantisation.
"""
import numpy as np
import pytest
import torch

from block_scaled_bit_amd import synth
from oracle import (fp8_e4m3_table, ue8m0_value, e2m1_table, decode_fp8_block_ref,
                    dequant_fp8_block_ref, decode_mxfp4_ref, dequant_mxfp4_ref)
from oracle.decode import OCP, FNUZ
from tests import exact
from tests.golden_io import table, parse_float


def _torch_decode(dtype):
    return torch.arange(256, dtype=torch.uint8).view(dtype).double().numpy()


@pytest.mark.parametrize("dialect,dtype", [(OCP, torch.float8_e4m3fn), (FNUZ, torch.float8_e4m3fnuz)])
def test_fp8_table_against_torch(dialect, dtype):
    ours, ref = fp8_e4m3_table(dialect), _torch_decode(dtype)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))   # -0 only in OCP


def test_fp8_golden_spot_values():
    ocp, fnuz = fp8_e4m3_table(OCP), fp8_e4m3_table(FNUZ)
    rows = table("fp8_e4m3_spot.txt")
    assert len(rows) == 13
    for b, vo, vf in rows:
        b = int(b, 16)
        for got, want in ((ocp[b], parse_float(vo)), (fnuz[b], parse_float(vf))):
            if np.isnan(want):
                assert np.isnan(got)
            else:
                assert got == want and np.signbit(got) == np.signbit(want)


def test_ocp_is_twice_fnuz_on_all_shared_codes():
    ocp, fnuz = fp8_e4m3_table(OCP), fp8_e4m3_table(FNUZ)
    codes = synth.FP8_CODES_FINITE_BOTH
    assert len(codes) == 253
    assert np.array_equal(ocp[codes], 2.0 * fnuz[codes])


def test_ue8m0_against_torch():
    ref = _torch_decode(torch.float8_e8m0fnu)
    ours = ue8m0_value(np.arange(256))
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])


def test_e2m1_table_golden_and_transformers():
    from transformers.integrations.mxfp4 import FP4_VALUES
    ours = e2m1_table()
    rows = table("e2m1_values.txt")
    want = np.array([float(v) for _, v in rows])
    assert np.array_equal(ours, want) and np.array_equal(np.signbit(ours), np.signbit(want))
    assert np.array_equal(ours, np.array(FP4_VALUES, np.float64))


def test_mxfp4_dequant_against_transformers():
    """Nibble order, block size 32 and 2^(E-127) scaling as in transformers' loader."""
    from transformers.integrations.mxfp4 import _convert_moe_packed_tensors
    rng = np.random.default_rng(0)
    E, N, K = 2, 8, 256
    packed, sc = synth.mxfp4_weights(rng, E, N, K)
    ours = dequant_mxfp4_ref(packed, sc)
    blocks = torch.from_numpy(packed.reshape(E, N, K // 32, 16))
    ref = _convert_moe_packed_tensors(blocks, torch.from_numpy(sc), dtype=torch.float32)
    ref = ref.transpose(1, 2).contiguous().numpy()          # helper returns [E, K, N]
    assert np.array_equal(ours, ref)


def test_fp8_dequant_against_torch():
    rng = np.random.default_rng(1)
    w, bs = synth.fp8_block_weights(rng, 256, 384)
    for dialect, dtype in ((OCP, torch.float8_e4m3fn), (FNUZ, torch.float8_e4m3fnuz)):
        ours = dequant_fp8_block_ref(w, bs, dialect)
        v = torch.from_numpy(w).view(dtype).float()
        e = torch.from_numpy(bs.astype(np.int32) - 127).repeat_interleave(128, 0).repeat_interleave(128, 1)
        ref = torch.ldexp(v, e.float()).numpy()
        assert np.array_equal(ours, ref)


def test_fp8_dialects_same_q_twice_scale():
    rng = np.random.default_rng(2)
    w, bs = synth.fp8_block_weights(rng, 256, 512)
    qo, so = decode_fp8_block_ref(w, bs, OCP)
    qf, sf = decode_fp8_block_ref(w, bs, FNUZ)
    assert np.array_equal(qo, qf)
    assert np.array_equal(so, (2 * sf).astype(np.float32))


def test_fp8_q_independent_of_block_exponent():
    rng = np.random.default_rng(3)
    w, bs = synth.fp8_block_weights(rng, 128, 256)
    q0, s0 = decode_fp8_block_ref(w, bs, OCP)
    bs2 = (bs.astype(np.int32) + np.array([[3, -5]])).astype(np.uint8)
    q1, s1 = decode_fp8_block_ref(w, bs2, OCP)
    assert np.array_equal(q0, q1)
    assert np.array_equal(s1[:, 0], (s0[:, 0] * np.float32(8)).astype(np.float32))
    assert np.array_equal(s1[:, 1], (s0[:, 1] / np.float32(32)).astype(np.float32))


def test_requant_against_exact_rationals():
    rng = np.random.default_rng(4)
    w, bs = synth.fp8_block_weights(rng, 128, 256)
    W = dequant_fp8_block_ref(w, bs, OCP)
    q, s = decode_fp8_block_ref(w, bs, OCP)
    for n in range(0, 128, 9):
        for g in range(2):
            qe, se = exact.quant_rule_exact(W[n, 128 * g:128 * (g + 1)].tolist())
            assert exact.f32_bits(se) == exact.f32_bits(s[n, g])
            assert q[n, 128 * g:128 * (g + 1)].tolist() == qe
    packed, sc = synth.mxfp4_weights(rng, 1, 16, 256)
    Wm = dequant_mxfp4_ref(packed, sc)
    qm, sm = decode_mxfp4_ref(packed, sc)
    for n in range(16):
        for g in range(2):
            qe, se = exact.quant_rule_exact(Wm[0, n, 128 * g:128 * (g + 1)].tolist())
            assert exact.f32_bits(se) == exact.f32_bits(sm[0, n, g])
            assert qm[0, n, 128 * g:128 * (g + 1)].tolist() == qe


def test_mxfp4_every_code_every_exponent():
    """All 16 codes under every block exponent in [-8, 4], one 128-group per (exponent set)."""
    codes = np.arange(128, dtype=np.uint8) % 16
    packed_row = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    for e0 in range(-8, 5):
        for spread in (0, 3, 12):
            exps = [e0, e0, min(4, e0 + spread), e0]
            packed = packed_row[None, None, :]
            sc = np.array([[[127 + e for e in exps]]], np.uint8)
            W = dequant_mxfp4_ref(packed, sc)
            q, s = decode_mxfp4_ref(packed, sc)
            qe, se = exact.quant_rule_exact(W[0, 0].tolist())
            assert exact.f32_bits(se) == exact.f32_bits(s[0, 0, 0])
            assert q[0, 0].tolist() == qe
            if spread == 0:      # equal exponents: q independent of the exponent
                q_ref = decode_mxfp4_ref(packed, np.full_like(sc, 127))[0]
                assert np.array_equal(q, q_ref)


def test_mxfp4_tie_case_rounds_to_even():
    """Value 3 next to a group maximum 6: fl32(3 / fl32(6/127)) is exactly 63.5, so q = 64."""
    s = np.float32(np.float32(6.0) / np.float32(127.0))
    t = exact.round_f32(exact.F(3.0) / exact.F(s))
    assert t == np.float32(63.5)
    codes = np.zeros(128, np.uint8)
    codes[0], codes[1] = 7, 5                      # 6.0 and 3.0
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)[None, None, :]
    q, _ = decode_mxfp4_ref(packed, np.full((1, 1, 4), 127, np.uint8))
    assert q[0, 0, 0] == 127 and q[0, 0, 1] == 64


@pytest.mark.parametrize("dialect", [OCP, FNUZ])
def test_subnormal_group_scale_and_clamp(dialect):
    """Block exponent byte 0 puts group maxima near 2^-136: the float32 scale amax/127 is
    subnormal with few significant bits, so the argmax need not map to 127. In the fnuz
    reading the smallest code gives x/scale = 128 exactly, and only the symmetric clamp
    keeps q at +-127 (never -128)."""
    w = np.zeros((128, 128), np.uint8)
    w[0, 0] = 0x81                       # -(smallest subnormal) in both dialects
    w[0, 1] = 0x01
    w[1, :3] = [0x02, 0x81, 0x83]
    bs = np.zeros((1, 1), np.uint8)      # 2^-127
    Wd = dequant_fp8_block_ref(w, bs, dialect)
    q, s = decode_fp8_block_ref(w, bs, dialect)
    for n in (0, 1):
        qe, se = exact.quant_rule_exact(Wd[n].tolist())
        assert exact.f32_bits(se) == exact.f32_bits(s[n, 0]) and 0 < s[n, 0] < 1e-38
        assert q[n].tolist() == qe
    if dialect == FNUZ:
        raw = exact.round_f32(exact.F(Wd[0, 0]) / exact.F(s[0, 0]))
        assert raw == -128.0                  # unclamped value would be -128
        assert q[0, 0] == -127 and q[0, 1] == 127
    else:
        assert q[0, 0] == -126 and q[0, 1] == 126     # scale rounded up: 127*64.5/65
