"""GPU parity: quantize_act, decode_fp8_block, decode_mxfp4 vs the oracle, bit-exact."""
import numpy as np
import pytest
import torch

import block_scaled_bit_amd as bsb
from block_scaled_bit_amd import synth
from oracle import quantize_act_ref, decode_fp8_block_ref, decode_mxfp4_ref
from oracle.decode import OCP, FNUZ
from tests.golden_io import keyed_blocks
from tests.gpu_util import require_gpu, dev, dev_bf16, host, say, Guarded

pytestmark = pytest.mark.gpu


def _quant_gpu(bits, d):
    M, K = bits.shape
    qg = Guarded((M, K), torch.int8, d)
    sg = Guarded((M,), torch.float32, d)
    bsb.quantize_act(dev_bf16(bits, d), q=qg.view, sa=sg.view)
    torch.cuda.synchronize()
    return qg.check(), sg.check()


def _assert_quant_equal(bits, d):
    q, s = _quant_gpu(bits, d)
    qr, sr = quantize_act_ref(bits)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32)), "scales differ"
    assert np.array_equal(q, qr), f"{np.sum(q != qr)} quantised values differ"


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill"])
def test_quantize_configs(name):
    d = require_gpu()
    cfg = synth.LINEAR_CONFIGS[name]
    say(f"quantize_act {name} M={cfg['M']} K={cfg['K']}")
    x = synth.activations(np.random.Generator(np.random.PCG64(0)), cfg["M"], cfg["K"],
                          cfg["outlier_p"], cfg["outlier_f"])
    _assert_quant_equal(x, d)


@pytest.mark.parametrize("M,K", [(1, 128), (3, 384), (5, 1152), (2, 7168), (7, 4096),
                                 (2, 16384), (3, 16512), (2, 40960)])
def test_quantize_shapes(M, K):
    """Every chunks-per-thread specialisation, ragged thread counts, the streaming path."""
    d = require_gpu()
    say(f"quantize_act M={M} K={K}")
    x = synth.activations(np.random.default_rng(M * K), M, K, 0.01, 20.0)
    _assert_quant_equal(x, d)


def test_quantize_golden_and_edge_rows():
    d = require_gpu()
    K = 256
    rows = []
    for blk in keyed_blocks("quant_cases.txt", ["x", "scale", "q"]):
        r = np.zeros(K, np.float32)
        v = np.array([float(t) for t in blk["x"]], np.float32)
        r[: len(v)] = v
        rows.append(r)
    rows.append(np.zeros(K, np.float32))                                   # all zero
    sub = np.zeros(K, np.float32)
    sub[:6] = [1e-37, -3e-38, 5e-38, 2.5e-39, 0.0, -1e-37]               # subnormal scale
    rows.append(sub)
    tiny = np.zeros(K, np.float32)
    tiny[:3] = [9.2e-41, -4.6e-41, 2.0e-40]                               # BF16 subnormals
    rows.append(tiny)
    rng = np.random.default_rng(3)
    for amax_mant in range(128, 256, 5):                                  # near-ties
        amax = np.float32(amax_mant) / 128.0
        scale = np.float32(amax / np.float32(127.0))
        r = np.zeros(K, np.float32)
        r[0] = amax
        r[1:121] = ((rng.integers(0, 127, 120) + 0.5) * scale).astype(np.float32)
        rows.append(r)
    bits = synth.to_bf16_bits(np.stack(rows))
    say(f"quantize_act golden/edge rows M={bits.shape[0]}")
    _assert_quant_equal(bits, d)
    q, s = _quant_gpu(bits, d)
    assert s[5] == 0.0 and not q[5].any()


def test_quantize_every_bf16_value():
    """All finite BF16 magnitudes as amax, each row holding a sweep of values below it."""
    d = require_gpu()
    rng = np.random.default_rng(11)
    mags = np.arange(1, 0x7F80, 37, dtype=np.uint32)           # finite positive BF16 codes
    K = 512
    rows = np.empty((len(mags), K), np.uint16)
    for i, m in enumerate(mags):
        lo = max(1, int(m) - 0x0600)                          # ~12 binades below amax
        vals = rng.integers(lo, int(m) + 1, K).astype(np.uint16)
        vals[0] = m
        sign = rng.integers(0, 2, K).astype(np.uint16) << 15
        rows[i] = vals | sign
    say(f"quantize_act BF16 sweep M={rows.shape[0]} K={K}")
    _assert_quant_equal(rows, d)


def test_quantize_empty_and_determinism():
    d = require_gpu()
    q, s = bsb.quantize_act(torch.empty((0, 256), dtype=torch.bfloat16, device=d))
    assert q.shape == (0, 256) and s.shape == (0,)
    x = synth.activations(np.random.default_rng(5), 64, 8192, 0.005, 30.0)
    xd = dev_bf16(x, d)
    outs = [tuple(host(t) for t in bsb.quantize_act(xd)) for _ in range(3)]
    for o in outs[1:]:
        assert np.array_equal(o[0], outs[0][0]) and np.array_equal(o[1], outs[0][1])


def _decode_fp8_gpu(w, bs, dialect, d):
    N, K = w.shape
    qg = Guarded((N, K), torch.int8, d)
    sg = Guarded((N, K // 128), torch.float32, d)
    bsb.decode_fp8_block(dev(w, d), dev(bs, d), dialect, qw=qg.view, sw=sg.view)
    torch.cuda.synchronize()
    return qg.check(), sg.check()


def test_decode_fp8_blockfmt_config_both_dialects():
    d = require_gpu()
    rng = np.random.Generator(np.random.PCG64(0))
    w, bs = synth.fp8_block_weights(rng, 4096, 7168)
    res = {}
    for dialect in (OCP, FNUZ):
        say(f"decode_fp8_block N=4096 K=7168 dialect={dialect}")
        q, s = _decode_fp8_gpu(w, bs, dialect, d)
        qr, sr = decode_fp8_block_ref(w, bs, dialect)
        assert np.array_equal(q, qr), f"{np.sum(q != qr)} INT8 values differ"
        assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))
        res[dialect] = (q, s)
    # same bytes, other dialect: identical INT8, scales exactly 2x
    assert np.array_equal(res[OCP][0], res[FNUZ][0])
    assert np.array_equal(res[OCP][1], (2 * res[FNUZ][1]).astype(np.float32))


@pytest.mark.parametrize("dialect", [OCP, FNUZ])
def test_decode_fp8_every_code_every_exponent(dialect):
    """Each 128x128 block holds every finite code; block exponents sweep 0..254."""
    d = require_gpu()
    N, K = 128 * 8, 128 * 32
    rng = np.random.default_rng(dialect)
    w = rng.choice(synth.FP8_CODES_FINITE_BOTH, size=(N, K))
    w[:, :253] = synth.FP8_CODES_FINITE_BOTH[None, :]
    # exponents 0..245: 448 * 2^(245-127) is the largest product still finite in float32
    bs = (np.arange(8 * 32).reshape(8, 32) % 246).astype(np.uint8)
    bs[0, 0] = 0                                            # subnormal block scale
    say(f"decode_fp8_block sweep dialect={dialect}")
    q, s = _decode_fp8_gpu(w, bs, dialect, d)
    qr, sr = decode_fp8_block_ref(w, bs, dialect)
    assert np.array_equal(q, qr) and np.array_equal(s.view(np.uint32), sr.view(np.uint32))


def test_decode_mxfp4_blockfmt_config():
    d = require_gpu()
    rng = np.random.Generator(np.random.PCG64(0))
    synth.fp8_block_weights(rng, 4096, 7168)                # same draw order as blockfmt_inputs
    packed, sc = synth.mxfp4_weights(rng, 8, 2048, 4096)
    say("decode_mxfp4 E=8 N=2048 K=4096")
    qg = Guarded((8, 2048, 4096), torch.int8, d)
    sg = Guarded((8, 2048, 32), torch.float32, d)
    bsb.decode_mxfp4(dev(packed, d), dev(sc, d), qw=qg.view, sw=sg.view)
    torch.cuda.synchronize()
    q, s = qg.check(), sg.check()
    qr, sr = decode_mxfp4_ref(packed, sc)
    assert np.array_equal(q, qr), f"{np.sum(q != qr)} INT8 values differ"
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))


def test_decode_mxfp4_all_exponents_small():
    d = require_gpu()
    rng = np.random.default_rng(9)
    packed = rng.integers(0, 256, size=(3, 5, 192), dtype=np.uint8)   # K = 384
    sc = rng.integers(0, 251, size=(3, 5, 12)).astype(np.uint8)        # 2^-127 .. 2^123 (finite)
    say("decode_mxfp4 exponent sweep")
    q, s = bsb.decode_mxfp4(dev(packed, d), dev(sc, d))
    qr, sr = decode_mxfp4_ref(packed, sc)
    assert np.array_equal(host(q), qr)
    assert np.array_equal(host(s).view(np.uint32), sr.view(np.uint32))
