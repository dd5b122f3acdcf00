"""GPU parity: the per-channel / per-tensor W8A8 GEMM vs the oracle.

FP32 outputs within 1e-5 of |y| of the float64 definition and BF16 outputs
within one BF16 ulp, both also bit-identical to the oracle's float32 steps
((float)P, times the weight scale, then the activation scale). Every kernel
runs the form: small-M (narrow and wide workgroups), 128x128 tiles and 256x256
tiles, with ragged edges, and the INT32 total at its bound (K = 131072).
"""
import numpy as np
import pytest
import torch

import block_scaled_bit_amd as bsb
from block_scaled_bit_amd import synth
from oracle import quantize_act_ref, gemm_channel_ref, gemm_channel_fp32_ordered_ref
from tests.gpu_util import require_gpu, dev, dev_bf16, host, say, Guarded, check_fp32, check_bf16

pytestmark = pytest.mark.gpu


def _gpu(q, sa, qw, sw, dtype, d):
    g = Guarded((q.shape[0], qw.shape[0]), dtype, d)
    bsb.gemm_w8a8_channel(dev(q, d), dev(sa, d), dev(qw, d), dev(sw, d), out_dtype=dtype,
                          out=g.view)
    torch.cuda.synchronize()
    return g.check()


def _check(q, sa, qw, sw, d):
    y64, mag = gemm_channel_ref(q, sa, qw, sw)
    c32, cb = gemm_channel_fp32_ordered_ref(q, sa, qw, sw)
    check_fp32(_gpu(q, sa, qw, sw, torch.float32, d), y64, mag, c32)
    check_bf16(_gpu(q, sa, qw, sw, torch.bfloat16, d), y64, mag, cb)


@pytest.mark.parametrize("per_tensor", [False, True])
@pytest.mark.parametrize("M,N,K", [
    (1, 1, 128), (17, 100, 384), (33, 64, 256), (64, 130, 640),   # small-M, 2-wave groups
    (32, 13000, 1152),                                             # small-M, wide groups
    (100, 300, 384), (130, 257, 512), (600, 300, 384),             # 128x128 tiles
    (2049, 7425, 256)])                                            # 256x256 tiles
def test_ragged_shapes(M, N, K, per_tensor):
    d = require_gpu()
    say(f"channel gemm M={M} N={N} K={K} per_tensor={per_tensor}")
    cfg = synth.linear_inputs(M, K, N, outlier_p=0.01, outlier_f=20.0, seed=M + N + K)
    q, sa = quantize_act_ref(cfg["x"])
    sw = synth.channel_scales(1 if per_tensor else N, seed=M + N + K)
    _check(q, sa, cfg["qw"], sw, d)


@pytest.mark.parametrize("M,N", [(2, 64), (130, 128)])
def test_int32_total_at_its_bound(M, N):
    """K = 131072 with rows of +127 against rows of +-127: totals of +-2,114,060,288,
    the largest the INT32 accumulator must hold; the other rows random."""
    d = require_gpu()
    K = 131072
    say(f"channel gemm at the INT32 bound M={M} N={N} K={K}")
    rng = np.random.default_rng(M * N)
    q = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    qw = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    q[0], qw[0], qw[1] = 127, 127, -127
    sa = np.exp(rng.normal(-3.0, 0.5, size=M)).astype(np.float32)
    sw = synth.channel_scales(N, seed=7)
    y64, _ = gemm_channel_ref(q, sa, qw, sw)
    assert abs(y64[0, 0] / (float(sa[0]) * float(sw[0])) - 2114060288) < 1
    _check(q, sa, qw, sw, d)


def test_decode_config_per_channel():
    """Decode-shaped linear (32 x 8192 x 28672) with per-channel scales, quantised on
    the GPU, every output checked."""
    d = require_gpu()
    say("channel gemm decode M=32 K=8192 N=28672")
    cfg = synth.linear_config("decode")
    q, sa = quantize_act_ref(cfg["x"])
    qd, sd = bsb.quantize_act(dev_bf16(cfg["x"], d))
    assert np.array_equal(host(qd), q) and np.array_equal(host(sd), sa)
    sw = synth.channel_scales(cfg["N"])
    y64, mag = gemm_channel_ref(q, sa, cfg["qw"], sw)
    c32, cb = gemm_channel_fp32_ordered_ref(q, sa, cfg["qw"], sw)
    yb = host(bsb.gemm_w8a8_channel(qd, sd, dev(cfg["qw"], d), dev(sw, d)))
    check_bf16(yb, y64, mag, cb)


def test_prefill_config_per_tensor_sampled():
    """Prefill-shaped linear (4096 x 8192 x 8192), one weight scale; eight 128x128 output
    tiles checked."""
    d = require_gpu()
    say("channel gemm prefill M=4096 K=8192 N=8192 per-tensor (sampled tiles)")
    cfg = synth.linear_config("prefill")
    q, sa = quantize_act_ref(cfg["x"])
    qw = cfg["qw"]
    sw = synth.channel_scales(1)
    y = host(bsb.gemm_w8a8_channel(dev(q, d), dev(sa, d), dev(qw, d), dev(sw, d),
                                   out_dtype=torch.float32))
    rng = np.random.default_rng(1)
    tiles = [(0, 0), (31, 63)] + [tuple(rng.integers(0, [32, 64])) for _ in range(6)]
    for tm, tn in tiles:
        rs, cs = slice(128 * tm, 128 * tm + 128), slice(128 * tn, 128 * tn + 128)
        y64, mag = gemm_channel_ref(q[rs], sa[rs], qw[cs], sw)
        c32, _ = gemm_channel_fp32_ordered_ref(q[rs], sa[rs], qw[cs], sw)
        check_fp32(y[rs, cs], y64, mag, c32)
