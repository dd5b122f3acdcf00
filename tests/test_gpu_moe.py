"""GPU parity: the MoE glue (gather of quantised rows, top-k weighted combine) vs the oracle.

Gathered rows and scales must match bit for bit; combined BF16 outputs must be
within one BF16 ulp of the float64 definition and bit-identical to the
oracle's float32 replay of the kernel's order. The routed MoE layer is also
run end to end (quantise the tokens, gather, grouped GEMM, combine) and
checked against quantising after the gather.
"""
import numpy as np
import pytest
import torch

import block_scaled_bit_amd as bsb
from block_scaled_bit_amd import synth
from oracle import (quantize_act_ref, gather_rows_ref, moe_combine_ref,
                    moe_combine_fp32_ordered_ref, gemm_ref, gemm_fp32_ordered_ref)
from tests.gpu_util import require_gpu, dev, dev_bf16, host, say, Guarded, check_bf16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,R,K", [(1, 1, 128), (7, 30, 256), (64, 500, 4096), (300, 2400, 1152)])
def test_gather_rows(T, R, K):
    d = require_gpu()
    say(f"gather T={T} R={R} K={K}")
    rng = np.random.default_rng(T + R + K)
    x = synth.activations(rng, T, K, 0.01, 20.0)
    q, sa = quantize_act_ref(x)
    index = rng.integers(0, T, size=R).astype(np.int32)
    gq, gs = Guarded((R, K), torch.int8, d), Guarded((R,), torch.float32, d)
    bsb.gather_rows(dev(q, d), dev(sa, d), dev(index, d), q_out=gq.view, sa_out=gs.view)
    torch.cuda.synchronize()
    qr, sr = gather_rows_ref(q, sa, index)
    assert np.array_equal(gq.check(), qr)
    assert np.array_equal(gs.check().view(np.uint32), sr.view(np.uint32))


def test_gather_out_of_range_rows_are_zero():
    """Indices outside [0, T) are outside the domain: never read, row written as zeros."""
    d = require_gpu()
    say("gather out-of-range indices")
    rng = np.random.default_rng(2)
    q = rng.integers(-127, 128, size=(5, 128)).astype(np.int8)
    sa = np.arange(1, 6, dtype=np.float32)
    index = np.array([0, -1, 4, 5, 1 << 30, 2], np.int32)
    qo, so = bsb.gather_rows(dev(q, d), dev(sa, d), dev(index, d))
    qo, so = host(qo), host(so)
    for r, i in enumerate(index):
        if 0 <= i < 5:
            assert np.array_equal(qo[r], q[i]) and so[r] == sa[i]
        else:
            assert not qo[r].any() and so[r] == 0.0


def _combine_case(rng, T, topk, R, N):
    y = synth.to_bf16_bits(rng.standard_normal((R, N)).astype(np.float32))
    rp = np.stack([rng.choice(R, topk, replace=False) for _ in range(T)]).astype(np.int32)
    return y, rp, synth.gate_weights(rng, T, topk)


@pytest.mark.parametrize("T,topk,R,N", [(1, 1, 1, 8), (5, 3, 17, 64), (40, 8, 400, 2048),
                                         (9, 9, 30, 2056), (3, 20, 64, 520)])
def test_combine_shapes(T, topk, R, N):
    """One slot, a partial slot batch (9, 20 > 8 in flight), columns past one
    workgroup pass (N = 2056), rows used by several tokens."""
    d = require_gpu()
    say(f"combine T={T} topk={topk} R={R} N={N}")
    rng = np.random.default_rng(T * 7 + topk + N)
    y, rp, gate = _combine_case(rng, T, topk, R, N)
    g = Guarded((T, N), torch.bfloat16, d)
    bsb.moe_combine(dev_bf16(y, d), dev(rp, d), dev(gate, d), out=g.view)
    torch.cuda.synchronize()
    out64, mag = moe_combine_ref(y, rp, gate)
    _, canon = moe_combine_fp32_ordered_ref(y, rp, gate)
    check_bf16(g.check(), out64, mag, canon)


def test_combine_out_of_range_slots_add_nothing():
    d = require_gpu()
    say("combine out-of-range slots")
    rng = np.random.default_rng(4)
    y, rp, gate = _combine_case(rng, 6, 4, 12, 16)
    bad = rp.copy()
    bad[:, 2] = -5
    bad[3, 0] = 12
    got = host(bsb.moe_combine(dev_bf16(y, d), dev(bad, d), dev(gate, d)))
    keep = np.ones_like(gate)
    keep[:, 2] = 0
    keep[3, 0] = 0
    _, canon = moe_combine_fp32_ordered_ref(y, np.where(keep > 0, bad, 0).astype(np.int32),
                                            (gate * keep).astype(np.float32))
    assert np.array_equal(got, canon)


def test_moe_layer_end_to_end():
    """The routed MoE layer (4096 tokens, top-8 of 64 experts): quantising the
    tokens then gathering equals quantising the gathered rows bit for bit; the
    combine over the grouped GEMM's output matches the oracle's float32 replay
    for every token; sampled tokens also match the whole layer computed by the
    oracle from the weights."""
    d = require_gpu()
    say("moe layer end to end (full size)")
    m = synth.moe_inputs()
    T, K, N, E, R = m["T"], m["K"], m["N"], m["E"], m["R"]
    xt = dev_bf16(m["x_tokens"], d)
    qt, st = bsb.quantize_act(xt)
    idx = dev(m["token_of_row"], d)
    qg, sg = bsb.gather_rows(qt, st, idx)
    qs, ss = bsb.quantize_act(dev_bf16(m["x_sorted"], d))
    assert torch.equal(qg, qs) and torch.equal(sg.view(torch.int32), ss.view(torch.int32))
    del qs, ss
    qw, sw, off = dev(m["qw"], d), dev(m["sw"], d), dev(m["offsets"], d)
    y = bsb.grouped_gemm_w8a8_g128(qg, sg, qw, sw, off)
    rp, gate = m["row_of_pair"], m["gate"]
    out = host(bsb.moe_combine(y, dev(rp, d), dev(gate, d)))
    yh = host(y)
    out64, mag = moe_combine_ref(yh, rp, gate)
    _, canon = moe_combine_fp32_ordered_ref(yh, rp, gate)
    check_bf16(out, out64, mag, canon)
    # whole layer from the weights for a few tokens
    q, sa = quantize_act_ref(m["x_tokens"])
    off_h = m["offsets"]
    expert_of_row = np.searchsorted(off_h, np.arange(R), side="right") - 1
    rng = np.random.default_rng(9)
    for t in rng.choice(T, 6, replace=False):
        rows = rp[t]
        yb = np.empty((len(rows), N), np.uint16)
        for k, r in enumerate(rows):
            e = int(expert_of_row[r])
            _, yb[k] = gemm_fp32_ordered_ref(q[t:t + 1], sa[t:t + 1], m["qw"][e], m["sw"][e])
        o64, mg = moe_combine_ref(yb, np.arange(len(rows), dtype=np.int32)[None], gate[t:t + 1])
        _, cb = moe_combine_fp32_ordered_ref(yb, np.arange(len(rows), dtype=np.int32)[None],
                                             gate[t:t + 1])
        check_bf16(out[t:t + 1], o64, mg, cb)
