"""GPU: the allocation-free decode attention (bsb_attention_decode_int8kv_noalloc)
called through the C ABI gives the same output bits as bsb_attention_decode_int8kv
with a caller workspace, on two calls in a row (the second smaller, so the static
workspace still holds the first call's partials), and both stay within the
derived bound of the oracle's float64 attention."""
import numpy as np
import pytest
import torch

from block_scaled_bit_amd import _lib
from oracle import kv_quantize_ref, attention_int8kv_ref, attention_tolerance, bf16_bits_to_f32_ref
from block_scaled_bit_amd import synth
from tests.gpu_util import require_gpu, dev, dev_bf16, host, say
from tests.test_gpu_kvcache import k_encode, v_encode

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, T, lens, seed):
    lens = np.asarray(lens, np.int32)
    inp = synth.kv_inputs(B, Hq, Hkv, T, lens=lens, seed=seed)
    kc, ks = kv_quantize_ref(inp["k"])
    vc, vs = kv_quantize_ref(inp["v"])
    return inp, lens, kc, ks, vc, vs


def _run(L, d, inp, lens, kc, ks, vc, vs, max_len, out_code):
    B, Hkv, T, _ = kc.shape
    Hq = inp["q"].shape[1]
    q = dev_bf16(inp["q"], d)
    dk, dks, dv, dvs = dev(k_encode(kc), d), dev(ks, d), dev(v_encode(vc), d), dev(vs, d)
    dl = dev(lens, d)
    odt = torch.bfloat16 if out_code == 0 else torch.float32
    out_ref = torch.empty((B, Hq, 128), dtype=odt, device=d)
    out_na = torch.full((B, Hq, 128), float("nan"), dtype=odt, device=d)
    need = L.bsb_attention_workspace_bytes(B, Hq, max_len)
    assert 0 < need <= _lib.ATTENTION_NOALLOC_MAX_BYTES
    work = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=d)
    st = torch.cuda.current_stream(d).cuda_stream
    s = L.bsb_attention_decode_int8kv(q.data_ptr(), dk.data_ptr(), dks.data_ptr(), dv.data_ptr(),
                                      dvs.data_ptr(), dl.data_ptr(), B, Hq, Hkv, T, 128, max_len,
                                      work.data_ptr(), need, out_ref.data_ptr(), out_code, st)
    assert s == 0, s
    s = L.bsb_attention_decode_int8kv_noalloc(q.data_ptr(), dk.data_ptr(), dks.data_ptr(),
                                              dv.data_ptr(), dvs.data_ptr(), dl.data_ptr(), B, Hq,
                                              Hkv, T, 128, max_len, out_na.data_ptr(), out_code, st)
    assert s == 0, s
    torch.cuda.synchronize()
    return host(out_ref), host(out_na)


@pytest.mark.parametrize("out_code", [0, 1])
def test_noalloc_attention_matches_workspace_form_twice(out_code):
    d = require_gpu()
    L = _lib.lib()
    # first call: 4 sequences over 3 splits of the 2048-token bound; second: smaller
    cases = [(4, 16, 2, 2048, [2048, 1500, 1, 700], 2048, 11),
             (2, 8, 1, 1024, [1024, 513], 1024, 12)]
    for B, Hq, Hkv, T, lens, max_len, seed in cases:
        say(f"noalloc attention B={B} Hq={Hq} Hkv={Hkv} T={T} max_len={max_len} out={out_code}")
        inp, lens, kc, ks, vc, vs = _case(B, Hq, Hkv, T, lens, seed)
        ref, na = _run(L, d, inp, lens, kc, ks, vc, vs, max_len, out_code)
        assert np.array_equal(ref.view(np.uint8), na.view(np.uint8)), \
            f"{np.sum(ref != na)} outputs differ from the workspace form"
        o64, wmag = attention_int8kv_ref(inp["q"], kc, ks, vc, vs, lens)
        got = bf16_bits_to_f32_ref(na).astype(np.float64) if out_code == 0 else na.astype(np.float64)
        t = attention_tolerance(out_code == 0)
        assert np.all(np.abs(got - o64) <= t * wmag)
