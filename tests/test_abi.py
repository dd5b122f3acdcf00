"""C-ABI checks that need no GPU: the library loads, exports what include/bsb.h
declares, and rejects bad arguments before anything is launched.

The argument checks pass fake device addresses. They run only where no GPU is
visible: with one, a call whose checks regressed would launch a kernel on those
addresses."""
import ctypes
import os
import re

import pytest
import torch  # noqa: F401  (loads the HIP runtime the library binds to)

import block_scaled_bit_amd as bsb
from block_scaled_bit_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsb.h")

OK, INVALID, UNSUPPORTED, MISALIGNED = 0, 1, 2, 3
no_gpu = pytest.mark.skipif(torch.cuda.is_available(),
                            reason="passes fake device addresses: host checks only, no GPU visible")
A = 0x10000          # fake, 16-byte aligned, never dereferenced
U = 0x10008          # fake, misaligned


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(bsb_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libbsb.so is not built (python -m block_scaled_bit_amd.build)")
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert set(names) == set(_lib.EXPORTED), names
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert L.bsb_abi_version() == 1
    for code, name in _lib.STATUS.items():
        assert L.bsb_status_string(code).decode().startswith(name)
    assert L.bsb_status_string(99).decode() == "BSB_ERR_UNKNOWN"


@no_gpu
def test_invalid_sizes_return_invalid_arg(L):
    # K not a multiple of 128, negative sizes, empty N
    assert L.bsb_quantize_act(A, 4, 100, A, A, None) == INVALID
    assert L.bsb_quantize_act(A, -1, 128, A, A, None) == INVALID
    assert L.bsb_gemm_w8a8_g128(A, A, A, A, 4, 0, 128, A, 0, None) == INVALID
    assert L.bsb_gemm_w8a8_g128(A, A, A, A, 4, 8, 130, A, 0, None) == INVALID
    assert L.bsb_gemm_w8a8_g128(A, A, A, A, -4, 8, 128, A, 0, None) == INVALID
    assert L.bsb_gemm_w8a8_g128_partials(A, A, 4, 8, 0, A, None) == INVALID
    assert L.bsb_grouped_gemm_w8a8_g128(A, A, A, A, A, 0, 4, 8, 128, A, 0, None) == INVALID
    assert L.bsb_decode_fp8_block(A, A, 100, 128, 0, A, A, None) == INVALID   # N % 128
    assert L.bsb_decode_mxfp4(A, A, 1, 8, 96, A, A, None) == INVALID
    # products of in-range extents that overflow int64 or the index limits
    big = 1 << 29
    assert L.bsb_grouped_gemm_w8a8_g128(A, A, A, A, A, 1 << 19, 4, big, big, A, 0, None) == INVALID
    assert L.bsb_decode_mxfp4(A, A, big, big, big, A, A, None) == INVALID
    assert L.bsb_gemm_w8a8_g128_partials(A, A, big, big, 1 << 20, A, None) == INVALID
    assert L.bsb_decode_fp8_block(A, A, 1 << 23, 1 << 13, 0, A, A, None) == INVALID   # 2^36
    # K below 2^24 for the row-major W8A8 GEMMs (128-row panels, 32-bit offsets)
    assert L.bsb_gemm_w8a8_g128(A, A, A, A, 4, 8, 1 << 24, A, 0, None) == INVALID
    assert L.bsb_gemm_w8a8_g128_partials(A, A, 4, 8, 1 << 24, A, None) == INVALID
    assert L.bsb_grouped_gemm_w8a8_g128(A, A, A, A, A, 1, 4, 8, 1 << 24, A, 0, None) == INVALID
    assert L.bsb_gather_rows(A, A, A, 4, 0, 128, A, A, None) == INVALID          # no tokens
    assert L.bsb_gather_rows(A, A, A, 4, 8, 100, A, A, None) == INVALID          # K % 128
    assert L.bsb_moe_combine(A, A, A, 4, 0, 16, 64, A, None) == INVALID          # topk 0
    assert L.bsb_moe_combine(A, A, A, 4, 257, 16, 64, A, None) == INVALID        # topk > 256
    assert L.bsb_moe_combine(A, A, A, 4, 2, 16, 60, A, None) == INVALID          # N % 8


@no_gpu
def test_bad_enums_return_invalid_arg(L):
    assert L.bsb_gemm_w8a8_g128(A, A, A, A, 4, 8, 128, A, 7, None) == INVALID
    assert L.bsb_grouped_gemm_w8a8_g128(A, A, A, A, A, 2, 4, 8, 128, A, -1, None) == INVALID
    assert L.bsb_decode_fp8_block(A, A, 128, 128, 2, A, A, None) == INVALID


@no_gpu
def test_null_pointers_return_invalid_arg(L):
    assert L.bsb_quantize_act(None, 4, 128, A, A, None) == INVALID
    assert L.bsb_gemm_w8a8_g128(A, None, A, A, 4, 8, 128, A, 0, None) == INVALID
    assert L.bsb_grouped_gemm_w8a8_g128(A, A, A, A, None, 2, 4, 8, 128, A, 0, None) == INVALID
    assert L.bsb_decode_fp8_block(A, A, 128, 128, 0, None, A, None) == INVALID
    assert L.bsb_decode_mxfp4(A, None, 1, 8, 128, A, A, None) == INVALID
    assert L.bsb_gemm_w8a8_g128_partials(A, A, 4, 8, 128, None, None) == INVALID
    assert L.bsb_gather_rows(A, A, None, 4, 8, 128, A, A, None) == INVALID
    assert L.bsb_moe_combine(A, None, A, 4, 2, 16, 64, A, None) == INVALID


@no_gpu
def test_misaligned_pointers(L):
    assert L.bsb_quantize_act(U, 4, 128, A, A, None) == MISALIGNED
    assert L.bsb_gemm_w8a8_g128(A, A, A, U, 4, 8, 128, A, 1, None) == MISALIGNED
    assert L.bsb_grouped_gemm_w8a8_g128(A, A, A, A, U, 2, 4, 8, 128, A, 0, None) == MISALIGNED
    assert L.bsb_decode_mxfp4(A, A, 1, 8, 128, U, A, None) == MISALIGNED
    assert L.bsb_gather_rows(A, A, U, 4, 8, 128, A, A, None) == MISALIGNED
    assert L.bsb_moe_combine(A, A, U, 4, 2, 16, 64, A, None) == MISALIGNED


@no_gpu
def test_empty_rows_are_a_successful_no_op(L):
    # M = 0 / R = 0: nothing to do, nothing launched, null pointers allowed
    assert L.bsb_quantize_act(None, 0, 128, None, None, None) == OK
    assert L.bsb_gemm_w8a8_g128(None, None, None, None, 0, 8, 128, None, 0, None) == OK
    assert L.bsb_grouped_gemm_w8a8_g128(None, None, None, None, None, 3, 0, 8, 128, None, 0,
                                        None) == OK
    assert L.bsb_gather_rows(None, None, None, 0, 8, 128, None, None, None) == OK
    assert L.bsb_moe_combine(None, None, None, 0, 2, 16, 64, None, None) == OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU path")
def test_no_gpu_is_unsupported_device(L):
    # valid arguments, but no gfx950 device is present: fail fast, launch nothing
    assert L.bsb_quantize_act(A, 4, 128, A, A, None) == UNSUPPORTED
    assert L.bsb_gemm_w8a8_g128(A, A, A, A, 4, 8, 128, A, 0, None) == UNSUPPORTED
    assert L.bsb_gather_rows(A, A, A, 4, 8, 128, A, A, None) == UNSUPPORTED
    assert L.bsb_moe_combine(A, A, A, 4, 2, 16, 64, A, None) == UNSUPPORTED


def test_python_binding_validates_before_calling():
    cpu = torch.zeros(4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        bsb.quantize_act(cpu)                      # not on a GPU
    with pytest.raises(ValueError):
        bsb.gemm_w8a8_g128(torch.zeros(4, 128, dtype=torch.int8), None, None, None)


@no_gpu
def test_channel_gemm_argument_checks(L):
    """Per-channel / per-tensor GEMM: stride 0 or 1 only, K within the INT32 total's
    bound, sw 4-byte aligned (one float for per-tensor), the usual null, enum and
    empty-input rules; with valid arguments and no gfx950 device it fails fast."""
    f = L.bsb_gemm_w8a8_channel
    assert f(A, A, A, A, 2, 4, 8, 128, A, 0, None) == INVALID          # stride
    assert f(A, A, A, A, -1, 4, 8, 128, A, 0, None) == INVALID
    assert f(A, A, A, A, 1, 4, 8, 131072 + 128, A, 0, None) == INVALID  # INT32 total bound
    assert f(A, A, A, A, 1, 4, 8, 130, A, 0, None) == INVALID
    assert f(A, A, A, A, 1, 4, 8, 128, A, 5, None) == INVALID          # out enum
    assert f(A, None, A, A, 1, 4, 8, 128, A, 0, None) == INVALID
    assert f(A, A, A, A + 2, 1, 4, 8, 128, A, 0, None) == MISALIGNED
    assert f(A, A, U, A, 0, 4, 8, 128, A, 0, None) == MISALIGNED
    assert f(None, None, None, None, 1, 0, 8, 128, None, 0, None) == OK
    if not torch.cuda.is_available():
        assert f(A, A, A, A + 4, 0, 4, 8, 131072, A, 1, None) == UNSUPPORTED


@no_gpu
def test_bf16_activation_routes_argument_checks(L):
    """W8A16 / BF16 GEMMs: K a multiple of 128 below 2^23, any number of rows; the FP8 -> BF16
    dequantisation: the decoder's size and dialect rules."""
    w16, b16, dq = L.bsb_gemm_w8a16_g128, L.bsb_gemm_bf16, L.bsb_dequant_fp8_block_bf16
    assert w16(A, A, A, -1, 8, 128, A, 0, None) == INVALID
    assert b16(A, A, 1 << 30, 8, 128, A, 0, None) == INVALID        # rows below 2^30
    assert w16(A, A, A, 4, 8, 1 << 23, A, 0, None) == INVALID       # 256*K >= 2^31
    assert w16(A, A, A, 100, 8, 1 << 23, A, 0, None) == INVALID
    if not torch.cuda.is_available():
        assert w16(A, A, A, 65, 8, 128, A, 0, None) == UNSUPPORTED   # tiled kernel beyond 64 rows
        assert b16(A, A, 65, 8, 128, A, 0, None) == UNSUPPORTED
    assert b16(A, A, 4, 8, 130, A, 0, None) == INVALID
    assert w16(A, A, A, 4, 8, 128, A, 3, None) == INVALID           # out enum
    assert w16(A, None, A, 4, 8, 128, A, 0, None) == INVALID
    assert b16(A, A, 4, 8, 128, None, 0, None) == INVALID
    assert w16(A, A, U, 4, 8, 128, A, 0, None) == MISALIGNED
    assert b16(U, A, 4, 8, 128, A, 0, None) == MISALIGNED
    assert w16(None, None, None, 0, 8, 128, None, 0, None) == OK
    assert b16(None, None, 0, 8, 128, None, 0, None) == OK
    assert dq(A, A, 100, 128, 0, A, None) == INVALID                # N % 128
    assert dq(A, A, 128, 128, 2, A, None) == INVALID                # dialect
    assert dq(A, A, 128, 128, 0, U, None) == MISALIGNED
    if not torch.cuda.is_available():
        assert w16(A, A, A, 64, 8, 128, A, 1, None) == UNSUPPORTED
        assert b16(A, A, 1, 8, 128, A, 0, None) == UNSUPPORTED
        assert dq(A, A, 128, 128, 1, A, None) == UNSUPPORTED


@no_gpu
def test_kv_cache_argument_checks(L):
    """KV cache write and decode attention: head dimension 128, T a multiple of 64,
    at most 16 query heads per KV head, max_len <= T, a large enough workspace;
    nothing to write is a no-op; with valid arguments and no gfx950 device they
    fail fast."""
    wr, at, wb = L.bsb_kv_cache_write, L.bsb_attention_decode_int8kv, L.bsb_attention_workspace_bytes
    assert wb(2, 16, 1000) == 2 * 16 * 2 * 130 * 4                    # two 512-token splits
    assert wb(2, 16, 0) == 0 and wb(0, 16, 10) == -1 and wb(2, 16, -1) == -1
    assert wr(A, A, A, A, 3, 2, 4, 128, 64, A, A, A, A, None) == INVALID     # D != 128
    assert wr(A, A, A, A, 3, 2, 4, 96, 128, A, A, A, A, None) == INVALID     # T % 64
    assert wr(A, A, A, None, 3, 2, 4, 128, 128, A, A, A, A, None) == INVALID
    assert wr(A, A, A, A, 3, 2, 4, 128, 128, A, A, U, A, None) == MISALIGNED
    assert wr(None, None, None, None, 0, 2, 4, 128, 128, None, None, None, None, None) == OK
    need = wb(2, 16, 128)
    ok = (A, A, A, A, A, A, 2, 16, 4, 128, 128, 128, A, need, A, 0, None)

    def call(**kw):
        names = ["q", "kc", "ks", "vc", "vs", "lens", "B", "Hq", "Hkv", "T", "D", "max_len",
                 "work", "work_bytes", "out", "dtype", "stream"]
        args = dict(zip(names, ok))
        args.update(kw)
        return at(*[args[n] for n in names])

    assert call(Hq=15) == INVALID                                   # Hq % Hkv
    assert call(Hq=68, Hkv=4) == INVALID                            # 17 heads per KV head
    assert call(D=64) == INVALID
    assert call(T=100) == INVALID
    assert call(max_len=129) == INVALID                             # above T
    assert call(work_bytes=need - 4) == INVALID
    assert call(dtype=2) == INVALID
    assert call(lens=None) == INVALID
    assert call(B=65536 // 4 + 1) == INVALID                        # B * Hkv > 65535
    assert call(vs=U) == MISALIGNED
    if not torch.cuda.is_available():
        assert call() == UNSUPPORTED
        assert call(max_len=0, work=None, work_bytes=0) == UNSUPPORTED
        assert wr(A, A, A, A, 3, 2, 4, 128, 128, A, A, A, A, None) == UNSUPPORTED


@no_gpu
def test_grouped_gather_argument_checks(L):
    """Grouped GEMM with the rows gathered by the kernel: the grouped GEMM's checks plus
    T >= 1, T * K + 128 < 2^31, a non-null 16-byte-aligned index; R = 0 is a no-op."""
    f = L.bsb_grouped_gemm_w8a8_g128_gather
    names = ["q", "sa", "index", "T", "qw", "sw", "off", "E", "R", "N", "K", "y", "out", "stream"]
    ok = (A, A, A, 100, A, A, A, 4, 300, 64, 256, A, 0, None)

    def call(**kw):
        args = dict(zip(names, ok))
        args.update(kw)
        return f(*[args[n] for n in names])

    assert call(T=0) == INVALID
    assert call(T=(1 << 23), K=256) == INVALID          # T * K reaches 2^31
    assert call(K=200) == INVALID
    assert call(E=0) == INVALID
    assert call(out=2) == INVALID
    assert call(index=None) == INVALID
    assert call(index=U) == MISALIGNED
    assert call(q=U) == MISALIGNED
    assert call(q=None, sa=None, index=None, qw=None, sw=None, off=None, y=None, R=0) == OK
    if not torch.cuda.is_available():
        assert call() == UNSUPPORTED
        assert call(T=(1 << 23) - 1, K=256) == UNSUPPORTED


@no_gpu
def test_chunk_attention_argument_checks(L):
    """Attention of several query tokens per sequence: the decode attention's checks
    plus 1 <= Qn and Qn * Hq / Hkv <= 16, a workspace sized for B * Qn query heads;
    with valid arguments and no gfx950 device it fails fast."""
    ch, wb = L.bsb_attention_chunk_int8kv, L.bsb_attention_workspace_bytes
    names = ["q", "kc", "ks", "vc", "vs", "lens", "B", "Qn", "Hq", "Hkv", "T", "D", "max_len",
             "work", "work_bytes", "out", "dtype", "stream"]
    need = wb(2, 4 * 8, 1000)
    ok = (A, A, A, A, A, A, 2, 4, 8, 2, 1024, 128, 1000, A, need, A, 0, None)

    def call(**kw):
        args = dict(zip(names, ok))
        args.update(kw)
        return ch(*[args[n] for n in names])

    assert call(Qn=0) == INVALID
    assert call(Qn=5) == INVALID                                    # 5 tokens x 4 heads > 16
    assert call(Qn=17, Hq=2) == INVALID
    assert call(work_bytes=wb(2, 8, 1000)) == INVALID               # sized for one token
    assert call(Hq=7) == INVALID                                    # Hq % Hkv
    assert call(D=64) == INVALID
    assert call(T=1000) == INVALID
    assert call(max_len=1025) == INVALID
    assert call(work_bytes=need - 4) == INVALID
    assert call(dtype=2) == INVALID
    assert call(q=None) == INVALID
    assert call(vs=U) == MISALIGNED
    if not torch.cuda.is_available():
        assert call() == UNSUPPORTED
        assert call(Qn=8, Hq=4) == UNSUPPORTED                       # 8 x 2 columns
        assert call(Qn=16, Hq=2) == UNSUPPORTED                      # 16 x 1
        assert call(max_len=0, work=None, work_bytes=0) == UNSUPPORTED


@no_gpu
def test_noalloc_attention_argument_checks(L):
    """The allocation-free decode attention: the attention's checks without a
    workspace argument, and sizes whose workspace exceeds the static array's
    BSB_ATTENTION_NOALLOC_MAX_BYTES are refused before anything is launched."""
    na, wb = L.bsb_attention_decode_int8kv_noalloc, L.bsb_attention_workspace_bytes
    limit = _lib.ATTENTION_NOALLOC_MAX_BYTES
    assert limit == 32 << 20
    names = ["q", "kc", "ks", "vc", "vs", "lens", "B", "Hq", "Hkv", "T", "D", "max_len", "out",
             "dtype", "stream"]
    ok = (A, A, A, A, A, A, 2, 16, 4, 128, 128, 128, A, 0, None)

    def call(**kw):
        args = dict(zip(names, ok))
        args.update(kw)
        return na(*[args[n] for n in names])

    assert call(Hq=15) == INVALID
    assert call(D=64) == INVALID
    assert call(max_len=129) == INVALID
    assert call(dtype=2) == INVALID
    assert call(out=None) == INVALID
    assert call(kc=None) == INVALID
    assert call(vs=U) == MISALIGNED
    # 1024 sequences x 64 heads x 2 splits of 512 tokens: 68 MB of partials, over the limit
    assert wb(1024, 64, 1024) > limit
    assert call(B=1024, Hq=64, Hkv=64, T=1024, max_len=1024) == INVALID
    # the largest workspace under the limit is accepted up to the device check
    assert wb(32, 64, 8192) <= limit
    if not torch.cuda.is_available():
        assert call() == UNSUPPORTED
        assert call(B=32, Hq=64, Hkv=8, T=8192, max_len=8192) == UNSUPPORTED


@no_gpu
def test_probe_argument_checks(L):
    """Measurement probes: sizes outside their stated ranges are refused before
    anything is launched; valid calls without a gfx950 device fail fast."""
    mf, hb = L.bsb_probe_mfma_i8, L.bsb_probe_hbm_read
    for m in (mf, L.bsb_probe_mfma_i8_epilogue):
        assert m(A, A, 8, 1, A, None) == INVALID            # under 16 bytes
        assert m(A, A, 24, 1, A, None) == INVALID           # not a multiple of 16
        assert m(A, A, 1024, 0, A, None) == INVALID         # no rounds
        assert m(A, A, 1024, (1 << 24) + 1, A, None) == INVALID
        assert m(A, A, (1 << 31) + 16, 1, A, None) == INVALID
        assert m(None, A, 1024, 1, A, None) == INVALID
        assert m(A, A, 1024, 1, U, None) == MISALIGNED
    sweep = 16 * 131072
    assert hb(A, sweep - 16, A, None) == INVALID
    assert hb(A, sweep + 16, A, None) == INVALID
    assert hb(None, sweep, A, None) == INVALID
    assert hb(U, sweep, A, None) == MISALIGNED
    cp = L.bsb_probe_hbm_copy
    assert cp(A, A, sweep + 16, None) == INVALID
    assert cp(A, None, sweep, None) == INVALID
    assert cp(A, U, sweep, None) == MISALIGNED
    if not torch.cuda.is_available():
        assert mf(A, A, 1024, 1, A, None) == UNSUPPORTED
        assert L.bsb_probe_mfma_i8_epilogue(A, A, 1024, 1, A, None) == UNSUPPORTED
        assert hb(A, 2 * sweep, A, None) == UNSUPPORTED
        assert cp(A, A, 2 * sweep, None) == UNSUPPORTED


@no_gpu
def test_bf16_kv_cache_argument_checks(L):
    wr, at, wb = L.bsb_kv_cache_write_bf16, L.bsb_attention_decode_bf16kv, L.bsb_attention_workspace_bytes
    assert wr(A, A, A, A, 3, 2, 4, 128, 64, A, A, None) == INVALID          # D != 128
    assert wr(A, A, A, A, 3, 2, 4, 96, 128, A, A, None) == INVALID          # T % 64
    assert wr(A, A, A, A, 3, 2, 4, 128, 128, A, None, None) == INVALID
    assert wr(A, A, A, A, 3, 2, 4, 128, 128, U, A, None) == MISALIGNED
    assert wr(None, None, None, None, 0, 2, 4, 128, 128, None, None, None) == OK
    need = wb(2, 16, 128)
    assert at(A, A, A, A, 2, 15, 4, 128, 128, 128, A, need, A, 0, None) == INVALID
    assert at(A, A, A, A, 2, 16, 4, 128, 128, 129, A, need, A, 0, None) == INVALID
    assert at(A, A, A, A, 2, 16, 4, 128, 128, 128, A, need - 4, A, 0, None) == INVALID
    assert at(A, None, A, A, 2, 16, 4, 128, 128, 128, A, need, A, 0, None) == INVALID
    assert at(A, A, U, A, 2, 16, 4, 128, 128, 128, A, need, A, 0, None) == MISALIGNED
    if not torch.cuda.is_available():
        assert at(A, A, A, A, 2, 16, 4, 128, 128, 128, A, need, A, 0, None) == UNSUPPORTED
        assert at(A, A, A, A, 2, 16, 4, 128, 128, 128, A, need, A, 1, None) == UNSUPPORTED
        assert wr(A, A, A, A, 3, 2, 4, 128, 128, A, A, None) == UNSUPPORTED


@no_gpu
def test_packed_weight_argument_checks(L):
    """Repack and packed GEMM: N a multiple of 16, K of 128, the GEMM at most 64
    rows and K <= 2^24, the usual null, enum, alignment and empty-input rules;
    with valid arguments and no gfx950 device they fail fast."""
    rp, g = L.bsb_repack_weights_mfma, L.bsb_gemm_w8a8_g128_packed
    assert rp(A, 24, 128, A, None) == INVALID            # N % 16
    assert rp(A, 16, 192, A, None) == INVALID            # K % 128
    assert rp(A, 0, 128, A, None) == INVALID             # empty weight
    assert rp(None, 16, 128, A, None) == INVALID
    assert rp(A, 16, 128, None, None) == INVALID
    assert rp(U, 16, 128, A, None) == MISALIGNED
    assert rp(A, 16, 128, U, None) == MISALIGNED
    assert rp(A, 1 << 23, 1 << 14, A, None) == INVALID   # 2^37 bytes
    assert g(A, A, A, A, 65, 16, 128, A, 0, None) == INVALID           # more than 64 rows
    assert g(A, A, A, A, 4, 24, 128, A, 0, None) == INVALID            # N % 16
    assert g(A, A, A, A, 4, 16, 130, A, 0, None) == INVALID            # K % 128
    assert g(A, A, A, A, 4, 16, (1 << 24) + 128, A, 0, None) == INVALID   # K limit
    assert g(A, A, A, A, -1, 16, 128, A, 0, None) == INVALID
    assert g(A, A, A, A, 4, 16, 128, A, 7, None) == INVALID            # out enum
    assert g(A, A, None, A, 4, 16, 128, A, 0, None) == INVALID
    assert g(A, A, U, A, 4, 16, 128, A, 0, None) == MISALIGNED
    assert g(None, None, None, None, 0, 16, 128, None, 0, None) == OK   # no rows
    gp = L.bsb_grouped_gemm_w8a8_g128_packed
    assert gp(A, A, A, A, A, 0, 4, 16, 128, A, 0, None) == INVALID       # no experts
    assert gp(A, A, A, A, A, 65536, 4, 16, 128, A, 0, None) == INVALID   # too many experts
    assert gp(A, A, A, A, A, 2, 4, 24, 128, A, 0, None) == INVALID       # N % 16
    assert gp(A, A, A, A, None, 2, 4, 16, 128, A, 0, None) == INVALID    # offsets
    assert gp(A, A, A, A, U, 2, 4, 16, 128, A, 0, None) == MISALIGNED
    assert gp(None, None, None, None, None, 2, 0, 16, 128, None, 0, None) == OK   # no rows
    dp = L.bsb_decode_fp8_block_packed
    assert dp(A, A, 64, 128, 0, A, A, None) == INVALID        # N % 128
    assert dp(A, A, 128, 128, 2, A, A, None) == INVALID       # dialect
    assert dp(A, A, 128, 128, 0, None, A, None) == INVALID
    assert dp(A, A, 128, 128, 0, U, A, None) == MISALIGNED
    mp = L.bsb_decode_mxfp4_packed
    assert mp(A, A, 1, 24, 128, A, A, None) == INVALID        # N % 16
    assert mp(A, A, 0, 16, 128, A, A, None) == INVALID        # no experts
    assert mp(A, A, 1, 16, 96, A, A, None) == INVALID         # K % 128
    assert mp(A, A, 1, 16, 128, None, A, None) == INVALID
    assert mp(A, A, 1, 16, 128, A, U, None) == MISALIGNED
    if not torch.cuda.is_available():
        assert mp(A, A, 1, 16, 128, A, A, None) == UNSUPPORTED
        assert dp(A, A, 128, 128, 1, A, A, None) == UNSUPPORTED
        assert gp(A, A, A, A, A, 2, 4, 16, 128, A, 1, None) == UNSUPPORTED
        assert rp(A, 16, 128, A, None) == UNSUPPORTED
        assert g(A, A, A, A, 64, 16, 1 << 24, A, 1, None) == UNSUPPORTED
