"""Block-scaled INT8 linear layer for AMD Instinct MI355X (gfx950).

The compute path is libbsb.so (hand-written HIP kernels behind the C ABI in
include/bsb.h); the functions exported here are its thin ctypes binding.
Importing the package does not load the library; the first call does, and
raises if it has not been built.
"""
from ._lib import (quantize_act, gemm_w8a8_g128, gemm_w8a8_g128_partials,  # noqa: F401
                   repack_weights_mfma, gemm_w8a8_g128_packed, decode_fp8_block_packed,
                   grouped_gemm_w8a8_g128_packed, grouped_gemm_w8a8_g128_gather,
                   gemm_w8a8_channel, gemm_w8a16_g128, gemm_bf16, dequant_fp8_block_bf16,
                   grouped_gemm_w8a8_g128, decode_fp8_block, decode_mxfp4, decode_mxfp4_packed,
                   gather_rows,
                   moe_combine, kv_cache_empty, kv_cache_write, attention_workspace_bytes,
                   attention_decode_int8kv, attention_decode_int8kv_noalloc,
                   attention_chunk_int8kv,
                   kv_cache_empty_bf16, kv_cache_write_bf16,
                   attention_decode_bf16kv, BsbError,
                   BSB_OUT_BF16, BSB_OUT_FP32, BSB_FP8_OCP, BSB_FP8_FNUZ, lib, LIB_PATH)
