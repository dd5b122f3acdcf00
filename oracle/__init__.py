"""CPU oracle for the block-scaled INT8 linear layer — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct NumPy versions of every step on the hot path.
Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package; the product path (the HIP library and its binding) never
does, and this package imports nothing from the product path.

Sources ("pages"):
  [P1] "Running DeepSeek-V4-Flash-Vision on 4x A800: adaptation"
       (yfxerp.com/news/113390), sec. 1 (the constraints table: FP8 e4m3
       [128,128] UE8M0 block-scaled linears, dynamic activations, MXFP4 E2M1
       UE8M0 routed experts) and sec. 2 (dequantise / repack to the INT8 route;
       the BF16 dense route and the weight-only INT8 expert route).
  [P2] "Deploying DeepSeek-V4-Flash on AMD MI300X: a hard-core retrospective"
       (aimsg.uk), section "FP8 dialect clash" (OCP vs fnuz: same bits, bias
       off by one, values exactly 2x apart) and "Loose ends" items 1-2 (MoE
       expert-mask layout; padding lanes masked by the logical block size).
  [P3] "Hunyuan 770B in INT8 on domestic accelerators" (pwwt.cn/news/4495474),
       sec. 3.1 (per-group-128 weights, per-token dynamic activations, INT8
       multiply-accumulate into INT32, FP32 scales applied last; per-tensor and
       per-channel weight scales as the coarser alternatives), sec. 1.3
       (MoE: few experts active per token) and sec. 4.4 (tokens dispatched to
       their experts and combined back); sec. 2.2, 3.4 and 4.1 (the INT8 KV
       cache: one dynamic scale per key / value vector, dequantised inside the
       attention kernel).

The pages state the method in prose only. The constants of the quantisation
rule (scale = amax/127 in float32, round-half-to-even, clamp to [-127, 127])
are the stated formula of the task; the pages print no worked example.

Parity pins (checked in tests/ with ``-m "not gpu"``): exact rational
re-computation, closed-form tables cross-checked against torch's float8
decoders and transformers' MXFP4 decoder, the OCP = 2 x fnuz identity, the
integer-matmul identity, brute force on tiny shapes. Nothing here is "parity
unpinned".
"""
from .quant import bf16_bits_to_f32, quantize_rows_ref, quantize_act_ref
from .gemm import (group_partials_ref, gemm_ref, gemm_fp32_ordered_ref, fmaf_ref,
                   f32_to_bf16_bits_ref, bf16_bits_to_f32_ref)
from .grouped import grouped_gemm_ref, grouped_gemm_fp32_ordered_ref
from .decode import (fp8_e4m3_table, ue8m0_value, e2m1_table, decode_fp8_block_ref,
                     dequant_fp8_block_ref, decode_mxfp4_ref, dequant_mxfp4_ref)
from .moe import gather_rows_ref, moe_combine_ref, moe_combine_fp32_ordered_ref
from .channel import gemm_channel_ref, gemm_channel_fp32_ordered_ref, channel_total_ref
from .a16 import gemm_w8a16_ref, gemm_bf16_ref, a16_tolerance, dequant_fp8_block_bf16_ref
from .kvcache import (kv_quantize_ref, dequant_kv_ref, attention_int8kv_ref,
                      attention_bf16kv_ref, attention_tolerance, chunk_lengths_ref,
                      attention_int8kv_chunk_ref)
from .packed import packed_position_ref, repack_mfma_ref, unpack_mfma_ref

__all__ = [
    "bf16_bits_to_f32", "quantize_rows_ref", "quantize_act_ref",
    "group_partials_ref", "gemm_ref", "gemm_fp32_ordered_ref", "fmaf_ref",
    "f32_to_bf16_bits_ref", "bf16_bits_to_f32_ref",
    "grouped_gemm_ref", "grouped_gemm_fp32_ordered_ref",
    "fp8_e4m3_table", "ue8m0_value", "e2m1_table", "decode_fp8_block_ref",
    "dequant_fp8_block_ref", "decode_mxfp4_ref", "dequant_mxfp4_ref",
    "gather_rows_ref", "moe_combine_ref", "moe_combine_fp32_ordered_ref",
    "gemm_channel_ref", "gemm_channel_fp32_ordered_ref", "channel_total_ref",
    "gemm_w8a16_ref", "gemm_bf16_ref", "a16_tolerance", "dequant_fp8_block_bf16_ref",
    "kv_quantize_ref", "dequant_kv_ref", "attention_int8kv_chunk_ref", "chunk_lengths_ref", "attention_int8kv_ref", "attention_bf16kv_ref",
    "attention_tolerance",
    "packed_position_ref", "repack_mfma_ref", "unpack_mfma_ref",
]
