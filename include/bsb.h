/*
 * bsb.h — block-scaled INT8 linear layer for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libbsb.so. Sources ("pages"):
 *   [P1] "Running DeepSeek-V4-Flash-Vision on 4x A800: adaptation"
 *        (yfxerp.com/news/113390), sec. 1 (constraints table) and sec. 2
 *        (per-segment re-routing: dequantise / repack onto the INT8 path).
 *   [P2] "Deploying DeepSeek-V4-Flash on AMD MI300X: a hard-core
 *        retrospective" (aimsg.uk), sections "FP8 dialect clash",
 *        "HIP Graphs limits" and "Loose ends".
 *   [P3] "Hunyuan 770B in INT8 on domestic accelerators"
 *        (pwwt.cn/news/4495474), sec. 3.1 and sec. 1.3 / 4.4 (MoE dispatch
 *        and combine).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor argument is a DEVICE pointer into memory the caller
 *    allocated and owns (PyTorch in the Python binding). The library
 *    allocates nothing, keeps no pointer after returning, never synchronises
 *    and never reads device memory on the host. Work is enqueued on `stream`
 *    (a hipStream_t passed as void*, NULL = the null stream) of the current
 *    device, so every call can be captured into a HIP graph: launch sizes
 *    come from the host-side size arguments only, as [P2] "HIP Graphs limits"
 *    requires of graph-safe kernels (device pointers and sizes, no host reads
 *    mid-way, no scratch allocation).
 *  - All matrices are row-major and contiguous. K is the reduction dimension
 *    and is contiguous in both operands; G = K / 128 is the number of
 *    128-wide K groups. Two exceptions, each with its layout stated at its
 *    calls: the packed weight form (written by bsb_repack_weights_mfma,
 *    bsb_decode_fp8_block_packed and bsb_decode_mxfp4_packed, read by
 *    bsb_gemm_w8a8_g128_packed and bsb_grouped_gemm_w8a8_g128_packed) and the
 *    INT8 KV cache's blocks.
 *  - Sizes: K % 128 == 0 and K > 0; N >= 1; M, R >= 0 (0 rows is a
 *    successful no-op that launches nothing). Every extent is below 2^30;
 *    a weight matrix (all experts together) holds at most 2^36 elements,
 *    2^35 for the decoders' inputs, and the partials at most 2^36 values.
 *    Larger sizes return BSB_ERR_INVALID_ARG.
 *  - Every pointer must be 16-byte aligned (BSB_ERR_MISALIGNED otherwise).
 *  - Arguments are validated before anything is launched: a NULL pointer
 *    with a non-empty size, a negative or inconsistent size, or a bad enum
 *    returns BSB_ERR_INVALID_ARG and launches nothing. Then, on the first
 *    call per device, the device's architecture is checked: anything other
 *    than gfx950 returns BSB_ERR_UNSUPPORTED_DEVICE (fail fast instead of
 *    running a kernel built for another chip, [P1] sec. 3). A launch failure
 *    reported by hipGetLastError() returns BSB_ERR_LAUNCH. Faults inside a
 *    kernel surface at the caller's next synchronisation, as usual for HIP.
 *  - Outputs are written exactly once for every in-range element; nothing
 *    outside the documented output extents is written.
 *  - Calls are reentrant; calls on different streams do not share state,
 *    except bsb_attention_decode_int8kv_noalloc, whose calls on one device
 *    share a static workspace (stated at its declaration).
 *  - No C++ exception crosses this boundary.
 */
#ifndef BSB_H
#define BSB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bsb_status {
    BSB_OK = 0,
    BSB_ERR_INVALID_ARG = 1,
    BSB_ERR_UNSUPPORTED_DEVICE = 2,
    BSB_ERR_MISALIGNED = 3,
    BSB_ERR_LAUNCH = 4
} bsb_status;

typedef enum bsb_out_dtype {
    BSB_OUT_BF16 = 0,   /* uint16 BF16 bits, round to nearest even */
    BSB_OUT_FP32 = 1    /* IEEE float32 */
} bsb_out_dtype;

typedef enum bsb_fp8_dialect {
    BSB_FP8_OCP = 0,    /* E4M3FN:   bias 7, max 448, 0x7F/0xFF NaN, 0x80 = -0 */
    BSB_FP8_FNUZ = 1    /* E4M3FNUZ: bias 8, max 240, 0x80 NaN, no -0, no inf  */
} bsb_fp8_dialect;

/*
 * Dynamic per-token INT8 quantisation of BF16 activations ([P3] sec. 3.1:
 * per-token scales computed at run time from each token's own range).
 * For each row m:
 *     amax  = max_k |x[m,k]|
 *     sa[m] = amax / 127                     (IEEE float32 divide)
 *     q[m,k] = clamp(rint(x[m,k] / sa[m]), -127, 127)
 * with a true IEEE divide by the stored scale and round-half-to-even; an
 * all-zero row gives sa = 0 and q = 0. Inputs must be finite.
 *   x_bf16  [M, K] BF16 bits (read)
 *   q       [M, K] int8      (written)
 *   sa      [M]    float32   (written)
 */
bsb_status bsb_quantize_act(const uint16_t *x_bf16, int64_t M, int64_t K,
                            int8_t *q, float *sa, void *stream);

/*
 * W8A8 GEMM with per-(output row, 128-wide K group) weight scales ([P3]
 * sec. 3.1: INT8 multiply-accumulate into INT32 inside the matmul, FP32
 * scales applied last):
 *     P[m,n,g] = sum_{k in group g} q[m,k] * qw[n,k]        (exact INT32)
 *     acc      = 0; for g = 0..G-1: acc = fmaf((float)P[m,n,g], sw[n,g], acc)
 *     y[m,n]   = acc * sa[m]        (float32), stored as BF16 (RNE) or FP32
 * The float32 accumulation runs over g in ascending order for every output
 * element (no split-K), so results do not depend on the launch shape.
 *   q   [M, K] int8, sa [M] float32       (output of bsb_quantize_act)
 *   qw  [N, K] int8, sw [N, G] float32    (weights, [out, in] layout)
 *   y   [M, N] BF16 bits or float32 per `out`
 *   K   a multiple of 128 below 2^24 (also for the partials and grouped forms)
 */
bsb_status bsb_gemm_w8a8_g128(const int8_t *q, const float *sa,
                              const int8_t *qw, const float *sw,
                              int64_t M, int64_t N, int64_t K,
                              void *y, bsb_out_dtype out, void *stream);

/*
 * Load-time repack of INT8 weights into the matrix cores' operand order ([P1]
 * sec. 2: quantised weights are rearranged once, when they are loaded, into the
 * layout of the kernel that consumes them). The [N, K] matrix is cut into
 * blocks of 16 rows x 64 columns, each stored as 1024 contiguous bytes:
 *     packed[((n/16)*(K/64) + k/64)*1024 + 16*l + (k%16)] = qw[n, k]
 *         with l = (n%16) + 16*((k%64)/16)
 * (a permutation of the bytes: packed holds exactly N*K bytes). The scales sw
 * keep their [N, G] layout.
 *   qw      [N, K] int8 (read), 16-byte aligned
 *   packed  [N*K] int8 (written), 16-byte aligned, caller-owned, must not
 *           overlap qw
 *   N       a multiple of 16;  K a multiple of 128
 * Errors: BSB_ERR_INVALID_ARG for bad sizes or null pointers (N*K = 0 is not
 * allowed), BSB_ERR_MISALIGNED, BSB_ERR_UNSUPPORTED_DEVICE, BSB_ERR_LAUNCH.
 */
bsb_status bsb_repack_weights_mfma(const int8_t *qw, int64_t N, int64_t K,
                                   int8_t *packed, void *stream);

/*
 * bsb_gemm_w8a8_g128 for decode-shaped M on weights repacked by
 * bsb_repack_weights_mfma: the same arithmetic in the same order ([P3] sec. 3.1),
 * so y is bit-identical to bsb_gemm_w8a8_g128(q, sa, qw, sw, ...) on the
 * unpacked qw. Each wave streams its 16 rows' weights as contiguous 1 KB loads
 * straight into its matrix-core operands.
 *   packed  [N*K] int8 from bsb_repack_weights_mfma
 *   M       0 .. 64 (M = 0: nothing to do);  N a multiple of 16;
 *           K a multiple of 128, at most 2^24
 * Other arguments, limits and errors as bsb_gemm_w8a8_g128; M > 64 is
 * BSB_ERR_INVALID_ARG (use the row-major weights there).
 */
bsb_status bsb_gemm_w8a8_g128_packed(const int8_t *q, const float *sa,
                                     const int8_t *packed, const float *sw,
                                     int64_t M, int64_t N, int64_t K,
                                     void *y, bsb_out_dtype out, void *stream);

/*
 * The MoE form ([P3] sec. 1.3: experts resident, each token runs through a few
 * of them; [P1] sec. 2: weights rearranged once at load time into the layout
 * of the kernel that consumes them) on packed expert weights: the
 * stacked experts qw [E*N, K] repacked by bsb_repack_weights_mfma (each expert's
 * [N, K] block is then contiguous, N*K bytes at e*N*K), scales sw [E, N, K/128]
 * unchanged. Same arithmetic and order, so y is bit-identical to
 * bsb_grouped_gemm_w8a8_g128 on the unpacked weights. Built for decode-shaped
 * MoE: each expert's rows are walked in passes of 32, and each pass streams the
 * expert's weights once.
 *   N a multiple of 16;  K a multiple of 128, at most 2^24;  E at most 65535
 * Other arguments, limits and errors as bsb_grouped_gemm_w8a8_g128.
 */
bsb_status bsb_grouped_gemm_w8a8_g128_packed(const int8_t *q, const float *sa,
                                             const int8_t *packed, const float *sw,
                                             const int32_t *offsets, int64_t E, int64_t R,
                                             int64_t N, int64_t K, void *y,
                                             bsb_out_dtype out, void *stream);

/*
 * W8A8 GEMM with one weight scale per output row (per-channel) or one for the
 * whole weight (per-tensor): the coarser granularities of [P3] sec. 3.1's
 * taxonomy, whose deployment checklist (sec. 6) runs per-tensor before moving
 * to per-group 128. Same operands as bsb_gemm_w8a8_g128 except the scales:
 *     P[m,n]  = sum_k q[m,k] * qw[n,k]              (exact INT32, all of K)
 *     y[m,n]  = ((float)P[m,n] * sw[n * sw_stride]) * sa[m]
 * (float)P rounds to nearest even, each product is rounded to float32, then
 * the store rounds to BF16 (RNE) or keeps FP32.
 *   sw         [N] float32 (sw_stride = 1, per-channel) or [1] (sw_stride = 0,
 *              per-tensor); 4-byte aligned
 *   sw_stride  0 or 1
 *   K          a multiple of 128, at most 131072, so that the INT32 total
 *              cannot overflow (127 * 127 * 131072 < 2^31)
 * Other arguments, limits and errors as bsb_gemm_w8a8_g128.
 */
bsb_status bsb_gemm_w8a8_channel(const int8_t *q, const float *sa,
                                 const int8_t *qw, const float *sw, int64_t sw_stride,
                                 int64_t M, int64_t N, int64_t K,
                                 void *y, bsb_out_dtype out, void *stream);

/*
 * Grouped (MoE) form: rows are sorted by expert and expert e owns rows
 * [offsets[e], offsets[e+1]) ([P3] sec. 1.3: experts resident, each token
 * runs through a few of them). Each segment is multiplied with its expert's
 * weights by the rule of bsb_gemm_w8a8_g128. Tail rows of a tile are masked
 * by the segment end, never by a padded bound ([P2] "Loose ends" item 2);
 * empty experts launch no work and read no weights.
 *   q       [R, K] int8, sa [R] float32
 *   qw      [E, N, K] int8, sw [E, N, G] float32
 *   offsets [E+1] int32, DEVICE memory; preconditions: offsets[0] = 0,
 *           non-decreasing, offsets[E] = R. The kernel clamps every segment
 *           to [0, R], so a violated precondition gives unspecified values in
 *           y but never an out-of-bounds access.
 *   y       [R, N] BF16 bits or float32
 * The launch grid is sized from host values only (the row tiles any split of
 * R rows over E experts can need); with R >= 128*E (and more than 128 tiles
 * of 256x256 without the experts' partial ones) the kernel uses 256-row
 * tiles, with R <= 32*E it walks each expert's rows in passes of 32, otherwise
 * it uses 128-row tiles. No choice changes a result bit.
 */
bsb_status bsb_grouped_gemm_w8a8_g128(const int8_t *q, const float *sa,
                                      const int8_t *qw, const float *sw,
                                      const int32_t *offsets,
                                      int64_t E, int64_t R, int64_t N, int64_t K,
                                      void *y, bsb_out_dtype out, void *stream);

/*
 * The grouped GEMM with the MoE dispatch gather folded into its activation
 * loads ([P3] sec. 1.3 / 4.4: each token runs through the experts it
 * selected): row r of the grouped problem is token index[r] of the T
 * quantised tokens, so the gathered rows are never written to memory. The
 * result is bit-identical to bsb_gather_rows followed by
 * bsb_grouped_gemm_w8a8_g128 (the same kernels and arithmetic; an index
 * outside [0, T) reads a zero row with scale 0, as the gather writes it).
 *   q       [T, K] int8, sa [T] float32 (bsb_quantize_act's outputs);
 *           T >= 1 and T * K + 128 < 2^31
 *   index   [R] int32, DEVICE memory, the token of each sorted row
 *   qw, sw, offsets, E, R, N, K, y, out: as bsb_grouped_gemm_w8a8_g128
 * Errors: as bsb_grouped_gemm_w8a8_g128, and BSB_ERR_INVALID_ARG for T out of
 * range or a null index (R > 0), BSB_ERR_MISALIGNED for an index not on a
 * 16-byte boundary.
 */
bsb_status bsb_grouped_gemm_w8a8_g128_gather(const int8_t *q, const float *sa,
                                             const int32_t *index, int64_t T,
                                             const int8_t *qw, const float *sw,
                                             const int32_t *offsets,
                                             int64_t E, int64_t R, int64_t N, int64_t K,
                                             void *y, bsb_out_dtype out, void *stream);

/*
 * The routes the pages run beside W8A8 ([P1] sec. 1-2): weight-only INT8
 * ("WNA16": INT8 weights with the per-group scales above, BF16 activations)
 * and BF16 weights dequantised from FP8 at load time. Both take BF16
 * activations as they are (no activation quantisation); up to 64 rows the
 * weights are streamed once (decode-shaped M), beyond that 128x128 output
 * tiles are used:
 *     W8A16: y[m,n] = sum_g sw[n,g] * sum_{k in g} x[m,k] * qw[n,k]
 *     BF16:  y[m,n] = sum_k x[m,k] * w[n,k]
 * Products are exact in float32; the matrix core sums each group's 128
 * products in float32 in its own order, and group sums are combined in group
 * order (a fused multiply-add with sw[n,g], or a float32 add), so results are
 * within (127 + G) * 2^-24 * sum |terms| of the exact value and do not depend
 * on the launch shape.
 *   x_bf16  [M, K] BF16 bits
 *   qw      [N, K] int8, sw [N, G] float32   (W8A16)
 *   w_bf16  [N, K] BF16 bits                 (BF16)
 *   y       [M, N] BF16 bits or float32 per `out`
 * K a multiple of 128 and below 2^23; other limits and errors as
 * bsb_gemm_w8a8_g128.
 */
bsb_status bsb_gemm_w8a16_g128(const uint16_t *x_bf16, const int8_t *qw, const float *sw,
                               int64_t M, int64_t N, int64_t K,
                               void *y, bsb_out_dtype out, void *stream);

bsb_status bsb_gemm_bf16(const uint16_t *x_bf16, const uint16_t *w_bf16,
                         int64_t M, int64_t N, int64_t K,
                         void *y, bsb_out_dtype out, void *stream);

/*
 * FP8 e4m3 weights with [128,128] UE8M0 block scales -> BF16, the load-time
 * dequantisation of the BF16 route ([P1] sec. 2):
 *     w_bf16[n,k] = RNE_bf16(e4m3_dialect(w[n,k]) * 2^(bs[n/128, k/128] - 127))
 * exact unless the value is a BF16 subnormal. Arguments and limits as
 * bsb_decode_fp8_block; w_bf16 [N, K] BF16 bits (written).
 */
bsb_status bsb_dequant_fp8_block_bf16(const uint8_t *w, const uint8_t *bs,
                                      int64_t N, int64_t K, bsb_fp8_dialect dialect,
                                      uint16_t *w_bf16, void *stream);

/*
 * FP8 e4m3 weights with [128,128] UE8M0 block scales ([P1] sec. 1) ->
 * INT8 per-group-128 ([P1] sec. 2 repack onto the INT8 path). The dialect is
 * explicit: the same bytes read as OCP are exactly twice their fnuz reading
 * ([P2] "FP8 dialect clash").
 *     W[n,k]  = e4m3_dialect(w[n,k]) * 2^(bs[n/128, k/128] - 127)
 *     then per (n, g) the rule of bsb_quantize_act over W[n, 128g .. 128g+127]
 *   w   [N, K] uint8 e4m3 bytes; N % 128 == 0
 *   bs  [N/128, K/128] uint8 UE8M0 exponents (255 = NaN: outside the domain)
 *   qw  [N, K] int8, sw [N, G] float32 (written)
 * Bytes that the dialect defines as NaN are outside the domain.
 */
bsb_status bsb_decode_fp8_block(const uint8_t *w, const uint8_t *bs,
                                int64_t N, int64_t K, bsb_fp8_dialect dialect,
                                int8_t *qw, float *sw, void *stream);

/*
 * FP8 [128,128]-block weights decoded to INT8 per-group-128 ([P1] sec. 1-2; the
 * dialect as in [P2] "FP8 dialect clash") with the INT8 weight written straight
 * into the matrix cores' operand order of bsb_repack_weights_mfma, the one
 * load-time rearrangement [P1] sec. 2 describes done in the same pass as the
 * decode: packed = bsb_repack_weights_mfma(qw) of the qw that
 * bsb_decode_fp8_block writes; sw is the same [N, G] array. Arguments, limits
 * and errors as bsb_decode_fp8_block; packed [N*K] int8 (written).
 */
bsb_status bsb_decode_fp8_block_packed(const uint8_t *w, const uint8_t *bs,
                                       int64_t N, int64_t K, bsb_fp8_dialect dialect,
                                       int8_t *packed, float *sw, void *stream);

/*
 * MXFP4 (E2M1 elements, 1x32 UE8M0 block scales along K) experts ([P1]
 * sec. 1) -> INT8 per-group-128 ([P1] sec. 2).
 *     W[e,n,k] = E2M1(nibble k of row (e,n)) * 2^(scale[e,n,k/32] - 127)
 *     then per (e, n, g) the rule of bsb_quantize_act
 *   packed [E, N, K/2] uint8: element 2j in the low nibble of byte j,
 *          element 2j+1 in the high nibble
 *   scale  [E, N, K/32] uint8 UE8M0 exponents
 *   qw     [E, N, K] int8, sw [E, N, G] float32 (written)
 */
bsb_status bsb_decode_mxfp4(const uint8_t *packed, const uint8_t *scale,
                            int64_t E, int64_t N, int64_t K,
                            int8_t *qw, float *sw, void *stream);

/*
 * MXFP4 experts ([P1] sec. 1: E2M1 elements with one UE8M0 exponent per 32
 * along K) decoded to INT8 per-group-128 with the INT8 weight written in the
 * matrix cores' operand order, ready for bsb_grouped_gemm_w8a8_g128_packed:
 * the decode of bsb_decode_mxfp4 and the load-time rearrangement of [P1]
 * sec. 2 in one pass. packed_qw = bsb_repack_weights_mfma of the stacked
 * [E*N, K] qw that bsb_decode_mxfp4 writes (expert e's block at e*N*K);
 * sw is the same [E, N, G] array.
 *   N a multiple of 16; other arguments, limits and errors as bsb_decode_mxfp4;
 *   packed_qw [E*N*K] int8 (written).
 */
bsb_status bsb_decode_mxfp4_packed(const uint8_t *packed, const uint8_t *scale,
                                   int64_t E, int64_t N, int64_t K,
                                   int8_t *packed_qw, float *sw, void *stream);

/*
 * Inspection form of bsb_gemm_w8a8_g128 for tests: the same kernels and
 * main loop selected by the same M, with the epilogue replaced by a store of
 * the exact INT32 group partials ([P3] sec. 3.1 INT32 accumulator).
 *   P [M, N, G] int32 (written)
 */
bsb_status bsb_gemm_w8a8_g128_partials(const int8_t *q, const int8_t *qw,
                                       int64_t M, int64_t N, int64_t K,
                                       int32_t *P, void *stream);

/*
 * MoE dispatch on one GPU ([P3] sec. 1.3 / 4.4: tokens are sent to the
 * experts they selected): gather quantised token rows into expert order.
 *     q_out[r, :] = q[index[r], :],  sa_out[r] = sa[index[r]]
 * Quantising T tokens with bsb_quantize_act and gathering gives the same
 * bits as quantising the R gathered BF16 rows (the rule works per row).
 *   q      [T, K] int8, sa [T] float32 (bsb_quantize_act's outputs)
 *   index  [R] int32 token of each sorted row (values outside [0, T) are
 *          outside the domain: that row is written as zeros with scale 0)
 *   q_out  [R, K] int8, sa_out [R] float32 (written)
 */
bsb_status bsb_gather_rows(const int8_t *q, const float *sa, const int32_t *index,
                           int64_t R, int64_t T, int64_t K,
                           int8_t *q_out, float *sa_out, void *stream);

/*
 * MoE combine ([P3] sec. 4.4: the experts' outputs come back to their token):
 *     out[t, :] = sum_{k = 0 .. topk-1} gate[t, k] * y[row_of_pair[t, k], :]
 * in float32, one fused multiply-add per slot with k ascending from 0, then
 * BF16 round to nearest even.
 *   y            [R, N] BF16 bits: the grouped GEMM's output rows
 *   row_of_pair  [T, topk] int32: the sorted row of token t's k-th expert
 *                (values outside [0, R) are outside the domain and add nothing)
 *   gate         [T, topk] float32 router weights
 *   out          [T, N] BF16 bits (written); N % 8 == 0, 1 <= topk <= 256
 */
bsb_status bsb_moe_combine(const uint16_t *y, const int32_t *row_of_pair,
                           const float *gate, int64_t T, int64_t topk,
                           int64_t R, int64_t N, uint16_t *out, void *stream);

/*
 * INT8 KV cache ([P3] sec. 2.2 / 3.4): one dynamic scale per key vector and
 * per value vector (one token of one KV head, D = 128 values), taken on write
 * by the rule of bsb_quantize_act over those 128 values.
 * Cache layout (T = token slots per sequence, a multiple of 64, 64 <= T < 2^24):
 *   k_cache [T/64, B, Hkv, 8192] int8: row (c, b, h) holds tokens 64c .. 64c+63
 *           of sequence b, KV head h (the same chunk of every sequence and head
 *           is adjacent, which is the order the attention reads them in), as
 *           four blocks of 16 tokens, 2048 bytes each; token tau of a block and
 *           dimension d sit at byte
 *           ((d/16)%2)*1024 + ((d/32)*16 + tau)*16 + d%16 of the block
 *   v_cache [T/64, B, Hkv, 8192] int8: rows as k_cache, each two blocks of 32
 *           tokens, 4096 bytes each; token tau of a block and dimension d sit
 *           at byte (d/32)*1024 + (((tau%16)/4)*16 + d%16)*16 + ((d/16)%2)*8 +
 *           (tau/16)*4 + tau%4 of the block
 *   k_scale, v_scale [B, Hkv, T] float32
 * The caller allocates and owns every buffer; nothing is written outside the
 * slots named by (seq, pos).
 */

/*
 * Write n new tokens' keys and values into the cache, quantised.
 *   k_bf16, v_bf16 [n, Hkv, 128] BF16 bits
 *   seq, pos [n] int32 (device): token i goes to sequence seq[i], slot pos[i];
 *            entries outside [0, B) x [0, T) are skipped (nothing written);
 *            two entries naming the same slot race.
 * n == 0 is a no-op. D must be 128, else BSB_ERR_INVALID_ARG.
 */
bsb_status bsb_kv_cache_write(const uint16_t *k_bf16, const uint16_t *v_bf16,
                              const int32_t *seq, const int32_t *pos, int64_t n,
                              int64_t B, int64_t Hkv, int64_t T, int64_t D,
                              int8_t *k_cache, float *k_scale,
                              int8_t *v_cache, float *v_scale, void *stream);

/*
 * Bytes of float32 workspace bsb_attention_decode_int8kv needs:
 * B * Hq * ceil(max_len / 512) * 130 * 4.
 */
int64_t bsb_attention_workspace_bytes(int64_t B, int64_t Hq, int64_t max_len);

/*
 * Decode attention of one query token per sequence over the INT8 cache, the
 * dequantisation fused into the kernel ([P3] sec. 3.4, sec. 4.1):
 *     K[t,d] = k_scale[t] * k_cache[t,d],  V[t,d] = v_scale[t] * v_cache[t,d]
 *     z[t] = q . K[t] / sqrt(128),  w = softmax(z over t < lens[b]),
 *     out[b, h, :] = sum_t w[t] * V[t, :]
 * query head h reads KV head h / (Hq / Hkv); lens[b] == 0 gives zeros. The
 * matrix cores take the BF16 query and the INT8 codes converted exactly to
 * BF16, with float32 accumulation; scores, exponentials and sums are float32;
 * the weights times the value scales enter the P.V product rounded to BF16.
 * Results are within 2^-7 * sum_t w[t] |V[t,d]| of the exact value (plus
 * 2^-8 of that for a BF16 output) for score terms sum_d |q[d] K[t,d]| / sqrt(128)
 * up to ~100.
 *   q_bf16   [B, Hq, 128] BF16 bits; 1 <= Hq / Hkv <= 16, Hq % Hkv == 0
 *   lens     [B] int32 (device): cached tokens per sequence; values are
 *            clamped to [0, min(max_len, T)] (tokens past max_len are not read)
 *   max_len  host bound on lens that sizes the launch, 0 <= max_len <= T
 *   work     float32 scratch of bsb_attention_workspace_bytes(B, Hq, max_len)
 *            bytes (contents on entry ignored); work_bytes its size
 *   out      [B, Hq, 128] BF16 bits or float32 per `out_dtype` (written)
 * B * Hkv <= 65535, B * Hq < 2^31; other errors as bsb_gemm_w8a8_g128.
 */
bsb_status bsb_attention_decode_int8kv(const uint16_t *q_bf16,
                                       const int8_t *k_cache, const float *k_scale,
                                       const int8_t *v_cache, const float *v_scale,
                                       const int32_t *lens, int64_t B, int64_t Hq,
                                       int64_t Hkv, int64_t T, int64_t D, int64_t max_len,
                                       float *work, int64_t work_bytes,
                                       void *out, bsb_out_dtype out_dtype, void *stream);

/*
 * Attention of several query tokens per sequence over the INT8 cache: the
 * blockwise attention of [P3] sec. 4.1 with the dequantisation fused as in
 * bsb_attention_decode_int8kv, for chunked prefill or for checking drafted
 * tokens. The Qn query tokens of sequence b are its newest Qn tokens, at
 * positions lens[b] - Qn .. lens[b] - 1, whose keys and values are already in
 * the cache; query i attends to tokens 0 .. lens[b] - Qn + i (causal):
 *     out[b, i, h, :] = the attention of bsb_attention_decode_int8kv for
 *                       query q[b, i, h, :] over tokens t <= lens[b] - Qn + i
 * and a query with no such token (lens[b] < Qn - i) gives zeros. All Qn
 * queries of a sequence share one read of its cache.
 *   q_bf16   [B, Qn, Hq, 128] BF16 bits; 1 <= Qn and Qn * Hq / Hkv <= 16
 *   work     float32 scratch of bsb_attention_workspace_bytes(B, Qn * Hq,
 *            max_len) bytes; work_bytes its size
 *   out      [B, Qn, Hq, 128] BF16 bits or float32 per `out_dtype` (written)
 * Other arguments, the bound and the errors as bsb_attention_decode_int8kv
 * (B * Qn * Hq < 2^31).
 */
bsb_status bsb_attention_chunk_int8kv(const uint16_t *q_bf16,
                                      const int8_t *k_cache, const float *k_scale,
                                      const int8_t *v_cache, const float *v_scale,
                                      const int32_t *lens, int64_t B, int64_t Qn, int64_t Hq,
                                      int64_t Hkv, int64_t T, int64_t D, int64_t max_len,
                                      float *work, int64_t work_bytes,
                                      void *out, bsb_out_dtype out_dtype, void *stream);

/*
 * bsb_attention_decode_int8kv for callers that cannot allocate: code under
 * HIP graph capture, tight serving loops and harnesses that forbid hipMalloc.
 * Same arguments, arithmetic and results (bit for bit) without the workspace:
 * the split partials live in a static array of BSB_ATTENTION_NOALLOC_MAX_BYTES
 * that each device the library runs on holds until the process ends, found
 * on the first call on a device (with that device current). The call
 * allocates and frees nothing. Sizes whose workspace,
 * bsb_attention_workspace_bytes(B, Hq, max_len), exceeds the limit return
 * BSB_ERR_INVALID_ARG and launch nothing. Calls on one device share the array:
 * calls that overlap on a device (different streams, or graphs replayed
 * concurrently) race and give undefined outputs; serialise them. Every value
 * the call reads back from the array is written earlier in the same call.
 */
#define BSB_ATTENTION_NOALLOC_MAX_BYTES ((int64_t)32 << 20)

bsb_status bsb_attention_decode_int8kv_noalloc(const uint16_t *q_bf16,
                                               const int8_t *k_cache, const float *k_scale,
                                               const int8_t *v_cache, const float *v_scale,
                                               const int32_t *lens, int64_t B, int64_t Hq,
                                               int64_t Hkv, int64_t T, int64_t D,
                                               int64_t max_len, void *out,
                                               bsb_out_dtype out_dtype, void *stream);

/*
 * The comparison route of the INT8 KV cache: the same cache and attention with
 * BF16 keys and values (no scales, nothing quantised), the cache the INT8 one
 * replaces ([P3] sec. 2.2 counts it at 2 bytes per element).
 * Cache layout (T as above):
 *   k_cache [T/64, B, Hkv, 8192] BF16 bits: rows as the INT8 cache, each four
 *           blocks of 16 tokens (2048 elements); token tau and dimension d at
 *           element ((d/8)%4)*512 + ((d/32)*16 + tau)*8 + d%8 of the block
 *   v_cache [T/64, B, Hkv, 8192] BF16 bits: rows of two blocks of 32 tokens
 *           (4096 elements); token tau and dimension d at element
 *           (d/16)*512 + (((tau%16)/4)*16 + d%16)*8 + (tau/16)*4 + tau%4
 * bsb_kv_cache_write_bf16 copies n tokens' keys and values into their slots
 * (arguments as bsb_kv_cache_write, without scales);
 * bsb_attention_decode_bf16kv computes the attention of
 * bsb_attention_decode_int8kv with K and V the cached BF16 values (arguments,
 * workspace, bound and errors as there).
 */
bsb_status bsb_kv_cache_write_bf16(const uint16_t *k_bf16, const uint16_t *v_bf16,
                                   const int32_t *seq, const int32_t *pos, int64_t n,
                                   int64_t B, int64_t Hkv, int64_t T, int64_t D,
                                   uint16_t *k_cache, uint16_t *v_cache, void *stream);

bsb_status bsb_attention_decode_bf16kv(const uint16_t *q_bf16,
                                       const uint16_t *k_cache, const uint16_t *v_cache,
                                       const int32_t *lens, int64_t B, int64_t Hq,
                                       int64_t Hkv, int64_t T, int64_t D, int64_t max_len,
                                       float *work, int64_t work_bytes,
                                       void *out, bsb_out_dtype out_dtype, void *stream);

/*
 * Measurement probes. Not steps of the method: they measure what this part
 * sustains, so that the benchmark can state its rooflines against measured
 * ceilings beside the published peaks ([P3] sec. 4.1 and its sec. 6
 * checklist: confirm by measurement what the INT8 path really achieves).
 * Each launches BSB_PROBE_THREADS threads, and each thread writes one int32 of
 * `out` (a value derived from what it read or computed, so nothing is skipped).
 *
 * bsb_probe_mfma_i8: only v_mfma_i32_32x32x32_i8, two waves per SIMD on 256
 * compute units, rounds * 64 MFMAs per wave; ops = BSB_PROBE_THREADS / 64 *
 * rounds * 64 * 65536. Operands are 16-byte chunks of `a` and `b` (each
 * `bytes` long), so the rate reflects those bytes (the matrix cores draw more
 * power on dense bit patterns and the clock follows).
 *   bytes a multiple of 16, 16 .. 2^31;  1 <= rounds <= 2^24
 * bsb_probe_mfma_i8_epilogue: the same MFMA stream (same ops, same operand
 * bytes and sizes) with the per-group epilogue of the W8A8-g128 GEMMs beside
 * it ([P3] sec. 3.1: the INT32 group sum converted and scaled in float32 per
 * 128-wide K group): after every MFMA, 4 conversions and 4 fused multiply-adds
 * of the previous 32x32 block into float32 totals, with no memory traffic.
 * Its rate is what the matrix cores keep beside the epilogue that the
 * per-group scales require; out as bsb_probe_mfma_i8.
 * bsb_probe_hbm_read: reads `bytes` of src once, 16 bytes per lane, four
 * loads in flight per lane, non-temporal.
 *   bytes a multiple of 16 * BSB_PROBE_THREADS (2 MiB), at most 2^40
 * out [BSB_PROBE_THREADS] int32 (written). Errors as bsb_gemm_w8a8_g128.
 * bsb_probe_hbm_copy: the same walk copying src to dst (`bytes` read and
 * `bytes` written, non-temporal loads and stores): a read + write stream.
 * Sizes as bsb_probe_hbm_read; src and dst must not overlap (the copied values
 * are otherwise unspecified); nothing is written to `out`.
 */
#define BSB_PROBE_THREADS 131072

bsb_status bsb_probe_mfma_i8(const int8_t *a, const int8_t *b, int64_t bytes, int64_t rounds,
                             int32_t *out, void *stream);

bsb_status bsb_probe_mfma_i8_epilogue(const int8_t *a, const int8_t *b, int64_t bytes,
                                      int64_t rounds, int32_t *out, void *stream);

bsb_status bsb_probe_hbm_read(const void *src, int64_t bytes, int32_t *out, void *stream);

bsb_status bsb_probe_hbm_copy(const void *src, void *dst, int64_t bytes, void *stream);

/* Static, human-readable name of a status code (never NULL). */
const char *bsb_status_string(bsb_status s);

/* ABI version of this header; bumped on any incompatible change. */
int bsb_abi_version(void);

#define BSB_ABI_VERSION 1

#ifdef __cplusplus
}
#endif

#endif /* BSB_H */
