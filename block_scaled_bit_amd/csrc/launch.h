// Host-side launchers of the gfx950 kernels (internal to libbsb).
// Arguments have been validated by the C-ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsb {

hipError_t launch_quantize_act(const uint16_t *x, int64_t M, int64_t K, int8_t *q,
                               float *sa, hipStream_t stream);

hipError_t launch_decode_fp8_block(const uint8_t *w, const uint8_t *bs, int64_t N,
                                   int64_t K, int fnuz, int8_t *qw, float *sw,
                                   hipStream_t stream, bool packed = false);

// FP8 e4m3 [N,K] with [N/128, K/128] UE8M0 block scales -> BF16 bits [N,K].
hipError_t launch_dequant_fp8_block_bf16(const uint8_t *w, const uint8_t *bs, int64_t N,
                                         int64_t K, int fnuz, uint16_t *out, hipStream_t stream);

hipError_t launch_decode_mxfp4(const uint8_t *packed, const uint8_t *scale, int64_t E,
                               int64_t N, int64_t K, int8_t *qw, float *sw,
                               hipStream_t stream, bool packed_out = false);

// out: 0 = BF16, 1 = FP32, 2 = INT32 group partials [M, N, G]
hipError_t launch_gemm(const int8_t *q, const float *sa, const int8_t *qw,
                       const float *sw, int64_t M, int64_t N, int64_t K, void *y,
                       int out, hipStream_t stream);

// gemm_big.hip: 256x256 tiles for prefill-shaped M. out as gemm_common.h's
// OUT_* forms; offsets non-null selects the grouped form (BF16 / FP32 only);
// with gidx non-null as well, q / sa are T tokens and row m is token gidx[m]
// (T * K < 2^31).
bool big_gemm_fits(int64_t K);
hipError_t launch_gemm_big(const int8_t *q, const float *sa, const int8_t *qw, const float *sw,
                           int M, int N, int K, void *y, int out, const int32_t *offsets, int E,
                           int sw_stride, hipStream_t stream, const int32_t *gidx = nullptr,
                           int T = 0);
// gemm_mid.hip: 128x128 tiles for mid-sized M (same arguments and forms)
bool mid_gemm_fits(int64_t K);
hipError_t launch_gemm_mid(const int8_t *q, const float *sa, const int8_t *qw, const float *sw,
                           int M, int N, int K, void *y, int out, const int32_t *offsets, int E,
                           int sw_stride, hipStream_t stream, const int32_t *gidx = nullptr,
                           int T = 0);

// gemm_a16.hip: BF16 activations beyond 64 rows, 128x128 tiles; am 1 = INT8
// weights with group scales (W8A16), 2 = BF16 weights
bool a16_tiles_fit(int64_t K);
hipError_t launch_gemm_a16_tiles(const uint16_t *x, const void *w, const float *sw, int M, int N,
                                 int K, void *y, int out, int am, hipStream_t stream);

// gemm_packed.hip: weights in the matrix cores' operand order (M <= 64)
hipError_t launch_repack_mfma(const int8_t *qw, int64_t N, int64_t K, int8_t *packed,
                              hipStream_t stream);
hipError_t launch_grouped_gemm_packed(const int8_t *q, const float *sa, const int8_t *packed,
                                      const float *sw, const int32_t *offsets, int64_t E,
                                      int64_t R, int64_t N, int64_t K, void *y, int out,
                                      hipStream_t stream);
hipError_t launch_gemm_packed(const int8_t *q, const float *sa, const int8_t *packed,
                              const float *sw, int64_t M, int64_t N, int64_t K, void *y, int out,
                              hipStream_t stream);

// Per-channel (sw_stride 1, sw[N]) or per-tensor (sw_stride 0, sw[1]) weight
// scales: out 0 = BF16, 1 = FP32.
hipError_t launch_gemm_channel(const int8_t *q, const float *sa, const int8_t *qw,
                               const float *sw, int64_t sw_stride, int64_t M, int64_t N,
                               int64_t K, void *y, int out, hipStream_t stream);

// BF16 activations x [M,K], M <= 64: am 1 = W8A16 (w INT8 [N,K], sw [N,K/128]),
// am 2 = BF16 weights (w BF16 bits [N,K], no scales); out 0 = BF16, 1 = FP32.
hipError_t launch_gemm_a16(const uint16_t *x, const void *w, const float *sw, int64_t M,
                           int64_t N, int64_t K, void *y, int out, int am, hipStream_t stream);

// gidx non-null: q / sa are T quantised tokens, row r of the grouped problem
// is token gidx[r] (an index outside [0, T) reads a zero row with scale 0)
hipError_t launch_grouped_gemm(const int8_t *q, const float *sa, const int8_t *qw,
                               const float *sw, const int32_t *offsets, int64_t E,
                               int64_t R, int64_t N, int64_t K, void *y, int out,
                               hipStream_t stream, const int32_t *gidx = nullptr, int64_t T = 0);

hipError_t launch_gather_rows(const int8_t *q, const float *sa, const int32_t *index, int64_t R,
                              int64_t T, int64_t K, int8_t *q_out, float *sa_out,
                              hipStream_t stream);

hipError_t launch_moe_combine(const uint16_t *y, const int32_t *row_of_pair, const float *gate,
                              int64_t T, int64_t topk, int64_t R, int64_t N, uint16_t *out,
                              hipStream_t stream);

// INT8 KV cache (head dimension 128): quantise-on-write and decode attention.
int64_t attention_splits(int64_t max_len);
int64_t attention_workspace_floats(int64_t B, int64_t Hq, int64_t max_len);

hipError_t launch_kv_cache_write(const uint16_t *k, const uint16_t *v, const int32_t *seq,
                                 const int32_t *pos, int64_t n, int B, int Hkv, int T, int8_t *kc,
                                 float *ks, int8_t *vc, float *vs, hipStream_t stream);

hipError_t launch_attention_decode(const uint16_t *q, const int8_t *kc, const float *ks,
                                   const int8_t *vc, const float *vs, const int32_t *lens, int B,
                                   int Hq, int Hkv, int T, int max_len, float *work, void *out,
                                   int out_bf16, hipStream_t stream);

// Attention of the Qn newest tokens of each sequence (causal), Qn * Hq / Hkv <= 16;
// q and out [B, Qn, Hq, 128]; work: attention_workspace_floats(B, Qn * Hq, max_len).
hipError_t launch_attention_chunk(const uint16_t *q, const int8_t *kc, const float *ks,
                                  const int8_t *vc, const float *vs, const int32_t *lens, int B,
                                  int Qn, int Hq, int Hkv, int T, int max_len, float *work,
                                  void *out, int out_bf16, hipStream_t stream);

// The same attention with its split partials in a static per-device array of
// kNoAllocScratchBytes (no workspace argument, nothing allocated); sizes whose
// workspace exceeds it are rejected by the caller.
constexpr int64_t kNoAllocScratchBytes = (int64_t)32 << 20;
hipError_t launch_attention_decode_noalloc(const uint16_t *q, const int8_t *kc, const float *ks,
                                           const int8_t *vc, const float *vs, const int32_t *lens,
                                           int B, int Hq, int Hkv, int T, int max_len, void *out,
                                           int out_bf16, hipStream_t stream);

// probe.hip: measurement probes (threads per launch; each writes one int32 to out)
constexpr int kProbeThreads = 131072;
hipError_t launch_probe_mfma_i8(const int8_t *a, const int8_t *b, int64_t bytes, int64_t rounds,
                                int32_t *out, hipStream_t stream);
hipError_t launch_probe_mfma_i8_epilogue(const int8_t *a, const int8_t *b, int64_t bytes, int64_t rounds,
                                int32_t *out, hipStream_t stream);
hipError_t launch_probe_hbm_read(const void *src, int64_t bytes, int32_t *out,
                                 hipStream_t stream);
hipError_t launch_probe_hbm_copy(const void *src, void *dst, int64_t bytes, hipStream_t stream);

// The BF16 KV cache of the comparison route (same blocks, 2-byte elements, no scales).
hipError_t launch_kv_cache_write_bf16(const uint16_t *k, const uint16_t *v, const int32_t *seq,
                                      const int32_t *pos, int64_t n, int B, int Hkv, int T,
                                      uint16_t *kc, uint16_t *vc, hipStream_t stream);

hipError_t launch_attention_decode_bf16kv(const uint16_t *q, const uint16_t *kc,
                                          const uint16_t *vc, const int32_t *lens, int B, int Hq,
                                          int Hkv, int T, int max_len, float *work, void *out,
                                          int out_bf16, hipStream_t stream);

}  // namespace bsb
