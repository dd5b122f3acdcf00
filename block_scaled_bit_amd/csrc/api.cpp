// C ABI of libbsb: argument validation, device check, dispatch to the gfx950
// kernels. Every entry point validates before it launches anything and
// returns a status code; nothing here allocates, synchronises or reads
// device memory.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "../../include/bsb.h"
#include "launch.h"

static_assert(BSB_ATTENTION_NOALLOC_MAX_BYTES == bsb::kNoAllocScratchBytes,
              "the header's limit is the size of the static workspace");

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other architecture
std::atomic<int> g_arch_state[kMaxDevices];

bsb_status check_device() noexcept {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return BSB_ERR_UNSUPPORTED_DEVICE;
    if (dev >= kMaxDevices) return BSB_ERR_UNSUPPORTED_DEVICE;
    int st = g_arch_state[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return BSB_ERR_UNSUPPORTED_DEVICE;
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_arch_state[dev].store(st, std::memory_order_relaxed);
    }
    return st == 1 ? BSB_OK : BSB_ERR_UNSUPPORTED_DEVICE;
}

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Largest extents the 32-bit index arithmetic inside the kernels accepts.
constexpr int64_t kMaxDim = (int64_t)1 << 30;
constexpr int64_t kMaxElems = (int64_t)1 << 36;
constexpr int64_t kMaxPackedK = (int64_t)1 << 24;

// a * b * c <= limit for positive extents, without overflowing int64.
inline bool prod_le(int64_t a, int64_t b, int64_t c, int64_t limit) {
    return a >= 1 && b >= 1 && c >= 1 && a <= limit && b <= limit / a && c <= limit / (a * b);
}

// The decoders index 16-byte chunks with 32-bit arithmetic: N*K/16 plus one
// workgroup of slack must stay below 2^32.
constexpr int64_t kMaxDecodeElems = (int64_t)1 << 35;

// K accepted by the per-channel / per-tensor GEMM: its INT32 total over the
// whole of K stays in range (127 * 127 * 131072 < 2^31).
constexpr int64_t kMaxChannelK = 131072;

// K accepted by the row-major W8A8 GEMMs: the kernels address a 128-row operand
// panel with 32-bit buffer offsets (128 * K + 128 < 2^31).
constexpr int64_t kGemmKLimit = (int64_t)1 << 24;   // K must be below it

// Experts per token accepted by the combine.
constexpr int64_t kMaxTopk = 256;

// KV cache: head dimension, and token slots per sequence (kept well inside
// the 32-bit token arithmetic of the attention kernel).
constexpr int64_t kKvHeadDim = 128;
constexpr int64_t kMaxKvSlots = (int64_t)1 << 24;

inline bool dims_ok(int64_t rows, int64_t N, int64_t K) {
    return rows >= 0 && N >= 1 && K >= 128 && (K % 128) == 0 && rows < kMaxDim && N < kMaxDim &&
           K < kMaxDim;
}

inline bsb_status finish(hipError_t e) noexcept { return e == hipSuccess ? BSB_OK : BSB_ERR_LAUNCH; }

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int bsb_abi_version(void) { return BSB_ABI_VERSION; }

const char *bsb_status_string(bsb_status s) {
    switch (s) {
        case BSB_OK: return "BSB_OK";
        case BSB_ERR_INVALID_ARG: return "BSB_ERR_INVALID_ARG: invalid argument";
        case BSB_ERR_UNSUPPORTED_DEVICE: return "BSB_ERR_UNSUPPORTED_DEVICE: current device is not gfx950";
        case BSB_ERR_MISALIGNED: return "BSB_ERR_MISALIGNED: pointer not 16-byte aligned";
        case BSB_ERR_LAUNCH: return "BSB_ERR_LAUNCH: kernel launch failed";
    }
    return "BSB_ERR_UNKNOWN";
}

bsb_status bsb_quantize_act(const uint16_t *x_bf16, int64_t M, int64_t K, int8_t *q, float *sa,
                            void *stream) {
    if (M < 0 || M >= kMaxDim || K < 128 || K % 128 || K >= kMaxDim) return BSB_ERR_INVALID_ARG;
    if (M == 0) return BSB_OK;
    if (!x_bf16 || !q || !sa) return BSB_ERR_INVALID_ARG;
    if (!aligned16(x_bf16) || !aligned16(q) || !aligned16(sa)) return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_quantize_act(x_bf16, M, K, q, sa, as_stream(stream)));
}

bsb_status bsb_gemm_w8a8_g128(const int8_t *q, const float *sa, const int8_t *qw, const float *sw,
                              int64_t M, int64_t N, int64_t K, void *y, bsb_out_dtype out,
                              void *stream) {
    if (!dims_ok(M, N, K) || N * K > kMaxElems || K >= kGemmKLimit) return BSB_ERR_INVALID_ARG;
    if (out != BSB_OUT_BF16 && out != BSB_OUT_FP32) return BSB_ERR_INVALID_ARG;
    if (M == 0) return BSB_OK;
    if (!q || !sa || !qw || !sw || !y) return BSB_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(sa) || !aligned16(qw) || !aligned16(sw) || !aligned16(y))
        return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_gemm(q, sa, qw, sw, M, N, K, y, (int)out, as_stream(stream)));
}

bsb_status bsb_repack_weights_mfma(const int8_t *qw, int64_t N, int64_t K, int8_t *packed,
                                   void *stream) {
    if (!dims_ok(0, N, K) || N % 16 || N * K > kMaxElems) return BSB_ERR_INVALID_ARG;
    if (!qw || !packed) return BSB_ERR_INVALID_ARG;
    if (!aligned16(qw) || !aligned16(packed)) return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_repack_mfma(qw, N, K, packed, as_stream(stream)));
}

bsb_status bsb_gemm_w8a8_g128_packed(const int8_t *q, const float *sa, const int8_t *packed,
                                     const float *sw, int64_t M, int64_t N, int64_t K, void *y,
                                     bsb_out_dtype out, void *stream) {
    // 32-bit buffer offsets: 64 activation rows of K bytes, 16*K weight bytes per wave
    if (!dims_ok(M, N, K) || N % 16 || M > 64 || K > kMaxPackedK || N * K > kMaxElems)
        return BSB_ERR_INVALID_ARG;
    if (out != BSB_OUT_BF16 && out != BSB_OUT_FP32) return BSB_ERR_INVALID_ARG;
    if (M == 0) return BSB_OK;
    if (!q || !sa || !packed || !sw || !y) return BSB_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(sa) || !aligned16(packed) || !aligned16(sw) || !aligned16(y))
        return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_gemm_packed(q, sa, packed, sw, M, N, K, y, (int)out,
                                          as_stream(stream)));
}

bsb_status bsb_grouped_gemm_w8a8_g128_packed(const int8_t *q, const float *sa,
                                             const int8_t *packed, const float *sw,
                                             const int32_t *offsets, int64_t E, int64_t R,
                                             int64_t N, int64_t K, void *y, bsb_out_dtype out,
                                             void *stream) {
    if (!dims_ok(R, N, K) || N % 16 || K > kMaxPackedK || E < 1 || E > 65535 ||
        !prod_le(E, N, K, kMaxElems))
        return BSB_ERR_INVALID_ARG;
    if (out != BSB_OUT_BF16 && out != BSB_OUT_FP32) return BSB_ERR_INVALID_ARG;
    if (R == 0) return BSB_OK;
    if (!q || !sa || !packed || !sw || !offsets || !y) return BSB_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(sa) || !aligned16(packed) || !aligned16(sw) ||
        !aligned16(offsets) || !aligned16(y))
        return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_grouped_gemm_packed(q, sa, packed, sw, offsets, E, R, N, K, y,
                                                  (int)out, as_stream(stream)));
}

bsb_status bsb_gemm_w8a8_channel(const int8_t *q, const float *sa, const int8_t *qw,
                                 const float *sw, int64_t sw_stride, int64_t M, int64_t N,
                                 int64_t K, void *y, bsb_out_dtype out, void *stream) {
    if (!dims_ok(M, N, K) || N * K > kMaxElems || K > kMaxChannelK) return BSB_ERR_INVALID_ARG;
    if (sw_stride != 0 && sw_stride != 1) return BSB_ERR_INVALID_ARG;
    if (out != BSB_OUT_BF16 && out != BSB_OUT_FP32) return BSB_ERR_INVALID_ARG;
    if (M == 0) return BSB_OK;
    if (!q || !sa || !qw || !sw || !y) return BSB_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(sa) || !aligned16(qw) || !aligned16(y) ||
        (reinterpret_cast<uintptr_t>(sw) & 3))
        return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_gemm_channel(q, sa, qw, sw, sw_stride, M, N, K, y, (int)out,
                                           as_stream(stream)));
}

bsb_status bsb_gemm_w8a8_g128_partials(const int8_t *q, const int8_t *qw, int64_t M, int64_t N,
                                       int64_t K, int32_t *P, void *stream) {
    if (!dims_ok(M, N, K) || N * K > kMaxElems || K >= kGemmKLimit ||
        (M > 0 && !prod_le(M, N, K / 128, kMaxElems)))
        return BSB_ERR_INVALID_ARG;
    if (M == 0) return BSB_OK;
    if (!q || !qw || !P) return BSB_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(qw) || !aligned16(P)) return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_gemm(q, nullptr, qw, nullptr, M, N, K, P, 2, as_stream(stream)));
}

bsb_status bsb_grouped_gemm_w8a8_g128(const int8_t *q, const float *sa, const int8_t *qw,
                                      const float *sw, const int32_t *offsets, int64_t E,
                                      int64_t R, int64_t N, int64_t K, void *y,
                                      bsb_out_dtype out, void *stream) {
    if (!dims_ok(R, N, K) || K >= kGemmKLimit || E < 1 || E >= (1 << 20) ||
        !prod_le(E, N, K, kMaxElems))
        return BSB_ERR_INVALID_ARG;
    if (out != BSB_OUT_BF16 && out != BSB_OUT_FP32) return BSB_ERR_INVALID_ARG;
    if (R == 0) return BSB_OK;
    if (!q || !sa || !qw || !sw || !offsets || !y) return BSB_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(sa) || !aligned16(qw) || !aligned16(sw) ||
        !aligned16(offsets) || !aligned16(y))
        return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_grouped_gemm(q, sa, qw, sw, offsets, E, R, N, K, y, (int)out,
                                           as_stream(stream)));
}

bsb_status bsb_grouped_gemm_w8a8_g128_gather(const int8_t *q, const float *sa,
                                             const int32_t *index, int64_t T, const int8_t *qw,
                                             const float *sw, const int32_t *offsets, int64_t E,
                                             int64_t R, int64_t N, int64_t K, void *y,
                                             bsb_out_dtype out, void *stream) {
    if (!dims_ok(R, N, K) || K >= kGemmKLimit || E < 1 || E >= (1 << 20) ||
        !prod_le(E, N, K, kMaxElems))
        return BSB_ERR_INVALID_ARG;
    // the tokens are addressed through one 32-bit buffer range
    if (T < 1 || T >= kMaxDim || T * K + 128 >= ((int64_t)1 << 31))
        return BSB_ERR_INVALID_ARG;
    if (out != BSB_OUT_BF16 && out != BSB_OUT_FP32) return BSB_ERR_INVALID_ARG;
    if (R == 0) return BSB_OK;
    if (!q || !sa || !index || !qw || !sw || !offsets || !y) return BSB_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(sa) || !aligned16(index) || !aligned16(qw) ||
        !aligned16(sw) || !aligned16(offsets) || !aligned16(y))
        return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_grouped_gemm(q, sa, qw, sw, offsets, E, R, N, K, y, (int)out,
                                           as_stream(stream), index, T));
}

bsb_status bsb_decode_fp8_block(const uint8_t *w, const uint8_t *bs, int64_t N, int64_t K,
                                bsb_fp8_dialect dialect, int8_t *qw, float *sw, void *stream) {
    if (N < 128 || N % 128 || K < 128 || K % 128 || N >= kMaxDim || K >= kMaxDim ||
        N * K > kMaxDecodeElems)
        return BSB_ERR_INVALID_ARG;
    if (dialect != BSB_FP8_OCP && dialect != BSB_FP8_FNUZ) return BSB_ERR_INVALID_ARG;
    if (!w || !bs || !qw || !sw) return BSB_ERR_INVALID_ARG;
    if (!aligned16(w) || !aligned16(bs) || !aligned16(qw) || !aligned16(sw))
        return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_decode_fp8_block(w, bs, N, K, dialect == BSB_FP8_FNUZ ? 1 : 0, qw,
                                               sw, as_stream(stream)));
}

bsb_status bsb_decode_fp8_block_packed(const uint8_t *w, const uint8_t *bs, int64_t N,
                                       int64_t K, bsb_fp8_dialect dialect, int8_t *packed,
                                       float *sw, void *stream) {
    if (N < 128 || N % 128 || K < 128 || K % 128 || N >= kMaxDim || K >= kMaxDim ||
        N * K > kMaxDecodeElems)
        return BSB_ERR_INVALID_ARG;
    if (dialect != BSB_FP8_OCP && dialect != BSB_FP8_FNUZ) return BSB_ERR_INVALID_ARG;
    if (!w || !bs || !packed || !sw) return BSB_ERR_INVALID_ARG;
    if (!aligned16(w) || !aligned16(bs) || !aligned16(packed) || !aligned16(sw))
        return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_decode_fp8_block(w, bs, N, K, dialect == BSB_FP8_FNUZ ? 1 : 0,
                                               packed, sw, as_stream(stream), true));
}

bsb_status bsb_dequant_fp8_block_bf16(const uint8_t *w, const uint8_t *bs, int64_t N, int64_t K,
                                      bsb_fp8_dialect dialect, uint16_t *w_bf16, void *stream) {
    if (N < 128 || N % 128 || K < 128 || K % 128 || N >= kMaxDim || K >= kMaxDim ||
        N * K > kMaxDecodeElems)
        return BSB_ERR_INVALID_ARG;
    if (dialect != BSB_FP8_OCP && dialect != BSB_FP8_FNUZ) return BSB_ERR_INVALID_ARG;
    if (!w || !bs || !w_bf16) return BSB_ERR_INVALID_ARG;
    if (!aligned16(w) || !aligned16(bs) || !aligned16(w_bf16)) return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_dequant_fp8_block_bf16(w, bs, N, K, dialect == BSB_FP8_FNUZ ? 1 : 0,
                                                     w_bf16, as_stream(stream)));
}

namespace {

// The BF16-activation GEMMs address 128 rows of 2K bytes (weights in the
// decode-shaped kernel, activations in the tiled one) with 32-bit offsets.
bsb_status a16_checks(int64_t M, int64_t N, int64_t K, bsb_out_dtype out) {
    if (!dims_ok(M, N, K) || N * K > kMaxElems || (int64_t)256 * K >= ((int64_t)1 << 31))
        return BSB_ERR_INVALID_ARG;
    if (out != BSB_OUT_BF16 && out != BSB_OUT_FP32) return BSB_ERR_INVALID_ARG;
    return BSB_OK;
}

}  // namespace

bsb_status bsb_gemm_w8a16_g128(const uint16_t *x_bf16, const int8_t *qw, const float *sw,
                               int64_t M, int64_t N, int64_t K, void *y, bsb_out_dtype out,
                               void *stream) {
    if (bsb_status s = a16_checks(M, N, K, out)) return s;
    if (M == 0) return BSB_OK;
    if (!x_bf16 || !qw || !sw || !y) return BSB_ERR_INVALID_ARG;
    if (!aligned16(x_bf16) || !aligned16(qw) || !aligned16(sw) || !aligned16(y))
        return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_gemm_a16(x_bf16, qw, sw, M, N, K, y, (int)out, 1, as_stream(stream)));
}

bsb_status bsb_gemm_bf16(const uint16_t *x_bf16, const uint16_t *w_bf16, int64_t M, int64_t N,
                         int64_t K, void *y, bsb_out_dtype out, void *stream) {
    if (bsb_status s = a16_checks(M, N, K, out)) return s;
    if (M == 0) return BSB_OK;
    if (!x_bf16 || !w_bf16 || !y) return BSB_ERR_INVALID_ARG;
    if (!aligned16(x_bf16) || !aligned16(w_bf16) || !aligned16(y)) return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_gemm_a16(x_bf16, w_bf16, nullptr, M, N, K, y, (int)out, 2,
                                       as_stream(stream)));
}

bsb_status bsb_decode_mxfp4(const uint8_t *packed, const uint8_t *scale, int64_t E, int64_t N,
                            int64_t K, int8_t *qw, float *sw, void *stream) {
    if (E < 1 || N < 1 || K < 128 || K % 128 || E >= kMaxDim || N >= kMaxDim || K >= kMaxDim ||
        !prod_le(E, N, K, kMaxDecodeElems))
        return BSB_ERR_INVALID_ARG;
    if (!packed || !scale || !qw || !sw) return BSB_ERR_INVALID_ARG;
    if (!aligned16(packed) || !aligned16(scale) || !aligned16(qw) || !aligned16(sw))
        return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_decode_mxfp4(packed, scale, E, N, K, qw, sw, as_stream(stream)));
}

bsb_status bsb_decode_mxfp4_packed(const uint8_t *packed, const uint8_t *scale, int64_t E,
                                   int64_t N, int64_t K, int8_t *packed_qw, float *sw,
                                   void *stream) {
    if (E < 1 || N < 16 || N % 16 || K < 128 || K % 128 || E >= kMaxDim || N >= kMaxDim ||
        K >= kMaxDim || !prod_le(E, N, K, kMaxDecodeElems))
        return BSB_ERR_INVALID_ARG;
    if (!packed || !scale || !packed_qw || !sw) return BSB_ERR_INVALID_ARG;
    if (!aligned16(packed) || !aligned16(scale) || !aligned16(packed_qw) || !aligned16(sw))
        return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_decode_mxfp4(packed, scale, E, N, K, packed_qw, sw,
                                           as_stream(stream), true));
}

bsb_status bsb_gather_rows(const int8_t *q, const float *sa, const int32_t *index, int64_t R,
                           int64_t T, int64_t K, int8_t *q_out, float *sa_out, void *stream) {
    if (R < 0 || R >= kMaxDim || T < 1 || T >= kMaxDim || K < 128 || K % 128 || K >= kMaxDim ||
        (R > 0 && !prod_le(R, K, 1, kMaxElems)) || !prod_le(T, K, 1, kMaxElems))
        return BSB_ERR_INVALID_ARG;
    if (R == 0) return BSB_OK;
    if (!q || !sa || !index || !q_out || !sa_out) return BSB_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(sa) || !aligned16(index) || !aligned16(q_out) ||
        !aligned16(sa_out))
        return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_gather_rows(q, sa, index, R, T, K, q_out, sa_out, as_stream(stream)));
}

bsb_status bsb_moe_combine(const uint16_t *y, const int32_t *row_of_pair, const float *gate,
                           int64_t T, int64_t topk, int64_t R, int64_t N, uint16_t *out,
                           void *stream) {
    if (T < 0 || T >= kMaxDim || topk < 1 || topk > kMaxTopk || R < 1 || R >= kMaxDim ||
        N < 8 || N % 8 || N >= kMaxDim || !prod_le(R, N, 1, kMaxElems) ||
        (T > 0 && !prod_le(T, N, 1, kMaxElems)) || (T > 0 && !prod_le(T, topk, 1, kMaxElems)))
        return BSB_ERR_INVALID_ARG;
    if (T == 0) return BSB_OK;
    if (!y || !row_of_pair || !gate || !out) return BSB_ERR_INVALID_ARG;
    if (!aligned16(y) || !aligned16(row_of_pair) || !aligned16(gate) || !aligned16(out))
        return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_moe_combine(y, row_of_pair, gate, T, topk, R, N, out,
                                          as_stream(stream)));
}

bsb_status bsb_kv_cache_write(const uint16_t *k_bf16, const uint16_t *v_bf16,
                              const int32_t *seq, const int32_t *pos, int64_t n, int64_t B,
                              int64_t Hkv, int64_t T, int64_t D, int8_t *k_cache, float *k_scale,
                              int8_t *v_cache, float *v_scale, void *stream) {
    if (n < 0 || n >= kMaxDim || B < 1 || B >= kMaxDim || Hkv < 1 || Hkv >= kMaxDim ||
        D != kKvHeadDim || T < 64 || T % 64 || T >= kMaxKvSlots ||
        !prod_le(B, Hkv, T, kMaxElems) || (n > 0 && !prod_le(n, Hkv, 2 * D, kMaxElems)))
        return BSB_ERR_INVALID_ARG;
    if (n == 0) return BSB_OK;
    if (!k_bf16 || !v_bf16 || !seq || !pos || !k_cache || !k_scale || !v_cache || !v_scale)
        return BSB_ERR_INVALID_ARG;
    if (!aligned16(k_bf16) || !aligned16(v_bf16) || !aligned16(seq) || !aligned16(pos) ||
        !aligned16(k_cache) || !aligned16(k_scale) || !aligned16(v_cache) || !aligned16(v_scale))
        return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_kv_cache_write(k_bf16, v_bf16, seq, pos, n, (int)B, (int)Hkv, (int)T,
                                             k_cache, k_scale, v_cache, v_scale,
                                             as_stream(stream)));
}

int64_t bsb_attention_workspace_bytes(int64_t B, int64_t Hq, int64_t max_len) {
    if (B < 1 || B >= kMaxDim || Hq < 1 || Hq >= kMaxDim || max_len < 0 || max_len >= kMaxKvSlots)
        return -1;
    return 4 * bsb::attention_workspace_floats(B, Hq, max_len);
}

}  // extern "C"

namespace {

// Shape, dtype and pointer checks shared by the attention entry points
// (caches checked by the caller, the workspace by attention_checks).
bsb_status attention_shape_checks(const uint16_t *q, const int32_t *lens, int64_t B, int64_t Hq,
                                  int64_t Hkv, int64_t T, int64_t D, int64_t max_len,
                                  const void *out, bsb_out_dtype out_dtype) noexcept {
    if (B < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv || Hq / Hkv > 16 || B * Hkv > 65535 ||
        B * Hq >= ((int64_t)1 << 31) || D != kKvHeadDim || T < 64 || T % 64 ||
        T >= kMaxKvSlots || max_len < 0 || max_len > T || !prod_le(B, Hkv, T, kMaxElems))
        return BSB_ERR_INVALID_ARG;
    if (out_dtype != BSB_OUT_BF16 && out_dtype != BSB_OUT_FP32) return BSB_ERR_INVALID_ARG;
    if (!q || !lens || !out) return BSB_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(lens) || !aligned16(out)) return BSB_ERR_MISALIGNED;
    return BSB_OK;
}

bsb_status attention_checks(const uint16_t *q, const int32_t *lens, int64_t B, int64_t Hq,
                            int64_t Hkv, int64_t T, int64_t D, int64_t max_len, const float *work,
                            int64_t work_bytes, const void *out, bsb_out_dtype out_dtype) noexcept {
    if (bsb_status s = attention_shape_checks(q, lens, B, Hq, Hkv, T, D, max_len, out, out_dtype))
        return s;
    const int64_t need = bsb_attention_workspace_bytes(B, Hq, max_len);
    if (need < 0 || work_bytes < need) return BSB_ERR_INVALID_ARG;
    if (need > 0 && !work) return BSB_ERR_INVALID_ARG;
    if (work && !aligned16(work)) return BSB_ERR_MISALIGNED;
    return BSB_OK;
}

}  // namespace

extern "C" {

bsb_status bsb_attention_decode_int8kv(const uint16_t *q_bf16, const int8_t *k_cache,
                                       const float *k_scale, const int8_t *v_cache,
                                       const float *v_scale, const int32_t *lens, int64_t B,
                                       int64_t Hq, int64_t Hkv, int64_t T, int64_t D,
                                       int64_t max_len, float *work, int64_t work_bytes,
                                       void *out, bsb_out_dtype out_dtype, void *stream) {
    if (bsb_status s = attention_checks(q_bf16, lens, B, Hq, Hkv, T, D, max_len, work, work_bytes,
                                        out, out_dtype))
        return s;
    if (!k_cache || !k_scale || !v_cache || !v_scale) return BSB_ERR_INVALID_ARG;
    if (!aligned16(k_cache) || !aligned16(k_scale) || !aligned16(v_cache) || !aligned16(v_scale))
        return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_attention_decode(q_bf16, k_cache, k_scale, v_cache, v_scale, lens,
                                               (int)B, (int)Hq, (int)Hkv, (int)T, (int)max_len,
                                               work, out, out_dtype == BSB_OUT_BF16 ? 1 : 0,
                                               as_stream(stream)));
}

bsb_status bsb_attention_chunk_int8kv(const uint16_t *q_bf16, const int8_t *k_cache,
                                      const float *k_scale, const int8_t *v_cache,
                                      const float *v_scale, const int32_t *lens, int64_t B,
                                      int64_t Qn, int64_t Hq, int64_t Hkv, int64_t T, int64_t D,
                                      int64_t max_len, float *work, int64_t work_bytes, void *out,
                                      bsb_out_dtype out_dtype, void *stream) {
    if (bsb_status s = attention_shape_checks(q_bf16, lens, B, Hq, Hkv, T, D, max_len, out,
                                              out_dtype))
        return s;
    // Qn query tokens x Hq / Hkv heads share the 16 query columns of a KV head
    if (Qn < 1 || Qn > 16 || Qn * (Hq / Hkv) > 16 || B * Qn * Hq >= ((int64_t)1 << 31))
        return BSB_ERR_INVALID_ARG;
    const int64_t need = bsb_attention_workspace_bytes(B, Qn * Hq, max_len);
    if (need < 0 || work_bytes < need) return BSB_ERR_INVALID_ARG;
    if (need > 0 && !work) return BSB_ERR_INVALID_ARG;
    if (work && !aligned16(work)) return BSB_ERR_MISALIGNED;
    if (!k_cache || !k_scale || !v_cache || !v_scale) return BSB_ERR_INVALID_ARG;
    if (!aligned16(k_cache) || !aligned16(k_scale) || !aligned16(v_cache) || !aligned16(v_scale))
        return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_attention_chunk(q_bf16, k_cache, k_scale, v_cache, v_scale, lens,
                                              (int)B, (int)Qn, (int)Hq, (int)Hkv, (int)T,
                                              (int)max_len, work, out,
                                              out_dtype == BSB_OUT_BF16 ? 1 : 0,
                                              as_stream(stream)));
}

bsb_status bsb_attention_decode_int8kv_noalloc(const uint16_t *q_bf16, const int8_t *k_cache,
                                               const float *k_scale, const int8_t *v_cache,
                                               const float *v_scale, const int32_t *lens,
                                               int64_t B, int64_t Hq, int64_t Hkv, int64_t T,
                                               int64_t D, int64_t max_len, void *out,
                                               bsb_out_dtype out_dtype, void *stream) {
    if (bsb_status s = attention_shape_checks(q_bf16, lens, B, Hq, Hkv, T, D, max_len, out,
                                              out_dtype))
        return s;
    const int64_t need = bsb_attention_workspace_bytes(B, Hq, max_len);
    if (need < 0 || need > BSB_ATTENTION_NOALLOC_MAX_BYTES) return BSB_ERR_INVALID_ARG;
    if (!k_cache || !k_scale || !v_cache || !v_scale) return BSB_ERR_INVALID_ARG;
    if (!aligned16(k_cache) || !aligned16(k_scale) || !aligned16(v_cache) || !aligned16(v_scale))
        return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_attention_decode_noalloc(
        q_bf16, k_cache, k_scale, v_cache, v_scale, lens, (int)B, (int)Hq, (int)Hkv, (int)T,
        (int)max_len, out, out_dtype == BSB_OUT_BF16 ? 1 : 0, as_stream(stream)));
}

bsb_status bsb_kv_cache_write_bf16(const uint16_t *k_bf16, const uint16_t *v_bf16,
                                   const int32_t *seq, const int32_t *pos, int64_t n, int64_t B,
                                   int64_t Hkv, int64_t T, int64_t D, uint16_t *k_cache,
                                   uint16_t *v_cache, void *stream) {
    if (n < 0 || n >= kMaxDim || B < 1 || B >= kMaxDim || Hkv < 1 || Hkv >= kMaxDim ||
        D != kKvHeadDim || T < 64 || T % 64 || T >= kMaxKvSlots ||
        !prod_le(B, Hkv, T, kMaxElems) || (n > 0 && !prod_le(n, Hkv, 2 * D, kMaxElems)))
        return BSB_ERR_INVALID_ARG;
    if (n == 0) return BSB_OK;
    if (!k_bf16 || !v_bf16 || !seq || !pos || !k_cache || !v_cache) return BSB_ERR_INVALID_ARG;
    if (!aligned16(k_bf16) || !aligned16(v_bf16) || !aligned16(seq) || !aligned16(pos) ||
        !aligned16(k_cache) || !aligned16(v_cache))
        return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_kv_cache_write_bf16(k_bf16, v_bf16, seq, pos, n, (int)B, (int)Hkv,
                                                  (int)T, k_cache, v_cache, as_stream(stream)));
}

bsb_status bsb_attention_decode_bf16kv(const uint16_t *q_bf16, const uint16_t *k_cache,
                                       const uint16_t *v_cache, const int32_t *lens, int64_t B,
                                       int64_t Hq, int64_t Hkv, int64_t T, int64_t D,
                                       int64_t max_len, float *work, int64_t work_bytes,
                                       void *out, bsb_out_dtype out_dtype, void *stream) {
    if (bsb_status s = attention_checks(q_bf16, lens, B, Hq, Hkv, T, D, max_len, work, work_bytes,
                                        out, out_dtype))
        return s;
    if (!k_cache || !v_cache) return BSB_ERR_INVALID_ARG;
    if (!aligned16(k_cache) || !aligned16(v_cache)) return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_attention_decode_bf16kv(
        q_bf16, k_cache, v_cache, lens, (int)B, (int)Hq, (int)Hkv, (int)T, (int)max_len, work, out,
        out_dtype == BSB_OUT_BF16 ? 1 : 0, as_stream(stream)));
}

bsb_status bsb_probe_mfma_i8(const int8_t *a, const int8_t *b, int64_t bytes, int64_t rounds,
                             int32_t *out, void *stream) {
    if (bytes < 16 || bytes % 16 || bytes > ((int64_t)1 << 31) || rounds < 1 ||
        rounds > ((int64_t)1 << 24))
        return BSB_ERR_INVALID_ARG;
    if (!a || !b || !out) return BSB_ERR_INVALID_ARG;
    if (!aligned16(a) || !aligned16(b) || !aligned16(out)) return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_probe_mfma_i8(a, b, bytes, rounds, out, as_stream(stream)));
}

bsb_status bsb_probe_mfma_i8_epilogue(const int8_t *a, const int8_t *b, int64_t bytes, int64_t rounds,
                             int32_t *out, void *stream) {
    if (bytes < 16 || bytes % 16 || bytes > ((int64_t)1 << 31) || rounds < 1 ||
        rounds > ((int64_t)1 << 24))
        return BSB_ERR_INVALID_ARG;
    if (!a || !b || !out) return BSB_ERR_INVALID_ARG;
    if (!aligned16(a) || !aligned16(b) || !aligned16(out)) return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_probe_mfma_i8_epilogue(a, b, bytes, rounds, out, as_stream(stream)));
}

bsb_status bsb_probe_hbm_read(const void *src, int64_t bytes, int32_t *out, void *stream) {
    const int64_t sweep = (int64_t)16 * bsb::kProbeThreads;
    if (bytes < sweep || bytes % sweep || bytes > ((int64_t)1 << 40)) return BSB_ERR_INVALID_ARG;
    if (!src || !out) return BSB_ERR_INVALID_ARG;
    if (!aligned16(src) || !aligned16(out)) return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_probe_hbm_read(src, bytes, out, as_stream(stream)));
}

bsb_status bsb_probe_hbm_copy(const void *src, void *dst, int64_t bytes, void *stream) {
    const int64_t sweep = (int64_t)16 * bsb::kProbeThreads;
    if (bytes < sweep || bytes % sweep || bytes > ((int64_t)1 << 40)) return BSB_ERR_INVALID_ARG;
    if (!src || !dst) return BSB_ERR_INVALID_ARG;
    if (!aligned16(src) || !aligned16(dst)) return BSB_ERR_MISALIGNED;
    if (bsb_status s = check_device()) return s;
    (void)hipGetLastError();
    return finish(bsb::launch_probe_hbm_copy(src, dst, bytes, as_stream(stream)));
}

}  // extern "C"
