// Block-scaled weight formats -> INT8 per-group-128 on gfx950.
//
// [P1] sec. 1: ordinary linears are FP8 e4m3 with [128,128] UE8M0 block
// scales, routed experts packed MXFP4 E2M1 with UE8M0 scales; [P1] sec. 2
// re-routes both onto the INT8 path by dequantise-and-repack. [P2] "FP8
// dialect clash": OCP and fnuz share the bit layout, biases 7 vs 8.
//
// The BF16 route's dequantisation (the same FP8 blocks to BF16, [P1] sec. 2's
// load-time path for the dense linears) shares the element decode.
//
// Both decoders are HBM streams (1 or 0.5 byte in, 1 byte + 4/128 out per
// element). A thread owns two 16-byte input chunks, 256 chunks apart, whose
// loads are issued together; the lanes that cover one 128-wide K group are
// consecutive, so the group maximum is a shuffle reduction inside the wave,
// and the quantised bytes leave as one 16-byte store per 16 elements. Every
// byte is read or written once, so loads and stores carry the non-temporal
// hint (measured: about a tenth off the launch time against cached accesses). Elements are decoded by the hardware converts (two
// per instruction), which are exact: FP8 values and E2M1 values are float32
// values with few significant bits, and the block scales are powers of two
// applied by an exact multiply. The converts read FP8 as OCP e4m3; the fnuz
// reading of the same byte is exactly half of it except for 0x7F / 0xFF,
// NaN in OCP and +-240 in fnuz, which are patched. Quantisation uses one
// reciprocal per group and fused corrections instead of a division per element.
#include "device_common.h"
#include "launch.h"

namespace bsb {

namespace {

typedef float v2f __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kChunksPerThread = 2;

// 16-byte non-temporal load / store (the data is touched once).
__device__ __forceinline__ v4u load_nt(const void *p, uint32_t i) {
    return __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p) + i);
}
__device__ __forceinline__ void store_nt(void *p, uint32_t i, v4u v) {
    __builtin_nontemporal_store(v, reinterpret_cast<v4u *>(p) + i);
}

// UE8M0 exponent byte -> 2^(E-127). E = 0 is the subnormal 2^-127.
__device__ __forceinline__ float ue8m0_to_f32(uint32_t E) {
    return E ? __uint_as_float(E << 23) : __uint_as_float(0x00400000u);
}

// Sixteen elements (four dwords of four INT8 codes) against the group scale.
__device__ __forceinline__ void quant16(const float *f, float s, float amax, uint32_t *o) {
    if (s >= kFastScaleMin) {
        const float y = 1.0f / s;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = quant4_refined(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3], s, y);
    } else if (amax == 0.0f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = 0u;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = quant4_divide(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3], s);
    }
}

// Sixteen FP8 bytes -> float32 as the OCP reading; with fnuz the caller folds
// the factor 1/2 into its block scale, and 0x7F / 0xFF (NaN in OCP, +-240 in
// fnuz) come out as +-480 so that the half gives +-240.
__device__ __forceinline__ void fp8x16_to_f32(v4u v, int fnuz, float *f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t wd = v[i];
        const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd, false);   // bytes 0, 1
        const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd, true);    // bytes 2, 3
        f[4 * i] = lo.x;
        f[4 * i + 1] = lo.y;
        f[4 * i + 2] = hi.x;
        f[4 * i + 3] = hi.y;
        if (fnuz) {
            // a byte with all of e and m set
            const uint32_t t = (wd & 0x7F7F7F7Fu) ^ 0x7F7F7F7Fu;
            if ((t - 0x01010101u) & ~t & 0x80808080u) {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint32_t byte = (wd >> (8 * b)) & 0xFFu;
                    if ((byte & 0x7Fu) == 0x7Fu) f[4 * i + b] = (byte & 0x80u) ? -480.0f : 480.0f;
                }
            }
        }
    }
}

// Sixteen E2M1 bytes (32 elements; byte b holds elements 2b, low nibble, and
// 2b+1) -> float32.
__device__ __forceinline__ void e2m1x32_to_f32(v4u v, float *f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // the byte select is an immediate operand
        const v2f p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v[i], 1.0f, 0);
        const v2f p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v[i], 1.0f, 1);
        const v2f p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v[i], 1.0f, 2);
        const v2f p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v[i], 1.0f, 3);
        f[8 * i] = p0.x;
        f[8 * i + 1] = p0.y;
        f[8 * i + 2] = p1.x;
        f[8 * i + 3] = p1.y;
        f[8 * i + 4] = p2.x;
        f[8 * i + 5] = p2.y;
        f[8 * i + 6] = p3.x;
        f[8 * i + 7] = p3.y;
    }
}

// Chunk j of a thread: chunk (blockIdx.x * 2 + j) * 256 + threadIdx.x.
__device__ __forceinline__ uint32_t chunk_of(int j) {
    return (blockIdx.x * (uint32_t)kChunksPerThread + (uint32_t)j) * 256u + threadIdx.x;
}

// PACKED: qw is written in the matrix cores' operand order (16-row x 64-column
// blocks of 1 KB; 16 consecutive K positions of one row stay one 16-byte chunk),
// the layout the packed GEMM reads; otherwise row-major [N, K]. The packed form
// walks the chunks tile by tile (128 threads per 16 rows x one 128-wide group,
// eight per row), so a wave reads whole 128-byte row segments and writes
// 128-byte runs; eight consecutive lanes still hold one (row, group).
template <bool PACKED>
__global__ void __launch_bounds__(256)
decode_fp8_block_kernel(const uint8_t *__restrict__ w, const uint8_t *__restrict__ bs,
                        uint32_t nchunks, uint32_t cpr, uint32_t gpr, int fnuz,
                        int8_t *__restrict__ qw, float *__restrict__ sw) {
    // cpr = chunks (16 B) per row = K/16; gpr = groups per row = K/128.
    v4u v[kChunksPerThread];
    float scale[kChunksPerThread];
    uint32_t n[kChunksPerThread], kc[kChunksPerThread];
#pragma unroll
    for (int j = 0; j < kChunksPerThread; ++j) {   // both loads in flight before any use
        const uint32_t chunk = chunk_of(j);
        v[j] = v4u{0u, 0u, 0u, 0u};
        scale[j] = 0.0f;
        n[j] = kc[j] = 0;
        if (chunk < nchunks) {   // 8-lane groups are valid as a whole
            uint32_t src = chunk;
            if (PACKED) {
                const uint32_t tile = chunk >> 7, within = chunk & 127u;
                const uint32_t nt = tile / gpr, gt = tile - nt * gpr;
                n[j] = nt * 16u + (within >> 3);
                kc[j] = gt * 8u + (within & 7u);
                src = n[j] * cpr + kc[j];
            } else {
                n[j] = chunk / cpr;
                kc[j] = chunk - n[j] * cpr;
            }
            v[j] = load_nt(w, src);
            scale[j] = ue8m0_to_f32(bs[(n[j] >> 7) * gpr + (kc[j] >> 3)]);
        }
    }
#pragma unroll
    for (int j = 0; j < kChunksPerThread; ++j) {
        const uint32_t chunk = chunk_of(j);
        // fnuz = OCP / 2: fold the half into the (power-of-two) block scale
        const float sc = fnuz ? scale[j] * 0.5f : scale[j];
        float f[16];
        fp8x16_to_f32(v[j], fnuz, f);
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            f[i] *= sc;
            amax = __builtin_fmaxf(amax, __builtin_fabsf(f[i]));
        }
        amax = group_max(amax, 8);
        const float s = absmax_scale(amax);
        uint32_t o[4];
        quant16(f, s, amax, o);
        if (chunk < nchunks) {
            // packed: block (n/16, kc/4), lane n%16 + 16*(kc%4), in 16-byte chunks
            const uint32_t dst = PACKED ? (((n[j] >> 4) * (cpr >> 2) + (kc[j] >> 2)) << 6) +
                                              (n[j] & 15u) + ((kc[j] & 3u) << 4)
                                        : chunk;
            store_nt(qw, dst, v4u{o[0], o[1], o[2], o[3]});
            if ((kc[j] & 7u) == 0u) sw[n[j] * gpr + (kc[j] >> 3)] = s;
        }
    }
}

// One input chunk = 16 packed bytes = one 32-element MX block = one scale
// byte; four consecutive chunks of a row form a 128-wide K group, and four
// consecutive lanes hold them. cpr = input chunks per row = K/32 over the
// E*N stacked rows. PACKED writes the operand order above (each 32-element
// block is two output chunks, 16 chunks apart in a 1 KB block) and walks the
// input in tiles of 16 rows x 2^lg_tw chunks (128-byte row segments when K is
// a multiple of 256, else 64-byte ones).
template <bool PACKED>
__global__ void __launch_bounds__(256)
decode_mxfp4_kernel(const uint8_t *__restrict__ packed, const uint8_t *__restrict__ scale,
                    uint32_t nchunks, uint32_t cpr, uint32_t lg_tw, int8_t *__restrict__ qw,
                    float *__restrict__ sw) {
    v4u v[kChunksPerThread];
    float sc[kChunksPerThread];
    uint32_t n[kChunksPerThread], c[kChunksPerThread];
#pragma unroll
    for (int j = 0; j < kChunksPerThread; ++j) {
        const uint32_t chunk = chunk_of(j);
        v[j] = v4u{0u, 0u, 0u, 0u};
        sc[j] = 0.0f;
        n[j] = c[j] = 0;
        if (chunk < nchunks) {
            uint32_t src = chunk;
            if (PACKED) {
                const uint32_t tile = chunk >> (4u + lg_tw);
                const uint32_t within = chunk & ((16u << lg_tw) - 1u);
                const uint32_t tpr = cpr >> lg_tw, nt = tile / tpr, ct = tile - nt * tpr;
                n[j] = nt * 16u + (within >> lg_tw);
                c[j] = (ct << lg_tw) + (within & ((1u << lg_tw) - 1u));
                src = n[j] * cpr + c[j];
            }
            v[j] = load_nt(packed, src);
            sc[j] = ue8m0_to_f32(scale[src]);
        }
    }
#pragma unroll
    for (int j = 0; j < kChunksPerThread; ++j) {
        const uint32_t chunk = chunk_of(j);
        float f[32];
        e2m1x32_to_f32(v[j], f);
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            f[i] *= sc[j];
            amax = __builtin_fmaxf(amax, __builtin_fabsf(f[i]));
        }
        amax = group_max(amax, 4);
        const float s = absmax_scale(amax);
        uint32_t o[8];
        quant16(f, s, amax, o);
        quant16(f + 16, s, amax, o + 4);
        if (chunk < nchunks) {
            uint32_t d0, d1;
            if (PACKED) {
                // output chunks 2c and 2c+1 of row n: block (n/16, c/2), lanes
                // n%16 + 32*(c%2) and 16 above it
                d0 = (((n[j] >> 4) * (cpr >> 1) + (c[j] >> 1)) << 6) + (n[j] & 15u) +
                     ((c[j] & 1u) << 5);
                d1 = d0 + 16u;
                if ((c[j] & 3u) == 0u) sw[n[j] * (cpr >> 2) + (c[j] >> 2)] = s;
            } else {
                d0 = 2u * chunk;
                d1 = d0 + 1u;
                if ((chunk & 3u) == 0u) sw[chunk >> 2] = s;
            }
            store_nt(qw, d0, v4u{o[0], o[1], o[2], o[3]});
            store_nt(qw, d1, v4u{o[4], o[5], o[6], o[7]});
        }
    }
}

// FP8 block -> BF16 (the load-time dequantisation of the BF16 route): each
// element is e4m3(w) * 2^(E-127), exact in float32, then rounded to BF16 to
// nearest even (exact unless it is a BF16 subnormal). One thread per 16 input
// bytes, two 16-byte stores.
__global__ void __launch_bounds__(256)
dequant_fp8_block_bf16_kernel(const uint8_t *__restrict__ w, const uint8_t *__restrict__ bs,
                              uint32_t nchunks, uint32_t cpr, uint32_t gpr, int fnuz,
                              uint16_t *__restrict__ out) {
    const uint32_t chunk = blockIdx.x * 256u + threadIdx.x;
    if (chunk >= nchunks) return;
    const uint32_t n = chunk / cpr, kc = chunk - n * cpr;
    const v4u v = load_nt(w, chunk);
    float scale = ue8m0_to_f32(bs[(n >> 7) * gpr + (kc >> 3)]);
    if (fnuz) scale *= 0.5f;
    float f[16];
    fp8x16_to_f32(v, fnuz, f);
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const __bf16 a = (__bf16)(f[2 * i] * scale), b = (__bf16)(f[2 * i + 1] * scale);
        o[i] = (uint32_t)__builtin_bit_cast(uint16_t, a) |
               ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
    }
    store_nt(out, 2u * chunk, v4u{o[0], o[1], o[2], o[3]});
    store_nt(out, 2u * chunk + 1u, v4u{o[4], o[5], o[6], o[7]});
}

}  // namespace

hipError_t launch_dequant_fp8_block_bf16(const uint8_t *w, const uint8_t *bs, int64_t N,
                                         int64_t K, int fnuz, uint16_t *out, hipStream_t stream) {
    const uint32_t nchunks = (uint32_t)(N * K / 16);
    const uint32_t blocks = (nchunks + 255u) / 256u;
    dequant_fp8_block_bf16_kernel<<<blocks, 256, 0, stream>>>(
        w, bs, nchunks, (uint32_t)(K / 16), (uint32_t)(K / 128), fnuz, out);
    return hipGetLastError();
}

hipError_t launch_decode_fp8_block(const uint8_t *w, const uint8_t *bs, int64_t N, int64_t K,
                                   int fnuz, int8_t *qw, float *sw, hipStream_t stream,
                                   bool packed) {
    const uint32_t nchunks = (uint32_t)(N * K / 16);
    const uint32_t per = 256u * kChunksPerThread, blocks = (nchunks + per - 1u) / per;
    if (packed)
        decode_fp8_block_kernel<true><<<blocks, 256, 0, stream>>>(
            w, bs, nchunks, (uint32_t)(K / 16), (uint32_t)(K / 128), fnuz, qw, sw);
    else
        decode_fp8_block_kernel<false><<<blocks, 256, 0, stream>>>(
            w, bs, nchunks, (uint32_t)(K / 16), (uint32_t)(K / 128), fnuz, qw, sw);
    return hipGetLastError();
}

hipError_t launch_decode_mxfp4(const uint8_t *packed, const uint8_t *scale, int64_t E,
                               int64_t N, int64_t K, int8_t *qw, float *sw,
                               hipStream_t stream, bool packed_out) {
    const uint32_t nchunks = (uint32_t)(E * N * K / 32), cpr = (uint32_t)(K / 32);
    const uint32_t per = 256u * kChunksPerThread, blocks = (nchunks + per - 1u) / per;
    const uint32_t lg_tw = cpr % 8u == 0u ? 3u : 2u;   // K % 128 == 0: cpr % 4 == 0
    if (packed_out)
        decode_mxfp4_kernel<true><<<blocks, 256, 0, stream>>>(packed, scale, nchunks, cpr, lg_tw,
                                                              qw, sw);
    else
        decode_mxfp4_kernel<false><<<blocks, 256, 0, stream>>>(packed, scale, nchunks, cpr,
                                                               lg_tw, qw, sw);
    return hipGetLastError();
}

}  // namespace bsb
