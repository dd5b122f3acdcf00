// Block-scaled weight formats -> INT8 per-group-128 on gfx950.
//
// [P1] sec. 1: ordinary linears are FP8 e4m3 with [128,128] UE8M0 block
// scales, routed experts packed MXFP4 E2M1 with UE8M0 scales; [P1] sec. 2
// re-routes both onto the INT8 path by dequantise-and-repack. [P2] "FP8
// dialect clash": OCP and fnuz share the bit layout, biases 7 vs 8.
//
// Both decoders are HBM streams (1 or 0.5 byte in, 1 byte + 4/128 out per
// element). A thread owns one 16-byte input chunk; the lanes that cover one
// 128-wide K group are consecutive, so the group maximum is a shuffle
// reduction inside the wave, and the quantised bytes leave as one 16-byte
// store per 16 elements. Values are decoded from the bit fields (exact in
// float32) rather than with the hardware FP8 converts, which implement only
// the OCP dialect.
#include "device_common.h"
#include "launch.h"

namespace bsb {

namespace {

// UE8M0 exponent byte -> 2^(E-127). E = 0 is the subnormal 2^-127.
__device__ __forceinline__ float ue8m0_to_f32(uint32_t E) {
    return E ? __uint_as_float(E << 23) : __uint_as_float(0x00400000u);
}

// e4m3 byte -> float32. fnuz: bias 8, else OCP bias 7.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b, int fnuz) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    const float sub = (float)m * (fnuz ? 0x1p-10f : 0x1p-9f);
    const float nrm = __uint_as_float(((e + (fnuz ? 119u : 120u)) << 23) | (m << 20));
    const float mag = e ? nrm : sub;
    return (b & 0x80u) ? -mag : mag;
}

// E2M1 nibble -> float32: {0, .5, 1, 1.5, 2, 3, 4, 6} with a sign bit.
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
    const uint32_t e = (c >> 1) & 3u, m = c & 1u;
    const float sub = m ? 0.5f : 0.0f;
    const float nrm = __uint_as_float(((e + 126u) << 23) | (m << 22));
    const float mag = e ? nrm : sub;
    return (c & 8u) ? -mag : mag;
}

__global__ void __launch_bounds__(256)
decode_fp8_block_kernel(const uint8_t *__restrict__ w, const uint8_t *__restrict__ bs,
                        uint32_t nchunks, uint32_t cpr, uint32_t gpr, int fnuz,
                        int8_t *__restrict__ qw, float *__restrict__ sw) {
    // cpr = chunks (16 B) per row = K/16; gpr = groups per row = K/128.
    const uint32_t chunk = blockIdx.x * 256u + threadIdx.x;
    const bool valid = chunk < nchunks;     // 8-lane groups are valid as a whole
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    float scale = 0.0f;
    uint32_t n = 0, kc = 0;
    if (valid) {
        n = chunk / cpr;
        kc = chunk - n * cpr;
        v = reinterpret_cast<const uint4 *>(w)[chunk];
        scale = ue8m0_to_f32(bs[(n >> 7) * gpr + (kc >> 3)]);
    }
    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
    float f[16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        f[i] = e4m3_to_f32((wd[i >> 2] >> (8 * (i & 3))) & 0xFFu, fnuz) * scale;
        amax = __builtin_fmaxf(amax, __builtin_fabsf(f[i]));
    }
    amax = group_max(amax, 8);
    const float s = absmax_scale(amax);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (amax == 0.0f) {
            o[i] = 0u;
        } else {
            o[i] = pack4_i8(quant_elem(f[4 * i], s), quant_elem(f[4 * i + 1], s),
                            quant_elem(f[4 * i + 2], s), quant_elem(f[4 * i + 3], s));
        }
    }
    if (valid) {
        reinterpret_cast<uint4 *>(qw)[chunk] = make_uint4(o[0], o[1], o[2], o[3]);
        if ((kc & 7u) == 0u) sw[n * gpr + (kc >> 3)] = s;
    }
}

__global__ void __launch_bounds__(256)
decode_mxfp4_kernel(const uint8_t *__restrict__ packed, const uint8_t *__restrict__ scale,
                    uint32_t nchunks, int8_t *__restrict__ qw, float *__restrict__ sw) {
    // One chunk = 16 packed bytes = one 32-element MX block = one scale byte;
    // four consecutive chunks form a 128-wide K group.
    const uint32_t chunk = blockIdx.x * 256u + threadIdx.x;
    const bool valid = chunk < nchunks;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    float sc = 0.0f;
    if (valid) {
        v = reinterpret_cast<const uint4 *>(packed)[chunk];
        sc = ue8m0_to_f32(scale[chunk]);
    }
    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
    float f[32];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const uint32_t byte = (wd[j >> 2] >> (8 * (j & 3))) & 0xFFu;
        f[2 * j] = e2m1_to_f32(byte & 0xFu) * sc;       // element 2j: low nibble
        f[2 * j + 1] = e2m1_to_f32(byte >> 4) * sc;     // element 2j+1: high nibble
        amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fabsf(f[2 * j]),
                                                     __builtin_fabsf(f[2 * j + 1])));
    }
    amax = group_max(amax, 4);
    const float s = absmax_scale(amax);
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (amax == 0.0f) {
            o[i] = 0u;
        } else {
            o[i] = pack4_i8(quant_elem(f[4 * i], s), quant_elem(f[4 * i + 1], s),
                            quant_elem(f[4 * i + 2], s), quant_elem(f[4 * i + 3], s));
        }
    }
    if (valid) {
        uint4 *dst = reinterpret_cast<uint4 *>(qw) + 2 * (size_t)chunk;
        dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
        dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
        if ((chunk & 3u) == 0u) sw[chunk >> 2] = s;
    }
}

}  // namespace

hipError_t launch_decode_fp8_block(const uint8_t *w, const uint8_t *bs, int64_t N, int64_t K,
                                   int fnuz, int8_t *qw, float *sw, hipStream_t stream) {
    const uint32_t nchunks = (uint32_t)(N * K / 16);
    const uint32_t blocks = (nchunks + 255u) / 256u;
    decode_fp8_block_kernel<<<blocks, 256, 0, stream>>>(w, bs, nchunks, (uint32_t)(K / 16),
                                                        (uint32_t)(K / 128), fnuz, qw, sw);
    return hipGetLastError();
}

hipError_t launch_decode_mxfp4(const uint8_t *packed, const uint8_t *scale, int64_t E,
                               int64_t N, int64_t K, int8_t *qw, float *sw,
                               hipStream_t stream) {
    const uint32_t nchunks = (uint32_t)(E * N * K / 32);
    const uint32_t blocks = (nchunks + 255u) / 256u;
    decode_mxfp4_kernel<<<blocks, 256, 0, stream>>>(packed, scale, nchunks, qw, sw);
    return hipGetLastError();
}

}  // namespace bsb
