// Dynamic per-token INT8 quantisation of BF16 activations on gfx950.
//
// [P3] sec. 3.1: per-token scales computed at run time from each token's own
// range. Rule: sa = amax/127 (IEEE float32), q = clamp(rint(x/sa), -127, 127).
//
// HBM-bound: 2 bytes in, 1 byte out per element. One workgroup per token row;
// the row is read once with 16-byte coalesced loads and kept in registers
// while the workgroup reduces the row maximum, then quantised from registers
// (one reciprocal per row and fused corrections instead of a division per
// element; the result is the same correctly rounded quotient). The codes are
// written once, with the non-temporal hint (inputs rotated through more than
// the caches hold: 4096 x 8192 20.5 -> 19.1 us, 4096 x 4096 12.5 -> 11.3 us,
// 1024 x 7168 7.5 -> 5.8 us; with the input left in the last-level cache,
// 32768 x 4096 70 -> 58 us). Non-temporal loads were faster only on inputs
// the caches do not hold, and slower (4096 x 8192 16.5 -> 17.7 us) on a
// freshly written input, the usual case; the loads stay cached.
#include "device_common.h"
#include "launch.h"

namespace bsb {

namespace {

typedef uint32_t v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void store8_nt(uint2 *p, int i, uint2 v) {
    const v2u t = {v.x, v.y};
    __builtin_nontemporal_store(t, reinterpret_cast<v2u *>(p) + i);
}

// Max of the 15-bit BF16 magnitudes in a dword holding two BF16 values. For
// finite BF16 the unsigned order of |bits| is the order of |values|, so the
// row maximum is an exact integer max.
__device__ __forceinline__ uint32_t mag2_max(uint32_t w, uint32_t cur) {
    uint32_t lo = w & 0x7FFFu, hi = (w >> 16) & 0x7FFFu;
    cur = cur > lo ? cur : lo;
    return cur > hi ? cur : hi;
}

__device__ __forceinline__ uint32_t row_reduce_max(uint32_t v, uint32_t *red) {
    v = group_max_u32(v, kWave);
    const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    uint32_t r = red[0];
    for (int i = 1; i < nw; ++i) r = r > red[i] ? r : red[i];
    return r;
}

// Eight BF16 elements -> eight INT8 codes. y = RN(1/s) when s takes the
// division-free path (s >= kFastScaleMin), unused otherwise.
__device__ __forceinline__ uint2 quant8(uint4 v, float s, float y, bool fast, bool zero) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
        f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
    if (fast)
        return make_uint2(quant4_refined(f[0], f[1], f[2], f[3], s, y),
                          quant4_refined(f[4], f[5], f[6], f[7], s, y));
    if (zero) return make_uint2(0u, 0u);
    return make_uint2(quant4_divide(f[0], f[1], f[2], f[3], s),
                      quant4_divide(f[4], f[5], f[6], f[7], s));
}

// CH 16-byte chunks per thread live in registers (K <= 8 * CH * blockDim).
template <int CH>
__global__ void __launch_bounds__(256)
quantize_act_kernel(const uint16_t *__restrict__ x, int64_t K, int8_t *__restrict__ q,
                    float *__restrict__ sa) {
    __shared__ uint32_t red[4];
    const int64_t m = blockIdx.x;
    const int nchunk = (int)(K >> 3);
    const uint4 *xr = reinterpret_cast<const uint4 *>(x + m * K);
    uint2 *qr = reinterpret_cast<uint2 *>(q + m * K);
    uint4 v[CH];
    uint32_t amax = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int idx = threadIdx.x + c * blockDim.x;
        v[c] = idx < nchunk ? xr[idx] : make_uint4(0u, 0u, 0u, 0u);
        amax = mag2_max(v[c].x, amax);
        amax = mag2_max(v[c].y, amax);
        amax = mag2_max(v[c].z, amax);
        amax = mag2_max(v[c].w, amax);
    }
    amax = row_reduce_max(amax, red);
    const float s = absmax_scale(bf16_to_f32(amax));
    const bool fast = s >= kFastScaleMin;
    const float y = fast ? 1.0f / s : 0.0f;
    if (threadIdx.x == 0) sa[m] = s;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int idx = threadIdx.x + c * blockDim.x;
        if (idx < nchunk) store8_nt(qr, idx, quant8(v[c], s, y, fast, amax == 0));
    }
}

// Rows longer than the register-resident limit: two passes over the row
// (the second pass re-reads from cache).
__global__ void __launch_bounds__(256)
quantize_act_stream_kernel(const uint16_t *__restrict__ x, int64_t K, int8_t *__restrict__ q,
                           float *__restrict__ sa) {
    __shared__ uint32_t red[4];
    const int64_t m = blockIdx.x;
    const int64_t nchunk = K >> 3;
    const uint4 *xr = reinterpret_cast<const uint4 *>(x + m * K);
    uint2 *qr = reinterpret_cast<uint2 *>(q + m * K);
    uint32_t amax = 0;
    for (int64_t idx = threadIdx.x; idx < nchunk; idx += blockDim.x) {
        const uint4 v = xr[idx];
        amax = mag2_max(v.x, amax);
        amax = mag2_max(v.y, amax);
        amax = mag2_max(v.z, amax);
        amax = mag2_max(v.w, amax);
    }
    amax = row_reduce_max(amax, red);
    const float s = absmax_scale(bf16_to_f32(amax));
    const bool fast = s >= kFastScaleMin;
    const float y = fast ? 1.0f / s : 0.0f;
    if (threadIdx.x == 0) sa[m] = s;
    for (int64_t idx = threadIdx.x; idx < nchunk; idx += blockDim.x)
        qr[idx] = quant8(xr[idx], s, y, fast, amax == 0);
}

}  // namespace

hipError_t launch_quantize_act(const uint16_t *x, int64_t M, int64_t K, int8_t *q, float *sa,
                               hipStream_t stream) {
    const int64_t nchunk = K / 8;
    const int threads = (int)(nchunk >= 256 ? 256 : ((nchunk + 63) / 64) * 64);
    const int64_t ch = (nchunk + threads - 1) / threads;
    const dim3 grid((unsigned)M), block((unsigned)threads);
    if (ch <= 1)
        quantize_act_kernel<1><<<grid, block, 0, stream>>>(x, K, q, sa);
    else if (ch <= 2)
        quantize_act_kernel<2><<<grid, block, 0, stream>>>(x, K, q, sa);
    else if (ch <= 4)
        quantize_act_kernel<4><<<grid, block, 0, stream>>>(x, K, q, sa);
    else if (ch <= 8)
        quantize_act_kernel<8><<<grid, block, 0, stream>>>(x, K, q, sa);
    else
        quantize_act_stream_kernel<<<grid, block, 0, stream>>>(x, K, q, sa);
    return hipGetLastError();
}

}  // namespace bsb
