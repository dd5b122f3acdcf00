// Measurement probes: the achievable rates on this part that the benchmark
// quotes its roofline fractions against, beside the published peaks.
//
//  * mfma_i8_probe_kernel: nothing but v_mfma_i32_32x32x32_i8, two waves per
//    SIMD on every CU, operands taken from caller bytes. The matrix cores'
//    power draw depends on the operand bits (zeros run near the published
//    rate; uniform INT8 codes well below it), so the probe runs on the
//    workload's own activation and weight bytes to give the INT8 rate those
//    operands allow.
//  * mfma_i8_epilogue_probe_kernel: the same MFMA stream with the GEMMs'
//    per-group epilogue beside it: every block of four MFMAs (one 32x32 block
//    over one 128-wide K group) is followed, next to the following block's
//    MFMAs, by the previous block's 16 conversions and 16 fused multiply-adds
//    into float32 totals (eight 32x32 blocks of them, as a GEMM wave holds),
//    8 VALU instructions after each MFMA. No memory access in the loop: the
//    rate the matrix cores keep while the VALU does the epilogue work that the
//    per-group scales require.
//  * hbm_read_probe_kernel: a streaming read of a buffer larger than the
//    last-level cache, 16 bytes per lane, four loads in flight, non-temporal.
//  * hbm_copy_probe_kernel: the same walk copying into a second buffer
//    (non-temporal stores): the rate of a read + write stream, the kind the
//    weight decoders run.
#include "device_common.h"
#include "launch.h"

namespace bsb {

namespace {

// Each wave takes 8 operand sets (16 bytes of a and of b per lane) and runs
// `rounds` rounds of 64 MFMAs over 4 accumulators, pairing a-set k with b-set
// k+u (u the round's step) so that consecutive MFMAs see different inputs.
__global__ void __launch_bounds__(512, 1)
mfma_i8_probe_kernel(const int8_t *a, const int8_t *b, uint32_t chunks, int rounds,
                     int32_t *out) {
    const uint32_t gt = blockIdx.x * 512u + threadIdx.x;
    v4i ra[8], rb[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t c = (gt * 8u + (uint32_t)k) % chunks;
        const uint4 x = reinterpret_cast<const uint4 *>(a)[c];
        const uint4 y = reinterpret_cast<const uint4 *>(b)[(c * 7u + 3u) % chunks];
        ra[k] = v4i{(int)x.x, (int)x.y, (int)x.z, (int)x.w};
        rb[k] = v4i{(int)y.x, (int)y.y, (int)y.z, (int)y.w};
    }
    v16i c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) c[j][r] = 0;
    for (int it = 0; it < rounds; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int k = 0; k < 8; ++k)
                c[k & 3] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ra[k], rb[(k + u) & 7], c[k & 3],
                                                                 0, 0, 0);
    }
    int32_t x = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) x ^= c[j][r];
    out[gt] = x;
}

// Operands as the plain probe; rounds of 16 blocks of four MFMAs.
__global__ void __launch_bounds__(512, 1)
mfma_i8_epilogue_probe_kernel(const int8_t *a, const int8_t *b, uint32_t chunks, int rounds,
                              int32_t *out) {
    const uint32_t gt = blockIdx.x * 512u + threadIdx.x;
    v4i ra[8], rb[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t c = (gt * 8u + (uint32_t)k) % chunks;
        const uint4 x = reinterpret_cast<const uint4 *>(a)[c];
        const uint4 y = reinterpret_cast<const uint4 *>(b)[(c * 7u + 3u) % chunks];
        ra[k] = v4i{(int)x.x, (int)x.y, (int)x.z, (int)x.w};
        rb[k] = v4i{(int)y.x, (int)y.y, (int)y.z, (int)y.w};
    }
    const float s = 1.0f + (float)(gt & 7u) * 0x1p-10f;
    v16f f[8];
    v16i prev;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) f[j][r] = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) prev[r] = 0;
    for (int it = 0; it < rounds; ++it) {
#pragma unroll
        for (int blk = 0; blk < 16; ++blk) {
            v16i c;
#pragma unroll
            for (int r = 0; r < 16; ++r) c[r] = 0;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int k = (blk * 4 + ks) & 7;
                c = __builtin_amdgcn_mfma_i32_32x32x32_i8(ra[k], rb[(k + (blk >> 1)) & 7], c, 0, 0,
                                                          0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                const int pj = (blk + 7) & 7;
#pragma unroll
                for (int r = 4 * ks; r < 4 * ks + 4; ++r)
                    f[pj][r] = __builtin_fmaf((float)prev[r], s, f[pj][r]);
                __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
            }
            prev = c;
        }
    }
    uint32_t x = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) x ^= __float_as_uint(f[j][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) x ^= (uint32_t)prev[r];
    out[gt] = (int32_t)x;
}

// 131072 threads; thread t reads chunks t, t + 131072, ... (16 bytes each),
// four loads in flight, and stores the XOR of what it read.
__global__ void __launch_bounds__(256)
hbm_read_probe_kernel(const void *src, uint32_t sweeps, int32_t *out) {
    const uint32_t gt = blockIdx.x * 256u + threadIdx.x;
    const uint64_t base = (uint64_t)src;
    v4i acc = {0, 0, 0, 0};
    // the buffer can exceed the 4 GiB a descriptor addresses: walk it in
    // windows of 512 sweeps (1 GiB), one descriptor per window
    for (uint32_t w = 0; w < sweeps; w += 512) {
        const uint32_t n = sweeps - w < 512 ? sweeps - w : 512;
        const __amdgpu_buffer_rsrc_t rw =
            make_rsrc((const void *)(base + (uint64_t)w * kProbeThreads * 16), 0xFFFFFFFFu);
        uint32_t s = 0;
        for (; s + 4 <= n; s += 4) {
            const v4i v0 = buf_load16s<kNonTemporal>(rw, (gt + (s + 0) * kProbeThreads) * 16u, 0);
            const v4i v1 = buf_load16s<kNonTemporal>(rw, (gt + (s + 1) * kProbeThreads) * 16u, 0);
            const v4i v2 = buf_load16s<kNonTemporal>(rw, (gt + (s + 2) * kProbeThreads) * 16u, 0);
            const v4i v3 = buf_load16s<kNonTemporal>(rw, (gt + (s + 3) * kProbeThreads) * 16u, 0);
            acc ^= v0 ^ v1 ^ v2 ^ v3;
        }
        for (; s < n; ++s) acc ^= buf_load16s<kNonTemporal>(rw, (gt + s * kProbeThreads) * 16u, 0);
    }
    out[gt] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Same walk as the read probe; every chunk read is stored at the same offset of dst.
__global__ void __launch_bounds__(256)
hbm_copy_probe_kernel(const void *src, void *dst, uint32_t sweeps) {
    const uint32_t gt = blockIdx.x * 256u + threadIdx.x;
    for (uint32_t w = 0; w < sweeps; w += 512) {
        const uint32_t n = sweeps - w < 512 ? sweeps - w : 512;
        const uint64_t base = (uint64_t)w * kProbeThreads;   // in 16-byte chunks
        const v4u *s4 = reinterpret_cast<const v4u *>(src) + base;
        v4u *d4 = reinterpret_cast<v4u *>(dst) + base;
        uint32_t s = 0;
        for (; s + 4 <= n; s += 4) {
            const v4u v0 = __builtin_nontemporal_load(s4 + gt + (s + 0) * kProbeThreads);
            const v4u v1 = __builtin_nontemporal_load(s4 + gt + (s + 1) * kProbeThreads);
            const v4u v2 = __builtin_nontemporal_load(s4 + gt + (s + 2) * kProbeThreads);
            const v4u v3 = __builtin_nontemporal_load(s4 + gt + (s + 3) * kProbeThreads);
            __builtin_nontemporal_store(v0, d4 + gt + (s + 0) * kProbeThreads);
            __builtin_nontemporal_store(v1, d4 + gt + (s + 1) * kProbeThreads);
            __builtin_nontemporal_store(v2, d4 + gt + (s + 2) * kProbeThreads);
            __builtin_nontemporal_store(v3, d4 + gt + (s + 3) * kProbeThreads);
        }
        for (; s < n; ++s)
            __builtin_nontemporal_store(__builtin_nontemporal_load(s4 + gt + s * kProbeThreads),
                                        d4 + gt + s * kProbeThreads);
    }
}

}  // namespace

hipError_t launch_probe_hbm_copy(const void *src, void *dst, int64_t bytes, hipStream_t stream) {
    hbm_copy_probe_kernel<<<dim3(kProbeThreads / 256), 256, 0, stream>>>(
        src, dst, (uint32_t)(bytes / (16 * (int64_t)kProbeThreads)));
    return hipGetLastError();
}

hipError_t launch_probe_mfma_i8(const int8_t *a, const int8_t *b, int64_t bytes, int64_t rounds,
                                int32_t *out, hipStream_t stream) {
    mfma_i8_probe_kernel<<<dim3(256), 512, 0, stream>>>(a, b, (uint32_t)(bytes / 16), (int)rounds,
                                                        out);
    return hipGetLastError();
}

hipError_t launch_probe_mfma_i8_epilogue(const int8_t *a, const int8_t *b, int64_t bytes,
                                         int64_t rounds, int32_t *out, hipStream_t stream) {
    mfma_i8_epilogue_probe_kernel<<<dim3(256), 512, 0, stream>>>(a, b, (uint32_t)(bytes / 16),
                                                                 (int)rounds, out);
    return hipGetLastError();
}

hipError_t launch_probe_hbm_read(const void *src, int64_t bytes, int32_t *out,
                                 hipStream_t stream) {
    hbm_read_probe_kernel<<<dim3(kProbeThreads / 256), 256, 0, stream>>>(
        src, (uint32_t)(bytes / (16 * (int64_t)kProbeThreads)), out);
    return hipGetLastError();
}

}  // namespace bsb
