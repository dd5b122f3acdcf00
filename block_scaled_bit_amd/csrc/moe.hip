// MoE glue either side of the grouped GEMM on gfx950.
//
// [P3] sec. 1.3 / 4.4: every expert stays resident and each token runs
// through a few of them; tokens are dispatched to their experts and the
// experts' outputs combined back per token. On one GPU:
//
//  * gather: the tokens are quantised once (bsb_quantize_act on [T, K]),
//    then row r of the expert-sorted batch is a copy of quantised token
//    index[r] and its scale. The rule is per row, so this equals quantising
//    the gathered BF16 rows, at an eighth of the quantisation traffic for
//    top-8 routing. One workgroup per sorted row, 16-byte chunks.
//
//  * combine: out[t] = sum over k ascending of gate[t,k] * y[row_of_pair[t,k]]
//    in float32, one fused multiply-add per slot, then BF16 round to nearest
//    even. One workgroup per token; each thread owns 8 consecutive columns
//    (one 16-byte chunk of every source row) and issues the loads of up to 8
//    slots before it multiplies any of them.
//
// Both are HBM streams. Indices outside their range are outside the domain:
// they are never dereferenced (a gathered row becomes zeros with scale 0, a
// combine slot contributes nothing).
#include "device_common.h"
#include "launch.h"

namespace bsb {

namespace {

__global__ void __launch_bounds__(256)
gather_rows_kernel(const int8_t *__restrict__ q, const float *__restrict__ sa,
                   const int32_t *__restrict__ index, int64_t T, int K,
                   int8_t *__restrict__ q_out, float *__restrict__ sa_out) {
    const int64_t r = blockIdx.x;
    const int32_t src = index[r];
    const bool ok = src >= 0 && src < T;
    const int nch = K >> 4;
    const uint4 *in = reinterpret_cast<const uint4 *>(q + (ok ? (int64_t)src * K : 0));
    uint4 *out = reinterpret_cast<uint4 *>(q_out + r * K);
    for (int c = threadIdx.x; c < nch; c += blockDim.x)
        out[c] = ok ? in[c] : make_uint4(0u, 0u, 0u, 0u);
    if (threadIdx.x == 0) sa_out[r] = ok ? sa[src] : 0.0f;
}

constexpr int kSlots = 8;   // slots whose loads are in flight together

__global__ void __launch_bounds__(256)
moe_combine_kernel(const uint16_t *__restrict__ y, const int32_t *__restrict__ row_of_pair,
                   const float *__restrict__ gate, int topk, int64_t R, int N,
                   uint16_t *__restrict__ out) {
    const int64_t t = blockIdx.x;
    const int nch = N >> 3;
    const int32_t *rp = row_of_pair + t * topk;
    const float *gt = gate + t * topk;
    for (int c = threadIdx.x; c < nch; c += blockDim.x) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
        for (int k0 = 0; k0 < topk; k0 += kSlots) {
            uint4 v[kSlots];
            float w[kSlots];
            bool ok[kSlots];
#pragma unroll
            for (int s = 0; s < kSlots; ++s) {
                const int k = k0 + s;
                const int32_t r = k < topk ? rp[k] : -1;
                ok[s] = r >= 0 && r < R;
                w[s] = ok[s] ? gt[k] : 0.0f;
                v[s] = ok[s] ? reinterpret_cast<const uint4 *>(y + (int64_t)r * N)[c]
                             : make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int s = 0; s < kSlots; ++s) {
                if (!ok[s]) continue;   // past topk, or outside the domain: no contribution
                const uint32_t wd[4] = {v[s].x, v[s].y, v[s].z, v[s].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] = __builtin_fmaf(w[s], bf16_to_f32(wd[i] & 0xFFFFu), acc[2 * i]);
                    acc[2 * i + 1] = __builtin_fmaf(w[s], bf16_to_f32(wd[i] >> 16), acc[2 * i + 1]);
                }
            }
        }
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = f32_to_bf16_rne(acc[2 * i]) | (f32_to_bf16_rne(acc[2 * i + 1]) << 16);
        reinterpret_cast<uint4 *>(out + t * N)[c] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

int threads_for(int64_t chunks) {
    return (int)(chunks >= 256 ? 256 : ((chunks + 63) / 64) * 64);
}

}  // namespace

hipError_t launch_gather_rows(const int8_t *q, const float *sa, const int32_t *index, int64_t R,
                              int64_t T, int64_t K, int8_t *q_out, float *sa_out,
                              hipStream_t stream) {
    gather_rows_kernel<<<dim3((unsigned)R), threads_for(K / 16), 0, stream>>>(
        q, sa, index, T, (int)K, q_out, sa_out);
    return hipGetLastError();
}

hipError_t launch_moe_combine(const uint16_t *y, const int32_t *row_of_pair, const float *gate,
                              int64_t T, int64_t topk, int64_t R, int64_t N, uint16_t *out,
                              hipStream_t stream) {
    moe_combine_kernel<<<dim3((unsigned)T), threads_for(N / 8), 0, stream>>>(
        y, row_of_pair, gate, (int)topk, R, (int)N, out);
    return hipGetLastError();
}

}  // namespace bsb
