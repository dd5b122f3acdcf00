// Output forms and stores shared by the W8A8 GEMM kernels of libbsb.
#pragma once

#include "device_common.h"

namespace bsb {

// Output forms. The *_CH forms take one weight scale per row n of the weight
// (or one for all rows: scale index n * sw_stride with stride 0): the INT32
// total over the whole of K is formed and rescaled once at the end.
// OUT_PARTIALS stores the exact INT32 group partials [M, N, G] instead of y.
enum { OUT_BF16 = 0, OUT_FP32 = 1, OUT_PARTIALS = 2, OUT_BF16_CH = 3, OUT_FP32_CH = 4 };

template <int OUT>
constexpr bool per_channel() {
    return OUT == OUT_BF16_CH || OUT == OUT_FP32_CH;
}

// (float)P, times the weight scale, then the activation scale, each rounded
// to float32 (the build does not contract multiplies into FMAs)
__device__ __forceinline__ float channel_value(int32_t p, float swn, float sa) {
    const float t = (float)p * swn;
    return t * sa;
}

template <int OUT>
__device__ __forceinline__ void store_out(void *y, int64_t idx, float v) {
    if (OUT == OUT_BF16 || OUT == OUT_BF16_CH)
        reinterpret_cast<uint16_t *>(y)[idx] = (uint16_t)f32_to_bf16_rne(v);
    else
        reinterpret_cast<float *>(y)[idx] = v;
}

}  // namespace bsb
