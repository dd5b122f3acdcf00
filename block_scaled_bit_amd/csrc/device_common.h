// Device helpers shared by the gfx950 kernels of libbsb.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsb {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kGroup = 128;   // K-group width of the weight scales
constexpr int kWave = 64;     // CDNA wavefront

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

// float32 -> BF16 bits, round to nearest even. Inputs are finite.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t b = __float_as_uint(f);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Two float32 values to BF16 in one instruction (v_cvt_pk_bf16_f32): lo in the
// low half. Round to nearest even, the same bits as f32_to_bf16_rne for every
// float32 that is not a NaN, denormals included (all 2^32 patterns compared on
// the device, with the denormal-preserving mode this library is built with).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// The absmax INT8 rule of [P3] sec. 3.1 for one element, given the row's
// scale s > 0: clamp(rint(x / s), -127, 127). The division is the IEEE
// correctly rounded one (the library is built without fast-math), and rint
// rounds half to even (v_rndne_f32).
__device__ __forceinline__ int quant_elem(float x, float s) {
    float t = x / s;
    t = __builtin_rintf(t);
    t = __builtin_fminf(__builtin_fmaxf(t, -127.0f), 127.0f);
    return (int)t;
}

// Scale of the absmax rule: amax / 127 as an IEEE float32 divide.
__device__ __forceinline__ float absmax_scale(float amax) {
    return amax / 127.0f;
}

// Quantising a group of elements against its scale s = RN(amax / 127) > 0
// without one division per element. For s >= 2^-100:
//   y  = RN(1 / s)                          (one IEEE division per group)
//   q0 = RN(x * y)                          (within 1.5 ulp of x / s)
//   q1 = RN(q0 + y * (x - s * q0))          (fused; faithful)
//   q2 = RN(q1 + y * (x - s * q1))          (fused; = RN(x / s))
// The first correction brings q within an ulp of x / s (its residual is
// rounded once, a relative error of 2^-24 on a correction that is itself
// within 1.5 ulp); the residual of such a faithful quotient is exact in one
// fused multiply-add, and with y the correctly rounded reciprocal the second
// correction returns the correctly rounded quotient (Markstein's theorem; the
// range condition keeps every step clear of overflow, and an element small
// enough to underflow quantises to 0 either way). Since |x| <= amax, |x / s| <= 127*(1 + 2^-23)
// and no clamp is needed. Adding 1.5 * 2^23 rounds the quotient to an integer,
// half to even, and leaves that integer in the low byte of the sum.
// Smaller s (subnormal scales, where rounding s loses precision and the clamp
// matters) take the per-element division of quant_elem.
constexpr float kFastScaleMin = 0x1p-100f;

__device__ __forceinline__ float div_refined(float x, float s, float y) {
    float q = x * y;
    q = __builtin_fmaf(__builtin_fmaf(-s, q, x), y, q);
    return __builtin_fmaf(__builtin_fmaf(-s, q, x), y, q);
}

// Four elements -> four INT8 codes packed little-endian into one dword.
__device__ __forceinline__ uint32_t quant4_refined(float a, float b, float c, float d, float s,
                                                   float y) {
    constexpr float kRound = 12582912.0f;   // 1.5 * 2^23
    const uint32_t ua = __float_as_uint(div_refined(a, s, y) + kRound);
    const uint32_t ub = __float_as_uint(div_refined(b, s, y) + kRound);
    const uint32_t uc = __float_as_uint(div_refined(c, s, y) + kRound);
    const uint32_t ud = __float_as_uint(div_refined(d, s, y) + kRound);
    // low bytes of a, b into bytes 0, 1 and of c, d into bytes 2, 3
    return __builtin_amdgcn_perm(ub, ua, 0x0c0c0400u) | __builtin_amdgcn_perm(ud, uc, 0x04000c0cu);
}

// The same four codes by the per-element rule (any s > 0).
__device__ __forceinline__ uint32_t quant4_divide(float a, float b, float c, float d, float s);

// Max over the `width` consecutive lanes that share an aligned lane group.
__device__ __forceinline__ float group_max(float v, int width) {
    for (int off = width >> 1; off > 0; off >>= 1)
        v = __builtin_fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

__device__ __forceinline__ uint32_t group_max_u32(uint32_t v, int width) {
    for (int off = width >> 1; off > 0; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, off, kWave);
        v = v > o ? v : o;
    }
    return v;
}

// Pack four int8 values (each already in [-127, 127]) into one dword.
__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) |
           ((uint32_t)(c & 0xFF) << 16) | ((uint32_t)(d & 0xFF) << 24);
}

__device__ __forceinline__ uint32_t quant4_divide(float a, float b, float c, float d, float s) {
    return pack4_i8(quant_elem(a, s), quant_elem(b, s), quant_elem(c, s), quant_elem(d, s));
}

}  // namespace bsb

namespace bsb {

// Raw buffer resource over [base, base + bytes). Loads at offsets >= bytes
// return zero without touching memory, which lets the kernels issue every
// prefetch unconditionally (no divergent branches around loads, so the
// compiler's memory-counter waits stay exact). Word 3 = 0x00020000: the
// untyped-buffer configuration for CDNA.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ v4i buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// Same, with a wave-uniform scalar part of the offset (kept in an SGPR).
template <int AUX = 0>
__device__ __forceinline__ v4i buf_load16s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, AUX);
}

__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

constexpr uint32_t kOOB = 0x80000000u;   // an offset past every resource used here

// Buffer descriptor as four words for inline assembly (same fields as
// make_rsrc: base, stride 0, size in bytes, raw-buffer flags).
__device__ __forceinline__ v4i make_rsrc_words(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    v4i r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at
// LDS address lds + 16*l (lds wave-uniform, passed in M0). Out-of-range
// offsets write zeros. Issued through inline assembly so that the compiler
// does not treat it as a write of unknown LDS and hold every later LDS read
// until it lands: the caller calls wait_vmem() and then a barrier before any
// wave reads the destination.
// The compiler cannot see that the assembly is a vector memory instruction,
// so it inserts none of the wait states the hardware needs before one; the
// s_nop supplies them. A VALU write of an SGPR the load reads needs five
// (the compiler writes soffset or the descriptor with v_readfirstlane, or
// restores a spilled SGPR from a VGPR lane with v_readlane, right before the
// assembly), which also covers the one wait state after an SALU write of M0.
__device__ __forceinline__ void buf_load16_lds(v4i rsrc, uint32_t lds, uint32_t voff,
                                               uint32_t soff) {
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "{m0}"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}

// The same with the non-temporal hint (data streamed once).
__device__ __forceinline__ void buf_load16_lds_nt(v4i rsrc, uint32_t lds, uint32_t voff,
                                                  uint32_t soff) {
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                 :: "{m0}"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}

// 4 bytes per lane straight into LDS: lane l's bytes land at lds + 4*l.
__device__ __forceinline__ void buf_load4_lds(v4i rsrc, uint32_t lds, uint32_t voff,
                                              uint32_t soff) {
    asm volatile("s_nop 4\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "{m0}"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}

// Wait until every vector memory load of this wave, including the LDS-bound
// ones above, has completed.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Cache-policy bits of a buffer load: non-temporal (streamed once, do not
// keep in the caches).
constexpr int kNonTemporal = 2;

}  // namespace bsb
