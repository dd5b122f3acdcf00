// GEMMs with BF16 activations for M above the decode-shaped range on gfx950:
// the two routes [P1] sec. 1-2 runs beside W8A8, on the same weights.
//     W8A16: y[m,n] = sum_g sw[n,g] * sum_{k in g} x[m,k] * qw[n,k]
//     BF16:  y[m,n] = sum_k x[m,k] * w[n,k]
// x is BF16 [M,K]; qw INT8 [N,K] with sw [N,K/128] float32, or w BF16 [N,K].
// Every product is exact in float32 (BF16 x INT8 has at most 15 significant
// bits, BF16 x BF16 16). Per 128-wide K group the matrix core sums the
// group's products into a fresh float32 accumulator in its own order
// (v_mfma_f32_32x32x16_bf16, eight per 32x32 block and group), and the group
// sums are folded in group order: acc = fmaf(P_g, sw[n,g], acc) (W8A16) or
// acc = acc + P_g (BF16). Results are therefore within (127 + G) * 2^-24 *
// sum |terms| of the exact value and do not depend on the tile shape, like the
// decode-shaped kernel's.
//
// Tile: 128x128 outputs per workgroup, 8 waves in a 2 (M) x 4 (N) grid, each
// owning 64 x 32 outputs (two 32x32 blocks stacked along M). K is walked in
// stages of 64 elements (half a group): the stage's A tile (128 rows x 128 B
// of BF16) and B tile (128 rows x 128 B of BF16, or 128 rows x 64 B of INT8)
// go from global memory straight into LDS (buffer loads with the
// LDS-destination bit, 1 KB per wave instruction), with the group's 128
// weight scales for W8A16. Four stages, one barrier per stage: the barrier of
// stage s publishes stage s+1, whose fragments are read while s is multiplied
// (each right after its last use), and frees stage s-1, into which s+3 is
// loaded at once. INT8 weight fragments (8 bytes: the 8 K positions a lane
// supplies) are converted to BF16 (exact: |w| <= 127 has at most 7
// significant bits) one stage ahead, beside the second block's MFMAs; the
// group epilogue (one fused multiply-add or add per output) runs beside the
// first block's MFMAs of the next group.
//
// Out-of-range rows, columns and stages read zero through the buffer
// descriptors (a zero group adds fmaf(0, 0, acc) = acc or acc + 0 = acc);
// stores are masked by the real extents.
#include <type_traits>

#include "gemm_common.h"
#include "launch.h"

namespace bsb {

namespace {

enum { A16_W8 = 1, A16_BF16 = 2 };   // the weight of the route: INT8 + scales, or BF16

constexpr int kA16TM = 128, kA16TN = 128;        // output tile per workgroup
constexpr int kA16ATile = 128 * 128;             // A tile of one stage (128 rows x 64 BF16)
constexpr int kA16Scales = 8 * 256;              // 128 scales + the spare waves' slots
constexpr int kA16Stages = 4;

template <int AM>
constexpr int a16_btile() {   // B tile of one stage
    return AM == A16_BF16 ? 128 * 128 : 128 * 64;
}
template <int AM>
constexpr int a16_stage() {
    return kA16ATile + a16_btile<AM>() + (AM == A16_W8 ? kA16Scales : 0);
}

// 16-byte chunk j of a 128-byte row r sits at j ^ ((r >> 1) & 7); of a 64-byte
// row (INT8 weights) at j ^ ((r >> 2) & 3): the 32 rows a fragment read spans
// then hit distinct bank groups (16 of them for the 8-byte INT8 reads).
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz4(int r) { return (r >> 2) & 3; }

// Eight INT8 weights (little-endian in w.x, w.y) -> eight BF16 values, exactly.
__device__ __forceinline__ bf16x8 int8x8_to_bf16(uint2 w) {
    bf16x8 b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        b[e] = (__bf16)(float)(int8_t)(w.x >> (8 * e));
        b[4 + e] = (__bf16)(float)(int8_t)(w.y >> (8 * e));
    }
    return b;
}

template <int OUT, int AM>
__global__ void __launch_bounds__(512, 1)
gemm_a16_kernel(const uint16_t *x, const void *w, const float *sw, int M, int N, int K, void *y,
                TileGrid tiles) {
    constexpr int kStage = a16_stage<AM>();
    constexpr int kB = kA16ATile;                                // B tile offset in a stage
    constexpr int kS = kA16ATile + a16_btile<AM>();              // scales offset in a stage
    __shared__ __align__(16) int8_t lds[kA16Stages * kStage];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int l32 = lane & 31, half = lane >> 5;
    const int G = K >> 7, S = K >> 6;   // groups, stages
    int bm, bn;
    xcd_tile_of(blockIdx.x, tiles, bm, bn);
    const int m0 = bm * kA16TM, n0 = bn * kA16TN;
    const int mrows = min(kA16TM, M - m0), ncols = min(kA16TN, N - n0);
    const int wrow = AM == A16_BF16 ? 2 * K : K;   // bytes per weight row

    const v4i ra = make_rsrc_words(x + (int64_t)m0 * K, (uint32_t)(mrows * 2 * K));
    const v4i rb = make_rsrc_words((const int8_t *)w + (int64_t)n0 * wrow, (uint32_t)(ncols * wrow));
    const v4i rs = make_rsrc_words(AM == A16_W8 ? sw + (int64_t)n0 * G : nullptr,
                                   AM == A16_W8 ? (uint32_t)(ncols * G * 4) : 0u);

    // ---- staging (global -> LDS) ----
    // A (and BF16 B): 1 KB blocks of 8 rows x 128 B, wave w fills blocks 2w and
    // 2w+1 (rows 16w .. 16w+15); lane l lands at byte 16*l of a block and
    // fetches the global chunk the swizzle puts there. INT8 B: 1 KB blocks of
    // 16 rows x 64 B, wave w fills block w. W8A16 scales: waves 0-1 load the
    // group's 128 scales in column order, waves 2-7 the same load past the end
    // into spare slots (equal load counts per wave).
    uint32_t dva[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = wave * 16 + 8 * j + (lane >> 3);
        dva[j] = (uint32_t)(row * 2 * K + (((lane & 7) ^ swz8(row)) << 4));
    }
    const int brow = wave * 16 + (lane >> 2);
    const uint32_t dvb = (uint32_t)(brow * K + (((lane & 3) ^ swz4(brow)) << 4));
    const uint32_t svoff = wave < 2 ? (uint32_t)((wave * 64 + lane) * G * 4) : 0u;
    const uint32_t lbase = (uint32_t)(uintptr_t)lds;

    // Stage s into buffer st (4 loads per wave), one statement; s_nop 4: the
    // wait states before a vector memory instruction reads an SGPR a VALU
    // instruction wrote; s_nop 0: one wait state after each M0 write.
    auto dma = [&](int st, int s) {
        const bool in = s < S;
        const uint32_t so = in ? (uint32_t)s * 128 : kOOB;        // A: 64 BF16 per stage
        const uint32_t ma = lbase + st * kStage + wave * 2048;
        uint32_t m0_out;
        if (AM == A16_BF16) {
            const uint32_t mb = lbase + st * kStage + kB + wave * 2048;
            asm volatile(
                "s_nop 4\n\t"
                "s_mov_b32 m0, %[a0]\n\ts_nop 0\n\t"
                "buffer_load_dwordx4 %[v0], %[ra], %[so] offen lds\n\t"
                "s_mov_b32 m0, %[a1]\n\ts_nop 0\n\t"
                "buffer_load_dwordx4 %[v1], %[ra], %[so] offen lds\n\t"
                "s_mov_b32 m0, %[b0]\n\ts_nop 0\n\t"
                "buffer_load_dwordx4 %[v0], %[rb], %[so] offen lds\n\t"
                "s_mov_b32 m0, %[b1]\n\ts_nop 0\n\t"
                "buffer_load_dwordx4 %[v1], %[rb], %[so] offen lds"
                : "=&{m0}"(m0_out)
                : [a0] "s"(ma), [a1] "s"(ma + 1024), [b0] "s"(mb), [b1] "s"(mb + 1024),
                  [v0] "v"(dva[0]), [v1] "v"(dva[1]), [ra] "s"(ra), [rb] "s"(rb), [so] "s"(so)
                : "memory");
        } else {
            const uint32_t sb = in ? (uint32_t)s * 64 : kOOB;     // INT8 B: 64 bytes per stage
            const uint32_t ss = (in && wave < 2) ? (uint32_t)(s >> 1) * 4 : kOOB;
            const uint32_t mb = lbase + st * kStage + kB + wave * 1024;
            const uint32_t ms = lbase + st * kStage + kS + wave * 256;
            asm volatile(
                "s_nop 4\n\t"
                "s_mov_b32 m0, %[a0]\n\ts_nop 0\n\t"
                "buffer_load_dwordx4 %[v0], %[ra], %[so] offen lds\n\t"
                "s_mov_b32 m0, %[a1]\n\ts_nop 0\n\t"
                "buffer_load_dwordx4 %[v1], %[ra], %[so] offen lds\n\t"
                "s_mov_b32 m0, %[b0]\n\ts_nop 0\n\t"
                "buffer_load_dwordx4 %[vb], %[rb], %[sb] offen lds\n\t"
                "s_mov_b32 m0, %[c0]\n\ts_nop 0\n\t"
                "buffer_load_dword %[vs], %[rs], %[ss] offen lds"
                : "=&{m0}"(m0_out)
                : [a0] "s"(ma), [a1] "s"(ma + 1024), [b0] "s"(mb), [c0] "s"(ms),
                  [v0] "v"(dva[0]), [v1] "v"(dva[1]), [vb] "v"(dvb), [vs] "v"(svoff),
                  [ra] "s"(ra), [rb] "s"(rb), [rs] "s"(rs), [so] "s"(so), [sb] "s"(sb),
                  [ss] "s"(ss)
                : "memory");
        }
        (void)m0_out;
    };
    // At the barrier of stage s the loads of s+1 must have landed; those of s+2
    // (4 per wave) may still be in flight.
    auto wait_next = [&]() { asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)" ::: "memory"); };

    // ---- fragment reads ----
    // A fragment (row block rb, K step ks of 16): 16 bytes of row 64 wm + 32 rb +
    // l32 at byte 32 ks + 16 half of the stage's 128-byte line; BF16 B likewise
    // for weight row 32 wn + l32; INT8 B: 8 bytes at byte 16 ks + 8 half of the
    // 64-byte line.
    uint32_t fa[4], fb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int r_a = wm * 64 + l32, r_b = wn * 32 + l32;
        fa[ks] = r_a * 128 + (((2 * ks + half) ^ swz8(r_a)) << 4);
        fb[ks] = AM == A16_BF16 ? kB + r_b * 128 + (((2 * ks + half) ^ swz8(r_b)) << 4)
                                : kB + r_b * 64 + ((ks ^ swz4(r_b)) << 4) + 8 * half;
    }
    const uint32_t fs = kS + (wn * 32 + l32) * 4;
    auto ldA = [&](int st, int rb_, int ks) {
        return *reinterpret_cast<const bf16x8 *>(lds + fa[ks] + st * kStage + rb_ * 4096);
    };
    auto ldB16 = [&](int st, int ks) {
        return *reinterpret_cast<const bf16x8 *>(lds + fb[ks] + st * kStage);
    };
    auto ldB8 = [&](int st, int ks) {
        return *reinterpret_cast<const uint2 *>(lds + fb[ks] + st * kStage);
    };
    auto ldS = [&](int st) { return *reinterpret_cast<const float *>(lds + fs + st * kStage); };

    const bool active = wm * 64 < mrows && wn * 32 < ncols;

    v16f facc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) facc[i][r] = 0.0f;

    // prologue: stages 0..2; wait for stage 0
    dma(0, 0);
    dma(1, 1);
    dma(2, 2);
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    __syncthreads();

    if (active) {
        bf16x8 a[2][4], b[4], bn[4];
        uint2 braw[4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) a[i][ks] = ldA(0, i, ks);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) b[ks] = AM == A16_BF16 ? ldB16(0, ks) : int8x8_to_bf16(ldB8(0, ks));
        v16f c[2], prev[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                c[i][r] = 0.0f;
                prev[i][r] = 0.0f;
            }
        float sc = 0.0f, prev_s = 0.0f;   // scale of the current group / of the pending one

        // Epilogue quarter qt of the pending group's block pi.
        auto epi = [&](int pi, int qt) {
#pragma unroll
            for (int r = 4 * qt; r < 4 * qt + 4; ++r)
                facc[pi][r] = AM == A16_W8 ? __builtin_fmaf(prev[pi][r], prev_s, facc[pi][r])
                                           : facc[pi][r] + prev[pi][r];
        };

        // One stage st (stage index s; the first of its group when s is even).
        auto step = [&](auto stc, int s) {
            constexpr int st = decltype(stc)::value, nx = (st + 1) % kA16Stages;
            constexpr bool first = (st & 1) == 0;   // four buffers: parity of st = parity of s
            wait_next();
            __builtin_amdgcn_s_setprio(0);
            __syncthreads();
            __builtin_amdgcn_s_setprio(2);
            dma((st + 3) % kA16Stages, s + 3);
            if (AM == A16_W8 && !first) sc = ldS(st);   // this group's scales
#pragma unroll
            for (int rb_ = 0; rb_ < 2; ++rb_) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    v16f cin = c[rb_];
                    if (first && ks == 0) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) cin[r] = 0.0f;
                    }
                    c[rb_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[rb_][ks], b[ks], cin, 0, 0, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    a[rb_][ks] = ldA(nx, rb_, ks);   // next stage, after the last use here
                    if (rb_ == 0) {
                        if (AM == A16_W8) {
                            braw[ks] = ldB8(nx, ks);
                            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                        } else {
                            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                        }
                        if (first) {   // the previous group's epilogue
                            epi(0, ks);
                            epi(1, ks);
                            __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                        }
                    } else {
                        if (AM == A16_W8) {
                            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                            bn[ks] = int8x8_to_bf16(braw[ks]);
                            __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
                        } else {
                            b[ks] = ldB16(nx, ks);
                            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                        }
                    }
                }
            }
            if (AM == A16_W8) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) b[ks] = bn[ks];
            }
            if (!first) {   // group complete: its epilogue runs beside the next group
                prev[0] = c[0];
                prev[1] = c[1];
                prev_s = sc;
            }
        };

        __builtin_amdgcn_s_setprio(2);
        int s = 0;
        for (; s + 3 < S; s += 4) {
            step(std::integral_constant<int, 0>{}, s);
            step(std::integral_constant<int, 1>{}, s + 1);
            step(std::integral_constant<int, 2>{}, s + 2);
            step(std::integral_constant<int, 3>{}, s + 3);
        }
        if (s < S) {   // S is even: two stages left
            step(std::integral_constant<int, 0>{}, s);
            step(std::integral_constant<int, 1>{}, s + 1);
        }
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
            epi(0, qt);
            epi(1, qt);
        }
        __builtin_amdgcn_s_setprio(0);
    } else {
        for (int s = 0; s < S; ++s) {
            wait_next();
            __syncthreads();
            dma((s + 3) % kA16Stages, s + 3);
        }
    }
    // loads past the last stage still write (zeros) into LDS: let them land
    wait_vmem();
    if (!active) return;

    const int n = n0 + wn * 32 + l32;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (m < M && n < N) store_out<OUT>(y, (int64_t)m * N + n, facc[i][r]);
        }
}

template <int OUT, int AM>
hipError_t launch_a16_t(const uint16_t *x, const void *w, const float *sw, int M, int N, int K,
                        void *y, hipStream_t stream) {
    const int64_t mt = (M + kA16TM - 1) / kA16TM, nt = (N + kA16TN - 1) / kA16TN;
    const int64_t total = mt * nt;
    if (total > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const TileGrid t{(int)mt, (int)nt};
    gemm_a16_kernel<OUT, AM><<<dim3((unsigned)total), 512, 0, stream>>>(x, w, sw, M, N, K, y, t);
    return hipGetLastError();
}

}  // namespace

bool a16_tiles_fit(int64_t K) {
    // 32-bit buffer offsets: a lane's row of a 128-row BF16 panel plus a stage
    return (int64_t)kA16TM * 2 * K + 128 < ((int64_t)1 << 31);
}

hipError_t launch_gemm_a16_tiles(const uint16_t *x, const void *w, const float *sw, int M, int N,
                                 int K, void *y, int out, int am, hipStream_t stream) {
    if (am == A16_W8)
        return out == OUT_BF16 ? launch_a16_t<OUT_BF16, A16_W8>(x, w, sw, M, N, K, y, stream)
                               : launch_a16_t<OUT_FP32, A16_W8>(x, w, sw, M, N, K, y, stream);
    return out == OUT_BF16 ? launch_a16_t<OUT_BF16, A16_BF16>(x, w, nullptr, M, N, K, y, stream)
                           : launch_a16_t<OUT_FP32, A16_BF16>(x, w, nullptr, M, N, K, y, stream);
}

}  // namespace bsb
