// W8A8 per-group-128 GEMM on INT8 weights stored in the matrix cores' operand
// order (decode-shaped M <= 64).
//
// [P1] sec. 2: the serving stack rearranges quantised weights once, at load
// time, into the layout the kernel that consumes them wants. Here that layout
// is the B-operand order of v_mfma_i32_16x16x64_i8: the weight matrix qw[N,K]
// is cut into 16-row x 64-column blocks, each stored as 1 KB,
//
//     packed[((n/16) * (K/64) + k/64) * 1024 + 16*l + j] = qw[n, k]
//         with l = (n % 16) + 16 * ((k % 64) / 16),  j = k % 16,
//
// so lane l of a wave reads its 16 operand bytes of one instruction as one
// 16-byte load and the wave's 64 lanes read 1 KB contiguous. A wave owns 16
// weight rows; its whole weight stream (K/64 blocks) is contiguous.
//
// The arithmetic is the row-major kernel's, step for step ([P3] sec. 3.1):
// per output element the exact INT32 sum of each 128-wide K group, then
// acc = fmaf((float)P, sw[n,g], acc) for g ascending, then y = acc * sa[m];
// the results are bit-identical to bsb_gemm_w8a8_g128 on the unpacked weights.
//
// Kernel: a workgroup of NW waves owns 16*NW weight rows and all M <= 16*MB
// tokens. Each wave streams its weights straight into registers, PD groups
// ahead (a ring of PD register buffers; groups past the end read zeros, which
// add fmaf(0, 0, acc) = acc). The activations are shared through LDS: chunks of
// CG groups (PD or 2*PD), double-buffered, loaded one chunk ahead with
// LDS-destination buffer loads, one barrier per chunk. Every wave runs the whole loop (waves
// past N read through empty descriptors and store nothing) so the barriers
// always complete.
#include "device_common.h"
#include "launch.h"

namespace bsb {

namespace {

// One thread per 16-byte output chunk c: block c / 64, lane c % 64.
__global__ void __launch_bounds__(256)
repack_mfma_kernel(const int8_t *__restrict__ qw, int N, int K, int8_t *__restrict__ packed) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= (int64_t)N * K / 16) return;
    const int l = (int)(c & 63);
    const int64_t blk = c >> 6;
    const int ks = K / 64;
    const int64_t nb = blk / ks;
    const int s = (int)(blk - nb * ks);
    const int64_t n = nb * 16 + (l & 15);
    const int64_t k = (int64_t)s * 64 + (l >> 4) * 16;
    *reinterpret_cast<uint4 *>(packed + c * 16) = *reinterpret_cast<const uint4 *>(qw + n * K + k);
}

template <int OUT>
__device__ __forceinline__ void store_packed_out(void *y, int64_t idx, float v) {
    if (OUT == 0)
        reinterpret_cast<uint16_t *>(y)[idx] = (uint16_t)f32_to_bf16_rne(v);
    else
        reinterpret_cast<float *>(y)[idx] = v;
}

// Groups in flight per wave for MB token blocks. Each group costs 3 loads per
// wave (2 weight, 1 scale) and a chunk of CG groups 2*CG*MB 1 KB activation
// blocks per workgroup, shared by its NW waves; a wave may have at most 63 loads
// outstanding: 3*CG + ceil(2*CG*MB/NW) <= 63.
template <int MB>
constexpr int packed_depth() {
    return MB == 1 ? 12 : MB == 2 ? 8 : 4;
}

constexpr int packed_loads(int cg, int mb, int nw) { return 3 * cg + (2 * cg * mb + nw - 1) / nw; }

// Groups per activation chunk: two rings' worth where that stays within the
// outstanding-load limit (half the barriers: measured 1-2 % faster at 4 or
// more waves), else one.
template <int MB, int NW>
constexpr int packed_chunk() {
    return NW >= 4 && packed_loads(2 * packed_depth<MB>(), MB, NW) <= 63 ? 2 * packed_depth<MB>()
                                                                          : packed_depth<MB>();
}

// The pointer arguments carry no __restrict__: with it the compiler treats the
// buffer loads as invariant and regroups them by kind across the fences below,
// which breaks the one-group-per-step issue order the waits are counted for.
// GROUPED (the MoE form): blockIdx.y is the expert e, its rows are
// offsets[e] .. offsets[e+1]-1 of q / sa / y (clamped to [0, M]), its weights the
// e-th [N, K] block of the packed array (the stacked [E*N, K] experts repacked),
// its scales sw[e]; the rows are walked in passes of 16*MB.
template <int MB, int NW, int OUT, bool NT, bool GROUPED = false>
__global__ void __launch_bounds__(64 * NW)
gemm_packed_kernel(const int8_t *q, const float *sa, const int8_t *packed, const float *sw, int M,
                   int N, int K, void *y, const int32_t *offsets = nullptr) {
    constexpr int PD = packed_depth<MB>();
    constexpr int CG = packed_chunk<MB, NW>();
    constexpr int ROWS = 16 * MB;
    constexpr int GT = ROWS * 128;           // one group of the activation tile (bytes)
    constexpr int CT = CG * GT;              // one chunk
    constexpr int TB = CT / 1024;            // 1 KB blocks per chunk
    constexpr int AB = (TB + NW - 1) / NW;   // blocks per wave (the last waves may have fewer)
    static_assert(packed_loads(CG, MB, NW) <= 63 && CG % PD == 0,
                  "more loads than a wave can have outstanding");
    __shared__ __align__(16) int8_t As[2][CT];
    const int lane = threadIdx.x & 63;
    const int wv = NW == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int nb = blockIdx.x * NW + wv;
    const bool live = nb * 16 < N;
    const int G = K / 128;
    const int nch = (G + CG - 1) / CG;
    const int col = lane & 15, slot = lane >> 4;
    int lo = 0, hi = M;
    if (GROUPED) {
        const int e = blockIdx.y;
        lo = offsets[e];
        hi = offsets[e + 1];
        lo = lo < 0 ? 0 : (lo > M ? M : lo);
        hi = hi < lo ? lo : (hi > M ? M : hi);
        if (hi == lo) return;   // the whole workgroup: an empty expert
        packed += (int64_t)e * N * K;
        sw += (int64_t)e * N * G;
    }
    const auto wr = make_rsrc(live ? packed + (int64_t)nb * K * 16 : packed,
                              live ? (uint32_t)(K * 16) : 0u);
    const auto sr = make_rsrc(live ? sw + (int64_t)nb * 16 * G : sw,
                              live ? (uint32_t)(16 * G * 4) : 0u);
    v4i ra;   // the pass's activation rows (rows past them read zero)
    const uint32_t wl = (uint32_t)lane * 16;
    const uint32_t sl = (uint32_t)(col * G * 4);

    // Activation staging: block b of a chunk is group b / (ROWS/8), rows
    // 8*rb .. 8*rb+7 with rb = b % (ROWS/8); chunk j of row r lands at position
    // j ^ ((r>>1)&7) of its 128-byte LDS row, so the 16 rows one fragment read
    // touches fall in distinct bank groups. Lane l of a block loads row
    // 8*rb + l/8 at LDS position l%8; that row's pattern is
    // (4*(rb&1) + l/16) & 7, so the lane part of the offset takes one of two
    // values and the rest (8*rb*K + 128*g) is wave-uniform.
    uint32_t avl[2];
#pragma unroll
    for (int e = 0; e < 2; ++e)
        avl[e] = (uint32_t)((lane >> 3) * K + (((lane & 7) ^ ((4 * e + (lane >> 4)) & 7)) << 4));
    auto lds_addr = [](const void *p) {
        return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
    };
    auto stage = [&](int c) {   // chunk c into buffer c & 1
#pragma unroll
        for (int i = 0; i < AB; ++i) {
            const int b = wv + i * NW;
            if (b < TB) {
                const int gl = b / (ROWS / 8), rb = b % (ROWS / 8);
                const int g = c * CG + gl;
                buf_load16_lds(ra, lds_addr(&As[c & 1][gl * GT + rb * 1024]), avl[rb & 1],
                               g < G ? (uint32_t)(g * 128 + rb * 8 * K) : kOOB);
            }
        }
    };

    v4i w[PD][2];
    float s[PD];
    auto load_w = [&](int d, int g) {
        const uint32_t so = g < G ? (uint32_t)g * 2048u : kOOB;
        w[d][0] = buf_load16s<NT ? kNonTemporal : 0>(wr, wl, so);
        w[d][1] = buf_load16s<NT ? kNonTemporal : 0>(wr, wl + 1024, so);
    };
    auto load_s = [&](int d, int g) {
        s[d] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             sr, (int)sl, g < G ? g * 4 : (int)kOOB, 0));
    };
    // The dense form's activation scales, loaded first (their latency passes
    // under the K walk instead of standing between the last MFMA and the
    // stores: decode GEMM median per call 44.1 -> 43.6 us); the oldest loads, so the in-order
    // waits below only ever wait for them too.
    float sam[MB][4];
    if (!GROUPED) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = i * 16 + slot * 4 + r;
                sam[i][r] = m < M ? sa[m] : 0.0f;
            }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int r0 = lo;; r0 += ROWS) {   // the dense form makes exactly one pass
        const int rows = hi - r0 < ROWS ? hi - r0 : ROWS;
        ra = make_rsrc_words(q + (int64_t)r0 * K, (uint32_t)(rows * K));
        float facc[MB][4];
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) facc[i][r] = 0.0f;

        // Issue order: chunk 0's activations, then groups 0 .. PD-1 one at a time.
        stage(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = 0; d < PD; ++d) {
            load_w(d, d);
            load_s(d, d);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int c = 0; c < nch; ++c) {
            // Exactly 3*CG loads (3*PD for chunk 0: the prologue's groups) were
            // issued after this wave's blocks of chunk c, the weights and scales
            // of the groups in between, and loads complete in order: the blocks
            // have landed. The barrier then publishes every wave's and also means
            // every wave is done reading chunk c-1's buffer, which chunk c+1 goes
            // into.
            if (c == 0)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * PD) : "memory");
            else
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * CG) : "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            if (c + 1 < nch) stage(c + 1);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            const int8_t *buf = As[c & 1];
#pragma unroll
            for (int dd = 0; dd < CG; ++dd) {
                const int d = dd % PD;           // weight ring slot
                const int g = c * CG + dd;
                v4i af[2][MB];
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    const int r = i * 16 + col;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int j = h * 4 + slot;   // K positions 64h + 16*slot .. +15
                        af[h][i] = *reinterpret_cast<const v4i *>(buf + dd * GT + r * 128 +
                                                                  ((j ^ ((r >> 1) & 7)) << 4));
                    }
                }
                v4i acc[MB];
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[0][i], w[d][0],
                                                                   v4i{0, 0, 0, 0}, 0, 0, 0);
                    acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[1][i], w[d][1], acc[i],
                                                                   0, 0, 0);
                }
                load_w(d, g + PD);
                // C layout of 16x16: lane holds weight row `col`, tokens 4*slot + r
#pragma unroll
                for (int i = 0; i < MB; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        facc[i][r] = __builtin_fmaf((float)acc[i][r], s[d], facc[i][r]);
                load_s(d, g + PD);   // after the epilogue: s[d] is reused in place
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (live) {
            const int n = nb * 16 + col;
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = i * 16 + slot * 4 + r;
                    if (m < rows)
                        store_packed_out<OUT>(y, (int64_t)(r0 + m) * N + n,
                                              facc[i][r] * (GROUPED ? sa[r0 + m] : sam[i][r]));
                }
        }
        if (!GROUPED || r0 + ROWS >= hi) break;
        // the next pass's chunk 0 goes into buffer 0, which the last chunk may still
        // be read from: every wave finishes this pass first
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }
}

// Narrow weights (at most one 16-row block per CU): one wave per workgroup and no
// LDS. The wave reads its activations straight from L2 into registers, together
// with its weights and scales, PD groups ahead. Loads retire in issue order, so
// activations are fetched as far ahead as the weights, or a wait for one would
// also wait for every older weight load. With this few waves the per-wave
// activation re-reads are small and no barrier holds a wave back; at full width
// they would move twice the weight bytes through L2.
template <int MB, int OUT, bool NT>
__global__ void __launch_bounds__(64)
gemm_packed_narrow_kernel(const int8_t *q, const float *sa, const int8_t *packed, const float *sw,
                          int M, int N, int K, void *y) {
    constexpr int PD = packed_depth<MB>();
    static_assert((3 + 2 * MB) * PD <= 63, "more loads than a wave can have outstanding");
    const int lane = threadIdx.x;
    const int nb = blockIdx.x;                // N is a multiple of 16: every block exists
    const int G = K / 128;
    const int col = lane & 15, slot = lane >> 4;
    const auto wr = make_rsrc(packed + (int64_t)nb * K * 16, (uint32_t)(K * 16));
    const auto ar = make_rsrc(q, (uint32_t)(M * K));   // rows >= M read zero
    const auto sr = make_rsrc(sw + (int64_t)nb * 16 * G, (uint32_t)(16 * G * 4));
    const uint32_t wl = (uint32_t)lane * 16;
    const uint32_t sl = (uint32_t)(col * G * 4);
    uint32_t al[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) al[i] = (uint32_t)((i * 16 + col) * K + slot * 16);

    v4i w[PD][2];
    v4i a[PD][2][MB];
    float s[PD];
    // group g (past the end: zeros, no bytes; fmaf(0, 0, acc) = acc)
    auto load_wa = [&](int d, int g) {
        const bool in = g < G;
        const uint32_t so = in ? (uint32_t)g * 2048u : kOOB;
        w[d][0] = buf_load16s<NT ? kNonTemporal : 0>(wr, wl, so);
        w[d][1] = buf_load16s<NT ? kNonTemporal : 0>(wr, wl + 1024, so);
        const uint32_t ao = in ? (uint32_t)g * 128u : kOOB;
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            a[d][0][i] = buf_load16s(ar, al[i], ao);
            a[d][1][i] = buf_load16s(ar, al[i] + 64, ao);
        }
    };
    auto load_s = [&](int d, int g) {
        s[d] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             sr, (int)sl, g < G ? g * 4 : (int)kOOB, 0));
    };
    float facc[MB][4];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) facc[i][r] = 0.0f;
#pragma unroll
    for (int d = 0; d < PD; ++d) {   // issued in group order
        load_wa(d, d);
        load_s(d, d);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int g0 = 0; g0 < G; g0 += PD) {
#pragma unroll
        for (int d = 0; d < PD; ++d) {
            const int g = g0 + d;
            v4i acc[MB];
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[d][0][i], w[d][0], v4i{0, 0, 0, 0},
                                                               0, 0, 0);
                acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[d][1][i], w[d][1], acc[i], 0, 0,
                                                               0);
            }
            load_wa(d, g + PD);
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    facc[i][r] = __builtin_fmaf((float)acc[i][r], s[d], facc[i][r]);
            load_s(d, g + PD);   // after the epilogue: s[d] is reused in place
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    const int n = nb * 16 + col;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = i * 16 + slot * 4 + r;
            if (m < M) store_packed_out<OUT>(y, (int64_t)m * N + n, facc[i][r] * sa[m]);
        }
}

// Narrow weights, K split across the waves of a workgroup: KW waves share one
// 16-row block, wave w taking the groups g = KW*t + w (t = 0, 1, ...), each
// streaming its weights, activations and scales PD of its groups ahead like
// the one-wave kernel above (KW times the bytes in flight per block). The
// float32 fold must still run over g in ascending order for every output:
// after each round t every wave writes its group's INT32 partials and scales to
// LDS (double-buffered), one barrier, and then each wave folds all KW groups of
// the round, in order, into its own share of the block's outputs (MB of the
// 4*MB accumulator positions of every lane), which it stores at the end.
// Groups past the end read zeros and add fmaf(0, 0, acc) = acc.
template <int MB, int KW, int OUT, bool NT>
__global__ void __launch_bounds__(64 * KW)
gemm_packed_split_kernel(const int8_t *q, const float *sa, const int8_t *packed, const float *sw,
                         int M, int N, int K, void *y) {
    static_assert(KW == 4, "the KW waves' shares cover the 4*MB positions of a lane");
    constexpr int PD = packed_depth<MB>();
    constexpr int NP = 4 * MB;   // accumulator positions per lane: (token block i, row r)
    static_assert((3 + 2 * MB) * PD <= 63, "more loads than a wave can have outstanding");
    __shared__ __align__(16) int32_t xp[2][KW][64][NP];   // partials: [buffer][wave][lane][pos]
    __shared__ float xs[2][KW][16];                        // scales: [buffer][wave][col]
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int nb = blockIdx.x;                // N is a multiple of 16: every block exists
    const int G = K / 128;
    const int rounds = (G + KW - 1) / KW;
    const int col = lane & 15, slot = lane >> 4;
    const auto wr = make_rsrc(packed + (int64_t)nb * K * 16, (uint32_t)(K * 16));
    const auto ar = make_rsrc(q, (uint32_t)(M * K));   // rows >= M read zero
    const auto sr = make_rsrc(sw + (int64_t)nb * 16 * G, (uint32_t)(16 * G * 4));
    const uint32_t wl = (uint32_t)lane * 16;
    const uint32_t sl = (uint32_t)(col * G * 4);
    uint32_t al[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) al[i] = (uint32_t)((i * 16 + col) * K + slot * 16);

    v4i w[PD][2];
    v4i a[PD][2][MB];
    float s[PD];
    // this wave's t-th group (g = KW*t + wv; past the end: zeros, no bytes)
    auto load_wa = [&](int d, int t) {
        const int g = KW * t + wv;
        const bool in = g < G;
        const uint32_t so = in ? (uint32_t)g * 2048u : kOOB;
        w[d][0] = buf_load16s<NT ? kNonTemporal : 0>(wr, wl, so);
        w[d][1] = buf_load16s<NT ? kNonTemporal : 0>(wr, wl + 1024, so);
        const uint32_t ao = in ? (uint32_t)g * 128u : kOOB;
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            a[d][0][i] = buf_load16s(ar, al[i], ao);
            a[d][1][i] = buf_load16s(ar, al[i] + 64, ao);
        }
    };
    auto load_s = [&](int d, int t) {
        const int g = KW * t + wv;
        s[d] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             sr, (int)sl, g < G ? g * 4 : (int)kOOB, 0));
    };
    float facc[MB];   // this wave's share: positions MB*wv .. MB*wv + MB-1
#pragma unroll
    for (int p = 0; p < MB; ++p) facc[p] = 0.0f;
#pragma unroll
    for (int d = 0; d < PD; ++d) {   // issued in group order
        load_wa(d, d);
        load_s(d, d);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int t0 = 0; t0 < rounds; t0 += PD) {
#pragma unroll
        for (int d = 0; d < PD; ++d) {
            const int t = t0 + d;
            if (t >= rounds) break;   // uniform over the workgroup
            v4i acc[MB];
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[d][0][i], w[d][0], v4i{0, 0, 0, 0},
                                                               0, 0, 0);
                acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[d][1][i], w[d][1], acc[i], 0, 0,
                                                               0);
            }
            const int b = t & 1;
#pragma unroll
            for (int i = 0; i < MB; ++i)
                *reinterpret_cast<v4i *>(&xp[b][wv][lane][4 * i]) = acc[i];
            if (lane < 16) xs[b][wv][lane] = s[d];
            load_wa(d, t + PD);
            load_s(d, t + PD);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            // fold the round's KW groups in ascending order into this wave's share
#pragma unroll
            for (int u = 0; u < KW; ++u) {
                const float su = xs[b][u][col];
#pragma unroll
                for (int p = 0; p < MB; ++p)
                    facc[p] = __builtin_fmaf((float)xp[b][u][lane][MB * wv + p], su, facc[p]);
            }
        }
    }
    const int n = nb * 16 + col;
#pragma unroll
    for (int p = 0; p < MB; ++p) {
        const int pos = MB * wv + p, i = pos >> 2, r = pos & 3;
        const int m = i * 16 + slot * 4 + r;
        if (m < M) store_packed_out<OUT>(y, (int64_t)m * N + n, facc[p] * sa[m]);
    }
}

constexpr int kPackedCUs = 256;

template <int NW, int OUT>
hipError_t launch_packed_grouped_nw(const int8_t *q, const float *sa, const int8_t *packed,
                                    const float *sw, const int32_t *offsets, int E, int R, int N,
                                    int K, void *y, hipStream_t stream) {
    const dim3 grid((unsigned)((N / 16 + NW - 1) / NW), (unsigned)E);
    if ((int64_t)E * N * K >= ((int64_t)1 << 27))
        gemm_packed_kernel<2, NW, OUT, true, true><<<grid, 64 * NW, 0, stream>>>(
            q, sa, packed, sw, R, N, K, y, offsets);
    else
        gemm_packed_kernel<2, NW, OUT, false, true><<<grid, 64 * NW, 0, stream>>>(
            q, sa, packed, sw, R, N, K, y, offsets);
    return hipGetLastError();
}

// Workgroup width as for the dense form, over all experts' 16-row blocks.
template <int OUT>
hipError_t launch_packed_grouped(const int8_t *q, const float *sa, const int8_t *packed,
                                 const float *sw, const int32_t *offsets, int E, int R, int N,
                                 int K, void *y, hipStream_t stream) {
    const int64_t blocks16 = (int64_t)(N / 16) * E;
    const int64_t rounds = (blocks16 + 8 * kPackedCUs - 1) / (8 * kPackedCUs);
    int nw = (int)((blocks16 + kPackedCUs * rounds - 1) / (kPackedCUs * rounds));
    nw = nw < 2 ? 2 : nw;
#define BSB_PACKED_GROUPED_CASE(W)                                                               \
    case W:                                                                                      \
        return launch_packed_grouped_nw<W, OUT>(q, sa, packed, sw, offsets, E, R, N, K, y, stream);
    switch (nw) {
        BSB_PACKED_GROUPED_CASE(2)
        BSB_PACKED_GROUPED_CASE(3)
        BSB_PACKED_GROUPED_CASE(4)
        BSB_PACKED_GROUPED_CASE(5)
        BSB_PACKED_GROUPED_CASE(6)
        BSB_PACKED_GROUPED_CASE(7)
        default: return launch_packed_grouped_nw<8, OUT>(q, sa, packed, sw, offsets, E, R, N, K, y,
                                                          stream);
    }
#undef BSB_PACKED_GROUPED_CASE
}

template <int MB, int NW, int OUT>
hipError_t launch_packed_nw(const int8_t *q, const float *sa, const int8_t *packed,
                            const float *sw, int M, int N, int K, void *y, hipStream_t stream) {
    const dim3 grid((unsigned)((N / 16 + NW - 1) / NW));
    // the non-temporal hint pays on weight streams far larger than the caches
    if ((int64_t)N * K >= ((int64_t)1 << 27))
        gemm_packed_kernel<MB, NW, OUT, true><<<grid, 64 * NW, 0, stream>>>(q, sa, packed, sw, M,
                                                                            N, K, y);
    else
        gemm_packed_kernel<MB, NW, OUT, false><<<grid, 64 * NW, 0, stream>>>(q, sa, packed, sw, M,
                                                                             N, K, y);
    return hipGetLastError();
}

// Workgroup width: the 16-row blocks spread over whole rounds of one
// workgroup per CU, at most 8 waves (the width the row-major kernel uses).
// At most one block per CU: the narrow kernel.
template <int MB, int OUT>
hipError_t launch_packed_mb(const int8_t *q, const float *sa, const int8_t *packed,
                            const float *sw, int M, int N, int K, void *y, hipStream_t stream) {
    const int64_t blocks16 = N / 16;
    if (blocks16 <= kPackedCUs) {   // narrow: at most one 16-row block per CU
        const bool nt = (int64_t)N * K >= ((int64_t)1 << 27);
        // up to 16 tokens, or few groups, the K split across four waves (measured at
        // N = 2048-4096: M = 1 12 -> 6 us, M = 16 12.2 -> 10 us, K = 1152 11.6 -> 6 us);
        // more tokens on long K run faster on one wave (M = 32, K = 7168: 12.2 against
        // 13.7 us, the per-round exchange and barrier costing more than they hide)
        if (MB == 1 || K / 128 <= 16) {
            if (nt)
                gemm_packed_split_kernel<MB, 4, OUT, true><<<(unsigned)blocks16, 256, 0, stream>>>(
                    q, sa, packed, sw, M, N, K, y);
            else
                gemm_packed_split_kernel<MB, 4, OUT, false><<<(unsigned)blocks16, 256, 0, stream>>>(
                    q, sa, packed, sw, M, N, K, y);
            return hipGetLastError();
        }
        if (nt)
            gemm_packed_narrow_kernel<MB, OUT, true><<<(unsigned)blocks16, 64, 0, stream>>>(
                q, sa, packed, sw, M, N, K, y);
        else
            gemm_packed_narrow_kernel<MB, OUT, false><<<(unsigned)blocks16, 64, 0, stream>>>(
                q, sa, packed, sw, M, N, K, y);
        return hipGetLastError();
    }
    const int64_t rounds = (blocks16 + 8 * kPackedCUs - 1) / (8 * kPackedCUs);
    const int nw = (int)((blocks16 + kPackedCUs * rounds - 1) / (kPackedCUs * rounds));
    switch (nw) {
        case 1: return launch_packed_nw<MB, 1, OUT>(q, sa, packed, sw, M, N, K, y, stream);
        case 2: return launch_packed_nw<MB, 2, OUT>(q, sa, packed, sw, M, N, K, y, stream);
        case 3: return launch_packed_nw<MB, 3, OUT>(q, sa, packed, sw, M, N, K, y, stream);
        case 4: return launch_packed_nw<MB, 4, OUT>(q, sa, packed, sw, M, N, K, y, stream);
        case 5: return launch_packed_nw<MB, 5, OUT>(q, sa, packed, sw, M, N, K, y, stream);
        case 6: return launch_packed_nw<MB, 6, OUT>(q, sa, packed, sw, M, N, K, y, stream);
        case 7: return launch_packed_nw<MB, 7, OUT>(q, sa, packed, sw, M, N, K, y, stream);
        default: return launch_packed_nw<MB, 8, OUT>(q, sa, packed, sw, M, N, K, y, stream);
    }
}

template <int OUT>
hipError_t launch_packed_out(const int8_t *q, const float *sa, const int8_t *packed,
                             const float *sw, int M, int N, int K, void *y, hipStream_t stream) {
    if (M <= 16) return launch_packed_mb<1, OUT>(q, sa, packed, sw, M, N, K, y, stream);
    if (M <= 32) return launch_packed_mb<2, OUT>(q, sa, packed, sw, M, N, K, y, stream);
    return launch_packed_mb<4, OUT>(q, sa, packed, sw, M, N, K, y, stream);
}

}  // namespace

hipError_t launch_repack_mfma(const int8_t *qw, int64_t N, int64_t K, int8_t *packed,
                              hipStream_t stream) {
    const int64_t chunks = N * K / 16;
    repack_mfma_kernel<<<(unsigned)((chunks + 255) / 256), 256, 0, stream>>>(qw, (int)N, (int)K,
                                                                             packed);
    return hipGetLastError();
}

hipError_t launch_grouped_gemm_packed(const int8_t *q, const float *sa, const int8_t *packed,
                                      const float *sw, const int32_t *offsets, int64_t E,
                                      int64_t R, int64_t N, int64_t K, void *y, int out,
                                      hipStream_t stream) {
    return out == 0 ? launch_packed_grouped<0>(q, sa, packed, sw, offsets, (int)E, (int)R, (int)N,
                                               (int)K, y, stream)
                    : launch_packed_grouped<1>(q, sa, packed, sw, offsets, (int)E, (int)R, (int)N,
                                               (int)K, y, stream);
}

hipError_t launch_gemm_packed(const int8_t *q, const float *sa, const int8_t *packed,
                              const float *sw, int64_t M, int64_t N, int64_t K, void *y, int out,
                              hipStream_t stream) {
    return out == 0 ? launch_packed_out<0>(q, sa, packed, sw, (int)M, (int)N, (int)K, y, stream)
                    : launch_packed_out<1>(q, sa, packed, sw, (int)M, (int)N, (int)K, y, stream);
}

}  // namespace bsb
