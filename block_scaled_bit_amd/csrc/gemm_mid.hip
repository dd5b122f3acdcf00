// W8A8 per-group-128 GEMM for mid-sized M on gfx950: 128x128 output tile per
// workgroup, for the shapes whose 256x256 tiles would leave CUs idle (a few
// hundred to a few thousand rows; grouped launches with fewer than 128 rows
// per expert on average).
//
// The arithmetic is that of [P3] sec. 3.1 in the order of the 256x256 kernel:
//     acc = 0
//     for g = 0 .. K/128-1:                  (ascending, never split)
//         P   = sum_{k in group g} q[m,k]*qw[n,k]        (INT32, MFMA)
//         acc = fmaf((float)P, sw[n,g], acc)             (VALU epilogue)
//     y = acc * sa[m]  -> BF16 (RNE) or FP32
// so every output is bit-identical whichever kernel the shape selects.
//
// Workgroup: 8 waves in a 2 (M) x 4 (N) grid, two per SIMD, each owning
// 64 x 32 outputs = two v_mfma_i32_32x32x32_i8 blocks stacked along M; per K
// group a block takes four MFMAs into a fresh INT32 accumulator, then 16
// conversions and 16 fused multiply-adds fold it into the float32 totals,
// issued beside the next block's MFMAs (8 VALU instructions after each).
//
// Staging: per K group the A tile (128 rows x 128 B), the B tile (128 weight
// rows x 128 B) and the group's 128 weight scales go from global memory
// straight into LDS (buffer loads with the LDS-destination bit, 1 KB per wave
// instruction, 16-byte chunk j of row r at j ^ ((r >> 1) & 7)), five loads per
// wave and group. Four stages, one barrier per group: the barrier of group g
// publishes the stage of g+1 (whose fragments are read into registers while g
// is multiplied, each right after its last use in g) and frees the stage of
// g-1, into which g+3 is loaded at once; a load has two groups of work to
// land. 136 KB of LDS. Loads complete in issue order, so the wait before each
// barrier is one vmcnt that leaves the next group's loads in flight.
//
// Out-of-range rows, columns and groups read zero through the buffer
// descriptors (a zero group adds fmaf(0, 0, acc) = acc); stores are masked by
// the real extents.
#include <type_traits>

#include "gemm_common.h"
#include "launch.h"

namespace bsb {

namespace {

constexpr int kMidTM = 128, kMidTN = 128;        // output tile per workgroup
constexpr int kMidTile = 128 * kGroup;           // A or B tile of one K group (bytes)
constexpr int kMidScales = 8 * 256;              // 128 scales + the spare waves' slots
constexpr int kMidStage = 2 * kMidTile + kMidScales;
constexpr int kMidStages = 4;
constexpr int kMidLdsRowS = kMidStages * kMidStage;   // the tile's 128 row scales
constexpr int kMidLds = kMidLdsRowS + 128 * 4;         // 139776 bytes of 160 KB

__device__ __forceinline__ int mid_swz(int r) { return (r >> 1) & 7; }

// GATHER (grouped only): q / sa are the T quantised tokens and row m of the
// problem is token gidx[m] (an index outside [0, T) reads a zero row, scale 0).
template <int OUT, bool GROUPED, bool GATHER = false>
__global__ void __launch_bounds__(512, 1)
gemm_mid_kernel(const int8_t *q, const float *sa, const int8_t *qw, const float *sw, int M, int N,
                int K, void *y, TileGrid tiles, const int32_t *offsets, int E, int sw_stride,
                const int32_t *gidx, int T) {
    constexpr bool CHN = per_channel<OUT>();             // one scale per row, applied at the end
    constexpr bool SCALES = !CHN && OUT != OUT_PARTIALS;   // per-group scales staged in LDS
    __shared__ __align__(16) int8_t lds[kMidLds];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int l32 = lane & 31, half = lane >> 5;
    const int G = K >> 7;
    int m0, row_end, bm, bn;
    if (GROUPED) {
        int e;
        if (!grouped_tile<kMidTM>(offsets, E, M, tiles, e, m0, row_end, bm, bn)) return;
        qw += (int64_t)e * N * K;
        sw += (int64_t)e * N * G;
    } else {
        xcd_tile_of(blockIdx.x, tiles, bm, bn);
        m0 = bm * kMidTM;
        row_end = M;
    }
    const int n0 = bn * kMidTN;
    const int mrows = min(kMidTM, row_end - m0), ncols = min(kMidTN, N - n0);

    const v4i ra = GATHER ? make_rsrc_words(q, (uint32_t)(T * K))
                          : make_rsrc_words(q + (int64_t)m0 * K, (uint32_t)(mrows * K));
    const v4i rb = make_rsrc_words(qw + (int64_t)n0 * K, (uint32_t)(ncols * K));
    const v4i rs = make_rsrc_words(SCALES ? sw + (int64_t)n0 * G : nullptr,
                                   SCALES ? (uint32_t)(ncols * G * 4) : 0u);

    // ---- staging (global -> LDS) ----
    // Each tile is filled in 1 KB blocks of 8 rows x 128 B; lane l lands at
    // byte 16*l of a block and fetches the global chunk that the swizzle puts
    // there. Wave w fills blocks 2w and 2w+1 of both tiles (rows 16w .. 16w+15).
    // Scales: waves 0-1 load the group's 128 scales, one per lane, in column
    // order; waves 2-7 issue the same load past the end into spare slots, which
    // keeps every wave's load count per stage equal.
    uint32_t dvoff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = wave * 16 + 8 * j + (lane >> 3);
        dvoff[j] = (uint32_t)(row * K + (((lane & 7) ^ mid_swz(row)) << 4));
    }
    // A rows: the same tile rows; gathered, each its token's row (rows past the
    // segment and invalid indices read zeros). The index loads (and the
    // row-scale one below) are issued together, unconditionally (rows past the
    // segment read the segment's last entry, then dropped).
    int tix[3] = {0, 0, 0};
    if (GATHER) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int m = m0 + wave * 16 + 8 * j + (lane >> 3);
            tix[j] = gidx[m < row_end ? m : row_end - 1];
        }
        const int m = m0 + (wave & 1) * 64 + lane;
        tix[2] = gidx[m < row_end ? m : row_end - 1];
    }
    uint32_t aoff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = wave * 16 + 8 * j + (lane >> 3);
        if (GATHER) {
            const int t = m0 + row < row_end ? tix[j] : -1;
            const uint32_t o = (uint32_t)t * (uint32_t)K + (uint32_t)(((lane & 7) ^ mid_swz(row)) << 4);
            aoff[j] = t >= 0 && t < T ? o : kOOB;
        } else {
            aoff[j] = dvoff[j];
        }
    }
    // The tile's 128 activation scales go straight into LDS ahead of the first
    // stage: waves 0-1 load rows 64w .. 64w+63, one per lane (rows past the
    // segment and invalid indices read zero; the partials form has none, and sa
    // may be null there).
    const bool row_scales = OUT != OUT_PARTIALS && wave < 2;
    const v4i rsa = OUT == OUT_PARTIALS ? make_rsrc_words(nullptr, 0u)
                    : GATHER            ? make_rsrc_words(sa, (uint32_t)(T * 4))
                                        : make_rsrc_words(sa + m0, (uint32_t)(mrows * 4));
    uint32_t saoff = (uint32_t)((wave * 64 + lane) * 4);
    if (GATHER) {
        const int t = m0 + (wave & 1) * 64 + lane < row_end ? tix[2] : -1;
        saoff = t >= 0 && t < T ? (uint32_t)t * 4u : kOOB;
    }
    const uint32_t svoff = wave < 2 ? (uint32_t)((wave * 64 + lane) * G * 4) : 0u;
    const uint32_t lbase = (uint32_t)(uintptr_t)lds;

    // Group g into stage st, as one statement so that nothing the compiler emits
    // lands between the loads. s_nop 4: a VALU write of an SGPR read by a vector
    // memory instruction needs five wait states (the compiler may form the
    // descriptors or offsets with v_readfirstlane right before); s_nop 0 after
    // each M0 write: one wait state before an LDS-destination load reads M0.
    auto dma = [&](int st, int g) {
        const bool in = g < G;
        const uint32_t so = in ? (uint32_t)g * kGroup : kOOB;
        const uint32_t ss = (in && wave < 2) ? (uint32_t)g * 4 : kOOB;
        const uint32_t ma = lbase + st * kMidStage + wave * 2048;
        const uint32_t mb = ma + kMidTile;
        const uint32_t ms = lbase + st * kMidStage + 2 * kMidTile + wave * 256;
        uint32_t m0_out;   // M0 is written inside: declared as an output
        asm volatile(
            "s_nop 4\n\t"
            "s_mov_b32 m0, %[a0]\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %[w0], %[ra], %[so] offen lds\n\t"
            "s_mov_b32 m0, %[a1]\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %[w1], %[ra], %[so] offen lds\n\t"
            "s_mov_b32 m0, %[b0]\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %[v0], %[rb], %[so] offen lds\n\t"
            "s_mov_b32 m0, %[b1]\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %[v1], %[rb], %[so] offen lds\n\t"
            "s_mov_b32 m0, %[c0]\n\ts_nop 0\n\t"
            "buffer_load_dword %[vs], %[rs], %[ss] offen lds"
            : "=&{m0}"(m0_out)
            : [a0] "s"(ma), [a1] "s"(ma + 1024), [b0] "s"(mb), [b1] "s"(mb + 1024),
              [c0] "s"(ms), [v0] "v"(dvoff[0]), [v1] "v"(dvoff[1]), [vs] "v"(svoff),
              [w0] "v"(aoff[0]), [w1] "v"(aoff[1]),
              [ra] "s"(ra), [rb] "s"(rb), [rs] "s"(rs), [so] "s"(so), [ss] "s"(ss)
            : "memory");
        (void)m0_out;
    };
    auto dma_rows = [&]() {
        const uint32_t mr = lbase + kMidLdsRowS + wave * 256;
        uint32_t m0_out;
        asm volatile(
            "s_nop 4\n\t"
            "s_mov_b32 m0, %[c0]\n\ts_nop 0\n\t"
            "buffer_load_dword %[vo], %[rs], %[so] offen lds"
            : "=&{m0}"(m0_out)
            : [c0] "s"(mr), [vo] "v"(saoff), [rs] "s"(rsa), [so] "s"(0u)
            : "memory");
        (void)m0_out;
    };
    // At the barrier of group g the loads of g+1 must have landed; those of
    // g+2 (5 per wave) may still be in flight.
    auto wait_next = [&]() { asm volatile("s_waitcnt vmcnt(5) lgkmcnt(0)" ::: "memory"); };

    // ---- fragment reads (LDS -> registers) ----
    // A fragment (row block rb, K step ks) of lane l: 16 bytes of row
    // 64 wm + 32 rb + l32 at K bytes 32 ks + 16 half; B likewise for weight row
    // 32 wn + l32. Rows 32 apart share the swizzle, so stage and block offsets
    // beyond the per-(ks) lane base are constants.
    uint32_t fa[4], fb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int r_a = wm * 64 + l32, r_b = wn * 32 + l32;
        fa[ks] = r_a * kGroup + (((2 * ks + half) ^ mid_swz(r_a)) << 4);
        fb[ks] = kMidTile + r_b * kGroup + (((2 * ks + half) ^ mid_swz(r_b)) << 4);
    }
    const uint32_t fs = 2 * kMidTile + (wn * 32 + l32) * 4;
    auto ldA = [&](int st, int rb_, int ks) {
        return *reinterpret_cast<const v4i *>(lds + fa[ks] + st * kMidStage + rb_ * 4096);
    };
    auto ldB = [&](int st, int ks) {
        return *reinterpret_cast<const v4i *>(lds + fb[ks] + st * kMidStage);
    };
    auto ldS = [&](int st) { return *reinterpret_cast<const float *>(lds + fs + st * kMidStage); };

    // rows and columns of this wave exist in the tile
    const bool active = wm * 64 < mrows && wn * 32 < ncols;

    v16f facc[2];   // float32 totals (per-group forms)
    v16i pacc[2];   // INT32 totals (per-channel forms)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            facc[i][r] = 0.0f;
            pacc[i][r] = 0;
        }

    // prologue: the row scales (waves 0-1), then groups 0..2 into stages 0..2;
    // wait for the row scales and group 0 (the same count with or without the
    // row-scale load in front)
    if (row_scales) dma_rows();
    dma(0, 0);
    dma(1, 1);
    dma(2, 2);
    asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
    __syncthreads();

    if (active) {
        v4i a[2][4], b[4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) a[i][ks] = ldA(0, i, ks);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) b[ks] = ldB(0, ks);
        float sc = ldS(0), scn = 0.0f;
        v16i prev;         // INT32 partials of the block whose epilogue is pending
        float prev_s = 0;  // its weight scale (0 with zero partials before the first group)
#pragma unroll
        for (int r = 0; r < 16; ++r) prev[r] = 0;

        // Epilogue quarter qt of the pending block (row block pi, group g).
        auto epi = [&](int pi, int qt, int g) {
            if (OUT == OUT_PARTIALS) {
                if (g < 0) return;
                const int n = n0 + wn * 32 + l32;
#pragma unroll
                for (int r = 4 * qt; r < 4 * qt + 4; ++r) {
                    const int m = m0 + wm * 64 + pi * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                    if (m < row_end && n < N)
                        reinterpret_cast<int32_t *>(y)[((int64_t)m * N + n) * G + g] = prev[r];
                }
            } else if (SCALES) {
#pragma unroll
                for (int r = 4 * qt; r < 4 * qt + 4; ++r)
                    facc[pi][r] = __builtin_fmaf((float)prev[r], prev_s, facc[pi][r]);
            }
        };

        // One K group on stage st (group g): row blocks rb = 0, 1, four MFMAs each.
        auto step = [&](auto stc, int g) {
            constexpr int st = decltype(stc)::value, nx = (st + 1) % kMidStages;
            // publish the stage of g+1; the stage of g-1 is free: load g+3 there
            wait_next();
            __builtin_amdgcn_s_setprio(0);
            __syncthreads();
            __builtin_amdgcn_s_setprio(2);
            dma((st + 3) % kMidStages, g + 3);
            scn = ldS(nx);
#pragma unroll
            for (int rb_ = 0; rb_ < 2; ++rb_) {
                // the pending block: row block 1 of g-1, then row block 0 of g
                const int pi = rb_ == 0 ? 1 : 0;
                v16i c;
#pragma unroll
                for (int r = 0; r < 16; ++r) c[r] = CHN ? pacc[rb_][r] : 0;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    c = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[rb_][ks], b[ks], c, 0, 0, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    // fragments of group g+1 after their last use in g
                    a[rb_][ks] = ldA(nx, rb_, ks);
                    if (rb_ == 1) {
                        b[ks] = ldB(nx, ks);
                        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    } else {
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                    epi(pi, ks, rb_ == 0 ? g - 1 : g);
                    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                }
                if (CHN) pacc[rb_] = c;
                prev = c;
                prev_s = sc;
            }
            sc = scn;
        };

        __builtin_amdgcn_s_setprio(2);   // the multiplying phases run at the raised priority
        int g = 0;
        for (; g + 3 < G; g += 4) {
            step(std::integral_constant<int, 0>{}, g);
            step(std::integral_constant<int, 1>{}, g + 1);
            step(std::integral_constant<int, 2>{}, g + 2);
            step(std::integral_constant<int, 3>{}, g + 3);
        }
        if (g < G) step(std::integral_constant<int, 0>{}, g);
        if (g + 1 < G) step(std::integral_constant<int, 1>{}, g + 1);
        if (g + 2 < G) step(std::integral_constant<int, 2>{}, g + 2);
        epi(1, 0, G - 1);
        epi(1, 1, G - 1);
        epi(1, 2, G - 1);
        epi(1, 3, G - 1);
        __builtin_amdgcn_s_setprio(0);
    } else {
        // rows or columns past the tile's end: stage this wave's share and meet
        // every barrier
        for (int g = 0; g < G; ++g) {
            wait_next();
            __syncthreads();
            dma((g + 3) % kMidStages, g + 3);
        }
    }
    // loads past the last group still write (zeros) into LDS: let them land
    // before the workgroup's LDS can be handed to another one
    wait_vmem();
    // BF16 results leave through LDS, as in the 256x256 kernel: the 128 x 128
    // tile as 256-byte rows (16-byte chunk c of row r at c ^ (r & 7)) in the
    // stages, free once every wave has passed the first barrier, then 16 bytes
    // per lane and 4 rows per wave instruction.
    if (OUT == OUT_BF16 || OUT == OUT_BF16_CH) {
        __syncthreads();
        if (active) {
            const float *rsc = reinterpret_cast<const float *>(lds + kMidLdsRowS);
            const int nc = n0 + wn * 32 + l32;
            const float swn = CHN && nc < N ? sw[(int64_t)nc * sw_stride] : 0.0f;
            auto val = [&](int i, int r, float s) {
                return CHN ? channel_value(pacc[i][r], swn, s) : facc[i][r] * s;
            };
            // rows ml and ml + 1 (r even, r + 1) converted as one pair
            const int c = wn * 32 + l32, co = (c & 7) * 2;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const int ml = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                    const uint32_t h = bf16x2_rne(val(i, r, rsc[ml]), val(i, r + 1, rsc[ml + 1]));
                    *reinterpret_cast<uint16_t *>(lds + ml * 256 + (((c >> 3) ^ (ml & 7)) << 4) + co) =
                        (uint16_t)h;
                    *reinterpret_cast<uint16_t *>(lds + (ml + 1) * 256 +
                                                  (((c >> 3) ^ ((ml + 1) & 7)) << 4) + co) =
                        (uint16_t)(h >> 16);
                }
        }
        __syncthreads();
        const bool wide = (N & 7) == 0;   // 16-byte aligned rows of 8 outputs
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int id = k * 512 + tid, row = id >> 4, c16 = id & 15;
            const v4i d = *reinterpret_cast<const v4i *>(lds + row * 256 + ((c16 ^ (row & 7)) << 4));
            const int m = m0 + row;
            const int n = n0 + c16 * 8;
            if (m >= row_end || row >= mrows) continue;
            uint16_t *dst = reinterpret_cast<uint16_t *>(y) + (int64_t)m * N + n;
            if (wide && n + 8 <= N) {
                *reinterpret_cast<v4i *>(dst) = d;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (n + e < N) dst[e] = (uint16_t)((uint32_t)d[e >> 1] >> (16 * (e & 1)));
            }
        }
        return;
    }
    if (!active) return;

    const int n = n0 + wn * 32 + l32;
    if (CHN) {
        const float swn = n < N ? sw[(int64_t)n * sw_stride] : 0.0f;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                if (m < row_end && n < N)
                    store_out<OUT>(y, (int64_t)m * N + n,
                                   channel_value(pacc[i][r], swn,
                                                 reinterpret_cast<const float *>(
                                                     lds + kMidLdsRowS)[m - m0]));
            }
    } else if (OUT != OUT_PARTIALS) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                if (m >= row_end || n >= N) continue;
                const float s = reinterpret_cast<const float *>(lds + kMidLdsRowS)[m - m0];
                store_out<OUT>(y, (int64_t)m * N + n, facc[i][r] * s);
            }
    }
}

template <int OUT, bool GROUPED, bool GATHER = false>
hipError_t launch_mid_t(const int8_t *q, const float *sa, const int8_t *qw, const float *sw, int M,
                        int N, int K, void *y, const int32_t *offsets, int E, int sw_stride,
                        hipStream_t stream, const int32_t *gidx = nullptr, int T = 0) {
    // Grouped: sum over experts of ceil(rows_e / 128) <= ceil(R / 128) + E tile rows.
    const int64_t mt = (M + kMidTM - 1) / kMidTM + (GROUPED ? E : 0), nt = (N + kMidTN - 1) / kMidTN;
    const int64_t total = mt * nt;
    if (total > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const TileGrid t{(int)mt, (int)nt};
    gemm_mid_kernel<OUT, GROUPED, GATHER><<<dim3((unsigned)total), 512, 0, stream>>>(
        q, sa, qw, sw, M, N, K, y, t, offsets, E, sw_stride, gidx, T);
    return hipGetLastError();
}

}  // namespace

bool mid_gemm_fits(int64_t K) {
    // 32-bit buffer offsets: a lane's row of a 128-row panel plus a group
    return (int64_t)kMidTM * K + kGroup < ((int64_t)1 << 31);
}

hipError_t launch_gemm_mid(const int8_t *q, const float *sa, const int8_t *qw, const float *sw,
                           int M, int N, int K, void *y, int out, const int32_t *offsets, int E,
                           int sw_stride, hipStream_t stream, const int32_t *gidx, int T) {
    if (offsets && gidx) {
        switch (out) {
            case OUT_BF16:
                return launch_mid_t<OUT_BF16, true, true>(q, sa, qw, sw, M, N, K, y, offsets, E, 1,
                                                          stream, gidx, T);
            case OUT_FP32:
                return launch_mid_t<OUT_FP32, true, true>(q, sa, qw, sw, M, N, K, y, offsets, E, 1,
                                                          stream, gidx, T);
            default: return hipErrorInvalidValue;
        }
    }
    if (offsets) {
        switch (out) {
            case OUT_BF16:
                return launch_mid_t<OUT_BF16, true>(q, sa, qw, sw, M, N, K, y, offsets, E, 1, stream);
            case OUT_FP32:
                return launch_mid_t<OUT_FP32, true>(q, sa, qw, sw, M, N, K, y, offsets, E, 1, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (out) {
        case OUT_BF16:
            return launch_mid_t<OUT_BF16, false>(q, sa, qw, sw, M, N, K, y, nullptr, 0, 1, stream);
        case OUT_FP32:
            return launch_mid_t<OUT_FP32, false>(q, sa, qw, sw, M, N, K, y, nullptr, 0, 1, stream);
        case OUT_PARTIALS:
            return launch_mid_t<OUT_PARTIALS, false>(q, sa, qw, sw, M, N, K, y, nullptr, 0, 1,
                                                     stream);
        case OUT_BF16_CH:
            return launch_mid_t<OUT_BF16_CH, false>(q, sa, qw, sw, M, N, K, y, nullptr, 0,
                                                    sw_stride, stream);
        case OUT_FP32_CH:
            return launch_mid_t<OUT_FP32_CH, false>(q, sa, qw, sw, M, N, K, y, nullptr, 0,
                                                    sw_stride, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace bsb
