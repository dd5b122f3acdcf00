// W8A8 per-group-128 GEMM for prefill-shaped M (and the grouped MoE form with
// many rows per expert) on gfx950: 256x256 output tile per workgroup.
//
// [P3] sec. 3.1: INT8 x INT8 multiply-accumulate into INT32 inside the
// matmul, the FP32 scales applied last. Per output element:
//     acc = 0
//     for g = 0 .. K/128-1:                  (ascending, never split)
//         P   = sum_{k in group g} q[m,k]*qw[n,k]        (INT32, MFMA)
//         acc = fmaf((float)P, sw[n,g], acc)             (VALU epilogue)
//     y = acc * sa[m]  -> BF16 (RNE) or FP32
//
// Workgroup: 8 waves in a 4 (M) x 2 (N) grid, two per SIMD, each owning
// 64 x 128 outputs = 2 x 4 blocks of v_mfma_i32_32x32x32_i8. Per K group a
// block takes four MFMAs (32 K each) into a fresh INT32 accumulator, then 16
// conversions and 16 fused multiply-adds fold it into the float32 totals.
// Those 32 VALU instructions take as long as the block's four MFMAs, so the
// kernel is built to keep both units issuing side by side: every MFMA is
// followed by a quarter of the previous block's epilogue (8 VALU
// instructions), and nothing else runs on the VALU inside the main loop. LDS
// fragment addresses are fixed per lane and differ between stages, blocks
// and K steps only by constants, so every fragment read is one ds_read_b128
// with an immediate offset.
//
// Staging: per K group the A tile (256 rows x 128 B), the B tile (256 weight
// rows x 128 B) and the group's 256 weight scales go from global memory
// straight into LDS (buffer loads with the LDS-destination bit, 1 KB per wave
// instruction, 8 lanes per 128-byte row line, 16-byte chunk j of row r at
// j ^ ((r >> 1) & 7)), each in two stages. The B tile is staged as two
// halves: B01 holds the rows of every wave's column blocks 0 and 1, B23 those
// of blocks 2 and 3. Two barriers per group, after column block 0 (S) and
// after column block 2 (M), each preceded by a wait for the stages it
// publishes:
//   S(g): publishes B23[g] (read from block 1 on); frees the stages of A[g]
//         (read during block 3 of g-1) and B01[g] (read up to block 0), into
//         which A[g+2] and B01[g+2] are loaded at once;
//   M(g): publishes A[g+1], B01[g+1] and the scales of g+1, whose fragments are
//         read while block 3 of g is multiplied (each A fragment right after
//         its last use, each B fragment after its last use in that block);
//         frees B23[g] and the scales of g, into which B23[g+2] and the scales
//         of g+2 are loaded.
// A and B01 thus have one and a half groups of work to land, B23 one and a
// quarter, instead of one. Loads complete in issue order, so each wait is a
// single vmcnt that leaves the later stages in flight. 132 KB of LDS. The last
// block's epilogue moves into the next group, behind its first MFMA.
//
// Out-of-range rows, columns and groups read zero through the buffer
// descriptors (a zero group adds fmaf(0, 0, acc) = acc), so no load sits
// behind a branch; stores are masked by the real extents.
#include <type_traits>

#include "gemm_common.h"
#include "launch.h"

namespace bsb {

namespace {

constexpr int kBigTM = 256, kBigTN = 256;        // output tile per workgroup
constexpr int kBigStage = 256 * kGroup;          // A tile of one K group (bytes)
constexpr int kBigHalf = 128 * kGroup;           // half a B tile (B01 or B23) of one K group
constexpr int kBigLdsA = 0;                      // A tiles of stages 0, 1
constexpr int kBigLdsB01 = 2 * kBigStage;        // B01 halves of stages 0, 1
constexpr int kBigLdsB23 = kBigLdsB01 + 2 * kBigHalf;   // B23 halves of stages 0, 1
constexpr int kBigLdsS = kBigLdsB23 + 2 * kBigHalf;     // scales of stages 0, 1
constexpr int kBigScaleStage = 512 * 4;          // 256 scales + 256 slots for the spare loads
constexpr int kBigLdsRowS = kBigLdsS + 2 * kBigScaleStage;   // the tile's 256 row scales
constexpr int kBigLds = kBigLdsRowS + 256 * 4;   // 136192 bytes of 160 KB

__device__ __forceinline__ int big_swz(int r) { return (r >> 1) & 7; }

// GROUPED: q holds R = M rows sorted by expert, rows [offsets[e], offsets[e+1])
// multiply expert e's weights qw[e] / sw[e]; tile rows are laid out expert
// after expert (a tile never spans two experts) and the host sizes the grid
// for the most tiles any split of R rows over E experts can need.
// GATHER (grouped only): q / sa are the T quantised tokens and row m of the
// problem is token gidx[m] (the MoE gather done by the A-tile loads; an index
// outside [0, T) reads a zero row with scale 0).
template <int OUT, bool GROUPED, bool GATHER = false>
__global__ void __launch_bounds__(512, 1)
gemm_big_kernel(const int8_t *q, const float *sa, const int8_t *qw, const float *sw, int M, int N,
                int K, void *y, TileGrid tiles, const int32_t *offsets, int E, int sw_stride,
                const int32_t *gidx, int T) {
    constexpr bool CHN = per_channel<OUT>();             // one scale per row, applied at the end
    constexpr bool SCALES = !CHN && OUT != OUT_PARTIALS;   // per-group scales staged in LDS
    __shared__ __align__(16) int8_t lds[kBigLds];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, half = lane >> 5;
    const int G = K >> 7;
    int m0, row_end, bm, bn;
    if (GROUPED) {
        int e;
        if (!grouped_tile<kBigTM>(offsets, E, M, tiles, e, m0, row_end, bm, bn)) return;
        qw += (int64_t)e * N * K;
        sw += (int64_t)e * N * G;
    } else {
        xcd_tile_of(blockIdx.x, tiles, bm, bn);
        m0 = bm * kBigTM;
        row_end = M;
    }
    const int n0 = bn * kBigTN;
    const int mrows = min(kBigTM, row_end - m0), ncols = min(kBigTN, N - n0);

    const v4i ra = GATHER ? make_rsrc_words(q, (uint32_t)(T * K))
                          : make_rsrc_words(q + (int64_t)m0 * K, (uint32_t)(mrows * K));
    const v4i rb = make_rsrc_words(qw + (int64_t)n0 * K, (uint32_t)(ncols * K));
    const v4i rs = make_rsrc_words(SCALES ? sw + (int64_t)n0 * G : nullptr,
                                   SCALES ? (uint32_t)(ncols * G * 4) : 0u);

    // ---- staging (global -> LDS) ----
    // Each tile is filled in 1 KB blocks of 8 rows x 128 B; lane l lands at
    // byte 16*l of a block and fetches the global chunk that the swizzle puts
    // there. Wave w fills blocks 2w and 2w+1 of each region (LDS rows
    // 16w .. 16w+15), and of the A tile also blocks 16+2w, 17+2w (rows 128
    // further on). Rows 16 apart share the swizzle, so every block of a wave
    // uses one of two per-lane offsets and differs only in the scalar offset.
    // B01 row r holds tile row r + (r >= 64 ? 64 : 0), B23 row r tile row
    // r + 64 + (r >= 64 ? 64 : 0): the rows of column blocks 0-1 and 2-3 of
    // both waves' 128-row halves.
    uint32_t dvoff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = wave * 16 + 8 * j + (lane >> 3);
        dvoff[j] = (uint32_t)(row * K + (((lane & 7) ^ big_swz(row)) << 4));
    }
    // A rows of this lane's four A loads: 16w + 8j + lane/8 (j = 0, 1), and the
    // same 128 rows further on (rows 128 apart share the swizzle). Gathered,
    // each is its token's row; rows past the segment and invalid indices read
    // zeros. The index loads (and the row-scale one below) are issued together,
    // unconditionally (rows past the segment read the segment's last entry,
    // then dropped), and only then turned into offsets.
    auto arow = [&](int j) { return wave * 16 + 8 * (j & 1) + (lane >> 3) + 128 * (j >> 1); };
    int tix[5] = {0, 0, 0, 0, 0};
    if (GATHER) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = m0 + arow(j);
            tix[j] = gidx[m < row_end ? m : row_end - 1];
        }
        const int m = m0 + (wave & 3) * 64 + lane;
        tix[4] = gidx[m < row_end ? m : row_end - 1];
    }
    uint32_t aoff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (GATHER) {
            const int t = m0 + arow(j) < row_end ? tix[j] : -1;
            const uint32_t o = (uint32_t)t * (uint32_t)K + (uint32_t)(((lane & 7) ^ big_swz(arow(j))) << 4);
            aoff[j] = t >= 0 && t < T ? o : kOOB;
        } else {
            aoff[j] = dvoff[j & 1];   // the second 128 rows through the scalar offset
        }
    }
    // The tile's 256 activation scales go straight into LDS like the operands:
    // waves 0-3 load rows 64w .. 64w+63, one per lane, ahead of the first stage
    // (rows past the segment and invalid indices read zero). The epilogue then
    // reads no global memory, and no load of the prologue waits for them (at the
    // MoE layer with rows gathered through an index, scales read in the
    // epilogue: 444.9 us; staged by the lanes before the first stage: 400.8 us).
    const bool row_scales = OUT != OUT_PARTIALS && wave < 4;
    const v4i rsa = OUT == OUT_PARTIALS ? make_rsrc_words(nullptr, 0u)
                    : GATHER            ? make_rsrc_words(sa, (uint32_t)(T * 4))
                                        : make_rsrc_words(sa + m0, (uint32_t)(mrows * 4));
    uint32_t saoff = (uint32_t)((wave * 64 + lane) * 4);
    if (GATHER) {
        const int t = m0 + (wave & 3) * 64 + lane < row_end ? tix[4] : -1;
        saoff = t >= 0 && t < T ? (uint32_t)t * 4u : kOOB;
    }
    const uint32_t boff01 = (uint32_t)((wave >= 4 ? 64 : 0) * K);
    const uint32_t boff23 = (uint32_t)((wave >= 4 ? 128 : 64) * K);
    // Scales: waves 0-3 load the group's 256 scales, one per lane, into the
    // order [wn][l32][cb] (column n = 128 wn + 32 cb + l32), so that each lane
    // later reads its four column blocks' scales in one 16-byte read; waves
    // 4-7 issue the same load past the end into spare slots, which keeps every
    // wave's load count per stage equal.
    const int sp = wave * 64 + lane;
    const uint32_t svoff =
        wave < 4 ? (uint32_t)((((sp >> 7) << 7) + ((sp & 3) << 5) + ((sp >> 2) & 31)) * G * 4) : 0u;
    const uint32_t lbase = (uint32_t)(uintptr_t)lds;

    // Each batch is one statement, so nothing the compiler emits lands between
    // the loads. s_nop 4: a VALU write of an SGPR read by a vector memory
    // instruction needs five wait states (the compiler may form the
    // descriptors or offsets with v_readfirstlane right before); s_nop 0 after
    // each M0 write: one wait state before an LDS-destination load reads M0.
    // S batch of group g into stage st: A (4 loads) and B01 (2 loads).
    auto dma_s = [&](int st, int g) {
        const bool in = g < G;
        const uint32_t so = in ? (uint32_t)g * kGroup : kOOB;
        const uint32_t sa2 = in ? (GATHER ? so : so + (uint32_t)(128 * K)) : kOOB;
        const uint32_t sb = in ? so + boff01 : kOOB;
        const uint32_t ma = lbase + kBigLdsA + st * kBigStage + wave * 2048;
        const uint32_t mb = lbase + kBigLdsB01 + st * kBigHalf + wave * 2048;
        uint32_t m0_out;   // M0 is written inside: declared as an output
        asm volatile(
            "s_nop 4\n\t"
            "s_mov_b32 m0, %[a0]\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %[w0], %[ra], %[s0] offen lds\n\t"
            "s_mov_b32 m0, %[a1]\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %[w1], %[ra], %[s0] offen lds\n\t"
            "s_mov_b32 m0, %[a2]\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %[w2], %[ra], %[s1] offen lds\n\t"
            "s_mov_b32 m0, %[a3]\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %[w3], %[ra], %[s1] offen lds\n\t"
            "s_mov_b32 m0, %[b0]\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %[v0], %[rb], %[s2] offen lds\n\t"
            "s_mov_b32 m0, %[b1]\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %[v1], %[rb], %[s2] offen lds"
            : "=&{m0}"(m0_out)
            : [a0] "s"(ma), [a1] "s"(ma + 1024), [a2] "s"(ma + 16384), [a3] "s"(ma + 17408),
              [b0] "s"(mb), [b1] "s"(mb + 1024), [v0] "v"(dvoff[0]), [v1] "v"(dvoff[1]),
              [w0] "v"(aoff[0]), [w1] "v"(aoff[1]), [w2] "v"(aoff[2]), [w3] "v"(aoff[3]),
              [ra] "s"(ra), [rb] "s"(rb), [s0] "s"(so), [s1] "s"(sa2), [s2] "s"(sb)
            : "memory");
        (void)m0_out;
    };
    // M batch of group g into stage st: the scales (1 load) and B23 (2 loads).
    auto dma_m = [&](int st, int g) {
        const bool in = g < G;
        const uint32_t sb = in ? (uint32_t)g * kGroup + boff23 : kOOB;
        const uint32_t sso = (in && wave < 4) ? (uint32_t)g * 4 : kOOB;
        const uint32_t mb = lbase + kBigLdsB23 + st * kBigHalf + wave * 2048;
        const uint32_t ms = lbase + kBigLdsS + st * kBigScaleStage + wave * 256;
        uint32_t m0_out;
        asm volatile(
            "s_nop 4\n\t"
            "s_mov_b32 m0, %[c0]\n\ts_nop 0\n\t"
            "buffer_load_dword %[vs], %[rs], %[ss] offen lds\n\t"
            "s_mov_b32 m0, %[b0]\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %[v0], %[rb], %[s2] offen lds\n\t"
            "s_mov_b32 m0, %[b1]\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %[v1], %[rb], %[s2] offen lds"
            : "=&{m0}"(m0_out)
            : [c0] "s"(ms), [b0] "s"(mb), [b1] "s"(mb + 1024), [v0] "v"(dvoff[0]),
              [v1] "v"(dvoff[1]), [vs] "v"(svoff), [rb] "s"(rb), [rs] "s"(rs), [s2] "s"(sb),
              [ss] "s"(sso)
            : "memory");
        (void)m0_out;
    };
    auto dma_rows = [&]() {
        const uint32_t mr = lbase + kBigLdsRowS + wave * 256;
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
    // Loads per wave: 6 in an S batch, 3 in an M batch (scales first).
    // At S(g) B23[g] (end of the M batch of g-2) must have landed: the S and M
    // batches of g-1 (9 loads) may still be in flight. At M(g) the S batch of
    // g-1 and the scales of g+1 (first load of the M batch of g-1) must have
    // landed: B23[g+1] and the S batch of g (8 loads) may be in flight.
    auto wait_s = [&]() { asm volatile("s_waitcnt vmcnt(9) lgkmcnt(0)" ::: "memory"); };
    auto wait_m = [&]() { asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory"); };

    // ---- fragment reads (LDS -> registers) ----
    // A fragment (row block rb, K step ks) of lane l: 16 bytes of row
    // 64 wm + 32 rb + l32 at K bytes 32 ks + 16 half; B likewise for weight row
    // 128 wn + 32 cb + l32. Rows 32 apart share the swizzle, so stage, block
    // and K-step offsets beyond the per-(ks) lane base are constants.
    // B fragments of column blocks 0-1 come from B01 row 64 wn + 32 cb + l32,
    // those of blocks 2-3 from the same row of B23 (one lane base for both).
    uint32_t fa[4], fb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int r_a = wm * 64 + l32, r_b = wn * 64 + l32;
        fa[ks] = kBigLdsA + r_a * kGroup + (((2 * ks + half) ^ big_swz(r_a)) << 4);
        fb[ks] = kBigLdsB01 + r_b * kGroup + (((2 * ks + half) ^ big_swz(r_b)) << 4);
    }
    const uint32_t fs = kBigLdsS + (wn * 128 + l32 * 4) * 4;
    auto ldA = [&](int st, int rb_, int ks) {
        return *reinterpret_cast<const v4i *>(lds + fa[ks] + st * kBigStage + rb_ * 4096);
    };
    auto ldB = [&](int st, int cb, int ks) {
        const int off = cb < 2 ? st * kBigHalf + cb * 4096
                               : (kBigLdsB23 - kBigLdsB01) + st * kBigHalf + (cb - 2) * 4096;
        return *reinterpret_cast<const v4i *>(lds + fb[ks] + off);
    };
    auto ldS = [&](int st) {
        return *reinterpret_cast<const v4f *>(lds + fs + st * kBigScaleStage);
    };

    const bool active = wm * 64 < mrows;   // rows of this wave exist in the tile

    v16f facc[2][4];   // float32 totals (per-group forms)
    v16i pacc[2][4];   // INT32 totals (per-channel forms)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                facc[i][j][r] = 0.0f;
                pacc[i][j][r] = 0;
            }

    // prologue: the row scales (waves 0-3), then groups 0 and 1 into stages 0
    // and 1; wait for the row scales, A[0], B01[0] and the scales of group 0
    // (B23[0] and group 1 may stay in flight: the same count with or without
    // the row-scale load in front)
    if (row_scales) dma_rows();
    dma_s(0, 0);
    dma_m(0, 0);
    dma_s(1, 1);
    dma_m(1, 1);
    asm volatile("s_waitcnt vmcnt(11)" ::: "memory");
    __syncthreads();

    if (active) {
        v4i a[2][4], b[4];
        v4f sc = ldS(0), scn;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) a[i][ks] = ldA(0, i, ks);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) b[ks] = ldB(0, 0, ks);
        v16i prev;         // INT32 partials of the block whose epilogue is pending
        float prev_s = 0;  // its weight scale (0 with zero partials before the first group)
#pragma unroll
        for (int r = 0; r < 16; ++r) prev[r] = 0;

        // Epilogue quarter qt of the pending block (row block pi, column block pj).
        auto epi = [&](int pi, int pj, int qt, int g) {
            if (OUT == OUT_PARTIALS) {
                if (g < 0) return;
                const int n = n0 + wn * 128 + pj * 32 + l32;
#pragma unroll
                for (int r = 4 * qt; r < 4 * qt + 4; ++r) {
                    const int m = m0 + wm * 64 + pi * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                    if (m < row_end && n < N)
                        reinterpret_cast<int32_t *>(y)[((int64_t)m * N + n) * G + g] = prev[r];
                }
            } else if (SCALES) {
#pragma unroll
                for (int r = 4 * qt; r < 4 * qt + 4; ++r)
                    facc[pi][pj][r] = __builtin_fmaf((float)prev[r], prev_s, facc[pi][pj][r]);
            }
        };

        // One K group on stage st (group g): column blocks cb = 0..3, row
        // blocks rb = 0..1, four MFMAs each.
        auto step = [&](auto stc, int g) {
            constexpr int st = decltype(stc)::value;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
                for (int rb_ = 0; rb_ < 2; ++rb_) {
                    const int j = 2 * cb + rb_;   // block unit; its predecessor's epilogue runs beside it
                    const int pi = j == 0 ? 1 : (j - 1) & 1, pj = j == 0 ? 3 : (j - 1) >> 1;
                    v16i c;
#pragma unroll
                    for (int r = 0; r < 16; ++r) c[r] = CHN ? pacc[rb_][cb][r] : 0;
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        c = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[rb_][ks], b[ks], c, 0, 0, 0);
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        if (cb == 3) {   // fragments of group g+1 after their last use in g
                            a[rb_][ks] = ldA(st ^ 1, rb_, ks);
                            if (rb_ == 1) {
                                b[ks] = ldB(st ^ 1, 0, ks);
                                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                            } else {
                                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                            }
                        } else if (rb_ == 1) {   // next column block of this group
                            b[ks] = ldB(st, cb + 1, ks);
                            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                        }
                        epi(pi, pj, ks, j == 0 ? g - 1 : g);
                        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                    }
                    if (CHN) pacc[rb_][cb] = c;
                    prev = c;
                    prev_s = sc[cb];
                }
                // Around the barriers the wave drops to the default priority, so a
                // wave of the same SIMD that is still multiplying issues first.
                if (cb == 0 || cb == 2) __builtin_amdgcn_s_setprio(0);
                if (cb == 0) {
                    // S(g): publish B23[g]; A[g] and B01[g] are read: load g+2 there
                    wait_s();
                    __syncthreads();
                    dma_s(st, g + 2);
                } else if (cb == 2) {
                    // M(g): publish A, B01 and the scales of g+1; B23[g] and the
                    // scales of g are read: load g+2 there
                    wait_m();
                    __syncthreads();
                    dma_m(st, g + 2);
                    scn = ldS(st ^ 1);
                }
                if (cb == 0 || cb == 2) __builtin_amdgcn_s_setprio(2);
            }
            sc = scn;
        };

        __builtin_amdgcn_s_setprio(2);   // the multiplying phases run at the raised priority
        int g = 0;
        for (; g + 1 < G; g += 2) {
            step(std::integral_constant<int, 0>{}, g);
            step(std::integral_constant<int, 1>{}, g + 1);
        }
        if (g < G) step(std::integral_constant<int, 0>{}, g);
        epi(1, 3, 0, G - 1);
        epi(1, 3, 1, G - 1);
        epi(1, 3, 2, G - 1);
        epi(1, 3, 3, G - 1);
        __builtin_amdgcn_s_setprio(0);
    } else {
        // rows past the tile's end: stage this wave's share and meet every barrier
        for (int g = 0; g < G; ++g) {
            const int st = g & 1;
            wait_s();
            __syncthreads();
            dma_s(st, g + 2);
            wait_m();
            __syncthreads();
            dma_m(st, g + 2);
        }
    }
    // loads past the last group still write (zeros) into LDS: let them land
    // before the workgroup's LDS can be handed to another one
    wait_vmem();
    // BF16 results leave through LDS: the MFMA layout gives a lane one column of
    // 16 rows per block, so direct stores write 2 bytes per lane (128 store
    // instructions per lane, ~8.5 us per tile); transposed through the stages
    // (free once every wave has passed this barrier) they leave as 16-byte
    // rows, 16 instructions per lane (~5.5 us per tile; measured on the whole
    // kernel: prefill 308 -> 304 us, the MoE grouped GEMM 423-430 -> 404-412 us).
    constexpr bool LDS_OUT = OUT == OUT_BF16 || OUT == OUT_BF16_CH;
    if (LDS_OUT) __syncthreads();
    if (!active) return;
    if (LDS_OUT) {
        // this wave's 64 x 128 outputs as 256-byte BF16 rows in the 16 KB at
        // 16384 * wave, 16-byte chunk c of row r at c ^ (r & 7) (the two rows one
        // write instruction covers, 4 apart, fall in different banks; a read of
        // 4 rows x 16 chunks covers every bank once)
        int8_t *wo = lds + wave * 16384;
        const float *rsc = reinterpret_cast<const float *>(lds + kBigLdsRowS) + wm * 64;
        float swn[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // per-channel forms: the columns' scales
        if (CHN) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = n0 + wn * 128 + j * 32 + l32;
                swn[j] = n < N ? sw[(int64_t)n * sw_stride] : 0.0f;
            }
        }
        auto val = [&](int i, int j, int r, float s) {
            return CHN ? channel_value(pacc[i][j][r], swn[j], s) : facc[i][j][r] * s;
        };
        // rows ml and ml + 1 (r even, r + 1) converted as one pair
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const int ml = i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                const float s0 = rsc[ml], s1 = rsc[ml + 1];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = j * 32 + l32;
                    const uint32_t h = bf16x2_rne(val(i, j, r, s0), val(i, j, r + 1, s1));
                    const int co = (c & 7) * 2;
                    *reinterpret_cast<uint16_t *>(wo + ml * 256 + (((c >> 3) ^ (ml & 7)) << 4) + co) =
                        (uint16_t)h;
                    *reinterpret_cast<uint16_t *>(wo + (ml + 1) * 256 +
                                                  (((c >> 3) ^ ((ml + 1) & 7)) << 4) + co) =
                        (uint16_t)(h >> 16);
                }
            }
        const bool wide = (N & 7) == 0;   // 16-byte aligned rows of 8 outputs
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int row = 4 * k + (lane >> 4), c16 = lane & 15;
            const v4i d = *reinterpret_cast<const v4i *>(wo + row * 256 + ((c16 ^ (row & 7)) << 4));
            const int m = m0 + wm * 64 + row;
            const int n = n0 + wn * 128 + c16 * 8;
            if (m >= row_end) continue;
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

    if (CHN) {
        float swn[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + wn * 128 + j * 32 + l32;
            swn[j] = n < N ? sw[(int64_t)n * sw_stride] : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                if (m >= row_end) continue;
                const float s = reinterpret_cast<const float *>(lds + kBigLdsRowS)[m - m0];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int n = n0 + wn * 128 + j * 32 + l32;
                    if (n < N)
                        store_out<OUT>(y, (int64_t)m * N + n, channel_value(pacc[i][j][r], swn[j], s));
                }
            }
    } else if (OUT != OUT_PARTIALS) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                if (m >= row_end) continue;
                const float s = reinterpret_cast<const float *>(lds + kBigLdsRowS)[m - m0];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int n = n0 + wn * 128 + j * 32 + l32;
                    if (n < N) store_out<OUT>(y, (int64_t)m * N + n, facc[i][j][r] * s);
                }
            }
    }
}

template <int OUT, bool GROUPED, bool GATHER = false>
hipError_t launch_big_t(const int8_t *q, const float *sa, const int8_t *qw, const float *sw, int M,
                        int N, int K, void *y, const int32_t *offsets, int E, int sw_stride,
                        hipStream_t stream, const int32_t *gidx = nullptr, int T = 0) {
    // Grouped: sum over experts of ceil(rows_e / 256) <= ceil(R / 256) + E tile rows.
    const int64_t mt = (M + kBigTM - 1) / kBigTM + (GROUPED ? E : 0), nt = (N + kBigTN - 1) / kBigTN;
    const int64_t total = mt * nt;
    if (total > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const TileGrid t{(int)mt, (int)nt};
    gemm_big_kernel<OUT, GROUPED, GATHER><<<dim3((unsigned)total), 512, 0, stream>>>(
        q, sa, qw, sw, M, N, K, y, t, offsets, E, sw_stride, gidx, T);
    return hipGetLastError();
}

}  // namespace

bool big_gemm_fits(int64_t K) {
    // 32-bit buffer offsets: a lane's row of a 256-row panel plus 16 rows and a group
    return (int64_t)(kBigTM + 16) * K + kGroup < ((int64_t)1 << 31);
}

hipError_t launch_gemm_big(const int8_t *q, const float *sa, const int8_t *qw, const float *sw,
                           int M, int N, int K, void *y, int out, const int32_t *offsets, int E,
                           int sw_stride, hipStream_t stream, const int32_t *gidx, int T) {
    if (offsets && gidx) {
        switch (out) {
            case OUT_BF16:
                return launch_big_t<OUT_BF16, true, true>(q, sa, qw, sw, M, N, K, y, offsets, E, 1,
                                                          stream, gidx, T);
            case OUT_FP32:
                return launch_big_t<OUT_FP32, true, true>(q, sa, qw, sw, M, N, K, y, offsets, E, 1,
                                                          stream, gidx, T);
            default: return hipErrorInvalidValue;
        }
    }
    if (offsets) {
        switch (out) {
            case OUT_BF16:
                return launch_big_t<OUT_BF16, true>(q, sa, qw, sw, M, N, K, y, offsets, E, 1, stream);
            case OUT_FP32:
                return launch_big_t<OUT_FP32, true>(q, sa, qw, sw, M, N, K, y, offsets, E, 1, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (out) {
        case OUT_BF16:
            return launch_big_t<OUT_BF16, false>(q, sa, qw, sw, M, N, K, y, nullptr, 0, 1, stream);
        case OUT_FP32:
            return launch_big_t<OUT_FP32, false>(q, sa, qw, sw, M, N, K, y, nullptr, 0, 1, stream);
        case OUT_PARTIALS:
            return launch_big_t<OUT_PARTIALS, false>(q, sa, qw, sw, M, N, K, y, nullptr, 0, 1,
                                                     stream);
        case OUT_BF16_CH:
            return launch_big_t<OUT_BF16_CH, false>(q, sa, qw, sw, M, N, K, y, nullptr, 0,
                                                    sw_stride, stream);
        case OUT_FP32_CH:
            return launch_big_t<OUT_FP32_CH, false>(q, sa, qw, sw, M, N, K, y, nullptr, 0,
                                                    sw_stride, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace bsb
