// W8A8 per-group-128 GEMM (dense and grouped/MoE) on gfx950 MFMA.
//
// [P3] sec. 3.1: INT8 x INT8 multiply-accumulate into INT32 inside the
// matmul, the FP32 scales applied last. Per output element:
//     acc = 0
//     for g = 0 .. K/128-1:                  (ascending, never split)
//         P   = sum_{k in group g} q[m,k]*qw[n,k]        (INT32, MFMA)
//         acc = fmaf((float)P, sw[n,g], acc)             (VALU epilogue)
//     y = acc * sa[m]  -> BF16 (RNE) or FP32
//
// The kernels share that per-group structure:
//
//  * smallm (M <= 64, decode-shaped): the weight matrix is the stream. A
//    workgroup of 4 waves owns 64 output columns; each wave owns 16 columns
//    and all M rows (v_mfma_i32_16x16x64_i8, one 16-row block per 16 tokens).
//    The activation tile of the current group is staged once per workgroup
//    in LDS (double-buffered); each lane prefetches its weight bytes PF groups
//    ahead straight into registers, so every weight byte is read from HBM
//    once with many bytes in flight per wave.
//
//  * the tiled kernels for larger M (gemm_mid.hip, 128x128 tiles, and
//    gemm_big.hip, 256x256 tiles for prefill-shaped M and the grouped MoE
//    form with many rows per expert), selected by the launchers below.
//
// MFMA operand pairing: lane l supplies 16 bytes of row (l % 16 or l % 32)
// of A and the same 16 K positions of column (l % 16 or l % 32) of B. Any
// assignment of K positions to (lane slot, instruction) that is identical for
// A and B gives the same exact INT32 sum; each lane here owns a contiguous
// span of the group so its loads are 16-byte aligned and contiguous.
#include "gemm_common.h"
#include "launch.h"

namespace bsb {

namespace {

__device__ __forceinline__ v4i as_v4i(uint4 u) {
    v4i r;
    r[0] = (int)u.x; r[1] = (int)u.y; r[2] = (int)u.z; r[3] = (int)u.w;
    return r;
}

// LDS position of 16-byte chunk j of row r is j ^ chunk_swizzle(r): rows of
// 128 B (8 chunks) share a pattern in pairs, rows of 256 B (16 chunks) each
// have their own, so 16 rows read at one chunk index hit 16 distinct bank groups.
template <int ROW_BYTES>
__device__ __forceinline__ int chunk_swizzle(int r) {
    return ROW_BYTES == 256 ? (r & 15) : ((r >> 1) & 7);
}

// --------------------------------------------------------------------------
// smallm: M <= 16*MB tokens, weight-streaming.
// --------------------------------------------------------------------------
// Workgroup = NW waves = 16*NW weight rows (output columns) n0 .. n0+16*NW-1;
// each wave owns 16 of them (v_mfma_i32_16x16x64_i8, MB 16-token blocks).
//
// K is walked in stages of S groups through a ring of D LDS buffers. A
// stage's weight tile (16*NW rows x S*128 B) and activation tile (16*MB rows
// x S*128 B) go from global memory straight into LDS: buffer
// loads with the LDS-destination bit, each wave instruction filling one 1 KB
// block of 8 rows x 128 B (8 lanes per row line, the pattern HBM streams
// fastest; lane l lands at byte 16*l and fetches the chunk the swizzle puts
// there), with the non-temporal hint on weight streams large enough to gain
// from it. Nothing is staged through registers, so D-1 stages stay in flight.
// A single wait with a constant count finds the oldest stage landed: in
// narrow workgroups every wave issues the same number of loads per stage
// (spare ones read zero into a sink); wider ones skip the spares and each wave
// waits with the smallest count any wave issues every stage, which the
// in-order completion of loads makes sufficient. One barrier per stage then
// publishes the stage to all waves and frees the buffer that the next stage
// is loaded into. The loads are issued through
// inline assembly and waited for by hand: the compiler would otherwise wait
// for all of them before any LDS read.
//
// Workgroups of 4 or more waves stage the weight scales in chunks of 16
// groups (double-buffered): a chunk
// is 16*NW rows x 64 contiguous bytes, loaded in pieces of 4 rows (one 4-byte
// load per lane, 4 row segments per instruction rather than a line per lane).
// Each wave adds one piece load to every stage (a spare one reads zero into
// the sink), so the per-stage count stays constant; the pieces of chunk c+1
// ride on stages of chunk c that are issued after the barrier that retires
// chunk c-1, whose buffer they reuse, and land before chunk c+1's first stage.
// Narrower workgroups (where that measured slower) load each stage's own S
// groups of scales with it instead, one entry per lane.
//
// LDS tile layout: [group][row][8 x 16-byte chunks], chunk j of row r stored
// at position j ^ ((r >> 1) & 7): fragment reads (16 rows, one chunk index)
// hit 16 distinct 16-byte bank groups.
//
// Out-of-range rows, columns and groups read zero through the buffer
// descriptors (a group past the end adds fmaf(0, 0, acc) = acc, bit for bit),
// so no load sits behind a branch. Requires 16*NW*K < 2^31 (checked by the
// launcher).
//
// GROUPED (MoE with few rows per expert): blockIdx.y is the expert; the
// workgroup walks that expert's rows [offsets[e], offsets[e+1]) in passes of
// 16*MB rows against its slice of the expert's weights.
constexpr int kScaleChunk = 16;   // groups per staged chunk of weight scales

template <int NW>
constexpr bool smallm_chunked_scales() {
    return NW >= 4;
}

template <int NW, int S>
constexpr int smallm_stage_scale_floats() {   // per-stage scales, padded to whole waves
    return ((S * 16 * NW + 63) / 64) * 64;
}

// Activation modes of the small-M kernel: INT8 activations with their
// per-token scales (W8A8), BF16 activations with INT8 weights and per-group
// scales (W8A16), BF16 activations with BF16 weights (no scales).
enum { AM_W8A8 = 0, AM_W8A16 = 1, AM_BF16 = 2 };

template <int MB, int NW, int S, int AM = AM_W8A8>
constexpr int smallm_stage_bytes() {
    return S * 16 * NW * kGroup * (AM == AM_BF16 ? 2 : 1) + S * 16 * MB * kGroup * (AM ? 2 : 1) +
           (smallm_chunked_scales<NW>() || AM == AM_BF16 ? 0
                                                         : 4 * smallm_stage_scale_floats<NW, S>());
}

template <int NW, int AM = AM_W8A8>
constexpr int smallm_fixed_bytes() {   // scale chunks + sink
    return (smallm_chunked_scales<NW>() && AM != AM_BF16 ? 2 * 16 * NW * kScaleChunk * 4 : 0) +
           1024;
}

template <int MB, int NW, int OUT, int S, int D, bool GROUPED, bool NT, int AM = AM_W8A8>
__global__ void __launch_bounds__(64 * NW)
gemm_smallm_kernel(const int8_t *__restrict__ q, const float *__restrict__ sa,
                   const int8_t *__restrict__ qw, const float *__restrict__ sw, int M, int N,
                   int K, void *__restrict__ y, const int32_t *__restrict__ offsets,
                   int sw_stride, const int32_t *__restrict__ gidx, int T) {
    constexpr int ROWS = 16 * MB;              // activation rows
    constexpr int WR = 16 * NW;                // weight rows per workgroup
    constexpr int RW = kGroup * (AM == AM_BF16 ? 2 : 1);   // bytes of a weight row per group
    constexpr int RA = kGroup * (AM ? 2 : 1);             // bytes of an activation row per group
    constexpr int BT = WR * RW;                // one group of the weight tile (bytes)
    constexpr int AT = ROWS * RA;              // one group of the activation tile
    constexpr int WBLK = S * BT / 1024 / NW;   // 1 KB weight blocks per wave per stage
    constexpr int ABLK = (S * AT / 1024 + NW - 1) / NW;   // activation blocks per wave
    constexpr bool CHN = per_channel<OUT>();   // one scale per row, applied at the end
    constexpr bool NOSCALE = CHN || AM == AM_BF16;   // no per-group scales to stage
    constexpr int NLD = WBLK + ABLK + (NOSCALE ? 0 : 1);   // load slots per wave per stage (+1: scales)
    constexpr int TBLK = S * AT / 1024;        // activation blocks per stage
    // Spare slots issue nothing (a load past the end still costs an
    // instruction on the LDS-destination path), so waves issue different
    // numbers of loads per stage; each waits with the smallest number any wave
    // issues every stage: weights plus the activation blocks of the last wave.
    // With loads completing in issue order, at most (D-2)*NLD_MIN outstanding
    // means the oldest stage has landed whatever this wave issued after it.
    // (workgroups of 4 or more waves; narrower ones, with at most one spare,
    // measured faster keeping it)
    constexpr bool NOSPARE = NW >= 4;
    constexpr int A_MIN = TBLK - (NW - 1) * ABLK > 0 ? TBLK - (NW - 1) * ABLK : 0;
    constexpr int NLD_MIN = NOSPARE ? WBLK + A_MIN : NLD;
    constexpr int SCH = kScaleChunk;
    constexpr int SPC = SCH / S;               // stages per scale chunk
    constexpr int NP = WR * SCH / 64;          // 4-row pieces per scale chunk (= 4*NW)
    constexpr bool CHUNKED = smallm_chunked_scales<NW>() && !NOSCALE;
    constexpr int SPAD = smallm_stage_scale_floats<NW, S>();
    static_assert(D >= 2 && (D - 2) * NLD <= 63 && NLD_MIN >= 1,
                  "ring depth or wait count out of range");
    static_assert(!CHUNKED || (SCH % S == 0 && NP == 4 * NW && SPC >= D + 3),
                  "scale pieces must fit the stages issued after a chunk's buffer is free");
    __shared__ __align__(16) int8_t Bs[D][S * BT];
    __shared__ __align__(16) int8_t As[D][S * AT];
    // scales: [2][WR][SCH] in chunks, or [D][SPAD] per stage (entry gl*WR + row)
    __shared__ __align__(16) float Sc[NOSCALE ? 64 : CHUNKED ? 2 * WR * SCH : D * SPAD];
    __shared__ __align__(16) int8_t sink[1024];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = K >> 7;
    const int col = lane & 15;          // B column / A row within a 16-block
    const int slot = lane >> 4;         // which 32-byte quarter of the group
    const int n0 = blockIdx.x * WR;
    const int nrows = min(WR, N - n0);
    const int nl = wave * 16 + col;     // this lane's weight row within the slice
    const int n = n0 + nl;
    const int wv = __builtin_amdgcn_readfirstlane(wave);

    int lo = 0, hi = M;                 // rows of this workgroup
    if (GROUPED) {
        const int e = blockIdx.y;       // segment clamped to [0, R]
        lo = offsets[e];
        hi = offsets[e + 1];
        lo = lo < 0 ? 0 : (lo > M ? M : lo);
        hi = hi < lo ? lo : (hi > M ? M : hi);
        if (hi == lo) return;           // whole workgroup: empty expert
        qw += (int64_t)e * N * K;
        sw += (int64_t)e * N * G;
    }

    const v4i rw = make_rsrc_words(qw + (int64_t)n0 * K * (RW / kGroup),
                                   (uint32_t)(nrows * K * (RW / kGroup)));
    // The partials form has no scales (sw may be null): an empty descriptor
    // makes its scale loads read zero without touching memory.
    const v4i rsc = make_rsrc_words(OUT == OUT_PARTIALS || NOSCALE ? nullptr : sw + (int64_t)n0 * G,
                                    OUT == OUT_PARTIALS || NOSCALE ? 0u : (uint32_t)(nrows * G * 4));
    v4i ra;                             // the current pass's activation rows
    int rows = 0, r0 = 0;

    // Per-lane parts of the staging offsets and LDS destinations. A block's
    // group (stage start + its group within the stage) travels in the scalar
    // offset, pushed past the end of the descriptor for groups past the last,
    // so those read zero.
    uint32_t wvo[WBLK], avo[ABLK];
    uint32_t wdst[WBLK], adst[ABLK];
    int wgl[WBLK], agl[ABLK];
    // A 1 KB block holds 1024 / R rows of R bytes (R = 128 or 256 per group),
    // R / 16 lanes per row; chunk j of row r sits at position j ^ swz(r).
#pragma unroll
    for (int i = 0; i < WBLK; ++i) {
        constexpr int LPR = RW / 16, RPB = 1024 / RW;
        const int blk = wv * WBLK + i;
        const int gl = blk / (BT / 1024), rb = blk % (BT / 1024);
        const int row = rb * RPB + lane / LPR, pos = lane % LPR;
        wvo[i] = (uint32_t)(row * K * (RW / kGroup) + ((pos ^ chunk_swizzle<RW>(row)) << 4));
        wdst[i] = (uint32_t)(gl * BT + rb * 1024);
        wgl[i] = gl;
    }
#pragma unroll
    for (int i = 0; i < ABLK; ++i) {
        constexpr int LPR = RA / 16, RPB = 1024 / RA;
        const int blk = wv * ABLK + i;
        const bool ok = blk < S * AT / 1024;
        const int gl = blk / (AT / 1024), rb = blk % (AT / 1024);
        const int row = rb * RPB + lane / LPR, pos = lane % LPR;
        avo[i] = ok ? (uint32_t)(row * K * (RA / kGroup) + ((pos ^ chunk_swizzle<RA>(row)) << 4))
                    : kOOB;
        adst[i] = ok ? (uint32_t)(gl * AT + rb * 1024) : 0xFFFFFFFFu;
        agl[i] = ok ? gl : 0;
    }
    auto goffw = [&](int g) { return g < G ? (uint32_t)g * RW : kOOB; };
    auto goffa = [&](int g) { return g < G ? (uint32_t)g * RA : kOOB; };

    auto lds_addr = [](const void *p) {
        return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
    };
    // piece p (wave-uniform) of scale chunk c: rows 4p .. 4p+3, lane l -> row
    // 4p + (l >> 4), group c*SCH + (l & 15); p outside [0, NP) is a spare
    auto piece = [&](int c, int p) {
        const bool ok = p >= 0 && p < NP;
        const int row = 4 * p + (lane >> 4), g = c * SCH + (lane & 15);
        const uint32_t vo = (OUT != OUT_PARTIALS && ok && g < G) ? (uint32_t)(row * G * 4 + g * 4)
                                                                  : kOOB;
        buf_load4_lds(rsc,
                      lds_addr(ok ? &Sc[(c & 1) * WR * SCH + p * 64]
                                  : reinterpret_cast<float *>(sink)),
                      vo, 0u);
    };
    // With G a multiple of 4 a piece can be 16 rows x 64 B, one 16-byte load
    // per lane (lane l -> row 16p + l/4, groups c*SCH + 4*(l%4) .. +3, all
    // inside or all past G): a chunk is then NW pieces, one per wave, all on
    // the first stage issued after the chunk's buffer is free.
    const bool g4 = (G & 3) == 0;
    auto piece4 = [&](int c, int p) {
        const int row = 16 * p + (lane >> 2), g = c * SCH + 4 * (lane & 3);
        const uint32_t vo = (OUT != OUT_PARTIALS && g < G) ? (uint32_t)(row * G * 4 + g * 4) : kOOB;
        buf_load16_lds(rsc, lds_addr(&Sc[(c & 1) * WR * SCH + p * 256]), vo, 0u);
    };
    // per-stage form: lane l of wave w stages entry 64w + l = (group within
    // stage, weight row) of the stage, in that order; its group is per lane
    const int sidx = wv * 64 + lane;
    const int sgl = sidx / WR;
    const uint32_t svo =
        (sidx < S * WR && OUT != OUT_PARTIALS) ? (uint32_t)((sidx % WR) * G * 4 + sgl * 4) : kOOB;
    const bool s_wave = wv * 64 < SPAD;
    auto issue = [&](int d, int s0) {   // stage of groups s0 .. s0+S-1 into buffer d
#pragma unroll
        for (int i = 0; i < WBLK; ++i) {
            if (NT)
                buf_load16_lds_nt(rw, lds_addr(&Bs[d][wdst[i]]), wvo[i], goffw(s0 + wgl[i]));
            else
                buf_load16_lds(rw, lds_addr(&Bs[d][wdst[i]]), wvo[i], goffw(s0 + wgl[i]));
        }
#pragma unroll
        for (int i = 0; i < ABLK; ++i) {
            if (NOSPARE && wv * ABLK + i >= TBLK) continue;   // wave-uniform
            buf_load16_lds(ra, lds_addr(adst[i] != 0xFFFFFFFFu ? &As[d][adst[i]] : sink), avo[i],
                           adst[i] != 0xFFFFFFFFu ? goffa(s0 + agl[i]) : 0u);   // spare: reads zero
        }
        if (NOSCALE) {
            // no per-group scales
        } else if (CHUNKED) {
            // the stage's scale piece: stage X = s0 / S, position sg in its chunk
            const int X = s0 / S, sg = X % SPC;
            if (g4) {
                if (sg == D - 1) piece4(X / SPC + 1, wv);
            } else {
                const int pc = sg >= D - 1 ? (sg - (D - 1)) * NW + wv : -1;
                if (!NOSPARE || (pc >= 0 && pc < NP)) piece(X / SPC + 1, pc);
            }
        } else if (!NOSPARE || s_wave) {
            buf_load4_lds(rsc,
                          lds_addr(s_wave ? &Sc[d * SPAD + wv * 64]
                                          : reinterpret_cast<float *>(sink)),
                          s0 + sgl < G ? svo : kOOB, (uint32_t)s0 * 4);
        }
    };
    auto swz = [](int row, int j) { return (j ^ ((row >> 1) & 7)) * 16; };

    float facc[MB][4];
    v4i iacc[MB];   // per-channel form: the INT32 total so far
    // One stage: every LDS fragment first, then all matrix instructions, then
    // the per-group epilogues in group order, so that the stage pays one LDS
    // round trip and one matrix-pipeline drain rather than one per instruction.
    // BF16 activations: per group four v_mfma_f32_16x16x32_bf16; lane (col,
    // slot) of instruction kk holds K elements 8*(4kk + slot) .. +7 of its row
    // (A: activation row i*16 + col, B: weight row nl), the same for both
    // operands. INT8 weights are read 8 bytes at a time and converted to BF16
    // (exact: |w| <= 127 has at most 7 significant bits).
    auto compute_a16 = [&](int d, int s0) {
#pragma unroll
        for (int gl = 0; gl < S; ++gl) {
            const int8_t *at = &As[d][gl * AT];
            const int8_t *bt = &Bs[d][gl * BT];
            bf16x8 a[4][MB], b[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int c = 4 * kk + slot;
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    const int ar = i * 16 + col;
                    a[kk][i] = *reinterpret_cast<const bf16x8 *>(
                        at + ar * RA + ((c ^ chunk_swizzle<RA>(ar)) << 4));
                }
                if (AM == AM_BF16) {
                    b[kk] = *reinterpret_cast<const bf16x8 *>(
                        bt + nl * RW + ((c ^ chunk_swizzle<RW>(nl)) << 4));
                } else {
                    const uint2 w8 = *reinterpret_cast<const uint2 *>(
                        bt + nl * RW + (((c >> 1) ^ chunk_swizzle<RW>(nl)) << 4) + (c & 1) * 8);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        b[kk][e] = (__bf16)(float)(int8_t)(w8.x >> (8 * e));
                        b[kk][4 + e] = (__bf16)(float)(int8_t)(w8.y >> (8 * e));
                    }
                }
            }
            v4f acc[MB];
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                acc[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kk][i], b[kk], acc[i], 0, 0,
                                                                     0);
            }
            if (AM == AM_BF16) {
                // groups past the end add zeros (+0 leaves the sum unchanged)
#pragma unroll
                for (int i = 0; i < MB; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) facc[i][r] = facc[i][r] + acc[i][r];
            } else {
                const int g = s0 + gl;
                const float sc = CHUNKED ? Sc[((g / SCH) & 1) * WR * SCH + nl * SCH + g % SCH]
                                         : Sc[d * SPAD + gl * WR + nl];
#pragma unroll
                for (int i = 0; i < MB; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        facc[i][r] = __builtin_fmaf(acc[i][r], sc, facc[i][r]);
            }
        }
    };
    auto compute = [&](int d, int s0) {
        if (AM != AM_W8A8) {
            compute_a16(d, s0);
            return;
        }
        v4i bf[S][2], af[S][2][MB];
#pragma unroll
        for (int gl = 0; gl < S; ++gl)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int j = slot * 2 + t;
                bf[gl][t] =
                    *reinterpret_cast<const v4i *>(&Bs[d][gl * BT + nl * kGroup + swz(nl, j)]);
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    const int ar = i * 16 + col;
                    af[gl][t][i] =
                        *reinterpret_cast<const v4i *>(&As[d][gl * AT + ar * kGroup + swz(ar, j)]);
                }
            }
        if (CHN) {
            // groups past the end hold zero weights and add nothing
#pragma unroll
            for (int gl = 0; gl < S; ++gl)
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    const v4i c = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[gl][0][i], bf[gl][0],
                                                                        iacc[i], 0, 0, 0);
                    iacc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[gl][1][i], bf[gl][1], c,
                                                                    0, 0, 0);
                }
            return;
        }
        float sc[S];
        if (OUT != OUT_PARTIALS) {
#pragma unroll
            for (int gl = 0; gl < S; ++gl)
                sc[gl] = CHUNKED ? Sc[(((s0 + gl) / SCH) & 1) * WR * SCH + nl * SCH + (s0 + gl) % SCH]
                                 : Sc[d * SPAD + gl * WR + nl];
        }
        v4i acc[S][MB];
#pragma unroll
        for (int gl = 0; gl < S; ++gl)
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                acc[gl][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[gl][0][i], bf[gl][0],
                                                                   v4i{0, 0, 0, 0}, 0, 0, 0);
                acc[gl][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[gl][1][i], bf[gl][1],
                                                                   acc[gl][i], 0, 0, 0);
            }
#pragma unroll
        for (int gl = 0; gl < S; ++gl) {
            const int g = s0 + gl;
            if (OUT == OUT_PARTIALS) {
                // C layout of 16x16: lane holds column `col`, rows 4*slot + r.
                if (nl < nrows && g < G) {
#pragma unroll
                    for (int i = 0; i < MB; ++i)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int m = i * 16 + slot * 4 + r;
                            if (m < rows)
                                reinterpret_cast<int32_t *>(
                                    y)[((int64_t)(r0 + m) * N + n) * G + g] = acc[gl][i][r];
                        }
                }
            } else {
#pragma unroll
                for (int i = 0; i < MB; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        facc[i][r] = __builtin_fmaf((float)acc[gl][i][r], sc[gl], facc[i][r]);
            }
        }
    };

    // Row m of the problem: token gidx[m] of the T quantised tokens when
    // gathering (grouped W8A8 only; an index outside [0, T) is a zero row with
    // scale 0), else row m itself.
    const bool gather = GROUPED && AM == AM_W8A8 && gidx != nullptr;
    auto sa_of = [&](int m) {
        if (!gather) return sa[m];
        const int t = gidx[m];
        return (t >= 0 && t < T) ? sa[t] : 0.0f;
    };

    // One pass: rows r0 .. r0+rows-1 (rows <= 16*MB) against the whole K walk.
    auto pass = [&]() {
        if (gather) {
            // the activation blocks' rows are this pass's gathered tokens
            ra = make_rsrc_words(q, (uint32_t)(T * K));
#pragma unroll
            for (int i = 0; i < ABLK; ++i) {
                constexpr int LPR = RA / 16, RPB = 1024 / RA;
                const int blk = wv * ABLK + i;
                const bool ok = blk < S * AT / 1024;
                const int rb = blk % (AT / 1024);
                const int row = rb * RPB + lane / LPR, pos = lane % LPR;
                const int t = (ok && row < rows) ? gidx[r0 + row] : -1;
                avo[i] = (t >= 0 && t < T)
                             ? (uint32_t)(t * K + ((pos ^ chunk_swizzle<RA>(row)) << 4))
                             : kOOB;
            }
        } else {
            ra = make_rsrc_words(q + (int64_t)r0 * K * (RA / kGroup),
                                 (uint32_t)(rows * K * (RA / kGroup)));
        }
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            iacc[i] = v4i{0, 0, 0, 0};
#pragma unroll
            for (int r = 0; r < 4; ++r) facc[i][r] = 0.0f;
        }
        const int nst = (G + S - 1) / S;
        if (CHUNKED) {   // scale chunk 0
            if (g4) {
                piece4(0, wv);
            } else {
#pragma unroll
                for (int j = 0; j < NP / NW; ++j) piece(0, j * NW + wv);
            }
        }
#pragma unroll
        for (int d = 0; d < D - 1; ++d) issue(d, d * S);
        for (int st0 = 0; st0 < nst; st0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {   // may run past the last stage: zeros
                // the oldest stage has landed (the D-2 younger ones may not) ...
                asm volatile("s_waitcnt vmcnt(%0)" :: "n"((D - 2) * NLD_MIN) : "memory");
                __syncthreads();            // ... for every wave; buffer d-1 is free
                issue((d + D - 1) % D, (st0 + d + D - 1) * S);
                compute(d, (st0 + d) * S);
            }
        }
        wait_vmem();                        // nothing may still write LDS past this pass
        if (CHN && nl < nrows) {
            const float swn = sw[(int64_t)n * sw_stride];
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = i * 16 + slot * 4 + r;
                    if (m < rows)
                        store_out<OUT>(y, (int64_t)(r0 + m) * N + n,
                                       channel_value(iacc[i][r], swn, sa[r0 + m]));
                }
        } else if (AM != AM_W8A8 && nl < nrows) {
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = i * 16 + slot * 4 + r;
                    if (m < rows) store_out<OUT>(y, (int64_t)(r0 + m) * N + n, facc[i][r]);
                }
        } else if (OUT != OUT_PARTIALS && nl < nrows) {
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = i * 16 + slot * 4 + r;
                    if (m < rows)
                        store_out<OUT>(y, (int64_t)(r0 + m) * N + n, facc[i][r] * sa_of(r0 + m));
                }
        }
    };

    if (!GROUPED) {
        rows = M;
        pass();
    } else {
        for (r0 = lo; r0 < hi; r0 += ROWS) {
            rows = min(ROWS, hi - r0);
            pass();
            __syncthreads();            // the next pass restages every LDS buffer
        }
    }
}

constexpr int kSmallS = 2;     // K groups per stage
constexpr int kSmallD = 4;     // LDS stage buffers (D-1 stages in flight)

// Ring depth: as many stage buffers as fit in the 160 KB of LDS beside the
// scale chunks, at most kSmallD.
template <int MB, int NW, int S = kSmallS, int AM = AM_W8A8>
constexpr int small_depth() {
    constexpr int st = smallm_stage_bytes<MB, NW, S, AM>();
    constexpr int room = 160 * 1024 - smallm_fixed_bytes<NW, AM>();
    return (kSmallD * st <= room) ? kSmallD : room / st;
}

// Groups per stage: BF16 tiles are twice as large, so one group per stage
// where two would leave fewer than three stage buffers.
template <int MB, int NW, int AM>
constexpr int small_stage() {
    return AM == AM_BF16 || (AM == AM_W8A16 && small_depth<MB, NW, kSmallS, AM>() < 3) ? 1
                                                                                     : kSmallS;
}

template <int MB, int NW, int OUT, bool GROUPED, int AM = AM_W8A8>
hipError_t launch_smallm_mb(const int8_t *q, const float *sa, const int8_t *qw, const float *sw,
                            int M, int N, int K, void *y, const int32_t *offsets, int E,
                            hipStream_t stream, int sw_stride, const int32_t *gidx, int T) {
    constexpr int S = small_stage<MB, NW, AM>();
    constexpr int D = small_depth<MB, NW, S, AM>();
    const dim3 grid((unsigned)((N + 16 * NW - 1) / (16 * NW)), GROUPED ? (unsigned)E : 1u);
    // the non-temporal hint pays on weight streams far larger than the caches
    // (measured: faster at 235 MB, slower at 29 MB)
    constexpr int64_t kNtMin = (int64_t)1 << 27;
    const bool nt = (int64_t)N * K * (GROUPED ? E : 1) * (AM == AM_BF16 ? 2 : 1) >= kNtMin;
    if (nt)
        gemm_smallm_kernel<MB, NW, OUT, S, D, GROUPED, true, AM>
            <<<grid, 64 * NW, 0, stream>>>(q, sa, qw, sw, M, N, K, y, offsets, sw_stride, gidx,
                                           T);
    else
        gemm_smallm_kernel<MB, NW, OUT, S, D, GROUPED, false, AM>
            <<<grid, 64 * NW, 0, stream>>>(q, sa, qw, sw, M, N, K, y, offsets, sw_stride, gidx,
                                           T);
    return hipGetLastError();
}

// Workgroup width NW waves (16 weight rows each): spread the 16-row column
// blocks over whole rounds of one workgroup per CU, as wide as possible (the
// wider the workgroup, the fewer times the activation tile is re-read), at
// most 8 waves, and at least what the activation tile needs (register ring).
constexpr int kCUs = 256;

template <int MB, int OUT, bool GROUPED, int AM = AM_W8A8>
hipError_t launch_smallm_nw(const int8_t *q, const float *sa, const int8_t *qw, const float *sw,
                            int M, int N, int K, void *y, const int32_t *offsets, int E,
                            hipStream_t stream, int sw_stride = 1, const int32_t *gidx = nullptr,
                            int T = 0) {
    const int64_t blocks16 = (int64_t)((N + 15) / 16) * (GROUPED ? E : 1);
    const int64_t rounds = (blocks16 + 8 * kCUs - 1) / (8 * kCUs);
    int nw = (int)((blocks16 + kCUs * rounds - 1) / (kCUs * rounds));
    // at least what the activation ring needs per thread: 4 waves for 64 rows,
    // 2 for up to 32 rows (one-wave workgroups, tried for small N so that more
    // CUs stream weights, were slower: one wave keeps too few bytes in flight)
    const int min_nw = MB >= 4 ? 4 : 2;
    nw = nw < min_nw ? min_nw : nw;
    // 64 rows across 8 waves would leave room for only two stage buffers
    if (MB >= 4 && nw > 7) nw = 7;
#define BSB_SMALLM_CASE(W)                                                                       \
    case W:                                                                                      \
        return launch_smallm_mb<MB, W, OUT, GROUPED, AM>(q, sa, qw, sw, M, N, K, y, offsets, E,   \
                                                         stream, sw_stride, gidx, T);
    switch (nw) {
        BSB_SMALLM_CASE(2)
        BSB_SMALLM_CASE(3)
        BSB_SMALLM_CASE(4)
        BSB_SMALLM_CASE(5)
        BSB_SMALLM_CASE(6)
        BSB_SMALLM_CASE(7)
        default: return launch_smallm_mb<MB, 8, OUT, GROUPED, AM>(q, sa, qw, sw, M, N, K, y,
                                                                   offsets, E, stream, sw_stride,
                                                                   gidx, T);
    }
#undef BSB_SMALLM_CASE
}

template <int OUT>
hipError_t launch_smallm(const int8_t *q, const float *sa, const int8_t *qw, const float *sw,
                         int M, int N, int K, void *y, hipStream_t stream, int sw_stride) {
    if (M <= 16)
        return launch_smallm_nw<1, OUT, false>(q, sa, qw, sw, M, N, K, y, nullptr, 1, stream,
                                               sw_stride);
    if (M <= 32)
        return launch_smallm_nw<2, OUT, false>(q, sa, qw, sw, M, N, K, y, nullptr, 1, stream,
                                               sw_stride);
    return launch_smallm_nw<4, OUT, false>(q, sa, qw, sw, M, N, K, y, nullptr, 1, stream,
                                           sw_stride);
}

constexpr int kBigMinM = 512;   // rows from which the 256x256 kernel is used
// The 256x256 kernel once the 128x128 kernel's four times as many tiles would
// take more than two rounds of the CUs: more than 128 of its own tiles. Both
// give the same bits; measured at N = 4096, K = 7168 (and 8192 x 8192):
// 128 tiles 122 against 98 us for the 128x128 kernel, 160 tiles 130 against
// 145, 192 tiles 136 against 154, 224 tiles 154 against 189.
constexpr int64_t kBigMinTiles = kCUs / 2 + 1;

template <int OUT>
hipError_t launch_dense(const int8_t *q, const float *sa, const int8_t *qw, const float *sw,
                        int M, int N, int K, void *y, hipStream_t stream, int sw_stride = 1) {
    // smallm addresses a weight slice (at most 128 rows) and the whole
    // activation matrix (at most 64 rows) with 32-bit buffer offsets
    if (M <= 64 && (int64_t)128 * K < ((int64_t)1 << 31))
        return launch_smallm<OUT>(q, sa, qw, sw, M, N, K, y, stream, sw_stride);
    // The 256x256 kernel (which addresses its operand panels with 32-bit
    // buffer offsets) from kBigMinTiles of its tiles; below that the 128x128
    // kernel's four times as many tiles finish sooner.
    const int64_t big_tiles = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
    if (M >= kBigMinM && big_gemm_fits(K) && big_tiles >= kBigMinTiles)
        return launch_gemm_big(q, sa, qw, sw, M, N, K, y, OUT, nullptr, 0, sw_stride, stream);
    if (!mid_gemm_fits(K)) return hipErrorInvalidValue;   // excluded by the C ABI's checks
    return launch_gemm_mid(q, sa, qw, sw, M, N, K, y, OUT, nullptr, 0, sw_stride, stream);
}

}  // namespace

hipError_t launch_gemm(const int8_t *q, const float *sa, const int8_t *qw, const float *sw,
                       int64_t M, int64_t N, int64_t K, void *y, int out, hipStream_t stream) {
    switch (out) {
        case OUT_BF16: return launch_dense<OUT_BF16>(q, sa, qw, sw, (int)M, (int)N, (int)K, y, stream);
        case OUT_FP32: return launch_dense<OUT_FP32>(q, sa, qw, sw, (int)M, (int)N, (int)K, y, stream);
        default: return launch_dense<OUT_PARTIALS>(q, nullptr, qw, nullptr, (int)M, (int)N, (int)K, y, stream);
    }
}

namespace {

// BF16 activations (M <= 64): W8A16 (am 1: qw INT8 + sw) or BF16 weights (am 2).
template <int OUT, int AM>
hipError_t launch_a16_rows(const uint16_t *x, const void *w, const float *sw, int M, int N, int K,
                           void *y, hipStream_t stream) {
    const int8_t *xq = reinterpret_cast<const int8_t *>(x);
    const int8_t *wq = reinterpret_cast<const int8_t *>(w);
    if (M <= 16)
        return launch_smallm_nw<1, OUT, false, AM>(xq, nullptr, wq, sw, M, N, K, y, nullptr, 1,
                                                   stream);
    if (M <= 32)
        return launch_smallm_nw<2, OUT, false, AM>(xq, nullptr, wq, sw, M, N, K, y, nullptr, 1,
                                                   stream);
    return launch_smallm_nw<4, OUT, false, AM>(xq, nullptr, wq, sw, M, N, K, y, nullptr, 1,
                                               stream);
}

}  // namespace

hipError_t launch_gemm_a16(const uint16_t *x, const void *w, const float *sw, int64_t M,
                           int64_t N, int64_t K, void *y, int out, int am, hipStream_t stream) {
    // beyond the decode-shaped range: 128x128 tiles (gemm_a16.hip)
    if (M > 64) {
        if (!a16_tiles_fit(K)) return hipErrorInvalidValue;   // excluded by the C ABI's checks
        return launch_gemm_a16_tiles(x, w, sw, (int)M, (int)N, (int)K, y, out, am, stream);
    }
    if (am == 1) {
        if (out == OUT_BF16)
            return launch_a16_rows<OUT_BF16, AM_W8A16>(x, w, sw, (int)M, (int)N, (int)K, y, stream);
        return launch_a16_rows<OUT_FP32, AM_W8A16>(x, w, sw, (int)M, (int)N, (int)K, y, stream);
    }
    if (out == OUT_BF16)
        return launch_a16_rows<OUT_BF16, AM_BF16>(x, w, nullptr, (int)M, (int)N, (int)K, y, stream);
    return launch_a16_rows<OUT_FP32, AM_BF16>(x, w, nullptr, (int)M, (int)N, (int)K, y, stream);
}

hipError_t launch_gemm_channel(const int8_t *q, const float *sa, const int8_t *qw,
                               const float *sw, int64_t sw_stride, int64_t M, int64_t N,
                               int64_t K, void *y, int out, hipStream_t stream) {
    if (out == OUT_BF16)
        return launch_dense<OUT_BF16_CH>(q, sa, qw, sw, (int)M, (int)N, (int)K, y, stream,
                                         (int)sw_stride);
    return launch_dense<OUT_FP32_CH>(q, sa, qw, sw, (int)M, (int)N, (int)K, y, stream,
                                     (int)sw_stride);
}

hipError_t launch_grouped_gemm(const int8_t *q, const float *sa, const int8_t *qw,
                               const float *sw, const int32_t *offsets, int64_t E, int64_t R,
                               int64_t N, int64_t K, void *y, int out, hipStream_t stream,
                               const int32_t *gidx, int64_t T) {
    // gidx: every kernel below loads its activation rows through the index
    // (same arithmetic, so the same bits as gathering the rows first)
    // Rows per expert are known only on the device; the mean decides. With
    // at least 128 rows per expert on average, and at least kBigMinTiles tiles
    // (counted without the experts' partial tiles, a lower bound), the 256x256
    // kernel is used (the busiest GPU's share of the MoE layer under 8-way
    // expert parallelism, 240 tiles: 93 against 136 us).
    const int64_t big_tiles = ((R + 255) / 256) * ((N + 255) / 256);
    if (R >= 128 * E && big_tiles >= kBigMinTiles && big_gemm_fits(K))
        return launch_gemm_big(q, sa, qw, sw, (int)R, (int)N, (int)K, y, out, offsets, (int)E, 1,
                               stream, gidx, (int)T);
    // At most 32 rows per expert on average (decode-shaped MoE): stream each
    // expert's weights once per 32 of its rows.
    if (R <= 32 * E && E <= 65535 && (int64_t)128 * K < ((int64_t)1 << 31)) {
        if (out == OUT_BF16)
            return launch_smallm_nw<2, OUT_BF16, true>(q, sa, qw, sw, (int)R, (int)N, (int)K, y,
                                                       offsets, (int)E, stream, 1, gidx, (int)T);
        return launch_smallm_nw<2, OUT_FP32, true>(q, sa, qw, sw, (int)R, (int)N, (int)K, y,
                                                   offsets, (int)E, stream, 1, gidx, (int)T);
    }
    if (!mid_gemm_fits(K)) return hipErrorInvalidValue;   // excluded by the C ABI's checks
    return launch_gemm_mid(q, sa, qw, sw, (int)R, (int)N, (int)K, y, out, offsets, (int)E, 1,
                           stream, gidx, (int)T);
}

}  // namespace bsb
