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

// Output tiles of a launch: mt tile rows x nt tile columns.
struct TileGrid {
    int mt, nt;
};

// Workgroup -> tile. The dispatcher deals workgroups to the 8 XCDs round
// robin; the remap gives each XCD a contiguous run of tiles, walked in groups
// of 4 tile rows, column after column, so that the tiles an XCD runs at once
// share their A panels (each read for all tile columns while it is in that
// XCD's L2) and their B panels (four tile rows at a time; in the grouped form
// the rows of one expert, which share its weight panel).
__device__ __forceinline__ void xcd_tile_of(int b, TileGrid t, int &bm, int &bn) {
    const int num = t.mt * t.nt;
    const int x = b & 7, per = num >> 3, rem = num & 7;
    const int start = x * per + (x < rem ? x : rem);
    const int tid = start + (b >> 3);                       // bijection onto [0, num)
    constexpr int GM = 4;
    const int grp = tid / (GM * t.nt);
    const int first = grp * GM;
    const int gsz = min(t.mt - first, GM);
    const int in = tid - grp * GM * t.nt;
    bm = first + in % gsz;
    bn = in / gsz;
}

// The tile of this workgroup in a grouped launch of 512-thread workgroups:
// rows [offsets[e], offsets[e+1]) of R sorted rows belong to expert e, tile
// rows of TM rows are laid out expert after expert (a tile never spans two
// experts), and the host sized the grid for the most tile rows any split of R
// rows can need (tiles.mt). The tiles that exist are known only here. Each
// thread takes one expert of a chunk of 512 (one coalesced load of its bounds
// per chunk); a block-wide sum gives the tile rows that exist, and the first
// mt*nt workgroups take them (the dispatcher deals workgroups round-robin to
// the XCDs, so the idle surplus spreads evenly). A block-wide exclusive scan
// then finds the expert holding this workgroup's tile row. (Offsets that
// overlap, which the contract excludes, could count more than the host bound;
// the count is capped at it, so every tile stays inside [0, R).) Returns false,
// for the whole workgroup, when it has no tile.
template <int TM>
__device__ __forceinline__ bool grouped_tile(const int32_t *offsets, int E, int R, TileGrid tiles,
                                             int &e_out, int &m0, int &row_end, int &bm,
                                             int &bn) {
    __shared__ int s_red[8];
    __shared__ int s_hit[4];   // expert, block within it, its first row, its row end
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    auto seg = [&](int e, int &lo, int &hi) {   // expert e's rows, clamped to [0, R]
        lo = offsets[e];
        hi = offsets[e + 1];
        lo = lo < 0 ? 0 : (lo > R ? R : lo);
        hi = hi < lo ? lo : (hi > R ? R : hi);
    };
    // tile rows of expert e (0 past E), with its clamped rows
    auto tiles_of = [&](int e, int &lo, int &hi) {
        lo = hi = 0;
        if (e >= E) return 0;
        seg(e, lo, hi);
        return (hi - lo + TM - 1) / TM;
    };
    // inclusive scan of v over the 512 threads; also returns the block total
    auto block_scan = [&](int v, int &total) {
        int x = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o, kWave);
            if (lane >= o) x += y;
        }
        if (lane == 63) s_red[wave] = x;
        __syncthreads();
        int before = 0;
        total = 0;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const int t = s_red[w];
            before += w < wave ? t : 0;
            total += t;
        }
        __syncthreads();
        return x + before;
    };
    if (tid == 0) s_hit[0] = -1;   // published by the scans' barriers
    if (E <= 512) {
        // one expert per thread: one scan gives both the tile rows that exist and
        // each expert's first tile row
        int lo, hi;
        const int c = tiles_of(tid, lo, hi);
        int tot;
        const int incl = block_scan(c, tot);
        const int mt = tot < tiles.mt ? tot : tiles.mt;
        if ((int64_t)blockIdx.x >= (int64_t)mt * tiles.nt) return false;
        tiles.mt = mt;
        xcd_tile_of(blockIdx.x, tiles, bm, bn);
        if (c > 0 && incl - c <= bm && bm < incl) {
            s_hit[0] = tid;
            s_hit[1] = bm - (incl - c);
            s_hit[2] = lo;
            s_hit[3] = hi;
        }
        __syncthreads();
    } else {
    int64_t mt = 0;
    for (int base = 0; base < E; base += 512) {
        int tot, lo, hi;
        block_scan(tiles_of(base + tid, lo, hi), tot);
        mt += tot;
    }
    mt = mt < tiles.mt ? mt : tiles.mt;
    if ((int64_t)blockIdx.x >= mt * tiles.nt) return false;
    tiles.mt = (int)mt;
    xcd_tile_of(blockIdx.x, tiles, bm, bn);
    // tile row bm -> (expert, TM-row block)
    int run = 0;
    for (int base = 0; base < E; base += 512) {
        int lo, hi;
        const int e = base + tid, c = tiles_of(e, lo, hi);
        int tot;
        const int incl = block_scan(c, tot) + run;
        if (c > 0 && incl - c <= bm && bm < incl) {
            s_hit[0] = e;
            s_hit[1] = bm - (incl - c);
            s_hit[2] = lo;
            s_hit[3] = hi;
        }
        run += tot;
        __syncthreads();
        if (s_hit[0] >= 0 || run > bm) break;   // uniform: every thread reads the same
    }
    }
    const int e = s_hit[0];
    if (e < 0) return false;   // unreachable: bm < mt
    // the expert's rows come from the thread that found it (no second load of
    // the offsets after the scan)
    e_out = e;
    m0 = s_hit[2] + s_hit[1] * TM;
    row_end = s_hit[3];
    return true;
}

}  // namespace bsb
