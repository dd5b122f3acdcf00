// INT8 KV cache on gfx950: quantisation on write, and decode attention with
// the dequantisation fused into the attention kernel.
//
// [P3] sec. 3.4: one dynamic scale per key vector and per value vector, taken
// when the vector is written; attention multiplies the INT8 keys and values by
// their scales while reading them, inside the attention kernel (sec. 4.1: a
// blockwise attention that dequantises the INT8 cache itself), so the cache is
// read once and never expanded in memory.
//
// Cache layout (head dimension 128; T = token slots per sequence, a multiple of 64):
//   k_cache [T/64, B, Hkv, 8192] INT8: the 64-token chunk c of (sequence b, KV
//           head h) is row (c, b, h), chunks of every (b, h) interleaved; a
//           chunk is four 16-token blocks of 2 KB; token tau of a block,
//           dimension d at byte ((d/16)%2)*1024 + ((d/32)*16 + tau)*16 + d%16
//   v_cache [T/64, B, Hkv, 8192] INT8: a chunk is two 32-token blocks of 4 KB;
//           token tau of a block, dimension d at byte (d/32)*1024 +
//           (((tau%16)/4)*16 + d%16)*16 + ((d/16)%2)*8 + (tau/16)*4 + tau%4
//   k_scale, v_scale [B, Hkv, T] float32
// Both block orders are the matrix cores' operand orders (lane l of a wave
// reads bytes 16l .. 16l+15 of each 1 KB quarter or half of a block), so every
// load instruction reads 1 KB contiguous and nothing is transposed. (A V
// order in which each lane's 64 bytes were contiguous made every load
// instruction touch 4 KB at a 64-byte stride; measured 1-2 % slower.)
// Chunk-major order puts the chunks that the workgroups of one launch read at
// the same time (the same chunk of every (sequence, KV head)) next to each
// other in memory: at 32 sequences x 8 KV heads x 4096 tokens the attention
// ran 53-54 us with each (sequence, head) contiguous and 50-52 us chunk-major
// (with the non-temporal hint below, 48-50 us).
//
// Decode attention (one query token per sequence, grouped-query heads, up to
// 16 query heads per KV head): a workgroup of 8 waves takes a split of the
// cached tokens of one (sequence, KV head), each wave chunks of 64 tokens.
// Per chunk:
//   scores  S^T[token, head] = K . Q^T   on v_mfma_f32_16x16x32_bf16, the INT8
//           codes converted to BF16 in registers (exact), the query in BF16;
//   x = S * k_scale * log2(e)/sqrt(128) (float32), masked past the sequence;
//   p = exp2(x - m) against the running maximum m per head (float32);
//   o^T[d, head] += V^T . (p * v_scale)^T on the same MFMA, the weights times
//           the value scales rounded to BF16, the value codes converted exactly.
// The 8 wave results are merged in LDS (max, rescaled sums). With one split
// per sequence the kernel then divides by the total weight and writes the
// output; otherwise it writes one partial (m, l, o[128]) per head and split and
// a second kernel merges the splits.
//
// The same kernel also runs over a BF16 cache (the cache the INT8 one
// replaces, kept as the comparison route): 2-byte elements in blocks of the
// same operand order, no conversion and no scales.
//
// Several query tokens per sequence (chunked prefill, verifying drafted
// tokens; [P3] sec. 4.1's blockwise attention): the matrix instructions'
// 16 query columns hold (query token, head) pairs, Qn tokens x G heads <= 16,
// so the cache is still read once per (sequence, KV head) for all of them.
// Query i of Qn is the sequence's token at position L - Qn + i and attends to
// tokens 0 .. L - Qn + i: each column carries its own length in the masks.
#include "device_common.h"
#include <atomic>

#include "launch.h"

namespace bsb {

namespace {

constexpr int kHD = 128;                       // head dimension
constexpr int kVBlk = 32;                      // tokens per V block
constexpr int kChunk = 64;                     // tokens per cache chunk (row of the layout)
constexpr int kAttnWaves = 8;                  // waves per attention workgroup
constexpr int kWaveTok = 64;                   // tokens per wave
constexpr int kSplitTok = kAttnWaves * kWaveTok;   // tokens per split per chunk step
constexpr int64_t kMinWorkgroups = 256;   // grid size the chunk count aims for (one per CU)
constexpr int kMaxChunks = 8;              // chunks per wave at most
constexpr int kPart = kHD + 2;                 // floats per (head, split) partial: o, m, l
constexpr int kORow = kHD + 4;                 // LDS row stride of the wave partials
constexpr float kNegInf = -__builtin_huge_valf();
// log2(e) / sqrt(128), rounded to float32
constexpr float kScoreScale = (float)(1.4426950408889634 / 11.313708498984761);

typedef float v4f_t __attribute__((ext_vector_type(4)));

// byte of (token tau in a 16-token block, dim d) in a 2 KB K block: one wave
// instruction j reads bytes 1024j .. 1024j+1023, lane 16g + tau getting dims
// 32g + 16j .. 32g + 16j + 15 of token tau
__device__ __forceinline__ int kblk_off(int tau, int d) {
    return ((d >> 4) & 1) * 1024 + ((d >> 5) * 16 + tau) * 16 + (d & 15);
}

// byte of (token tau in a 32-token block, dim d) in a 4 KB V block: lane
// 16((tau%16)/4) + d%16 holds, in quarter d/32 of the block, the 16 bytes of
// dims d and d+16 (of that 32-dim slab) for its tokens 4 (tau/16) + tau%4
__device__ __forceinline__ int vblk_off(int tau, int d) {
    return (d >> 5) * 1024 + ((((tau & 15) >> 2) * 16 + (d & 15)) * 16) + ((d >> 4) & 1) * 8 +
           (tau >> 4) * 4 + (tau & 3);
}

// The BF16 cache of the comparison route keeps the same blocks with 2-byte
// elements: a 4 KB K block of 16 tokens (instruction s of a tile reads bytes
// 1024s .. 1024s+1023, lane 16g + tau getting dims 32g + 8s .. 32g + 8s + 7)
// and an 8 KB V block of 32 tokens (instruction i reads the d-tile 16i ..
// 16i+15, lane 16g + r getting dim 16i + r of the 8 tokens of slot group g).
__device__ __forceinline__ int kblk16_off(int tau, int d) {
    return ((d >> 3) & 3) * 1024 + ((d >> 5) * 16 + tau) * 16 + (d & 7) * 2;
}

__device__ __forceinline__ int vblk16_off(int tau, int d) {
    return (d >> 4) * 1024 + (((tau & 15) >> 2) * 16 + (d & 15)) * 16 + ((tau >> 4) * 4 + (tau & 3)) * 2;
}

// Byte offset of the chunk holding token t of (sequence, KV head) bh in a cache
// of BH = B * Hkv rows per chunk index, chunk_bytes per chunk.
__device__ __forceinline__ int64_t chunk_at(int64_t bh, int64_t BH, int t, int chunk_bytes) {
    return ((int64_t)(t / kChunk) * BH + bh) * chunk_bytes;
}

// eight INT8 codes (little-endian in two dwords) -> eight BF16 values (exact)
__device__ __forceinline__ bf16x8 i8x8_to_bf16(uint32_t lo, uint32_t hi) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = (__bf16)(float)(int8_t)(lo >> (8 * e));
        r[4 + e] = (__bf16)(float)(int8_t)(hi >> (8 * e));
    }
    return r;
}

// One wave per (token, KV head, K or V) vector of 128 BF16 values: two per lane.
__global__ void __launch_bounds__(256)
kv_write_kernel(const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
                const int32_t *__restrict__ seq, const int32_t *__restrict__ pos, int64_t n,
                int B, int Hkv, int T, int8_t *__restrict__ kc, float *__restrict__ ks,
                int8_t *__restrict__ vc, float *__restrict__ vs) {
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (item >= n * Hkv * 2) return;                     // whole wave
    const int which = (int)(item & 1);
    const int64_t th = item >> 1;                        // token * Hkv + head
    const int64_t tok = th / Hkv;
    const int h = (int)(th - tok * Hkv);
    const int b = seq[tok], t = pos[tok];
    if (b < 0 || b >= B || t < 0 || t >= T) return;     // whole wave: nothing written
    const uint32_t w = reinterpret_cast<const uint32_t *>((which ? v : k) + th * kHD)[lane];
    uint32_t amax = w & 0x7FFFu;
    amax = amax > ((w >> 16) & 0x7FFFu) ? amax : ((w >> 16) & 0x7FFFu);
    amax = group_max_u32(amax, kWave);
    const float s = absmax_scale(bf16_to_f32(amax));
    int c0 = 0, c1 = 0;
    if (amax != 0) {
        c0 = quant_elem(bf16_to_f32(w & 0xFFFFu), s);
        c1 = quant_elem(bf16_to_f32(w >> 16), s);
    }
    const int64_t bh = (int64_t)b * Hkv + h, vec = bh * T + t;
    const int64_t chunk = chunk_at(bh, (int64_t)B * Hkv, t, kChunk * kHD);
    if (which == 0) {
        const uint16_t pair = (uint16_t)((uint32_t)(c0 & 0xFF) | ((uint32_t)(c1 & 0xFF) << 8));
        int8_t *blk = kc + chunk + ((t % kChunk) / 16) * (16 * kHD);
        *reinterpret_cast<uint16_t *>(blk + kblk_off(t & 15, 2 * lane)) = pair;
        if (lane == 0) ks[vec] = s;
    } else {
        int8_t *blk = vc + chunk + ((t % kChunk) / kVBlk) * (kVBlk * kHD);
        const int tau = t % kVBlk;
        blk[vblk_off(tau, 2 * lane)] = (int8_t)c0;
        blk[vblk_off(tau, 2 * lane + 1)] = (int8_t)c1;
        if (lane == 0) vs[vec] = s;
    }
}

// BF16 keys and values copied into the BF16 block layouts (no quantisation):
// one wave per (token, KV head, K or V) vector, two values per lane.
__global__ void __launch_bounds__(256)
kv_write_bf16_kernel(const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
                     const int32_t *__restrict__ seq, const int32_t *__restrict__ pos, int64_t n,
                     int B, int Hkv, int T, uint16_t *__restrict__ kc, uint16_t *__restrict__ vc) {
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (item >= n * Hkv * 2) return;                     // whole wave
    const int which = (int)(item & 1);
    const int64_t th = item >> 1;
    const int64_t tok = th / Hkv;
    const int h = (int)(th - tok * Hkv);
    const int b = seq[tok], t = pos[tok];
    if (b < 0 || b >= B || t < 0 || t >= T) return;     // whole wave: nothing written
    const uint32_t w = reinterpret_cast<const uint32_t *>((which ? v : k) + th * kHD)[lane];
    const int64_t bh = (int64_t)b * Hkv + h;
    const int64_t chunk = chunk_at(bh, (int64_t)B * Hkv, t, kChunk * 2 * kHD);
    if (which == 0) {
        uint8_t *blk = reinterpret_cast<uint8_t *>(kc) + chunk + ((t % kChunk) / 16) * (16 * 2 * kHD);
        *reinterpret_cast<uint32_t *>(blk + kblk16_off(t & 15, 2 * lane)) = w;   // d, d+1 adjacent
    } else {
        uint8_t *blk = reinterpret_cast<uint8_t *>(vc) + chunk + ((t % kChunk) / kVBlk) * (kVBlk * 2 * kHD);
        *reinterpret_cast<uint16_t *>(blk + vblk16_off(t & 31, 2 * lane)) = (uint16_t)(w & 0xFFFFu);
        *reinterpret_cast<uint16_t *>(blk + vblk16_off(t & 31, 2 * lane + 1)) = (uint16_t)(w >> 16);
    }
}

// The cached tokens of one (sequence, KV head) this wave owns: chunks of 64.
// INT8: 8 KB of key codes, 8 KB of value codes and the 64 tokens' scales;
// BF16: 16 KB of keys and 16 KB of values.
enum { kKvInt8 = 0, kKvBf16 = 1 };

template <int KVT> struct KvChunk;
template <> struct KvChunk<kKvInt8> {
    v4i kd[4][2];   // keys: 16-token tile c, half j
    v4i vd[2][4];   // values: 32-token block s, quarter j
    float skl, svl; // scales of token t0 + lane
};
template <> struct KvChunk<kKvBf16> {
    v4i kd[4][4];   // keys: 16-token tile c, k-step s
    v4i vd[2][8];   // values: 32-token block s, d-tile i
};

// grid (splits, B * Hkv); 512 threads; a split is 8 * 64 * R tokens. Wave w
// takes chunks r * 8 + w (r < R) of its split, so at each step the 8 waves
// read adjacent regions of the keys and of the values; a wave issues the loads
// of one chunk (BF16) or of two chunks (INT8) together and keeps a running
// maximum, weight sum and output across its chunks (online softmax).
// part: [B*Hkv, splits, G, kPart] float32.
// OUT: kPartials writes the split's (o, m, l) for the merge kernel; with a
// single split the kernel writes the normalised output itself (kDirectBf16,
// kDirectF32) and no merge runs.
enum { kPartials = 0, kDirectBf16 = 1, kDirectF32 = 2 };

template <int KVT, int R, int OUT>
__global__ void __launch_bounds__(512)
attn_split_kernel(const uint16_t *__restrict__ q, const void *__restrict__ kc,
                  const float *__restrict__ ks, const void *__restrict__ vc,
                  const float *__restrict__ vs, const int32_t *__restrict__ lens, int Hq, int Hkv,
                  int T, int max_len, int Qn, float *__restrict__ part, void *__restrict__ out) {
    constexpr bool I8 = KVT == kKvInt8;
    constexpr int EB = I8 ? 1 : 2;                     // bytes per cached element
    __shared__ __align__(16) float s_o[kAttnWaves][16][kORow];
    __shared__ float s_m[kAttnWaves][16], s_l[kAttnWaves][16];

    const int split = blockIdx.x, nsplit = gridDim.x;
    const int bh = blockIdx.y;
    const int b = bh / Hkv, hk = bh - b * Hkv;
    const int G = Hq / Hkv, NC = Qn * G;   // query columns: (token qi, head hh) = (c / G, c % G)
    // wave index as a uniform value, so the offsets derived from it stay scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int col = lane & 15, grp = lane >> 4;
    int L = lens[b];
    const int lim = max_len < T ? max_len : T;
    L = L < 0 ? 0 : (L > lim ? lim : L);
    // this lane's column: its query token and head, and the tokens it attends
    const int qi = col / G, hh = col - qi * G;
    int Lc = L - Qn + qi + 1;
    Lc = Lc < 0 ? 0 : (Lc > L ? L : Lc);
    const int base = split * kSplitTok * R + wave * kWaveTok;
    auto t0_of = [&](int r) { return base + r * kSplitTok; };

    // one chunk of keys and one of values per load step, each through a buffer
    // descriptor over that chunk (range-checked; offset kOOB reads zeros); the
    // lane's part of an offset is in a VGPR, the rest scalar. Chunks are read
    // once and carry the non-temporal hint (at 32 sequences x 4096 tokens: INT8
    // 2-3 us faster, BF16 92.6 -> 82.7 us; with the (sequence, head)-contiguous
    // layout the hint had cost the INT8 cache 12-15 us).
    constexpr int kCB = kChunk * kHD * EB;   // bytes per chunk
    constexpr int kAux = kNonTemporal;
    const int64_t BH = (int64_t)gridDim.y;
    const uint32_t kvo = (uint32_t)lane * 16;
    const uint32_t vvo = (uint32_t)lane * 16;

    auto load = [&](KvChunk<KVT> &ch, int r) {
        const int t0 = t0_of(r);
        const bool ok = r < R && t0 < L;
        const uint32_t so = ok ? 0u : kOOB;
        const int64_t cb = chunk_at(bh, BH, ok ? t0 : 0, kCB);
        const __amdgpu_buffer_rsrc_t rk =
            make_rsrc(reinterpret_cast<const uint8_t *>(kc) + cb, (uint32_t)kCB);
        const __amdgpu_buffer_rsrc_t rv =
            make_rsrc(reinterpret_cast<const uint8_t *>(vc) + cb, (uint32_t)kCB);
        if constexpr (I8) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    ch.kd[c][j] = buf_load16s<kAux>(rk, kvo, ok ? so + c * 2048 + j * 1024 : kOOB);
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    ch.vd[s][j] =
                        buf_load16s<kAux>(rv, vvo, ok ? so + s * (kVBlk * kHD) + 1024 * j : kOOB);
            const __amdgpu_buffer_rsrc_t rks = make_rsrc(ks + (int64_t)bh * T, (uint32_t)T * 4);
            const __amdgpu_buffer_rsrc_t rvs = make_rsrc(vs + (int64_t)bh * T, (uint32_t)T * 4);
            const uint32_t ss = ok ? (uint32_t)t0 * 4 : kOOB;
            ch.skl = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(rks, (int)(lane * 4), (int)ss, 0));
            ch.svl = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(rvs, (int)(lane * 4), (int)ss, 0));
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    ch.kd[c][s] = buf_load16s<kAux>(rk, kvo, ok ? so + c * 4096 + s * 1024 : kOOB);
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    ch.vd[s][i] = buf_load16s<kAux>(rv, vvo, ok ? so + s * 8192 + i * 1024 : kOOB);
        }
        // keep the whole chunk's loads here, ahead of the computation that follows
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    // queries: token qi, head hk*G + hh (zero rows for col >= NC), dims 32grp .. 32grp+31
    uint4 qd[4];
    {
        const bool hv = col < NC;
        const uint16_t *qr =
            q + (((int64_t)b * Qn + (hv ? qi : 0)) * Hq + hk * G + (hv ? hh : 0)) * kHD + 32 * grp;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            qd[j] = hv ? *reinterpret_cast<const uint4 *>(qr + 8 * j) : make_uint4(0u, 0u, 0u, 0u);
    }

    // running maximum (log2 units), this lane's partial weight sum, unnormalised o^T
    float m = kNegInf, lpart = 0.0f;
    v4f_t o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](const KvChunk<KVT> &ch, int t0) {
        // scores: tile c holds tokens t0 + 16c + 4grp + r (rows) for head col
        float x[4][4];
        float mc = kNegInf;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            v4f_t acc = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf16x8 a;
                if constexpr (I8) {
                    const v4i &kk = ch.kd[c][s >> 1];
                    a = i8x8_to_bf16((uint32_t)kk[2 * (s & 1)], (uint32_t)kk[2 * (s & 1) + 1]);
                } else {
                    a = __builtin_bit_cast(bf16x8, ch.kd[c][s]);
                }
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, qd[s]),
                                                              acc, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tt = 16 * c + 4 * grp + r;
                float sv;
                if constexpr (I8) sv = (acc[r] * __shfl(ch.skl, tt, kWave)) * kScoreScale;
                else sv = acc[r] * kScoreScale;
                x[c][r] = (t0 + tt < Lc) ? sv : kNegInf;
                mc = __builtin_fmaxf(mc, x[c][r]);
            }
        }
        mc = __builtin_fmaxf(mc, __shfl_xor(mc, 16, kWave));
        mc = __builtin_fmaxf(mc, __shfl_xor(mc, 32, kWave));
        const float mn = __builtin_fmaxf(m, mc);
        // a column none of whose tokens so far is attended (a chunk's earlier
        // queries) keeps m = -inf: exponents against 0 then give 0, not NaN
        const float ms = mn == kNegInf ? 0.0f : mn;
        const float alpha = __builtin_amdgcn_exp2f(m - ms);   // 0 on the first chunk
        m = mn;
        lpart *= alpha;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] *= alpha;
        float p[4][4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[c][r] = __builtin_amdgcn_exp2f(x[c][r] - ms);
                lpart += p[c][r];
            }
        // P.V over two 32-token blocks; slot j < 4 is token 32s + 4grp + j,
        // slot 4 + j is token 32s + 16 + 4grp + j (the V block order above)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int ta = 32 * s + 4 * grp, tbk = ta + 16;
            bf16x8 pw;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float pa = p[2 * s][j], pb2 = p[2 * s + 1][j];
                if constexpr (I8) {
                    pa *= __shfl(ch.svl, ta + j, kWave);
                    pb2 *= __shfl(ch.svl, tbk + j, kWave);
                }
                pw[j] = (__bf16)(t0 + ta + j < Lc ? pa : 0.0f);
                pw[4 + j] = (__bf16)(t0 + tbk + j < Lc ? pb2 : 0.0f);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                bf16x8 a;
                if constexpr (I8) {
                    const v4i &vv = ch.vd[s][i >> 1];
                    a = i8x8_to_bf16((uint32_t)vv[2 * (i & 1)], (uint32_t)vv[2 * (i & 1) + 1]);
                } else {
                    a = __builtin_bit_cast(bf16x8, ch.vd[s][i]);
                }
                o[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pw, o[i], 0, 0, 0);
            }
        }
    };

    if (t0_of(0) < L) {   // whole wave
        if constexpr (I8 && R >= 2) {
            // two chunks' loads in flight together (33 KB per wave, as one BF16
            // chunk), then both computed
            KvChunk<KVT> A, B;
#pragma unroll
            for (int r = 0; r < R; r += 2) {
                if (t0_of(r) >= L) break;
                load(A, r);
                load(B, r + 1);
                compute(A, t0_of(r));
                if (t0_of(r + 1) < L) compute(B, t0_of(r + 1));
            }
        } else {
            KvChunk<KVT> A;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if (t0_of(r) >= L) break;
                load(A, r);
                compute(A, t0_of(r));
            }
        }
    }
    float l = lpart + __shfl_xor(lpart, 16, kWave);
    l += __shfl_xor(l, 32, kWave);

    // merge the 8 waves: lane (col, grp) holds o[head col][16i + 4grp + r]
    if (grp == 0) {
        s_m[wave][col] = m;
        s_l[wave][col] = l;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
        *reinterpret_cast<float4 *>(&s_o[wave][col][16 * i + 4 * grp]) =
            make_float4(o[i][0], o[i][1], o[i][2], o[i][3]);
    __syncthreads();
    float *pb = part + ((int64_t)bh * nsplit + split) * NC * kPart;
    for (int idx = threadIdx.x; idx < NC * kHD; idx += kAttnWaves * kWave) {
        const int h = idx / kHD, d = idx - h * kHD;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) M = __builtin_fmaxf(M, s_m[w][h]);
        float O = 0.0f, Ls = 0.0f;
        if (M != kNegInf) {
#pragma unroll
            for (int w = 0; w < kAttnWaves; ++w) {
                const float f = __builtin_amdgcn_exp2f(s_m[w][h] - M);   // 0 for an empty wave
                O += s_o[w][h][d] * f;
                Ls += s_l[w][h] * f;
            }
        }
        if (OUT == kPartials) {
            pb[h * kPart + d] = O;
            if (d == 0) {
                pb[h * kPart + kHD] = M;
                pb[h * kPart + kHD + 1] = Ls;
            }
        } else {
            // the only split: this is the whole sequence, finish here
            const float y = M != kNegInf ? O / Ls : 0.0f;
            const int hq = h / G, hhd = h - hq * G;   // column h: query token hq, head hhd
            const int64_t oi = (((int64_t)b * Qn + hq) * Hq + hk * G + hhd) * kHD + d;
            if (OUT == kDirectBf16)
                reinterpret_cast<uint16_t *>(out)[oi] = (uint16_t)f32_to_bf16_rne(y);
            else
                reinterpret_cast<float *>(out)[oi] = y;
        }
    }
}

// one wave per (sequence, query token, query head); lane holds dimensions 2 lane,
// 2 lane + 1.
// Splits are read eight at a time, all loads of a batch issued together, and
// merged with a running maximum.
template <bool OUT_BF16>
__global__ void __launch_bounds__(64)
attn_combine_kernel(const float *__restrict__ part, int Hq, int Hkv, int Qn, int nsplit,
                    void *__restrict__ out) {
    constexpr int kBatch = 8;
    const int bq = blockIdx.x;             // (sequence, query token, query head), row-major
    const int G = Hq / Hkv;
    const int b = bq / (Qn * Hq), rq = bq - b * Qn * Hq;
    const int qi = rq / Hq, hq = rq - qi * Hq;
    const int hk = hq / G, h = hq - hk * G;
    const int lane = threadIdx.x;
    const int64_t stride = (int64_t)Qn * G * kPart;
    const float *pp = part + ((int64_t)(b * Hkv + hk) * nsplit) * stride + (qi * G + h) * kPart;
    float M = kNegInf, Lt = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int s0 = 0; s0 < nsplit; s0 += kBatch) {
        float ms[kBatch], ls[kBatch];
        float2 os[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int s = s0 + j < nsplit ? s0 + j : nsplit - 1;   // in range; masked below
            const float *ps = pp + s * stride;
            ms[j] = ps[kHD];
            ls[j] = ps[kHD + 1];
            os[j] = *reinterpret_cast<const float2 *>(ps + 2 * lane);
        }
        float Mn = M;
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (s0 + j >= nsplit) ms[j] = kNegInf;
            Mn = __builtin_fmaxf(Mn, ms[j]);
        }
        if (Mn == kNegInf) continue;                 // no tokens so far
        const float a = __builtin_amdgcn_exp2f(M - Mn);   // 0 while M is -inf
        Lt *= a;
        o0 *= a;
        o1 *= a;
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const float f = __builtin_amdgcn_exp2f(ms[j] - Mn);   // 0 for empty splits
            Lt += ls[j] * f;
            o0 += os[j].x * f;
            o1 += os[j].y * f;
        }
        M = Mn;
    }
    if (M != kNegInf) {
        o0 = o0 / Lt;
        o1 = o1 / Lt;
    }
    const int64_t oi = (int64_t)bq * kHD + 2 * lane;
    if (OUT_BF16) {
        reinterpret_cast<uint32_t *>(out)[oi >> 1] = f32_to_bf16_rne(o0) | (f32_to_bf16_rne(o1) << 16);
    } else {
        *reinterpret_cast<float2 *>(reinterpret_cast<float *>(out) + oi) = make_float2(o0, o1);
    }
}

template <int KVT, int R, int OUT>
hipError_t launch_split(dim3 grid, const uint16_t *q, const void *kc, const float *ks,
                        const void *vc, const float *vs, const int32_t *lens, int Hq, int Hkv,
                        int T, int max_len, int Qn, float *work, void *out, hipStream_t stream) {
    attn_split_kernel<KVT, R, OUT><<<grid, kAttnWaves * kWave, 0, stream>>>(
        q, kc, ks, vc, vs, lens, Hq, Hkv, T, max_len, Qn, work, out);
    return hipGetLastError();
}

template <int KVT, int OUT>
hipError_t launch_split_o(int R, dim3 grid, const uint16_t *q, const void *kc, const float *ks,
                          const void *vc, const float *vs, const int32_t *lens, int Hq, int Hkv,
                          int T, int max_len, int Qn, float *work, void *out, hipStream_t stream) {
    switch (R) {
        case 1: return launch_split<KVT, 1, OUT>(grid, q, kc, ks, vc, vs, lens, Hq, Hkv, T, max_len, Qn, work, out, stream);
        case 2: return launch_split<KVT, 2, OUT>(grid, q, kc, ks, vc, vs, lens, Hq, Hkv, T, max_len, Qn, work, out, stream);
        case 4: return launch_split<KVT, 4, OUT>(grid, q, kc, ks, vc, vs, lens, Hq, Hkv, T, max_len, Qn, work, out, stream);
        default: return launch_split<KVT, 8, OUT>(grid, q, kc, ks, vc, vs, lens, Hq, Hkv, T, max_len, Qn, work, out, stream);
    }
}

// the split kernel for R chunks per wave over ceil(max_len / (512 R)) splits
template <int KVT>
hipError_t launch_split_r(int R, int out_mode, const uint16_t *q, const void *kc, const float *ks,
                          const void *vc, const float *vs, const int32_t *lens, int B, int Hq,
                          int Hkv, int T, int max_len, int Qn, float *work, void *out,
                          hipStream_t stream) {
    const int64_t ns = (max_len + (int64_t)kSplitTok * R - 1) / ((int64_t)kSplitTok * R);
    const dim3 grid((unsigned)ns, (unsigned)(B * Hkv));
    if (out_mode == kDirectBf16)
        return launch_split_o<KVT, kDirectBf16>(R, grid, q, kc, ks, vc, vs, lens, Hq, Hkv, T, max_len, Qn, work, out, stream);
    if (out_mode == kDirectF32)
        return launch_split_o<KVT, kDirectF32>(R, grid, q, kc, ks, vc, vs, lens, Hq, Hkv, T, max_len, Qn, work, out, stream);
    return launch_split_o<KVT, kPartials>(R, grid, q, kc, ks, vc, vs, lens, Hq, Hkv, T, max_len, Qn, work, out, stream);
}

// Both cache types: R chunks per wave, one or several splits, then the merge.
// Qn query tokens per sequence (1 for decode), Qn * Hq / Hkv <= 16.
template <int KVT>
hipError_t attention_decode(const uint16_t *q, const void *kc, const float *ks, const void *vc,
                            const float *vs, const int32_t *lens, int B, int Hq, int Hkv, int T,
                            int max_len, float *work, void *out, int out_bf16, hipStream_t stream,
                            int Qn = 1) {
    // chunks per wave (1, 2, 4 or 8): the most that keep at least kMinWorkgroups
    // workgroups in the grid (long-lived waves, fewer partials to merge)
    const int64_t units = (int64_t)B * Hkv * attention_splits(max_len);
    int R = 1;
    while (R < kMaxChunks && units / (2 * R) >= kMinWorkgroups) R *= 2;
    const int64_t ns = (max_len + kSplitTok * R - 1) / (kSplitTok * R);
    if (ns == 1)   // one split holds every sequence: it writes the output, no merge
        return launch_split_r<KVT>(R, out_bf16 ? kDirectBf16 : kDirectF32, q, kc, ks, vc, vs, lens,
                                   B, Hq, Hkv, T, max_len, Qn, work, out, stream);
    if (ns > 0) {   // max_len == 0: no split to run, the combine writes zeros
        hipError_t e = launch_split_r<KVT>(R, kPartials, q, kc, ks, vc, vs, lens, B, Hq, Hkv, T,
                                           max_len, Qn, work, out, stream);
        if (e != hipSuccess) return e;
    }
    const dim3 rows((unsigned)((int64_t)B * Qn * Hq));
    if (out_bf16)
        attn_combine_kernel<true><<<rows, 64, 0, stream>>>(work, Hq, Hkv, Qn, (int)ns, out);
    else
        attn_combine_kernel<false><<<rows, 64, 0, stream>>>(work, Hq, Hkv, Qn, (int)ns, out);
    return hipGetLastError();
}

}  // namespace

int64_t attention_splits(int64_t max_len) { return (max_len + kSplitTok - 1) / kSplitTok; }

// ---- the allocation-free entry point's workspace ----
// The split partials of bsb_attention_decode_int8kv_noalloc live in this
// array instead of a caller-provided workspace; each device the library runs
// on holds its own copy until the process ends. Every partial the merge reads
// is written by the split kernel of the same call, so nothing is cleared
// between calls; calls that overlap on one device share it and race.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / 4];

namespace {

constexpr int kMaxScratchDevices = 64;
std::atomic<float *> g_scratch[kMaxScratchDevices];

// Device address of `scratch` on the current device, looked up once per
// device. In host code the array's name is a host-side stand-in, never a
// device address, so kernels only ever receive this pointer.
hipError_t scratch_ptr(float **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    float *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        void *a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (a == nullptr) return hipErrorInvalidSymbol;
        p = static_cast<float *>(a);
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

hipError_t launch_attention_decode_noalloc(const uint16_t *q, const int8_t *kc, const float *ks,
                                           const int8_t *vc, const float *vs, const int32_t *lens,
                                           int B, int Hq, int Hkv, int T, int max_len, void *out,
                                           int out_bf16, hipStream_t stream) {
    if (attention_workspace_floats(B, Hq, max_len) * 4 > kNoAllocScratchBytes)
        return hipErrorInvalidValue;   // the entry point rejects these sizes first
    float *work = nullptr;
    hipError_t e = scratch_ptr(&work);
    if (e != hipSuccess) return e;
    return attention_decode<kKvInt8>(q, kc, ks, vc, vs, lens, B, Hq, Hkv, T, max_len, work, out,
                                     out_bf16, stream);
}

int64_t attention_workspace_floats(int64_t B, int64_t Hq, int64_t max_len) {
    return B * Hq * attention_splits(max_len) * kPart;
}

hipError_t launch_kv_cache_write(const uint16_t *k, const uint16_t *v, const int32_t *seq,
                                 const int32_t *pos, int64_t n, int B, int Hkv, int T, int8_t *kc,
                                 float *ks, int8_t *vc, float *vs, hipStream_t stream) {
    const int64_t items = n * Hkv * 2;
    const int64_t blocks = (items + 3) / 4;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    kv_write_kernel<<<dim3((unsigned)blocks), 256, 0, stream>>>(k, v, seq, pos, n, B, Hkv, T, kc,
                                                                ks, vc, vs);
    return hipGetLastError();
}

hipError_t launch_attention_decode(const uint16_t *q, const int8_t *kc, const float *ks,
                                   const int8_t *vc, const float *vs, const int32_t *lens, int B,
                                   int Hq, int Hkv, int T, int max_len, float *work, void *out,
                                   int out_bf16, hipStream_t stream) {
    return attention_decode<kKvInt8>(q, kc, ks, vc, vs, lens, B, Hq, Hkv, T, max_len, work, out,
                                     out_bf16, stream);
}

hipError_t launch_attention_chunk(const uint16_t *q, const int8_t *kc, const float *ks,
                                  const int8_t *vc, const float *vs, const int32_t *lens, int B,
                                  int Qn, int Hq, int Hkv, int T, int max_len, float *work,
                                  void *out, int out_bf16, hipStream_t stream) {
    return attention_decode<kKvInt8>(q, kc, ks, vc, vs, lens, B, Hq, Hkv, T, max_len, work, out,
                                     out_bf16, stream, Qn);
}

hipError_t launch_kv_cache_write_bf16(const uint16_t *k, const uint16_t *v, const int32_t *seq,
                                      const int32_t *pos, int64_t n, int B, int Hkv, int T,
                                      uint16_t *kc, uint16_t *vc, hipStream_t stream) {
    const int64_t items = n * Hkv * 2;
    const int64_t blocks = (items + 3) / 4;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    kv_write_bf16_kernel<<<dim3((unsigned)blocks), 256, 0, stream>>>(k, v, seq, pos, n, B, Hkv, T,
                                                                     kc, vc);
    return hipGetLastError();
}

hipError_t launch_attention_decode_bf16kv(const uint16_t *q, const uint16_t *kc,
                                          const uint16_t *vc, const int32_t *lens, int B, int Hq,
                                          int Hkv, int T, int max_len, float *work, void *out,
                                          int out_bf16, hipStream_t stream) {
    return attention_decode<kKvBf16>(q, kc, nullptr, vc, nullptr, lens, B, Hq, Hkv, T, max_len,
                                     work, out, out_bf16, stream);
}

}  // namespace bsb
