// Split-prefix decode attention ("Paying attention to the attention!" on the
// page "Doubling LLM token rates in ComfyUI"): a short query -- one token, or
// the committed token and the MTP draft rows with their causal verification --
// against a bf16 KV cache, with no materialised mask.  The cached prefix is
// split across many workgroups so that the tiny query still fills the GPU,
// and the last workgroup of each key/value head to finish combines the
// partial results in the same launch.
//
// Workgroup (kv head g, split s): 256 threads, positions in blocks of 64,
// staged in LDS (keys row-major, values transposed) while the next block is
// loaded into registers.  The query rows of the head group (r = token * qpg +
// head-in-group, at most 64) form up to four 16-row tiles, one per wave; a
// wave's tile products run on the matrix cores (bf16, 16 x 16 x 32):
//   scores   S = Q K^T, the query tile held in registers for the whole walk;
//   softmax  online per row (running max m and sum l, base 2); the score and
//            the output tiles put row 4 (lane / 16) + j of the tile in the
//            same lane register, so rescaling needs no data movement;
//   values   O += P V, with P as a bf16 high part plus a bf16 residual (two
//            products, about 16 significant bits; bf16 alone loses a percent
//            where values cancel), going through LDS to take the operand
//            layout.
// Each workgroup publishes (m, l, o) per row (the only split of a head writes
// the output itself), and the splits are merged: M = max m_s, L = sum l_s
// 2^(m_s - M), O = sum o_s 2^(m_s - M) / L.  Two combines:
//   a second kernel (the default), wide over (head, output columns);
//   in the same launch (MBQ_ATTN_COMBINE=inline in the environment): the
//     launch is cooperative, so every split is resident; a split counts in on
//     its head's counter, waits for the head's other splits, and merges a
//     share of the head's output columns.
// The cooperative launch alone costs more on this device than the second
// kernel does, so the second kernel is the default.  (Having the last split
// of a head merge everything leaves 64 rows x 256 columns over up to 128
// splits to one workgroup: slower still.)
#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "mbq.h"
#include "mbq_internal.h"
#include "mbq_kernels.h"

namespace mbq {

namespace {

constexpr int kBlock = 64;        // positions per block (32 for four row tiles)
constexpr int kMaxSplits = 128;
constexpr int kAttnThreads = 256;
#ifndef MBQ_ATTN_MIN_BLOCKS
#define MBQ_ATTN_MIN_BLOCKS 2
#endif

struct AttnArgs {
    const uint16_t *q;            // [M][n_q][D]
    const uint16_t *k, *v;        // [n_kv][L][D]
    uint16_t *o;                  // [M][n_q][D]
    float *part_o;                // [n_kv][n_split][rows][D]
    float *part_ml;               // [n_kv][n_split][rows][2]
    int64_t L;                    // cache row stride (positions)
    int32_t M, n_q, n_kv, qpg, rows, P, n_split, blocks_per_split, n_blocks;
    float scale_log2;             // log2(e) / sqrt(D)
    // The combine inside the launch (a cooperative one: every workgroup is
    // resident): per kv head g, cnt[32 g] counts the splits that have
    // published and cnt[32 g + 16] the ones done merging; the last of those
    // zeroes both.  merge_inline 0: attn_merge_kernel merges afterwards.
    uint32_t *cnt;
    int32_t merge_inline, tpq;
};

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

// Reductions over the 16 lanes of a DPP row, every lane ending with the result.
template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                                                 CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_row<0xB1>(v));    // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp_row<0x4E>(v));    // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp_row<0x141>(v));   // row_half_mirror
    return fmaxf(v, dpp_row<0x140>(v));   // row_mirror
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_row<0xB1>(v);
    v += dpp_row<0x4E>(v);
    v += dpp_row<0x141>(v);
    return v + dpp_row<0x140>(v);
}

struct MergeArgs {
    const float *part_o, *part_ml;   // as in AttnArgs
    uint16_t *o;
    int32_t n_split, rows, qpg, n_q, tpq;
};

// Loads of the partials: plain, or at agent scope when they were stored in
// the same launch by other CUs (a plain load could hit a stale cache line).
template <bool COH>
__device__ __forceinline__ f4 load_part4(const float *p) {
    if constexpr (COH) {
        const uint64_t *q = reinterpret_cast<const uint64_t *>(p);
        const uint64_t x = load_shared(q), y = load_shared(q + 1);
        return f4{__uint_as_float((uint32_t)x), __uint_as_float((uint32_t)(x >> 32)),
                  __uint_as_float((uint32_t)y), __uint_as_float((uint32_t)(y >> 32))};
    } else {
        return *reinterpret_cast<const f4 *>(p);
    }
}
template <bool COH>
__device__ __forceinline__ float load_part(const float *p) {
    if constexpr (COH) return load_shared(p);
    else return *p;
}

// Merge of one chunk of a head's outputs, wide: the chunk is the 256 / tpq
// groups of four adjacent outputs from output e_lo on; lanes t of a group of
// tpq consecutive lanes sum splits t, t + tpq, ... (at most 8, so tpq * 8 >=
// the split count) with one 16-byte load each, and the group adds its lanes'
// sums.  The weights 2^(m_s - M) / L of the rows the chunk touches (at most
// 16) are staged first.  Scratch (LDS): w_s, l_s kMaxSplits x kMaxRowsWg
// floats each, red kMaxRowsWg x 2.  Every thread of the workgroup calls it.
constexpr int kMaxRowsWg = kAttnThreads * 4 / 64;   // rows a chunk touches, at most
// a lane sums at most 8 splits and a group has at most 16 lanes
static_assert(kMaxSplits <= 16 * 8, "the merge covers every split");
constexpr int kMergeScratchBytes = (2 * kMaxSplits * kMaxRowsWg + 2 * kMaxRowsWg) * 4;
template <int D, bool COH>
__device__ __forceinline__ void merge_chunk(const MergeArgs &a, int g, int64_t e_lo, float *w_s, float *l_s,
                                            float *red) {
    const int tid = threadIdx.x;
    const int n = a.n_split, rows = a.rows, tpq = a.tpq;
    const int groups = kAttnThreads / tpq;
    const int r_lo = (int)(e_lo / D);
    const int r_hi = min(rows, (int)((e_lo + groups * 4 - 1) / D) + 1);
    const int nr = r_hi - r_lo;
    // the lane's partials (at most 8 splits: tpq * 8 >= n) go out first, so
    // that their round trip overlaps the weights' one.  A wave holds 64 / tpq
    // groups, lane gw + (64 / tpq) t being lane t of group gw: consecutive
    // lanes read consecutive outputs of one split (whole lines), not one
    // output of consecutive splits.
    const int gpw = 64 / tpq;                              // groups per wave
    const int t = (tid & 63) / gpw;
    const int64_t e0 = e_lo + (int64_t)((tid >> 6) * gpw + (tid & 63) % gpw) * 4;   // the group's first output
    const int r = (int)(e0 / D), d = (int)(e0 % D);
    const bool real = r < rows;
    f4 v[8];
    {
        const float *op = a.part_o + ((int64_t)g * n * rows + (real ? r : 0)) * D + d;
        const int64_t stride = (int64_t)rows * D;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int s = t + u * tpq;
            v[u] = real && s < n ? load_part4<COH>(op + s * stride) : f4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }
    const float *ml = a.part_ml + (int64_t)g * n * rows * 2;
    for (int idx = tid; idx < n * nr; idx += kAttnThreads) {
        const int s = idx / nr, rr = idx % nr;
        w_s[s * kMaxRowsWg + rr] = load_part<COH>(ml + ((int64_t)s * rows + r_lo + rr) * 2);
        l_s[s * kMaxRowsWg + rr] = load_part<COH>(ml + ((int64_t)s * rows + r_lo + rr) * 2 + 1);
    }
    __syncthreads();
    {   // a wave per row: its lanes stride over the splits
        const int lane = tid & 63, wave = tid >> 6;
        for (int rr = wave; rr < nr; rr += kAttnThreads / 64) {
            float mx = -INFINITY;
            for (int s = lane; s < n; s += 64) mx = fmaxf(mx, w_s[s * kMaxRowsWg + rr]);
            for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
            float den = 0.0f;
            for (int s = lane; s < n; s += 64)
                if (w_s[s * kMaxRowsWg + rr] != -INFINITY)
                    den += l_s[s * kMaxRowsWg + rr] * exp2f(w_s[s * kMaxRowsWg + rr] - mx);
            for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off);
            if (lane == 0) {
                red[rr * 2] = mx;
                red[rr * 2 + 1] = den;
            }
        }
    }
    __syncthreads();
    for (int idx = tid; idx < n * nr; idx += kAttnThreads) {
        const int s = idx / nr, rr = idx % nr;
        const float mt = w_s[s * kMaxRowsWg + rr];
        w_s[s * kMaxRowsWg + rr] = mt == -INFINITY ? 0.0f : exp2f(mt - red[rr * 2]) / red[rr * 2 + 1];
    }
    __syncthreads();
    f4 acc = f4{0.0f, 0.0f, 0.0f, 0.0f};
    if (real) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int s = t + u * tpq;
            if (s < n) acc += w_s[s * kMaxRowsWg + r - r_lo] * v[u];
        }
    }
    for (int off = gpw; off < 64; off <<= 1)   // the group's lanes are gpw apart: the same tree over t
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] += __shfl_xor(acc[c], off);
    if (real && t == 0) {
        const int i = r / a.qpg, j = r % a.qpg;
        uint32_t *dst = reinterpret_cast<uint32_t *>(a.o + ((int64_t)i * a.n_q + g * a.qpg + j) * D + d);
        dst[0] = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
        dst[1] = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
    }
    __syncthreads();   // the scratch is reused by the next chunk
}

// The merge inside the split launch: after this split's partials have reached
// memory it counts in on its head's counter and waits for every split of the
// head; then the head's chunks are dealt to its splits in turn, and the last
// split to finish merging zeroes the two counters for the next call.  Every
// split of the head is resident (cooperative launch), so the wait ends.
constexpr int64_t kMergeSpinLimit = 1ll << 26;
template <int D>
__device__ __forceinline__ void merge_in_launch(const AttnArgs &a, int g, int s, uint8_t *scratch) {
    uint32_t *arrived = a.cnt + 32 * g, *merged = a.cnt + 32 * g + 16;
    wait_memory();      // this thread's partial stores have reached memory
    __syncthreads();    // and every thread's
    if (threadIdx.x == 0) {
        counter_add(arrived, 1u);
        int64_t spins = 0;
        while (load_shared(arrived) < (uint32_t)a.n_split && ++spins < kMergeSpinLimit) __builtin_amdgcn_s_sleep(2);
    }
    __syncthreads();   // the whole workgroup waits for thread 0
    MergeArgs ma;
    ma.part_o = a.part_o;
    ma.part_ml = a.part_ml;
    ma.o = a.o;
    ma.n_split = a.n_split;
    ma.rows = a.rows;
    ma.qpg = a.qpg;
    ma.n_q = a.n_q;
    ma.tpq = a.tpq;
    float *w_s = reinterpret_cast<float *>(scratch);
    float *l_s = w_s + kMaxSplits * kMaxRowsWg;
    float *red = l_s + kMaxSplits * kMaxRowsWg;
    const int64_t per_chunk = kAttnThreads / a.tpq * 4;
    const int64_t n_chunks = ((int64_t)a.rows * D + per_chunk - 1) / per_chunk;
    for (int64_t c = s; c < n_chunks; c += a.n_split) merge_chunk<D, true>(ma, g, c * per_chunk, w_s, l_s, red);
    if (threadIdx.x == 0 && counter_add(merged, 1u) == (uint32_t)(a.n_split - 1)) {
        store_shared(arrived, 0u);
        store_shared(merged, 0u);
    }
}

// WPR: waves per 16-row query tile (4, 2 or 1 for up to 16, 32 or 64 rows);
// the waves of a tile split its score position tiles and output column tiles.
// BLK: positions per block, 64 or 32 (32 halves the staging LDS and the
// load registers, so the one-wave-per-tile form fits two workgroups per CU).
template <int D, int WPR, int BLK>
__device__ __forceinline__ void attention_split(const AttnArgs &a) {
    static_assert(BLK == 64 || BLK == 32, "block of 64 or 32 positions");
    constexpr int kPt = BLK / 16;                 // position tiles per block
    static_assert(WPR <= kPt, "a wave takes whole position tiles");
    constexpr int kKStride = D * 2 + 16;          // LDS bytes per key row
    constexpr int kVtStride = BLK * 2 + 16;       // LDS bytes per transposed value row (one column)
    constexpr int kPStride = BLK * 2 + 16;        // LDS bytes per probability row
    constexpr int kChunks = D / 8;                // 16-byte pieces of a row
    constexpr int kLoads = BLK * kChunks / kAttnThreads;   // 16-byte loads per thread per tensor
    constexpr int kKs = D / 32;                   // k steps of the score product
    constexpr int kCt = D / 16;                   // column tiles of the output
    constexpr int kPtW = kPt / WPR;               // position tiles per wave
    constexpr int kCtW = kCt / WPR;               // column tiles per wave
    extern __shared__ __align__(16) uint8_t lds[];
    uint8_t *k_lds = lds;                                  // [BLK][kKStride]
    uint8_t *vt_lds = k_lds + BLK * kKStride;              // [D][kVtStride]
    uint8_t *p_lds = vt_lds + D * kVtStride;               // [4 row tiles][hi 16, lo 16][kPStride]
    __shared__ float s_red[4][16];                         // per wave: its part of a row-tile reduction

    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    const int s = blockIdx.x, g = blockIdx.y;
    const int rows = a.rows;
    const int qpg = a.qpg;
    const int lr = lane & 15, lq = lane >> 4;     // operand row / column, k group
    const int rt = wave / WPR, sw = wave % WPR;   // the wave's row tile, and its part of it
    const bool computes = rt * 16 < rows;

    // the wave's query tile as score operands (rows past the group read zeros)
    bf8 qa[kKs];
    {
        const int r = rt * 16 + lr;
        const int i = r / qpg, j = r % qpg;
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) {
            v4i v = v4i{0, 0, 0, 0};
            if (r < rows) v = *gptr(reinterpret_cast<const v4i *>(a.q + ((int64_t)i * a.n_q + g * qpg + j) * D + 32 * ks + 8 * lq));
            qa[ks] = __builtin_bit_cast(bf8, v);
        }
    }

    // blocks_per_split blocks per split, and one more for each of the last
    // (n_blocks mod n_split) splits: the last split holds the cache's tail
    // block, which may hold no more than the new rows
    const int extra0 = a.n_split - (a.n_blocks - a.n_split * a.blocks_per_split);   // first split with one more
    const int b0 = s * a.blocks_per_split + max(0, s - extra0);
    const int b1 = b0 + a.blocks_per_split + (s >= extra0 ? 1 : 0);
    const int64_t used = (int64_t)a.P + a.M;       // positions in the cache
    const uint16_t *kg = a.k + (int64_t)g * a.L * D, *vg = a.v + (int64_t)g * a.L * D;

    // Loads: wave w covers positions 16 w .. 16 w + 15.  Keys held as score
    // operands (WPR = 4) take, in load u, chunks 4 u .. 4 u + 3 (lane >> 4)
    // of the 16 rows (lane & 15), 64 contiguous bytes of each.  Values, and
    // keys staged in LDS, need no operand layout, so where a thread makes an
    // even number of loads, load u takes whole 128-byte lines instead: rows
    // 8 (u & 1) + lane / 8, chunks 8 (u / 2) + lane % 8 (eight consecutive
    // lanes read one line; measured faster than the operand layout, where
    // consecutive lanes read 16 different rows).  Value loads
    // carry the non-temporal hint; key loads do not (measured: the hint
    // speeds the values and slows the keys).  The
    // transposed value tile keeps a column's positions contiguous, rotated by
    // 8 (d / 8 mod 8) positions, so the lanes of a write land on different
    // banks while every 8-position operand run stays contiguous.
    // With one position tile per wave (WPR = 4) the keys are not staged:
    // load u of a wave is exactly its score operand for k step u (position
    // 16 w + lr, k 32 u + 8 lq .. +7), kept in registers until the block's
    // scores.
    // With 32-position blocks two waves share a 16-position group, each
    // loading half of the row's 16-byte chunks.
    v4i kbuf[kLoads], vbuf[kLoads];
    const int pp = 16 * (wave % kPt) + lr;
    const int cbase = (wave / kPt) * (kChunks * kPt / 4);
    constexpr bool kVLines = kLoads % 2 == 0;
    auto vpos = [&](int u) { return kVLines ? 16 * (wave % kPt) + 8 * (u & 1) + (lane >> 3) : pp; };
    auto vchunk = [&](int u) { return kVLines ? cbase + 8 * (u >> 1) + (lane & 7) : cbase + 4 * u + lq; };
    // keys staged in LDS take the values' layout; keys held as operands (WPR = 4) their own
    auto kpos = [&](int u) { return WPR == 4 ? pp : vpos(u); };
    auto kchunk = [&](int u) { return WPR == 4 ? cbase + 4 * u + lq : vchunk(u); };
    auto fetch = [&](int b) {
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int64_t pos = (int64_t)b * BLK + kpos(u), vp = (int64_t)b * BLK + vpos(u);
            kbuf[u] = v4i{0, 0, 0, 0};
            vbuf[u] = v4i{0, 0, 0, 0};
            if (pos < used) kbuf[u] = *gptr(reinterpret_cast<const v4i *>(kg + pos * D) + kchunk(u));
            if (vp < used) vbuf[u] = load_stream(reinterpret_cast<const v4i *>(vg + vp * D) + vchunk(u));
        }
    };
    static_assert(WPR != 4 || (BLK == 64 && kLoads == kKs), "one key load per k step");
    v4i kop[WPR == 4 ? kKs : 1];
    auto stage = [&]() {
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int c = cbase + 4 * u + lq;
            if constexpr (WPR == 4) kop[u] = kbuf[u];
            else *reinterpret_cast<v4i *>(k_lds + kpos(u) * kKStride + kchunk(u) * 16) = kbuf[u];
            const uint32_t w[4] = {(uint32_t)vbuf[u].x, (uint32_t)vbuf[u].y, (uint32_t)vbuf[u].z, (uint32_t)vbuf[u].w};
            const int vc = vchunk(u);
            const int col = (vpos(u) + 8 * (vc & 7)) & (BLK - 1);   // rows 8 vc .. 8 vc + 7: d / 8 = vc
#pragma unroll
            for (int e = 0; e < 8; ++e)
                *reinterpret_cast<uint16_t *>(vt_lds + (8 * vc + e) * kVtStride + col * 2) =
                    (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        }
    };

    // m: the row's running max (the same in every wave of the tile); l: this
    // wave's part of the running sum (its positions); o: its column tiles
    float m[4], l[4];
    f4 o[kCtW];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.0f;
    }
#pragma unroll
    for (int c = 0; c < kCtW; ++c) o[c] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    uint8_t *pw = p_lds + rt * 32 * kPStride;     // rows 0-15: bf16 of p, rows 16-31: bf16 of the rest

    if (b0 < b1) fetch(b0);
    for (int b = b0; b < b1; ++b) {
        __syncthreads();   // the previous block's LDS is consumed
        stage();
        __syncthreads();
        if (b + 1 < b1) fetch(b + 1);
        // scores of the wave's position tiles: sc[q][j] = S[row 4 lq + j][position 16 (sw + q WPR) + lr]
        f4 sc[kPtW];
        float x[kPtW][4];
        if (computes) {
#pragma unroll
            for (int q = 0; q < kPtW; ++q) {
                const int pt = sw + q * WPR;
                f4 acc = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int ks = 0; ks < kKs; ++ks) {
                    bf8 kb;
                    if constexpr (WPR == 4) kb = __builtin_bit_cast(bf8, kop[ks < (WPR == 4 ? kKs : 1) ? ks : 0]);
                    else kb = *reinterpret_cast<const bf8 *>(k_lds + (16 * pt + lr) * kKStride + (32 * ks + 8 * lq) * 2);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kb, acc, 0, 0, 0);
                }
                sc[q] = acc;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = rt * 16 + 4 * lq + j;
                const int64_t lim = r < rows ? (int64_t)a.P + r / qpg : -1;   // last attended position
                float bm = -INFINITY;
#pragma unroll
                for (int q = 0; q < kPtW; ++q) {
                    const int64_t pos = (int64_t)b * BLK + 16 * (sw + q * WPR) + lr;
                    x[q][j] = pos <= lim ? sc[q][j] * a.scale_log2 : -INFINITY;
                    bm = fmaxf(bm, x[q][j]);
                }
                bm = row16_max(bm);
                if (WPR > 1 && lr == 0) s_red[wave][4 * lq + j] = bm;
            }
        }
        if (WPR > 1) __syncthreads();   // the row maxima of the tile's other waves
        if (computes) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float bm = x[0][j];
                if (WPR > 1) {
                    bm = s_red[rt * WPR][4 * lq + j];
#pragma unroll
                    for (int k = 1; k < WPR; ++k) bm = fmaxf(bm, s_red[rt * WPR + k][4 * lq + j]);
                } else {
#pragma unroll
                    for (int q = 1; q < kPtW; ++q) bm = fmaxf(bm, x[q][j]);
                    bm = row16_max(bm);
                }
                const float mn = fmaxf(m[j], bm);
                float alpha = 1.0f, ps = 0.0f;
                uint32_t pb[kPtW], pr[kPtW];
#pragma unroll
                for (int q = 0; q < kPtW; ++q) pb[q] = pr[q] = 0;
                if (mn != -INFINITY) {
                    alpha = exp2f(m[j] - mn);                 // 0 when m was -inf
#pragma unroll
                    for (int q = 0; q < kPtW; ++q) {
                        const float pv = exp2f(x[q][j] - mn);   // 0 at masked positions
                        pb[q] = f32_to_bf16_bits(pv);
                        pr[q] = f32_to_bf16_bits(pv - bf16_bits_to_f32(pb[q]));
                        ps += pv;
                    }
                    m[j] = mn;
                }
                l[j] = l[j] * alpha + row16_sum(ps);
#pragma unroll
                for (int c = 0; c < kCtW; ++c) o[c][j] *= alpha;
#pragma unroll
                for (int q = 0; q < kPtW; ++q) {
                    const int col = 16 * (sw + q * WPR) + lr;
                    *reinterpret_cast<uint16_t *>(pw + (4 * lq + j) * kPStride + col * 2) = (uint16_t)pb[q];
                    *reinterpret_cast<uint16_t *>(pw + (16 + 4 * lq + j) * kPStride + col * 2) = (uint16_t)pr[q];
                }
            }
        }
        if (WPR > 1) {
            __syncthreads();   // the tile's probabilities from every wave
        } else {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        if (!computes) continue;
        // values: O += P V over the wave's column tiles
#pragma unroll
        for (int ks = 0; ks < BLK / 32; ++ks) {
            const bf8 pa = *reinterpret_cast<const bf8 *>(pw + lr * kPStride + (32 * ks + 8 * lq) * 2);
            const bf8 pl = *reinterpret_cast<const bf8 *>(pw + (16 + lr) * kPStride + (32 * ks + 8 * lq) * 2);
#pragma unroll
            for (int c = 0; c < kCtW; ++c) {
                const int d = 16 * (sw + c * WPR) + lr;
                const int col = (32 * ks + 8 * lq + 8 * ((d >> 3) & 7)) & (BLK - 1);
                const bf8 vb = *reinterpret_cast<const bf8 *>(vt_lds + d * kVtStride + col * 2);
                o[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, o[c], 0, 0, 0);
                o[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vb, o[c], 0, 0, 0);
            }
        }
    }

    // publish this split's (m, l, o) per row; l is the sum of the tile's waves' parts
    const int64_t base = ((int64_t)g * a.n_split + s) * rows;
    if (WPR > 1) {
        __syncthreads();
        if (computes && lr == 0)
#pragma unroll
            for (int j = 0; j < 4; ++j) s_red[wave][4 * lq + j] = l[j];
        __syncthreads();
        if (computes)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float t = s_red[rt * WPR][4 * lq + j];
#pragma unroll
                for (int k = 1; k < WPR; ++k) t += s_red[rt * WPR + k][4 * lq + j];
                l[j] = t;
            }
    }
    if (computes) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = rt * 16 + 4 * lq + j;
            if (r >= rows) continue;
            if (a.n_split == 1) {   // the head's only split: its result is the output
                const float inv = 1.0f / l[j];
                const int i = r / qpg, jj = r % qpg;
                uint16_t *dst = a.o + ((int64_t)i * a.n_q + g * qpg + jj) * D;
#pragma unroll
                for (int c = 0; c < kCtW; ++c) dst[16 * (sw + c * WPR) + lr] = (uint16_t)f32_to_bf16_bits(o[c][j] * inv);
                continue;
            }
            float *po = a.part_o + (base + r) * D + 16 * sw + lr, *pml = a.part_ml + (base + r) * 2;
            if (a.merge_inline) {   // read in this launch, maybe on another XCD: agent scope
#pragma unroll
                for (int c = 0; c < kCtW; ++c) store_shared(po + 16 * c * WPR, o[c][j]);
                if (lr == 0 && sw == 0) {
                    store_shared(pml, m[j]);
                    store_shared(pml + 1, l[j]);
                }
            } else {
#pragma unroll
                for (int c = 0; c < kCtW; ++c) po[16 * c * WPR] = o[c][j];
                if (lr == 0 && sw == 0) {
                    pml[0] = m[j];
                    pml[1] = l[j];
                }
            }
        }
    }
    if (a.merge_inline && a.n_split > 1) {
        __syncthreads();   // the staging LDS is free: the merge's scratch
        merge_in_launch<D>(a, g, s, lds);
    }
}

template <int D, int WPR, int BLK>
__global__ __launch_bounds__(kAttnThreads) void decode_attention_kernel(AttnArgs a) {
    attention_split<D, WPR, BLK>(a);
}
// The same with at most 256 registers, so that two workgroups fit on a CU
// (two waves per SIMD): the forms for two row tiles, and for four with
// 32-position blocks, whose LDS allows two.
template <int D, int WPR, int BLK>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_attention_kernel_x2(
    AttnArgs a) {
    attention_split<D, WPR, BLK>(a);
}

// The merge as a second launch: a workgroup per chunk of a head.
template <int D>
__global__ __launch_bounds__(kAttnThreads) void attn_merge_kernel(MergeArgs a) {
    __shared__ float w_s[kMaxSplits * kMaxRowsWg];
    __shared__ float l_s[kMaxSplits * kMaxRowsWg];
    __shared__ float red[kMaxRowsWg * 2];
    const int64_t e_lo = (int64_t)blockIdx.x * (kAttnThreads / a.tpq) * 4;
    merge_chunk<D, false>(a, blockIdx.y, e_lo, w_s, l_s, red);
}

}  // namespace

AttnPlan plan_attention(int64_t M, int64_t n_q, int64_t n_kv, int64_t D, int64_t P, int n_cu) {
    AttnPlan pl;
    const int64_t used = P + M;
    pl.rows = (n_q / n_kv) * M;
    const int64_t row_tiles = (pl.rows + 15) / 16;
    pl.block = row_tiles > 2 ? kBlock / 2 : kBlock;
    pl.n_blocks = (used + pl.block - 1) / pl.block;
    // keys, transposed values, the row tiles' probabilities
    pl.lds_bytes = (int)(pl.block * (D * 2 + 16) + D * (pl.block * 2 + 16) + row_tiles * 32 * (pl.block * 2 + 16));
    // a workgroup per CU, two where their LDS fits (one hides the other's
    // load latency; the one-tile form's registers allow it, and the others
    // have a form capped at 256 registers), and at least MBQ_ATTN_MIN_BLOCKS
    // 64-position blocks' worth of positions each (a split's fixed cost --
    // the query load, the first fetch, publishing -- is latency)
    const int64_t kMinBlocks = MBQ_ATTN_MIN_BLOCKS * kBlock / pl.block;
    const int64_t per_cu = pl.lds_bytes <= 80 * 1024 ? 2 : 1;
    pl.two_per_cu = per_cu == 2;
    const int64_t target = std::max<int64_t>(
        1, std::min<int64_t>({kMaxSplits, per_cu * n_cu / n_kv, (pl.n_blocks + kMinBlocks - 1) / kMinBlocks}));
    // Every split the target allows, the blocks dealt as evenly as they go
    // with any remainder on the last splits: equal splits of the rounded-up
    // size leave workgroups idle.  A 32768-token cache plus the new row is
    // 513 blocks: 128 splits of 4, the last with a fifth of one row, took
    // M = 1 from 38.0 to 36.9 us against 103 splits of 5 (512 blocks: 35.5).
    pl.n_split = std::min<int64_t>(pl.n_blocks, target);
    pl.blocks_per_split = pl.n_blocks / pl.n_split;
    // merge: lanes per group of four outputs, so that a lane sums at most 8 splits
    pl.merge_tpq = 1;
    while (pl.merge_tpq < 16 && pl.merge_tpq * 8 < pl.n_split) pl.merge_tpq *= 2;
    // [merge counters: 128 bytes per kv head][m, l per split and row][o per split and row]
    const int64_t part_ml = n_kv * pl.n_split * pl.rows * 2 * 4;
    const int64_t part_o = n_kv * pl.n_split * pl.rows * D * 4;
    auto up = [](int64_t v) { return (v + 255) / 256 * 256; };
    pl.off_cnt = 0;
    pl.off_ml = up(n_kv * 128);
    pl.off_o = pl.off_ml + up(part_ml);
    pl.ws_bytes = pl.off_o + up(part_o);
    // the combine inside the launch, when asked for, borrows the staging LDS
    // for its scratch
    const char *combine = getenv("MBQ_ATTN_COMBINE");
    pl.merge_inline = combine && strcmp(combine, "inline") == 0 && pl.n_split > 1 &&
                      pl.lds_bytes >= kMergeScratchBytes;
    return pl;
}

hipError_t launch_attention(const AttnPlan &pl, int64_t M, int64_t n_q, int64_t n_kv, int64_t D, int64_t P,
                            int64_t L, const void *q, const void *k, const void *v, void *o, void *ws,
                            hipStream_t st) {
    AttnArgs a;
    a.q = (const uint16_t *)q;
    a.k = (const uint16_t *)k;
    a.v = (const uint16_t *)v;
    a.o = (uint16_t *)o;
    a.part_o = (float *)((char *)ws + pl.off_o);
    a.part_ml = (float *)((char *)ws + pl.off_ml);
    a.L = L;
    a.M = (int32_t)M;
    a.n_q = (int32_t)n_q;
    a.n_kv = (int32_t)n_kv;
    a.qpg = (int32_t)(n_q / n_kv);
    a.rows = (int32_t)pl.rows;
    a.P = (int32_t)P;
    a.n_split = (int32_t)pl.n_split;
    a.blocks_per_split = (int32_t)pl.blocks_per_split;
    a.n_blocks = (int32_t)pl.n_blocks;
    a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    a.cnt = (uint32_t *)((char *)ws + pl.off_cnt);
    a.tpq = (int32_t)pl.merge_tpq;
    const int wpr = pl.rows <= 16 ? 4 : pl.rows <= 32 ? 2 : 1;
#define MBQ_ATTN(DD)                                                                                   \
    (wpr == 4   ? reinterpret_cast<const void *>(&decode_attention_kernel<DD, 4, 64>)                   \
     : wpr == 2 ? (pl.two_per_cu ? reinterpret_cast<const void *>(&decode_attention_kernel_x2<DD, 2, 64>) \
                                 : reinterpret_cast<const void *>(&decode_attention_kernel<DD, 2, 64>))  \
                : (pl.two_per_cu ? reinterpret_cast<const void *>(&decode_attention_kernel_x2<DD, 1, 32>) \
                                 : reinterpret_cast<const void *>(&decode_attention_kernel<DD, 1, 32>)))
    const void *fn = D == 64 ? MBQ_ATTN(64) : D == 128 ? MBQ_ATTN(128) : MBQ_ATTN(256);
#undef MBQ_ATTN
    void *args[] = {(void *)&a};
    const dim3 grid((unsigned)pl.n_split, (unsigned)n_kv);
    if (pl.merge_inline) {
        // one launch: every split resident, the merge at its end
        a.merge_inline = 1;
        const hipError_t e =
            hipLaunchCooperativeKernel(fn, grid, dim3(kAttnThreads), args, (unsigned)pl.lds_bytes, st);
        if (e == hipSuccess) return e;
        (void)hipGetLastError();   // refused (the grid does not fit at once): merge in a second launch
    }
    a.merge_inline = 0;
    const hipError_t e = hipLaunchKernel(fn, grid, dim3(kAttnThreads), args, (size_t)pl.lds_bytes, st);
    if (e != hipSuccess || pl.n_split == 1) return e;
    MergeArgs ma;
    ma.part_o = a.part_o;
    ma.part_ml = a.part_ml;
    ma.o = a.o;
    ma.n_split = a.n_split;
    ma.rows = a.rows;
    ma.qpg = a.qpg;
    ma.n_q = a.n_q;
    ma.tpq = (int32_t)pl.merge_tpq;
    const int64_t per_wg = kAttnThreads / pl.merge_tpq * 4;   // outputs per workgroup
    const unsigned gx = (unsigned)((pl.rows * D + per_wg - 1) / per_wg);
    const void *mf = D == 64 ? reinterpret_cast<const void *>(&attn_merge_kernel<64>)
                     : D == 128 ? reinterpret_cast<const void *>(&attn_merge_kernel<128>)
                                : reinterpret_cast<const void *>(&attn_merge_kernel<256>);
    void *margs[] = {(void *)&ma};
    return hipLaunchKernel(mf, dim3(gx, (unsigned)n_kv), dim3(kAttnThreads), margs, 0, st);
}

}  // namespace mbq
