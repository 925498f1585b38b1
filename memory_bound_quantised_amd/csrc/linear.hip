// The skinny W4A8 / W6A8 linear, one launch per matrix.
//
// "What is the bottleneck?" (page "Doubling LLM token rates in ComfyUI"):
// one activation row (M = 1) or a thin block (M = 2..8) times a dense weight
// matrix; every weight is read once for about one operation, so the kernel is
// a stream over the packed weights.
//
// Two forms.  Split form: each wave owns one row block (64 rows, one per
// lane) and a contiguous range of its k groups (a "split"), the next tile
// loading while the current one is summed.  Row-block form (below, for
// matrices whose row blocks fill the chip in one round): one workgroup per
// row block, its waves splitting the k groups and adding their sums through
// LDS, so nothing is combined across workgroups.  For every 64x128 tile the
// lane unpacks its 128 codes to int8, takes int8 dot products against the
// activation (wave-uniform, so it is read through the scalar unit and shared
// by all 64 rows), sums them exactly in int32, and adds the group's
// scale * sum into an fp32 accumulator.  When a row block has several splits,
// each writes its fp32 partial to the workspace and the last split to arrive
// (device-scope counter) sums the partials in split order -- a fixed order, so
// results are bitwise reproducible -- and writes the bf16 output.  The same
// last-arriver combine inside one launch is what the page uses for its
// split-prefix decode attention ("Paying attention to the attention!").
#include "mbq_internal.h"
#include "mbq_kernels.h"
#include "quant_rows.h"

namespace mbq {

namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kTargetWaves = 2048;   // about 8 waves per CU on 256 CUs
#ifndef MBQ_LIN_TILES
#define MBQ_LIN_TILES 4
#endif
constexpr int kTilesPerWave = MBQ_LIN_TILES;   // a split's tiles, at least (when the matrix has enough)
constexpr int kMaxSplits = 16;       // a row block's partials, at most
// Shapes of the row-block form (see plan_linear).
constexpr int64_t kRbAnyBlocksGroups = 48;   // any row-block count up to this many k groups
constexpr int64_t kRbMinBlocks = 48;         // more groups: at least this many row blocks,
constexpr int64_t kRbMaxGroups = 160;        // and at most this many groups
constexpr int64_t kRbMaxBlocks = 512;
constexpr int64_t kRsMaxBlocks = 64;         // the row-set form up to this many row blocks
// The form with the prologue inside keeps the M x K activation codes in LDS,
// next to at most 16 KiB of the kernel's own.
constexpr int64_t kRbPrologueMaxCodes = 140 * 1024;
// Static LDS of the row-block and row-set kernels with the prologue inside:
// the wave partials, the row scales and the prologue's two reductions.
constexpr int64_t rb_static_lds(int W, int M) { return (int64_t)W * M * 64 * 4 + M * 4 + W * 12; }
constexpr int64_t rs_static_lds(int W, int M) { return (int64_t)W * M * 16 * 4 + M * 4 + W * 12; }
// Codes plus static LDS within the CU's 160 KiB, less 1 KiB of alignment
// slack, for every (waves, k groups) pair launch_rb and launch_rs pick: 16
// waves only up to 32 groups (K <= 4096) in the row-block form.
constexpr int64_t kCuLds = 160 * 1024 - 1024;
static_assert(kRbPrologueMaxCodes + rb_static_lds(4, kMaxM) <= kCuLds &&
                  (int64_t)kMaxM * 32 * 128 + rb_static_lds(16, kMaxM) <= kCuLds &&
                  kRbPrologueMaxCodes + rb_static_lds(8, kMaxM) <= kCuLds &&
                  kRbPrologueMaxCodes + rs_static_lds(16, kMaxM) <= kCuLds,
              "prologue codes and the kernels' own LDS fit a CU");
#ifndef MBQ_LIN_MFMA_MIN_M
#define MBQ_LIN_MFMA_MIN_M 1
#endif

template <int BITS, int M>
__global__ __launch_bounds__(64 * kWavesPerBlock) void linear_kernel(
    const uint8_t *__restrict__ packed, const int8_t *__restrict__ q, const float *__restrict__ s,
    uint16_t *__restrict__ y, int64_t y_stride, float *__restrict__ partials,
    unsigned *__restrict__ counters, int N, int K, int splits) {
    using L = Layout<BITS>;
    const int lane = threadIdx.x & 63;
    const int item = blockIdx.x * kWavesPerBlock + uniform(threadIdx.x >> 6);
    const int G = K >> 7;
    const int n_rb = (N + 63) >> 6;
    const int rb = item / splits;
    const int sp = item - rb * splits;
    if (rb >= n_rb) return;
    const int g0 = (int)(((int64_t)sp * G) / splits);
    const int g1 = (int)(((int64_t)(sp + 1) * G) / splits);

    const uint8_t *tiles = packed + (int64_t)rb * G * L::kTileBytes;

    // Matrix cores from MBQ_LIN_MFMA_MIN_M rows on: lane l then holds the sums
    // of weight rows 4 (l & 15) + i for activation rows 4 (l >> 4) + j (rows
    // past M are computed from row 0 and dropped); with v_dot4 every lane
    // holds all M activation rows of its k slice.
    constexpr bool kMfma = M >= MBQ_LIN_MFMA_MIN_M;
    constexpr int AR = kMfma ? (M > 4 ? 4 : M) : M;
    float facc[4][AR];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < AR; ++m) facc[i][m] = 0.0f;
    const int slice = lane >> 4;   // this lane's k slice
    v4i wc[L::kSlabs];
    v2u sc = {0u, 0u};
    if constexpr (kMfma) {
        const int am = (lane & 15) < M ? (lane & 15) : 0;
        const v4i *qrow = reinterpret_cast<const v4i *>(q + (int64_t)am * K + slice * 32);   // 8 v4i per group
        v4i ac0 = v4i{0, 0, 0, 0}, ac1 = v4i{0, 0, 0, 0};
        if (g0 < g1) {
            load_tile<BITS>(tiles + (int64_t)g0 * L::kTileBytes, lane, wc, sc);
            ac0 = *gptr(qrow + g0 * 8);
            ac1 = *gptr(qrow + g0 * 8 + 1);
        }
        for (int g = g0; g < g1; ++g) {
            v4i wn[L::kSlabs];
            v2u sn = {0u, 0u};
            v4i an0 = v4i{0, 0, 0, 0}, an1 = v4i{0, 0, 0, 0};
            if (g + 1 < g1) {
                load_tile<BITS>(tiles + (int64_t)(g + 1) * L::kTileBytes, lane, wn, sn);
                an0 = *gptr(qrow + (g + 1) * 8);
                an1 = *gptr(qrow + (g + 1) * 8 + 1);
            }
            v4i acc[4];
            mfma_tile_regs<BITS>(wc, ac0, ac1, acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float S = row_scale(sc, i);
#pragma unroll
                for (int j = 0; j < AR; ++j) facc[i][j] = fmaf((float)acc[i][j], S, facc[i][j]);
            }
#pragma unroll
            for (int j = 0; j < L::kSlabs; ++j) wc[j] = wn[j];
            sc = sn;
            ac0 = an0;
            ac1 = an1;
        }
    } else {
        const int *qa = reinterpret_cast<const int *>(q);
        const int kdw = K >> 2;  // dwords per activation row
        if (g0 < g1) load_tile<BITS>(tiles + (int64_t)g0 * L::kTileBytes, lane, wc, sc);
        for (int g = g0; g < g1; ++g) {
            v4i wn[L::kSlabs];
            v2u sn = {0u, 0u};
            if (g + 1 < g1) load_tile<BITS>(tiles + (int64_t)(g + 1) * L::kTileBytes, lane, wn, sn);
            int acc[4][M];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int m = 0; m < M; ++m) acc[i][m] = 0;
            const int *qg = qa + g * 32 + slice * 8;
            dot_tile<BITS, M>(wc, [&](int m, int d) { return qg[m * kdw + d]; }, acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float S = row_scale(sc, i);
#pragma unroll
                for (int m = 0; m < M; ++m) facc[i][m] = fmaf((float)acc[i][m], S, facc[i][m]);
            }
#pragma unroll
            for (int j = 0; j < L::kSlabs; ++j) wc[j] = wn[j];
            sc = sn;
        }
    }
    const float unscale = 1.0f / (float)(1 << L::kAccShift);   // exact power of two
    // the combine below works in the dot form: lane l gathers row slice_row(l), every m
    const int r = slice_row(lane);
    const int n = rb * 64 + r;
    float *part = partials + ((int64_t)item * M) * 64;
    if constexpr (kMfma) {
#pragma unroll
        for (int j = 0; j < AR; ++j) {
            const int m = 4 * (lane >> 4) + j;
            if (m >= M) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = 4 * (lane & 15) + i;
                if (splits == 1) {
                    if (rb * 64 + rr < N)
                        y[m * y_stride + rb * 64 + rr] = (uint16_t)f32_to_bf16_bits(s[m] * (facc[i][j] * unscale));
                } else {
                    store_shared(part + m * 64 + rr, facc[i][j]);
                }
            }
        }
        if (splits == 1) return;
    } else {
        // sum the four k slices: lane l ends with row r = slice_row(l)
        float frow[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float f[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) f[i] = facc[i][m];
            frow[m] = slice_reduce(f);
        }
        if (splits == 1) {
            if (n < N) {
#pragma unroll
                for (int m = 0; m < M; ++m)
                    y[m * y_stride + n] = (uint16_t)f32_to_bf16_bits(s[m] * (frow[m] * unscale));
            }
            return;
        }
#pragma unroll
        for (int m = 0; m < M; ++m) store_shared(part + m * 64 + r, frow[m]);
    }
    wait_memory();
    unsigned prev = 0;
    if (lane == 0) prev = counter_add(&counters[rb], 1u);
    prev = (unsigned)__builtin_amdgcn_readfirstlane((int)prev);
    if (prev != (unsigned)(splits - 1)) return;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    float tot[M];
#pragma unroll
    for (int m = 0; m < M; ++m) tot[m] = 0.0f;
    const float *rbp = partials + ((int64_t)rb * splits * M) * 64;
    // issue 32 / M partial loads at a time, then add them in split order
    constexpr int B = 32 / M;
    for (int p0 = 0; p0 < splits; p0 += B) {
        float v[B][M];
#pragma unroll
        for (int u = 0; u < B; ++u)
#pragma unroll
            for (int m = 0; m < M; ++m)
                v[u][m] = p0 + u < splits ? load_shared(rbp + ((p0 + u) * M + m) * 64 + r) : 0.0f;
#pragma unroll
        for (int u = 0; u < B; ++u)
#pragma unroll
            for (int m = 0; m < M; ++m) tot[m] += v[u][m];
    }
    if (n < N) {
#pragma unroll
        for (int m = 0; m < M; ++m)
            y[m * y_stride + n] = (uint16_t)f32_to_bf16_bits(s[m] * (tot[m] * unscale));
    }
    if (lane == 0) store_shared(&counters[rb], 0u);
}

// Row-block form: one workgroup of W waves per row block, wave w taking the
// contiguous k groups [G w / W, G (w + 1) / W),
// the waves' sums added in wave order through LDS.  No partials leave the
// workgroup, so no counter or second pass: with enough row blocks to fill
// the chip this is a single memory round trip deep.  A wave loads up to
// SHOT tiles all at once; a longer range goes in batches of two through a
// ping-pong pair of register sets.  Loads are unconditional, at an index
// clamped into the range, so that none is waited for early; the repeats of
// the last tile hit the cache and are never summed.
// (W, SHOT) per shape, never per row count, so that row m of an M-row call
// sums in the same order as the one-row call; measured on 4096 x 4096,
// 16384 x 5120, 5120 x 8192 and 8192 .. 32000 x 1024 .. 4096:
//   k groups <= 32: W4 16 x 2 (8 x 4 was 5-10 % slower at one row and 10-22 %
//                   slower at four, although 16 waves spill 8 registers from
//                   four rows on), W6 8 x 4 (16 waves spill 50-120 registers);
//   more k groups:   4 x 8 (a wave's longer range keeps more tiles in flight).
template <int BITS>
constexpr int rb_batch() { return 2; }

template <int BITS, int M, int TB>
struct RbBatch {
    v4i w[TB][Layout<BITS>::kSlabs];
    v2u sc[TB];
    v4i a0[TB], a1[TB];
};

// The activation halves of group g come from global memory (qrow) or, when
// the workgroup quantised its rows itself, from LDS (qlds).
template <int BITS, int M, int TB, bool QLDS>
__device__ __forceinline__ void rb_load(RbBatch<BITS, M, TB> &b, const uint8_t *tiles, const v4i *qrow,
                                        const __attribute__((address_space(3))) v4i *qlds, int gb, int g_last,
                                        int lane) {
#pragma unroll
    for (int u = 0; u < TB; ++u) {
        const int g = min(gb + u, g_last);
        load_tile<BITS>(tiles + (int64_t)g * Layout<BITS>::kTileBytes, lane, b.w[u], b.sc[u]);
        if constexpr (QLDS) {
            b.a0[u] = qlds[g * 8];
            b.a1[u] = qlds[g * 8 + 1];
        } else {
            b.a0[u] = *gptr(qrow + g * 8);
            b.a1[u] = *gptr(qrow + g * 8 + 1);
        }
    }
}

template <int BITS, int M, int TB, int AR>
__device__ __forceinline__ void rb_sum(const RbBatch<BITS, M, TB> &b, int gb, int g1, float (&facc)[4][AR]) {
#pragma unroll
    for (int u = 0; u < TB; ++u) {
        if (gb + u < g1) {
            v4i acc[4];
            mfma_tile_regs<BITS>(b.w[u], b.a0[u], b.a1[u], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float S = row_scale(b.sc[u], i);
#pragma unroll
                for (int j = 0; j < AR; ++j) facc[i][j] = fmaf((float)acc[i][j], S, facc[i][j]);
            }
        }
    }
}

// One activation row into LDS through prologue PRO and the quantisation.
template <int PRO, int NT>
__device__ __forceinline__ float rb_quant_row(int8_t *q_row, const uint16_t *x, const uint16_t *u, const uint16_t *wn,
                                              int K, double *red_d, float *red_f) {
    const auto put = [&](int64_t c, uint32_t lo, uint32_t hi) {
        *reinterpret_cast<uint2 *>(q_row + 8 * c) = make_uint2(lo, hi);
    };
    const auto none = [](int64_t, const float (&)[8]) {};
    return quant_row<PRO, NT, false>(x, u, wn, K, red_d, red_f, put, none);
}

// The workgroup's own prologue `pro` (an MBQ_PRO_* value) and quantisation
// of the bf16 rows x (and u, wn) into q_lds (M x K codes) and s_lds.
template <int M, int W>
__device__ __forceinline__ void rb_prologue(int8_t *q_lds, float *s_lds, int K, int pro, const uint16_t *x,
                                            const uint16_t *u, const uint16_t *wn) {
    __shared__ double red_d[W];
    __shared__ float red_f[W];
    for (int m = 0; m < M; ++m) {
        int8_t *qr = q_lds + (int64_t)m * K;
        const uint16_t *xr = x + (int64_t)m * K, *ur = u ? u + (int64_t)m * K : nullptr;
        float sc;
        switch (pro) {
            case MBQ_PRO_RMSNORM_QUANT:
                sc = rb_quant_row<MBQ_PRO_RMSNORM_QUANT, 64 * W>(qr, xr, ur, wn, K, red_d, red_f);
                break;
            case MBQ_PRO_WRMSNORM_QUANT:
                sc = rb_quant_row<MBQ_PRO_WRMSNORM_QUANT, 64 * W>(qr, xr, ur, wn, K, red_d, red_f);
                break;
            case MBQ_PRO_SWIGLU_QUANT:
                sc = rb_quant_row<MBQ_PRO_SWIGLU_QUANT, 64 * W>(qr, xr, ur, wn, K, red_d, red_f);
                break;
            default:
                sc = rb_quant_row<MBQ_PRO_QUANT, 64 * W>(qr, xr, ur, wn, K, red_d, red_f);
                break;
        }
        if (threadIdx.x == 0) s_lds[m] = sc;
    }
    __syncthreads();
}

// QF false: q and s come quantised from global memory.  QF true: the
// workgroup runs prologue `pro` (an MBQ_PRO_* value) and the quantisation on
// the bf16 rows x (and u, wn) itself, into dynamic LDS (M x K codes), first.
template <int BITS, int M, int W, int SHOT, bool QF>
__global__ __launch_bounds__(64 * W) void linear_rb_kernel(
    const uint8_t *__restrict__ packed, const int8_t *__restrict__ q, const float *__restrict__ s,
    uint16_t *__restrict__ y, int64_t y_stride, int N, int K, int pro, const uint16_t *__restrict__ x,
    const uint16_t *__restrict__ u, const uint16_t *__restrict__ wn) {
    using L = Layout<BITS>;
    constexpr int TB = rb_batch<BITS>();
    constexpr int AR = M > 4 ? 4 : M;
    constexpr bool kQlds = QF;
    __shared__ float red[W][M][64];
    __shared__ float s_lds[M];
    extern __shared__ __align__(16) int8_t q_lds[];
    if constexpr (QF) rb_prologue<M, W>(q_lds, s_lds, K, pro, x, u, wn);
    const int lane = threadIdx.x & 63;
    const int w = uniform(threadIdx.x >> 6);
    const int rb = blockIdx.x;
    const int G = K >> 7;
    const int g0 = (int)((int64_t)G * w / W), g1 = (int)((int64_t)G * (w + 1) / W);
    const uint8_t *tiles = packed + (int64_t)rb * G * L::kTileBytes;
    // lane l sums weight rows 4 (l & 15) + i for activation rows 4 (l >> 4) + j
    // (rows past M are computed from row 0 and dropped), as the split form
    const int am = (lane & 15) < M ? (lane & 15) : 0;
    const v4i *qrow = kQlds ? nullptr : reinterpret_cast<const v4i *>(q + (int64_t)am * K + (lane >> 4) * 32);
    const __attribute__((address_space(3))) v4i *qlds =
        reinterpret_cast<const __attribute__((address_space(3))) v4i *>(
            (const __attribute__((address_space(3))) int8_t *)q_lds + (int64_t)am * K + (lane >> 4) * 32);
    float facc[4][AR];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < AR; ++j) facc[i][j] = 0.0f;
    if (g1 - g0 > 0 && g1 - g0 <= SHOT) {
        // every tile of the wave in flight at once, summed in the same branch
        RbBatch<BITS, M, SHOT> A;
        rb_load<BITS, M, SHOT, kQlds>(A, tiles, qrow, qlds, g0, g1 - 1, lane);
        rb_sum<BITS, M, SHOT, AR>(A, g0, g1, facc);
    } else if (g1 - g0 > SHOT) {
        RbBatch<BITS, M, TB> A, B;
        rb_load<BITS, M, TB, kQlds>(A, tiles, qrow, qlds, g0, g1 - 1, lane);
        {
            for (int gb = g0;;) {
                rb_load<BITS, M, TB, kQlds>(B, tiles, qrow, qlds, gb + TB, g1 - 1, lane);
                rb_sum<BITS, M, TB, AR>(A, gb, g1, facc);
                gb += TB;
                if (gb >= g1) break;
                rb_load<BITS, M, TB, kQlds>(A, tiles, qrow, qlds, gb + TB, g1 - 1, lane);
                rb_sum<BITS, M, TB, AR>(B, gb, g1, facc);
                gb += TB;
                if (gb >= g1) break;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < AR; ++j) {
        const int m = 4 * (lane >> 4) + j;
        if (m < M) {
#pragma unroll
            for (int i = 0; i < 4; ++i) red[w][m][4 * (lane & 15) + i] = facc[i][j];
        }
    }
    __syncthreads();
    const float unscale = 1.0f / (float)(1 << L::kAccShift);   // exact power of two
    for (int t = threadIdx.x; t < M * 64; t += 64 * W) {
        const int m = t >> 6, r = t & 63;
        float tot = 0.0f;
#pragma unroll
        for (int ww = 0; ww < W; ++ww) tot += red[ww][m][r];
        const int n = rb * 64 + r;
        const float sm = kQlds ? s_lds[m] : s[m];
        if (n < N) y[m * y_stride + n] = (uint16_t)f32_to_bf16_bits(sm * (tot * unscale));
    }
}

// Row-set form: one workgroup per (row block, row set).  A 64-row tile holds
// its rows in four sets of 16 (rows 4n + i, n = 0..15: W4 slab i, W6 dwords
// 6i .. 6i + 5 of each lane, a slab and a half), and the products of set i
// need only those bytes, so four workgroups share a row block without any
// combine: each loads a quarter of every tile (plus the tile's scales of its
// rows) and issues a quarter of the products.  A matrix of few row blocks so
// spreads over four times the CUs.  Waves split the k groups as in the
// row-block form and their sums are added in wave order; each output row sums
// its groups in the same order as the row-block form with the same W.
// Where row set `set` lies in a lane's share of a tile: W4 the 16 bytes of
// slab `set`; W6 a 16-byte part (slab 0, 2, 3 or 5) and an 8-byte part (a half
// of slab 1 or 4) that hold its six dwords, the 8-byte part first for odd
// sets; offsc: the byte of the fp16 scale of the lane's row 4 (lane & 15) + set.
struct RowsetAt {
    int off16, off8, offsc;
    bool odd;
};
template <int BITS>
__device__ __forceinline__ RowsetAt rowset_at(int set, int lane) {
    RowsetAt r;
    r.off16 = (BITS == 4 ? set : (set == 0 ? 0 : set == 1 ? 2 : set == 2 ? 3 : 5)) * kSlab + lane * 16;
    r.off8 = (set < 2 ? 1 : 4) * kSlab + lane * 16 + (set & 1) * 8;
    r.offsc = Layout<BITS>::kWeightBytes + 2 * (4 * (lane & 15) + set);
    r.odd = set & 1;
    return r;
}
// The set's two unpacked k halves from its bytes (v unused for W4).
template <int BITS>
__device__ __forceinline__ void rowset_unpack(v4i w, v2u v, bool odd, v4i &h0, v4i &h1) {
    if constexpr (BITS == 4) {
        h0 = unpack_row_w4(w, 0);
        h1 = unpack_row_w4(w, 1);
    } else {
        const uint32_t d0 = odd ? v.x : w.x, d1 = odd ? v.y : w.y, d2 = odd ? w.x : w.z;
        const uint32_t d3 = odd ? w.y : w.w, d4 = odd ? w.z : v.x, d5 = odd ? w.w : v.y;
        h0 = unpack_row_w6(d0, d1, d2);
        h1 = unpack_row_w6(d3, d4, d5);
    }
}

template <int BITS, int TB>
struct RsBatch {
    v4i w[TB];           // W4: the row set's slab; W6: its 16-byte part
    v2u w2[TB];          // W6: its 8-byte part (unused for W4)
    uint32_t sc[TB];     // fp16 bits of the lane's row scale
    v4i a0[TB], a1[TB];
};

template <int BITS, int TB, bool QLDS>
__device__ __forceinline__ void rs_load(RsBatch<BITS, TB> &b, const uint8_t *tiles, const RowsetAt &at,
                                        const v4i *qrow, const __attribute__((address_space(3))) v4i *qlds, int gb,
                                        int g_last) {
#pragma unroll
    for (int u = 0; u < TB; ++u) {
        const int g = min(gb + u, g_last);
        const uint8_t *t = tiles + (int64_t)g * Layout<BITS>::kTileBytes;
        b.w[u] = load_stream(reinterpret_cast<const v4i *>(t + at.off16));
        if constexpr (BITS == 6)
            b.w2[u] = __builtin_nontemporal_load(gptr(reinterpret_cast<const v2u *>(t + at.off8)));
        b.sc[u] = __builtin_nontemporal_load(gptr(reinterpret_cast<const uint16_t *>(t + at.offsc)));
        if constexpr (QLDS) {
            b.a0[u] = qlds[g * 8];
            b.a1[u] = qlds[g * 8 + 1];
        } else {
            b.a0[u] = *gptr(qrow + g * 8);
            b.a1[u] = *gptr(qrow + g * 8 + 1);
        }
    }
}

template <int BITS, int TB, int AR>
__device__ __forceinline__ void rs_sum(const RsBatch<BITS, TB> &b, bool odd, int gb, int g1, float (&facc)[AR]) {
#pragma unroll
    for (int u = 0; u < TB; ++u) {
        if (gb + u < g1) {
            v4i h0, h1;
            rowset_unpack<BITS>(b.w[u], b.w2[u], odd, h0, h1);
            const v4i acc = mfma_rowset(b.a0[u], b.a1[u], h0, h1);
            const float S = f16_bits_to_f32(b.sc[u] & 0xFFFFu);
#pragma unroll
            for (int j = 0; j < AR; ++j) facc[j] = fmaf((float)acc[j], S, facc[j]);
        }
    }
}

template <int BITS, int M, int W, int SHOT, bool QF>
__global__ __launch_bounds__(64 * W) void linear_rs_kernel(
    const uint8_t *__restrict__ packed, const int8_t *__restrict__ q, const float *__restrict__ s,
    uint16_t *__restrict__ y, int64_t y_stride, int N, int K, int pro, const uint16_t *__restrict__ x,
    const uint16_t *__restrict__ u, const uint16_t *__restrict__ wn) {
    using L = Layout<BITS>;
    constexpr int TB = rb_batch<BITS>();
    constexpr int AR = M > 4 ? 4 : M;
    __shared__ float red[W][M][16];
    __shared__ float s_lds[M];
    extern __shared__ __align__(16) int8_t q_lds[];
    if constexpr (QF) rb_prologue<M, W>(q_lds, s_lds, K, pro, x, u, wn);
    const int lane = threadIdx.x & 63;
    const int w = uniform(threadIdx.x >> 6);
    // The four workgroups of a row block on one XCD, which share its scale
    // lines in that XCD's L2 (workgroups go to the XCDs in turn): in each run
    // of 32 workgroups, workgroup 32 g + 8 s + j is set s of row block 8 g + j;
    // a last, partial run of r row blocks is dealt as 4 sets of r.
    int rb, set;
    {
        const int b = blockIdx.x, n_rb = (N + 63) >> 6, full = n_rb >> 3;
        if ((b >> 5) < full) {
            rb = 8 * (b >> 5) + (b & 7);
            set = (b >> 3) & 3;
        } else {
            const int r = n_rb - 8 * full, o = b - 32 * full;
            rb = 8 * full + o % r;
            set = o / r;
        }
    }
    const int G = K >> 7;
    const int g0 = (int)((int64_t)G * w / W), g1 = (int)((int64_t)G * (w + 1) / W);
    const uint8_t *tiles = packed + (int64_t)rb * G * L::kTileBytes;
    const RowsetAt at = rowset_at<BITS>(set, lane);
    // lane l sums weight row 4 (l & 15) + set for activation rows 4 (l >> 4) + j
    const int am = (lane & 15) < M ? (lane & 15) : 0;
    const v4i *qrow = QF ? nullptr : reinterpret_cast<const v4i *>(q + (int64_t)am * K + (lane >> 4) * 32);
    const __attribute__((address_space(3))) v4i *qlds =
        reinterpret_cast<const __attribute__((address_space(3))) v4i *>(
            (const __attribute__((address_space(3))) int8_t *)q_lds + (int64_t)am * K + (lane >> 4) * 32);
    float facc[AR];
#pragma unroll
    for (int j = 0; j < AR; ++j) facc[j] = 0.0f;
    if (g1 - g0 > 0 && g1 - g0 <= SHOT) {
        RsBatch<BITS, SHOT> A;
        rs_load<BITS, SHOT, QF>(A, tiles, at, qrow, qlds, g0, g1 - 1);
        rs_sum<BITS, SHOT, AR>(A, at.odd, g0, g1, facc);
    } else if (g1 - g0 > SHOT) {
        RsBatch<BITS, TB> A, B;
        rs_load<BITS, TB, QF>(A, tiles, at, qrow, qlds, g0, g1 - 1);
        for (int gb = g0;;) {
            rs_load<BITS, TB, QF>(B, tiles, at, qrow, qlds, gb + TB, g1 - 1);
            rs_sum<BITS, TB, AR>(A, at.odd, gb, g1, facc);
            gb += TB;
            if (gb >= g1) break;
            rs_load<BITS, TB, QF>(A, tiles, at, qrow, qlds, gb + TB, g1 - 1);
            rs_sum<BITS, TB, AR>(B, at.odd, gb, g1, facc);
            gb += TB;
            if (gb >= g1) break;
        }
    }
#pragma unroll
    for (int j = 0; j < AR; ++j) {
        const int m = 4 * (lane >> 4) + j;
        if (m < M) red[w][m][lane & 15] = facc[j];
    }
    __syncthreads();
    const float unscale = 1.0f / (float)(1 << L::kAccShift);   // exact power of two
    for (int t = threadIdx.x; t < M * 16; t += 64 * W) {
        const int m = t >> 4, r = t & 15;
        float tot = 0.0f;
#pragma unroll
        for (int ww = 0; ww < W; ++ww) tot += red[ww][m][r];
        const int n = rb * 64 + 4 * r + set;
        const float sm = QF ? s_lds[m] : s[m];
        if (n < N) y[m * y_stride + n] = (uint16_t)f32_to_bf16_bits(sm * (tot * unscale));
    }
}

// Exact int32 group sums for the tests: one wave per tile, through the same
// tile functions the product runs.  FORM 1: mfma_tile_regs, the whole-tile
// form of the per-op linear's split and row-block forms and of the fused
// walk, with the activation halves loaded exactly as the linear loads them;
// FORM 2: the row-set form's loads (rowset_at), unpack (rowset_unpack) and
// products (mfma_rowset), one row set after another; FORM 0: group_sums_dot,
// the v_dot4 form the walk is built with when MBQ_MFMA_MIN_M is raised.
template <int BITS, int M, int FORM>
__global__ __launch_bounds__(64) void group_acc_kernel(const uint8_t *__restrict__ packed,
                                                       const int8_t *__restrict__ q,
                                                       int32_t *__restrict__ acc_out, int N, int K) {
    using L = Layout<BITS>;
    const int G = K >> 7;
    const int tile = blockIdx.x;
    const int rb = tile / G, g = tile % G;
    const int lane = threadIdx.x;
    if constexpr (FORM == 2) {
        const int am = (lane & 15) < M ? (lane & 15) : 0;
        const v4i *qrow = reinterpret_cast<const v4i *>(q + (int64_t)am * K + (lane >> 4) * 32);
        const v4i a0 = *gptr(qrow + g * 8), a1 = *gptr(qrow + g * 8 + 1);
        const uint8_t *t = packed + (int64_t)tile * L::kTileBytes;
#pragma unroll
        for (int set = 0; set < 4; ++set) {
            const RowsetAt at = rowset_at<BITS>(set, lane);
            const v4i wq = *gptr(reinterpret_cast<const v4i *>(t + at.off16));
            const v2u wv = BITS == 6 ? *gptr(reinterpret_cast<const v2u *>(t + at.off8)) : v2u{0u, 0u};
            v4i h0, h1;
            rowset_unpack<BITS>(wq, wv, at.odd, h0, h1);
            const v4i acc = mfma_rowset(a0, a1, h0, h1);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int m = 4 * (lane >> 4) + j;
                const int n = rb * 64 + 4 * (lane & 15) + set;
                if (m < M && n < N) acc_out[((int64_t)m * N + n) * G + g] = acc[j] >> L::kAccShift;
            }
        }
        return;
    }
    v4i w[L::kSlabs];
    v2u sb;
    load_tile<BITS>(packed + (int64_t)tile * L::kTileBytes, lane, w, sb);
    if constexpr (FORM == 1) {
        const int am = (lane & 15) < M ? (lane & 15) : 0;
        const v4i *qrow = reinterpret_cast<const v4i *>(q + (int64_t)am * K + (lane >> 4) * 32);
        v4i acc[4];
        mfma_tile_regs<BITS>(w, *gptr(qrow + g * 8), *gptr(qrow + g * 8 + 1), acc);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = 4 * (lane >> 4) + j;
            if (m >= M) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int n = rb * 64 + 4 * (lane & 15) + i;
                if (n < N) acc_out[((int64_t)m * N + n) * G + g] = acc[i][j] >> L::kAccShift;
            }
        }
    } else {
        const int *qg = reinterpret_cast<const int *>(q) + g * 32 + (lane >> 4) * 8;
        const int kdw = K >> 2;
        int gs[M];
        group_sums_dot<BITS, M>(w, [&](int m, int d) { return qg[m * kdw + d]; }, gs);
        const int n = rb * 64 + slice_row(lane);
#pragma unroll
        for (int m = 0; m < M; ++m)
            if (n < N) acc_out[((int64_t)m * N + n) * G + g] = gs[m] >> L::kAccShift;
    }
}

template <int BITS, int M, bool QF>
void launch_rb(const uint8_t *pk, const int8_t *q, const float *s, uint16_t *y, int64_t y_stride, int64_t N,
               int64_t K, int64_t n_rb, int64_t groups, int pro, const uint16_t *x, const uint16_t *u,
               const uint16_t *wn, hipStream_t st) {
    const dim3 grid((unsigned)n_rb);
    const size_t lds = QF ? (size_t)(M * K) : 0;
    if (groups > 32) {
        linear_rb_kernel<BITS, M, 4, 8, QF><<<grid, dim3(64 * 4), lds, st>>>(pk, q, s, y, y_stride, (int)N, (int)K,
                                                                             pro, x, u, wn);
    } else if constexpr (BITS == 4) {
        linear_rb_kernel<BITS, M, 16, 2, QF><<<grid, dim3(64 * 16), lds, st>>>(pk, q, s, y, y_stride, (int)N,
                                                                               (int)K, pro, x, u, wn);
    } else {
        linear_rb_kernel<BITS, M, 8, 4, QF><<<grid, dim3(64 * 8), lds, st>>>(pk, q, s, y, y_stride, (int)N, (int)K,
                                                                             pro, x, u, wn);
    }
}

// Row-set form: W = 16 waves whatever M is, so a row's sum order never
// depends on the row count; up to 2 or 4 tiles per wave at once, longer
// ranges in two-deep batches.
template <int BITS, int M, bool QF>
void launch_rs(const uint8_t *pk, const int8_t *q, const float *s, uint16_t *y, int64_t y_stride, int64_t N,
               int64_t K, int64_t n_rb, int64_t groups, int pro, const uint16_t *x, const uint16_t *u,
               const uint16_t *wn, hipStream_t st) {
    const dim3 grid((unsigned)(n_rb * 4));
    const size_t lds = QF ? (size_t)(M * K) : 0;
    if (groups <= 32)
        linear_rs_kernel<BITS, M, 16, 2, QF><<<grid, dim3(64 * 16), lds, st>>>(pk, q, s, y, y_stride, (int)N, (int)K,
                                                                               pro, x, u, wn);
    else
        linear_rs_kernel<BITS, M, 16, 4, QF><<<grid, dim3(64 * 16), lds, st>>>(pk, q, s, y, y_stride, (int)N, (int)K,
                                                                               pro, x, u, wn);
}

template <int BITS, int M, bool QF>
void launch_rows(const LinearPlan &plan, const uint8_t *pk, const int8_t *q, const float *s, uint16_t *y,
                 int64_t y_stride, int64_t N, int64_t K, int pro, const uint16_t *x, const uint16_t *u,
                 const uint16_t *wn, hipStream_t st) {
    if (plan.rs_form)
        launch_rs<BITS, M, QF>(pk, q, s, y, y_stride, N, K, plan.n_rb, plan.groups, pro, x, u, wn, st);
    else
        launch_rb<BITS, M, QF>(pk, q, s, y, y_stride, N, K, plan.n_rb, plan.groups, pro, x, u, wn, st);
}

template <int BITS>
hipError_t launch_linear_bits(int64_t M, int64_t N, int64_t K, const int8_t *q, const float *s,
                              const void *packed, void *y, int64_t y_stride, void *ws,
                              const LinearPlan &plan, hipStream_t st) {
    const uint8_t *pk = (const uint8_t *)packed;
    uint16_t *yv = (uint16_t *)y;
    if (plan.rb_form) {
#define MBQ_RB(MM) launch_rows<BITS, MM, false>(plan, pk, q, s, yv, y_stride, N, K, 0, nullptr, nullptr, nullptr, st)
        switch (M) {
            case 1: MBQ_RB(1); break;
            case 2: MBQ_RB(2); break;
            case 3: MBQ_RB(3); break;
            case 4: MBQ_RB(4); break;
            case 5: MBQ_RB(5); break;
            case 6: MBQ_RB(6); break;
            case 7: MBQ_RB(7); break;
            default: MBQ_RB(8); break;
        }
#undef MBQ_RB
        return hipGetLastError();
    }
    const int64_t items = plan.n_rb * plan.splits;
    const dim3 grid((unsigned)((items + kWavesPerBlock - 1) / kWavesPerBlock));
    const dim3 block(64 * kWavesPerBlock);
    unsigned *counters = (unsigned *)ws;
    float *partials = (float *)((char *)ws + kCounterBytes);
    const uint8_t *p = (const uint8_t *)packed;
    uint16_t *yo = (uint16_t *)y;
#define MBQ_LAUNCH(MM)                                                                          \
    linear_kernel<BITS, MM><<<grid, block, 0, st>>>(p, q, s, yo, y_stride, partials, counters, \
                                                    (int)N, (int)K, (int)plan.splits)
    switch (M) {
        case 1: MBQ_LAUNCH(1); break;
        case 2: MBQ_LAUNCH(2); break;
        case 3: MBQ_LAUNCH(3); break;
        case 4: MBQ_LAUNCH(4); break;
        case 5: MBQ_LAUNCH(5); break;
        case 6: MBQ_LAUNCH(6); break;
        case 7: MBQ_LAUNCH(7); break;
        default: MBQ_LAUNCH(8); break;
    }
#undef MBQ_LAUNCH
    return hipGetLastError();
}

template <int BITS, int FORM>
hipError_t launch_group_acc_form(int64_t M, int64_t N, int64_t K, const int8_t *q, const void *packed,
                                 int32_t *acc, hipStream_t st) {
    const dim3 grid((unsigned)(row_blocks(N) * (K / kGroup)));
    const uint8_t *p = (const uint8_t *)packed;
#define MBQ_GA(MM) group_acc_kernel<BITS, MM, FORM><<<grid, 64, 0, st>>>(p, q, acc, (int)N, (int)K)
    switch (M) {
        case 1: MBQ_GA(1); break;
        case 2: MBQ_GA(2); break;
        case 3: MBQ_GA(3); break;
        case 4: MBQ_GA(4); break;
        case 5: MBQ_GA(5); break;
        case 6: MBQ_GA(6); break;
        case 7: MBQ_GA(7); break;
        default: MBQ_GA(8); break;
    }
#undef MBQ_GA
    return hipGetLastError();
}

}  // namespace

LinearPlan plan_linear(int bits, int64_t M, int64_t N, int64_t K) {
    (void)bits;
    LinearPlan p;
    p.n_rb = row_blocks(N);
    p.groups = K / kGroup;
    // enough waves to fill the chip, but kTilesPerWave tiles each where the
    // matrix has them and at most kMaxSplits splits per row block: a split
    // pays the load latency once, and the last arriver gathers every partial
    // of its row block, so a one-tile split (4096 x 4096 at 2048 waves) or a
    // 26-way split (5120 x 17408) costs more than it spreads.
    int64_t waves = p.n_rb * p.groups / kTilesPerWave;
    if (waves > kTargetWaves) waves = kTargetWaves;
    if (waves < p.n_rb) waves = p.n_rb;
    int64_t sp = (waves + p.n_rb - 1) / p.n_rb;
    if (sp > kMaxSplits) sp = kMaxSplits;
    if (sp > p.groups) sp = p.groups;
    if (sp < 1) sp = 1;
    p.splits = sp;
    p.ws_bytes = kCounterBytes + (sp > 1 ? p.n_rb * sp * M * 64 * 4 : 0);
    // The row-block form (a workgroup per row block, no partials, no combine)
    // wherever one workgroup's share stays modest or the row blocks fill most
    // of the chip; the split form's combine costs a counter and a gather round
    // trip.  Measured against the split form (M = 1 / 4, per call in a graph):
    // 1024 x 5120 5.7 / 6.3 against 7.3 / 9.2 us, 17408 x 5120 12.4 / 13.5
    // against 13.5 / 15.6 us, 5120 x 17408 15.2 / 16.3 against 15.5 / 18.6 us.
    // A few row blocks over many groups (a workgroup streaming half a MB
    // alone) stay split.
    p.rb_form = p.n_rb <= kRbMaxBlocks &&
                (p.groups <= kRbAnyBlocksGroups || (p.n_rb >= kRbMinBlocks && p.groups <= kRbMaxGroups));
    // Four workgroups per row block (the row-set form) while they fit the
    // chip in one round: 4096 x 4096 4.4 / 4.6 against 5.2 / 6.3 us at M = 1
    // / 4, 1024 x 5120 5.3 / 5.6 against 5.7 / 6.3 us; at 80 and more row
    // blocks it was 13-90 % slower.
    p.rs_form = p.rb_form && p.n_rb <= kRsMaxBlocks;
    return p;
}

hipError_t launch_linear(int bits, int64_t M, int64_t N, int64_t K, const int8_t *q, const float *s,
                         const void *packed, void *y, int64_t y_stride, void *ws, const LinearPlan &plan,
                         hipStream_t st) {
    return bits == 4 ? launch_linear_bits<4>(M, N, K, q, s, packed, y, y_stride, ws, plan, st)
                     : launch_linear_bits<6>(M, N, K, q, s, packed, y, y_stride, ws, plan, st);
}

int64_t linear_prologue_ws_bytes(int bits, int64_t M, int64_t N, int64_t K) {
    return (M * K + 255) / 256 * 256 + 256 + plan_linear(bits, M, N, K).ws_bytes;
}

hipError_t launch_linear_prologue(int bits, int pro, int64_t M, int64_t N, int64_t K, const void *x, const void *u,
                                  const void *w, const void *packed, void *y, void *ws, hipStream_t st) {
    const LinearPlan plan = plan_linear(bits, M, N, K);
    if (plan.rb_form && M * K <= kRbPrologueMaxCodes) {
        const uint8_t *pk = (const uint8_t *)packed;
        uint16_t *yv = (uint16_t *)y;
        const uint16_t *xs = (const uint16_t *)x, *us = (const uint16_t *)u, *wn = (const uint16_t *)w;
#define MBQ_RBF(B, MM) launch_rows<B, MM, true>(plan, pk, nullptr, nullptr, yv, N, N, K, pro, xs, us, wn, st)
#define MBQ_RBF_M(B)                   \
    switch (M) {                       \
        case 1: MBQ_RBF(B, 1); break;  \
        case 2: MBQ_RBF(B, 2); break;  \
        case 3: MBQ_RBF(B, 3); break;  \
        case 4: MBQ_RBF(B, 4); break;  \
        case 5: MBQ_RBF(B, 5); break;  \
        case 6: MBQ_RBF(B, 6); break;  \
        case 7: MBQ_RBF(B, 7); break;  \
        default: MBQ_RBF(B, 8); break; \
    }
        if (bits == 4) {
            MBQ_RBF_M(4)
        } else {
            MBQ_RBF_M(6)
        }
#undef MBQ_RBF_M
#undef MBQ_RBF
        return hipGetLastError();
    }
    // other shapes: the prologue kernel, then the linear, through the workspace
    int8_t *q = (int8_t *)ws;
    float *s = (float *)((char *)ws + (M * K + 255) / 256 * 256);
    void *lin_ws = (char *)ws + (M * K + 255) / 256 * 256 + 256;
    hipError_t e = launch_prologue_quant(pro, M, K, x, K, u, K, w, nullptr, q, s, st);
    if (e != hipSuccess) return e;
    return launch_linear(bits, M, N, K, q, s, packed, y, N, lin_ws, plan, st);
}

hipError_t launch_group_acc(int bits, int form, int64_t M, int64_t N, int64_t K, const int8_t *q,
                            const void *packed, int32_t *acc, hipStream_t st) {
    if (bits == 4)
        return form == 2 ? launch_group_acc_form<4, 2>(M, N, K, q, packed, acc, st)
               : form == 1 ? launch_group_acc_form<4, 1>(M, N, K, q, packed, acc, st)
                           : launch_group_acc_form<4, 0>(M, N, K, q, packed, acc, st);
    return form == 2 ? launch_group_acc_form<6, 2>(M, N, K, q, packed, acc, st)
           : form == 1 ? launch_group_acc_form<6, 1>(M, N, K, q, packed, acc, st)
                       : launch_group_acc_form<6, 0>(M, N, K, q, packed, acc, st);
}

}  // namespace mbq
