// Internal definitions shared by the HIP kernels of libmbq (gfx950 only).
//
// Kernel-order weight layout ("Optimizing the Linear Kernel" on the page
// "Doubling LLM token rates in ComfyUI": weights and their per-group scales
// interleaved in the order the kernel consumes them, so that a block streams
// one contiguous run):
//
//   A matrix is cut into row blocks of 64 rows and 128-wide k groups.  Tile
//   (rb, g) lives at byte offset (rb * G + g) * TILE_BYTES and holds SLABS
//   slabs of 1024 B followed by the 64 rows' fp16 scales (S[rb*64 + r][g] at
//   WEIGHT_BYTES + 2*r).  One slab is exactly one wave-wide dwordx4 load
//   (1 KiB, 8 full 128-B lines).
//
//   Lane l of a wave owns rows 4*(l & 15) + i (i = 0..3) of the tile and the
//   k slice s = l >> 4, i.e. k = g*128 + 32*s + (0..31): each activation
//   dword it reads is reused for four rows.  The lane's four scales are the 8
//   bytes at WEIGHT_BYTES + 8*(l & 15).
//
//   W4 (4 slabs): slab i holds the lane's row i; lane dword d (0..3) covers
//   k0 = 32*s + 8*d:
//     byte b low nibble  = code(k0 + b)      (two's complement)
//     byte b high nibble = code(k0 + 4 + b)  (two's complement)
//   so (x << 4) & 0xF0F0F0F0 and x & 0xF0F0F0F0 are four int8 lanes holding
//   16*w, matching activation dwords k0/4 and k0/4 + 1.
//
//   W6 (6 slabs): the lane's 24 dwords D = 4*slab + (dword in slab) form
//   triples D = 6*i + 3*t + (0, 1, 2) for row i and half t (t = 0, 1), which
//   cover k0 = 32*s + 16*t + (0..15):
//     dword c of the triple, byte b, bits 7..2 = code(k0 + 4c + b)      (c = 0, 1, 2)
//     dword c of the triple, byte b, bits 1..0 = bits (5-2c)..(4-2c) of code(k0 + 12 + b)
//   so x & 0xFCFCFCFC gives int8 lanes holding 4*w for k0+4c..k0+4c+3, and
//   ((x0&3)<<6)|((x1&3)<<4)|((x2&3)<<2) gives 4*w for k0+12..k0+15.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mbq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

constexpr int kRows = 64;     // rows per row block = lanes per wave
constexpr int kGroup = 128;   // k per scale group
constexpr int kSlab = 1024;   // bytes of one wave-wide dwordx4 load

// Every workspace starts with one fixed region of 32-bit counters, one per
// row block of the largest supported matrix.  Because its size never depends
// on the call's shape, counters that one call leaves at zero are still zero
// for any later call, whatever its shape.
constexpr int64_t kMaxN = (int64_t)1 << 20;
constexpr int kMaxM = 8;      // activation rows per call (a token plus up to 7 verify rows)
constexpr int64_t kCounterBytes = (kMaxN / kRows) * 4;   // 64 KiB

template <int BITS> struct Layout;
template <> struct Layout<4> {
    static constexpr int kSlabs = 4;
    static constexpr int kWeightBytes = 4096;
    static constexpr int kTileBytes = 4096 + 128;
    static constexpr int kAccShift = 4;     // unpacked lanes hold 16*w
};
template <> struct Layout<6> {
    static constexpr int kSlabs = 6;
    static constexpr int kWeightBytes = 6144;
    static constexpr int kTileBytes = 6144 + 128;
    static constexpr int kAccShift = 2;     // unpacked lanes hold 4*w
};

inline int64_t tile_bytes(int bits) { return bits == 4 ? Layout<4>::kTileBytes : Layout<6>::kTileBytes; }
inline int64_t row_blocks(int64_t N) { return (N + kRows - 1) / kRows; }

// ------------------------------------------------------------------ number formats

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

// Round to nearest even bf16; finite inputs only (inf stays inf, overflow -> inf).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// SwiGLU gate of one element, rounded to bf16 and returned as fp32:
// silu(g) * u with silu(g) = g / (1 + exp(-g)) in fp32 (g -> -inf gives -0).
__device__ __forceinline__ float swiglu_bf16f(float g, float u) {
    const float sg = g / (1.0f + expf(-g));
    return bf16_bits_to_f32(f32_to_bf16_bits(sg * u));
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)h);
}

// ------------------------------------------------------------------ integer dot product

__device__ __forceinline__ int dot4(int a, int b, int c) {
    return __builtin_amdgcn_sdot4(a, b, c, false);
}

// Wave-uniform value (the compiler keeps it in an SGPR).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Every pointer these kernels dereference in global memory goes through the
// global address space: generic (flat) accesses also count on the LDS/scalar
// counter, so an LDS read would then wait for every weight load in flight.
#define MBQ_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ MBQ_GLOBAL T *gptr(T *p) { return (MBQ_GLOBAL T *)p; }
template <typename T>
__device__ __forceinline__ const MBQ_GLOBAL T *gptr(const T *p) { return (const MBQ_GLOBAL T *)p; }

// Streaming 16-byte load of packed weights: read once, keep it out of the caches.
__device__ __forceinline__ v4i load_stream(const v4i *p) {
    return __builtin_nontemporal_load(gptr(p));
}

// ------------------------------------------------------------------ cross-wave communication
//
// Waves on different XCDs see each other's data only at the memory-side
// coherence point: each XCD has its own L2.  Rather than the compiler's
// agent-scope fences (which write back and invalidate the whole L2), every
// value that crosses waves is stored and loaded with agent-scope relaxed
// atomics (write-through / coherent-read instructions), and the only ordering
// needed -- "my data is at the coherence point before my counter increment"
// -- is a wait for this wave's outstanding memory operations.

template <typename T>
__device__ __forceinline__ void store_shared(T *p, T v) {
    __hip_atomic_store(gptr(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T load_shared(const T *p) {
    return __hip_atomic_load(gptr(const_cast<T *>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_memory() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);   // vmcnt(0) expcnt(0) lgkmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ unsigned counter_add(unsigned *p, unsigned v) {
    return __hip_atomic_fetch_add(gptr(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ one tile, one lane
//
// acc[i][m] += sum over the lane's 32 k of (2^kAccShift * w[row i]) * q[m][k]
// for the lane's four rows; `act(m, d)` returns activation dword d (k = 32*s +
// 4d .. +3 of the group, d = 0..7) of row m as four packed int8.

template <int M, typename Act>
__device__ __forceinline__ void dot_tile_w4(const v4i (&w)[4], Act act, int (&acc)[4][M]) {
    int a[M][8];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int d = 0; d < 8; ++d) a[m][d] = act(m, d);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t wd[4] = {(uint32_t)w[i].x, (uint32_t)w[i].y, (uint32_t)w[i].z, (uint32_t)w[i].w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int lo = (int)((wd[d] << 4) & 0xF0F0F0F0u);
            const int hi = (int)(wd[d] & 0xF0F0F0F0u);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                acc[i][m] = dot4(lo, a[m][2 * d], acc[i][m]);
                acc[i][m] = dot4(hi, a[m][2 * d + 1], acc[i][m]);
            }
        }
    }
}

template <int M, typename Act>
__device__ __forceinline__ void dot_tile_w6(const v4i (&w)[6], Act act, int (&acc)[4][M]) {
    int a[M][8];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int d = 0; d < 8; ++d) a[m][d] = act(m, d);
    uint32_t wd[24];
#pragma unroll
    for (int j = 0; j < 6; ++j) {
        wd[4 * j + 0] = (uint32_t)w[j].x;
        wd[4 * j + 1] = (uint32_t)w[j].y;
        wd[4 * j + 2] = (uint32_t)w[j].z;
        wd[4 * j + 3] = (uint32_t)w[j].w;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t x0 = wd[6 * i + 3 * t], x1 = wd[6 * i + 3 * t + 1], x2 = wd[6 * i + 3 * t + 2];
            const uint32_t m6 = 0xFCFCFCFCu;
            const int a0 = (int)(x0 & m6), a1 = (int)(x1 & m6), a2 = (int)(x2 & m6);
            const int a3 = (int)(((x0 << 6) & 0xC0C0C0C0u) | ((x1 << 4) & 0x30303030u) |
                                 ((x2 << 2) & 0x0C0C0C0Cu));
#pragma unroll
            for (int m = 0; m < M; ++m) {
                acc[i][m] = dot4(a0, a[m][4 * t], acc[i][m]);
                acc[i][m] = dot4(a1, a[m][4 * t + 1], acc[i][m]);
                acc[i][m] = dot4(a2, a[m][4 * t + 2], acc[i][m]);
                acc[i][m] = dot4(a3, a[m][4 * t + 3], acc[i][m]);
            }
        }
}

// ------------------------------------------------------------------ one tile on the matrix cores
//
// The same products through v_mfma_i32_16x16x64_i8 (16 x 16 int32 outputs, a
// 64-deep int8 dot each).  Lane l supplies bytes b = 0..15 of k group
// (l >> 4) for row l & 15 of A and column l & 15 of B; the product pairs A and
// B bytes of the same lane group and byte, so any fixed map from (lane group,
// byte) to k serves, provided A and B use the same one.  Here the lane's k
// slice s = l >> 4 (32 k) is split into two halves h, one product each:
//   B column n = l & 15 is weight row 4n + i of the tile (one product set per i),
//   A row l & 15 is activation row m (rows >= M only feed unused outputs),
// and output lane l holds D[4 * (l >> 4) + j][l & 15]: lanes 0..15 hold
// activation rows j = 0..3 of weight row 4 * l + i.  Rows past M cost nothing
// extra: a 16-row product is one instruction whatever M is.

// The lane's unpacked weights (2^kAccShift * w) of one row set, k half h
// (k = 32s + 16h + 0..15, in order) as four int8x4 dwords.  A row set's bytes
// in a lane: W4 the four dwords of one slab; W6 six consecutive dwords of the
// lane's 24 (row set i: dwords 6i .. 6i + 5, a slab and a half).
__device__ __forceinline__ v4i unpack_row_w4(v4i slab, int h) {
    const uint32_t d0 = (uint32_t)(h ? slab.z : slab.x), d1 = (uint32_t)(h ? slab.w : slab.y);
    return v4i{(int)((d0 << 4) & 0xF0F0F0F0u), (int)(d0 & 0xF0F0F0F0u), (int)((d1 << 4) & 0xF0F0F0F0u),
               (int)(d1 & 0xF0F0F0F0u)};
}
__device__ __forceinline__ v4i unpack_row_w6(uint32_t x0, uint32_t x1, uint32_t x2) {
    const uint32_t m6 = 0xFCFCFCFCu;
    return v4i{(int)(x0 & m6), (int)(x1 & m6), (int)(x2 & m6),
               (int)(((x0 << 6) & 0xC0C0C0C0u) | ((x1 << 4) & 0x30303030u) | ((x2 << 2) & 0x0C0C0C0Cu))};
}
// The same for row i of a whole tile held in registers.
template <int BITS>
__device__ __forceinline__ v4i unpack_half(const v4i (&w)[Layout<BITS>::kSlabs], int i, int h) {
    if constexpr (BITS == 4) {
        return unpack_row_w4(w[i], h);
    } else {
        uint32_t wd[24];
#pragma unroll
        for (int j = 0; j < 6; ++j) {
            wd[4 * j + 0] = (uint32_t)w[j].x;
            wd[4 * j + 1] = (uint32_t)w[j].y;
            wd[4 * j + 2] = (uint32_t)w[j].z;
            wd[4 * j + 3] = (uint32_t)w[j].w;
        }
        return unpack_row_w6(wd[6 * i + 3 * h], wd[6 * i + 3 * h + 1], wd[6 * i + 3 * h + 2]);
    }
}

// acc[i][j] = group sum (2^kAccShift * w times q, exact int32) of weight
// row 4 * (lane & 15) + i of the tile against activation row 4 * (lane >> 4)
// + j; a0 / a1 are the lane's two 16-byte halves of its 32-k activation slice
// (row lane & 15 of the group's k slice lane >> 4).  This is the one
// matrix-core implementation: the per-op linear, the fused walk and the
// group-sum test entry point all call it.
// The two products of one row set (its unpacked k halves h0, h1).
__device__ __forceinline__ v4i mfma_rowset(v4i a0, v4i a1, v4i h0, v4i h1) {
    const v4i z = {0, 0, 0, 0};
    const v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, h0, z, 0, 0, 0);
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, h1, acc, 0, 0, 0);
}
template <int BITS>
__device__ __forceinline__ void mfma_tile_regs(const v4i (&w)[Layout<BITS>::kSlabs], v4i a0, v4i a1,
                                               v4i (&acc)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = mfma_rowset(a0, a1, unpack_half<BITS>(w, i, 0), unpack_half<BITS>(w, i, 1));
}
// The same with the lane's activation slice read from memory at qa.
template <int BITS>
__device__ __forceinline__ void mfma_tile(const v4i (&w)[Layout<BITS>::kSlabs], const int8_t *qa, v4i (&acc)[4]) {
    mfma_tile_regs<BITS>(w, *reinterpret_cast<const v4i *>(qa), *reinterpret_cast<const v4i *>(qa + 16), acc);
}

template <int BITS, int M, typename Act>
__device__ __forceinline__ void dot_tile(const v4i (&w)[Layout<BITS>::kSlabs], Act act, int (&acc)[4][M]) {
    if constexpr (BITS == 4)
        dot_tile_w4<M>(w, act, acc);
    else
        dot_tile_w6<M>(w, act, acc);
}

// The lane's slabs and its four rows' fp16 scales (packed in two dwords).
template <int BITS>
__device__ __forceinline__ void load_tile(const uint8_t *tile, int lane, v4i (&w)[Layout<BITS>::kSlabs],
                                          v2u &scales) {
#pragma unroll
    for (int j = 0; j < Layout<BITS>::kSlabs; ++j)
        w[j] = load_stream(reinterpret_cast<const v4i *>(tile + j * kSlab) + lane);
    scales = __builtin_nontemporal_load(
        gptr(reinterpret_cast<const v2u *>(tile + Layout<BITS>::kWeightBytes) + (lane & 15)));
}

// fp32 scale of row i (0..3) of the lane from its packed scales.
__device__ __forceinline__ float row_scale(v2u s, int i) {
    const uint32_t word = i < 2 ? s.x : s.y;
    return f16_bits_to_f32((word >> (16 * (i & 1))) & 0xFFFFu);
}

// Sum a per-lane value over the four k slices (lanes l, l^16, l^32, l^48) in a
// fixed order; every lane of the group gets the same total.
// ------------------------------------------------------------------ cross-lane reductions
//
// DPP moves and gfx950's lane-swap instructions run on the vector ALU; the
// generic shuffles go through the LDS crossbar and cost a round trip each.

// dst = src of the lane picked by the DPP control; lanes of rows outside
// ROW_MASK (and lanes with no source) read 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float v) {
    return __uint_as_float(dpp_u32<CTRL, ROW_MASK>(__float_as_uint(v)));
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint64_t lo = dpp_u32<CTRL, ROW_MASK>((uint32_t)b), hi = dpp_u32<CTRL, ROW_MASK>((uint32_t)(b >> 32));
    return __longlong_as_double((long long)(lo | (hi << 32)));
}
constexpr int kDppQuadSwap1 = 0xB1;    // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuadSwap2 = 0x4E;    // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppHalfMirror = 0x141;  // lane 7 - i within 8
constexpr int kDppMirror = 0x140;      // lane 15 - i within 16
constexpr int kDppBcast15 = 0x142;     // lane 15 of a row into the next row
constexpr int kDppBcast31 = 0x143;     // lane 31 into rows 2 and 3

// Sum (or max of non-negative values) over the wave, in a fixed tree order;
// the result is valid in lane 63.
template <int CTRL, int ROW_MASK = 0xF, typename T>
__device__ __forceinline__ T dpp_any(T v) {
    if constexpr (sizeof(T) == 8) return dpp_f64<CTRL, ROW_MASK>(v);
    else return dpp_f32<CTRL, ROW_MASK>(v);
}
template <typename T>
__device__ __forceinline__ T wave_sum63(T v) {
    v += dpp_any<kDppQuadSwap1>(v);
    v += dpp_any<kDppQuadSwap2>(v);
    v += dpp_any<kDppHalfMirror>(v);
    v += dpp_any<kDppMirror>(v);
    v += dpp_any<kDppBcast15, 0xA>(v);
    v += dpp_any<kDppBcast31, 0xC>(v);
    return v;
}
__device__ __forceinline__ float wave_max63(float v) {   // v >= 0
    v = fmaxf(v, dpp_f32<kDppQuadSwap1>(v));
    v = fmaxf(v, dpp_f32<kDppQuadSwap2>(v));
    v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f32<kDppMirror>(v));
    v = fmaxf(v, dpp_f32<kDppBcast15, 0xA>(v));
    v = fmaxf(v, dpp_f32<kDppBcast31, 0xC>(v));
    return v;
}

// Pairwise reduce-scatter across the two halves (lanes l, l ^ 32) or across
// row pairs (l, l ^ 16): the lower (even) lanes return a + its partner's a,
// the upper (odd) lanes b + its partner's b.
__device__ __forceinline__ uint32_t bits_of(float v) { return __float_as_uint(v); }
__device__ __forceinline__ uint32_t bits_of(int v) { return (uint32_t)v; }
__device__ __forceinline__ float from_bits(uint32_t b, float) { return __uint_as_float(b); }
__device__ __forceinline__ int from_bits(uint32_t b, int) { return (int)b; }
template <typename T>
__device__ __forceinline__ T swap32_sum(T a, T b) {
    const auto r = __builtin_amdgcn_permlane32_swap(bits_of(a), bits_of(b), false, false);
    return from_bits(r[0], T()) + from_bits(r[1], T());
}
template <typename T>
__device__ __forceinline__ T swap16_sum(T a, T b) {
    const auto r = __builtin_amdgcn_permlane16_swap(bits_of(a), bits_of(b), false, false);
    return from_bits(r[0], T()) + from_bits(r[1], T());
}

// Sum a tile's per-lane row partials f[i] (row 4*(l % 16) + i of lane l, one
// k slice s = l / 16 per lane) over the four k slices.  Lane l returns the
// total of row slice_row(l) = 4*(l % 16) + l / 16.
template <typename T>
__device__ __forceinline__ T slice_reduce(const T (&f)[4]) {
    const T g0 = swap32_sum(f[0], f[2]);   // lanes 0-31: row 0, lanes 32-63: row 2
    const T g1 = swap32_sum(f[1], f[3]);   // rows 1 / 3
    return swap16_sum(g0, g1);             // even 16-lane rows keep g0, odd keep g1
}
__device__ __forceinline__ int slice_row(int lane) { return 4 * (lane & 15) + (lane >> 4); }

// The v_dot4 form of a tile's group sums: lane l ends with gs[m] = the exact
// int32 group sum (2^kAccShift * w times q over the group's 128 k) of weight
// row slice_row(l) against activation row m.  The four k slices' sums are
// added in int32 before any scaling, so the value is the same exact integer
// the matrix-core form produces.
template <int BITS, int M, typename Act>
__device__ __forceinline__ void group_sums_dot(const v4i (&w)[Layout<BITS>::kSlabs], Act act, int (&gs)[M]) {
    int acc[4][M];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[i][m] = 0;
    dot_tile<BITS, M>(w, act, acc);
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int f[4] = {acc[0][m], acc[1][m], acc[2][m], acc[3][m]};
        gs[m] = slice_reduce(f);
    }
}

}  // namespace mbq
