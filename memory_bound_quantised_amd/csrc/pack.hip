// Weight re-layout: canonical (checkpoint-order) codes + fp16 group scales <->
// the kernel-order tiles described in mbq_internal.h.  Runs once per matrix at
// load time ("Optimizing the Linear Kernel": the re-layout is done once per
// model load).  One block per tile; every thread moves 16 B (W4) or 12 B (W6).
#include <string.h>

#include <algorithm>
#include <mutex>

#include "mbq.h"
#include "mbq_internal.h"
#include "mbq_kernels.h"

namespace mbq {

namespace {

// W4: the 32 canonical codes at src (16 bytes: code e is nibble e & 1 of
// byte e >> 1) as one 16-byte lane chunk of slab order.
__device__ __forceinline__ void w4_chunk(const uint8_t *src, uint32_t (&out)[4]) {
    const int4 c = *reinterpret_cast<const int4 *>(src);
    const uint32_t cw[4] = {(uint32_t)c.x, (uint32_t)c.y, (uint32_t)c.z, (uint32_t)c.w};
    auto nib = [&](int e) -> uint32_t { return (cw[e >> 3] >> (4 * (e & 7))) & 0xFu; };
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t d = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b)
            d |= (nib(8 * i + b) | (nib(8 * i + 4 + b) << 4)) << (8 * b);
        out[i] = d;
    }
}

// W4: thread (slab i, lane l) turns the 32 canonical codes of row
// rb*64 + 4*(l & 15) + i, k = g*128 + 32*(l >> 4) .. +31 (16 canonical bytes)
// into one 16-byte lane chunk.
__global__ __launch_bounds__(256) void pack_w4_kernel(const uint8_t *__restrict__ canon,
                                                      const uint16_t *__restrict__ scales,
                                                      uint8_t *__restrict__ packed, int64_t N,
                                                      int64_t K) {
    const int64_t G = K / kGroup;
    const int64_t tile = blockIdx.x;
    const int64_t rb = tile / G, g = tile % G;
    const int j = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int64_t n = rb * kRows + 4 * (l & 15) + j;
    uint8_t *t = packed + tile * Layout<4>::kTileBytes;
    uint32_t out[4] = {0, 0, 0, 0};
    if (n < N) w4_chunk(canon + n * (K / 2) + g * 64 + (l >> 4) * 16, out);
    reinterpret_cast<int4 *>(t + j * kSlab)[l] = make_int4((int)out[0], (int)out[1], (int)out[2], (int)out[3]);
    if (j == 0) {
        const int64_t r = rb * kRows + l;
        reinterpret_cast<uint16_t *>(t + Layout<4>::kWeightBytes)[l] = r < N ? scales[r * G + g] : 0;
    }
}

__global__ __launch_bounds__(256) void unpack_w4_kernel(const uint8_t *__restrict__ packed,
                                                        uint8_t *__restrict__ canon,
                                                        uint16_t *__restrict__ scales, int64_t N,
                                                        int64_t K) {
    const int64_t G = K / kGroup;
    const int64_t tile = blockIdx.x;
    const int64_t rb = tile / G, g = tile % G;
    const int j = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int64_t n = rb * kRows + 4 * (l & 15) + j;
    const uint8_t *t = packed + tile * Layout<4>::kTileBytes;
    if (j == 0 && rb * kRows + l < N)
        scales[(rb * kRows + l) * G + g] = reinterpret_cast<const uint16_t *>(t + Layout<4>::kWeightBytes)[l];
    if (n >= N) return;
    const int4 p = reinterpret_cast<const int4 *>(t + j * kSlab)[l];
    const uint32_t pw[4] = {(uint32_t)p.x, (uint32_t)p.y, (uint32_t)p.z, (uint32_t)p.w};
    uint32_t cw[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t byte = (pw[i] >> (8 * b)) & 0xFFu;
            const int e_lo = 8 * i + b, e_hi = 8 * i + 4 + b;
            cw[e_lo >> 3] |= (byte & 0xFu) << (4 * (e_lo & 7));
            cw[e_hi >> 3] |= (byte >> 4) << (4 * (e_hi & 7));
        }
    *reinterpret_cast<int4 *>(canon + n * (K / 2) + g * 64 + (l >> 4) * 16) =
        make_int4((int)cw[0], (int)cw[1], (int)cw[2], (int)cw[3]);
}

// W6: thread (triple q, lane l) turns the 16 canonical codes of row
// rb*64 + 4*(l & 15) + q/2, k = g*128 + 32*(l >> 4) + 16*(q & 1) .. +15
// (12 canonical bytes) into lane dwords 3q..3q+2.
__device__ __forceinline__ uint32_t *w6_lane_dword(uint8_t *tile, int l, int D) {
    return reinterpret_cast<uint32_t *>(tile + (D >> 2) * kSlab + l * 16 + (D & 3) * 4);
}

// W6: the 16 canonical codes at src (12 bytes, four little-endian 24-bit
// words of four codes) as the lane's dwords 3q..3q+2 of slab order.
__device__ __forceinline__ void w6_chunk(const uint8_t *src, uint32_t (&d)[3]) {
    const uint32_t *s32 = reinterpret_cast<const uint32_t *>(src);
    const uint32_t b0 = s32[0], b1 = s32[1], b2 = s32[2];
    const uint32_t w24[4] = {b0 & 0xFFFFFFu, (b0 >> 24) | ((b1 & 0xFFFFu) << 8),
                             (b1 >> 16) | ((b2 & 0xFFu) << 16), b2 >> 8};
    auto code = [&](int e) -> uint32_t { return (w24[e >> 2] >> (6 * (e & 3))) & 0x3Fu; };
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b)
            v |= ((code(4 * c + b) << 2) | ((code(12 + b) >> (4 - 2 * c)) & 3u)) << (8 * b);
        d[c] = v;
    }
}

__global__ __launch_bounds__(512) void pack_w6_kernel(const uint8_t *__restrict__ canon,
                                                      const uint16_t *__restrict__ scales,
                                                      uint8_t *__restrict__ packed, int64_t N,
                                                      int64_t K) {
    const int64_t G = K / kGroup;
    const int64_t tile = blockIdx.x;
    const int64_t rb = tile / G, g = tile % G;
    const int t = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int64_t n = rb * kRows + 4 * (l & 15) + (t >> 1);
    const int64_t koff = g * 96 + (l >> 4) * 24 + (t & 1) * 12;   // canonical byte offset in the row
    uint8_t *tp = packed + tile * Layout<6>::kTileBytes;
    uint32_t d[3] = {0, 0, 0};
    if (n < N) w6_chunk(canon + n * (3 * K / 4) + koff, d);
#pragma unroll
    for (int c = 0; c < 3; ++c) *w6_lane_dword(tp, l, 3 * t + c) = d[c];
    if (t == 0) {
        const int64_t r = rb * kRows + l;
        reinterpret_cast<uint16_t *>(tp + Layout<6>::kWeightBytes)[l] = r < N ? scales[r * G + g] : 0;
    }
}

__global__ __launch_bounds__(512) void unpack_w6_kernel(const uint8_t *__restrict__ packed,
                                                        uint8_t *__restrict__ canon,
                                                        uint16_t *__restrict__ scales, int64_t N,
                                                        int64_t K) {
    const int64_t G = K / kGroup;
    const int64_t tile = blockIdx.x;
    const int64_t rb = tile / G, g = tile % G;
    const int t = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int64_t n = rb * kRows + 4 * (l & 15) + (t >> 1);
    const int64_t koff = g * 96 + (l >> 4) * 24 + (t & 1) * 12;
    uint8_t *tp = const_cast<uint8_t *>(packed + tile * Layout<6>::kTileBytes);
    if (t == 0 && rb * kRows + l < N)
        scales[(rb * kRows + l) * G + g] = reinterpret_cast<const uint16_t *>(tp + Layout<6>::kWeightBytes)[l];
    if (n >= N) return;
    const uint32_t d[3] = {*w6_lane_dword(tp, l, 3 * t), *w6_lane_dword(tp, l, 3 * t + 1),
                           *w6_lane_dword(tp, l, 3 * t + 2)};
    uint32_t code[16];
#pragma unroll
    for (int c = 0; c < 3; ++c)
#pragma unroll
        for (int b = 0; b < 4; ++b) code[4 * c + b] = (d[c] >> (8 * b + 2)) & 0x3Fu;
#pragma unroll
    for (int b = 0; b < 4; ++b)
        code[12 + b] = (((d[0] >> (8 * b)) & 3u) << 4) | (((d[1] >> (8 * b)) & 3u) << 2) |
                       ((d[2] >> (8 * b)) & 3u);
    uint32_t w24[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
        w24[p] = code[4 * p] | (code[4 * p + 1] << 6) | (code[4 * p + 2] << 12) | (code[4 * p + 3] << 18);
    uint32_t *dst = reinterpret_cast<uint32_t *>(canon + n * (3 * K / 4) + koff);
    dst[0] = w24[0] | (w24[1] << 24);
    dst[1] = (w24[1] >> 8) | (w24[2] << 16);
    dst[2] = (w24[2] >> 16) | (w24[3] << 8);
}


// ---------------------------------------------------------------- in-place re-layout
//
// The re-layout done where the weights already are, with no second copy
// ("Optimizing the Linear Kernel": the kernel-order re-layout happens in
// place in VRAM, once per load, with no extra RAM or VRAM).  The buffer starts
// as the canonical codes of N rows followed by their fp16 scales, and ends as
// the packed tiles.  Three steps, each moving bytes only inside the buffer:
//   P  (N not a multiple of 64) make room for the padding rows: rotate
//      [scales | free tail] to [free | scales], then zero the pad rows of
//      codes and of scales;
//   A  interleave row blocks: [C_0 .. C_R-1][S_0 .. S_R-1] becomes
//      [C_0 S_0][C_1 S_1] .. by recursive halving, each level one block
//      rotation per interval, every rotation three in-place reversals;
//   B  each row block is now a closed region: a cooperative pass stages
//      whole row blocks' tiles in LDS (every workgroup reads the bytes of
//      the tiles it will write), waits at a grid barrier until every
//      workgroup has read, then writes the tiles in slab order.

__global__ __launch_bounds__(256) void reverse_u16_kernel(uint16_t *buf, int64_t start, int64_t n) {
    const int64_t half = n / 2;
    for (int64_t p = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; p < half; p += (int64_t)gridDim.x * blockDim.x) {
        uint16_t *a = buf + start + p, *b = buf + start + n - 1 - p;
        const uint16_t va = *gptr(a), vb = *gptr(b);
        *gptr(a) = vb;
        *gptr(b) = va;
    }
}

__global__ __launch_bounds__(256) void zero_bytes_kernel(uint8_t *buf, int64_t start, int64_t n) {
    for (int64_t p = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; p < n; p += (int64_t)gridDim.x * blockDim.x)
        *gptr(buf + start + p) = 0;
}

// One level of step A: block y reverses, for interval node y of the level,
// part `which` (0: the codes being moved, 1: the scales, 2: both) of its
// rotation region, in 16-byte elements.
__global__ __launch_bounds__(256) void interleave_level_kernel(v4i *buf, RelayoutGeom geo, int level, int which) {
    int64_t a, b;
    relayout_node(geo.R, level, blockIdx.y, a, b);
    if (b - a < 2) return;
    const int64_t m = (a + b) / 2;
    const int64_t base = (a * geo.T + (m - a) * geo.C) / 16;
    const int64_t nx = (b - m) * geo.C / 16, ny = (m - a) * geo.S / 16;
    const int64_t start = which == 1 ? base + nx : base;
    const int64_t n = which == 0 ? nx : which == 1 ? ny : nx + ny;
    const int64_t half = n / 2;
    for (int64_t p = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; p < half; p += (int64_t)gridDim.x * blockDim.x) {
        v4i *pa = buf + start + p, *pb = buf + start + n - 1 - p;
        const v4i va = *gptr(pa), vb = *gptr(pb);
        *gptr(pa) = vb;
        *gptr(pb) = va;
    }
}

// Grid-barrier word and error flag of step B (the only state the re-layout
// keeps; calls on one device must not overlap).
__device__ uint32_t g_relayout_sync[2];

constexpr int64_t kRelayoutSpinLimit = 1ll << 24;

// Step B.  A staged tile holds its 64 row pieces (the row's canonical bytes
// of the tile's group, pc bytes each) and then its 64 scales, as the
// canonical layout of a 64 x 128 matrix would; the slab order is made from
// it exactly as pack_w4/w6_kernel make it from the canonical tensors.
template <int BITS>
__global__ __launch_bounds__(256) void relayout_tiles_kernel(uint8_t *buf, RelayoutGeom geo, int per_wg,
                                                             int64_t rb_per_batch, uint32_t *sync) {
    extern __shared__ __align__(16) uint8_t raw[];
    constexpr int kTile = Layout<BITS>::kTileBytes;
    constexpr int kPc = BITS == 4 ? 64 : 96;   // canonical bytes of one row's group
    constexpr int kChunks = 64 * kPc / 16;     // 16-byte chunks of a tile's codes
    const int tid = threadIdx.x;
    const int grid = gridDim.x, wg = blockIdx.x;
    int64_t batch = 0;
    for (int64_t rb0 = 0; rb0 < geo.R; rb0 += rb_per_batch, ++batch) {
        const int64_t rb1 = rb0 + rb_per_batch < geo.R ? rb0 + rb_per_batch : geo.R;
        const int64_t t_lo = rb0 * geo.G + (int64_t)wg * per_wg;
        const int64_t t_end = rb1 * geo.G;
        const int n_my = t_lo >= t_end ? 0 : (int)(t_end - t_lo < per_wg ? t_end - t_lo : per_wg);
        for (int idx = tid; idx < n_my * kChunks; idx += 256) {
            const int k = idx / kChunks, c = idx % kChunks;
            const int64_t t = t_lo + k, rb = t / geo.G, g = t % geo.G;
            const int r = c / (kPc / 16), q = c % (kPc / 16);
            const v4i v = *gptr(reinterpret_cast<const v4i *>(buf + rb * geo.T + r * geo.Cr + g * kPc + q * 16));
            *reinterpret_cast<v4i *>(raw + k * kTile + r * kPc + q * 16) = v;
        }
        for (int idx = tid; idx < n_my * 64; idx += 256) {
            const int k = idx / 64, r = idx % 64;
            const int64_t t = t_lo + k, rb = t / geo.G, g = t % geo.G;
            *reinterpret_cast<uint16_t *>(raw + k * kTile + 64 * kPc + 2 * r) =
                *gptr(reinterpret_cast<const uint16_t *>(buf + rb * geo.T + geo.C + r * 2 * geo.G + 2 * g));
        }
        __syncthreads();
        // grid barrier: every workgroup has read what it will write over
        if (tid == 0) {
            counter_add(sync, 1u);
            const uint32_t want = (uint32_t)((batch + 1) * grid);
            int64_t spins = 0;
            while (load_shared(sync) < want) {
                if (++spins > kRelayoutSpinLimit) {
                    store_shared(sync + 1, 1u);
                    break;
                }
                __builtin_amdgcn_s_sleep(8);
            }
        }
        __syncthreads();
        for (int k = 0; k < n_my; ++k) {
            const uint8_t *src = raw + k * kTile;
            uint8_t *dst = buf + (t_lo + k) * kTile;
            if constexpr (BITS == 4) {
                const int j = tid >> 6, l = tid & 63;
                uint32_t out[4];
                w4_chunk(src + (4 * (l & 15) + j) * kPc + (l >> 4) * 16, out);
                *gptr(reinterpret_cast<v4i *>(dst + j * kSlab) + l) =
                    v4i{(int)out[0], (int)out[1], (int)out[2], (int)out[3]};
                if (j == 0)
                    *gptr(reinterpret_cast<uint16_t *>(dst + Layout<4>::kWeightBytes) + l) =
                        *reinterpret_cast<const uint16_t *>(src + 64 * kPc + 2 * l);
            } else {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int tt = tid + 256 * h, t = tt >> 6, l = tt & 63;
                    uint32_t d[3];
                    w6_chunk(src + (4 * (l & 15) + (t >> 1)) * kPc + (l >> 4) * 24 + (t & 1) * 12, d);
#pragma unroll
                    for (int c = 0; c < 3; ++c) *gptr(w6_lane_dword(dst, l, 3 * t + c)) = d[c];
                    if (t == 0)
                        *gptr(reinterpret_cast<uint16_t *>(dst + Layout<6>::kWeightBytes) + l) =
                            *reinterpret_cast<const uint16_t *>(src + 64 * kPc + 2 * l);
                }
            }
        }
        __syncthreads();   // the staging area is refilled by the next batch
    }
}

}  // namespace

hipError_t launch_pack(int bits, int64_t N, int64_t K, const void *canon, const void *scales,
                       void *packed, hipStream_t s) {
    const int64_t tiles = row_blocks(N) * (K / kGroup);
    if (bits == 4)
        pack_w4_kernel<<<dim3((unsigned)tiles), dim3(256), 0, s>>>(
            (const uint8_t *)canon, (const uint16_t *)scales, (uint8_t *)packed, N, K);
    else
        pack_w6_kernel<<<dim3((unsigned)tiles), dim3(512), 0, s>>>(
            (const uint8_t *)canon, (const uint16_t *)scales, (uint8_t *)packed, N, K);
    return hipGetLastError();
}

hipError_t launch_unpack(int bits, int64_t N, int64_t K, const void *packed, void *canon,
                         void *scales, hipStream_t s) {
    const int64_t tiles = row_blocks(N) * (K / kGroup);
    if (bits == 4)
        unpack_w4_kernel<<<dim3((unsigned)tiles), dim3(256), 0, s>>>(
            (const uint8_t *)packed, (uint8_t *)canon, (uint16_t *)scales, N, K);
    else
        unpack_w6_kernel<<<dim3((unsigned)tiles), dim3(512), 0, s>>>(
            (const uint8_t *)packed, (uint8_t *)canon, (uint16_t *)scales, N, K);
    return hipGetLastError();
}


// ---------------------------------------------------------------- in-place re-layout, host side

namespace {

// Reverse n 2-byte elements from `start` (host buffer).
void reverse_u16_host(uint16_t *b, int64_t start, int64_t n) {
    for (int64_t p = 0; p < n / 2; ++p) std::swap(b[start + p], b[start + n - 1 - p]);
}
void reverse_u128_host(uint8_t *buf, int64_t start, int64_t n) {   // 16-byte elements
    uint8_t tmp[16];
    for (int64_t p = 0; p < n / 2; ++p) {
        uint8_t *a = buf + 16 * (start + p), *b = buf + 16 * (start + n - 1 - p);
        memcpy(tmp, a, 16);
        memcpy(a, b, 16);
        memcpy(b, tmp, 16);
    }
}

int relayout_levels(int64_t R) {
    int L = 0;
    while (((int64_t)1 << L) < R) ++L;
    return L;
}

// Every rotation of step A lies inside the buffer (the kernels do not check).
bool relayout_schedule_ok(const RelayoutGeom &g) {
    const int L = relayout_levels(g.R);
    for (int l = 0; l < L; ++l)
        for (int64_t i = 0; i < ((int64_t)1 << l); ++i) {
            int64_t a, b;
            relayout_node(g.R, l, i, a, b);
            if (a < 0 || b > g.R || a > b) return false;
            if (b - a < 2) continue;
            const int64_t m = (a + b) / 2;
            const int64_t base = a * g.T + (m - a) * g.C, len = (b - m) * g.C + (m - a) * g.S;
            if (base < 0 || base + len > g.packed_bytes || base % 16 || len % 16) return false;
        }
    return true;
}

uint32_t *relayout_sync_ptr(int dev) {
    static std::mutex mu;
    static uint32_t *ptr[64] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (dev < 0 || dev >= 64) return nullptr;
    if (!ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_relayout_sync)) != hipSuccess) return nullptr;
        ptr[dev] = (uint32_t *)p;
    }
    return ptr[dev];
}

}  // namespace

int relayout_interleave_host(int bits, int64_t N, int64_t K, uint8_t *buf) {
    const RelayoutGeom g = relayout_geom(bits, N, K);
    if (!relayout_schedule_ok(g)) return MBQ_ERR_SHAPE;
    if (g.Np > N) {   // step P
        const int64_t x = N * 2 * g.G, y = (g.Np - N) * g.Cr, st = N * g.Cr;
        uint16_t *b16 = reinterpret_cast<uint16_t *>(buf);
        reverse_u16_host(b16, st / 2, x / 2);
        reverse_u16_host(b16, (st + x) / 2, y / 2);
        reverse_u16_host(b16, st / 2, (x + y) / 2);
        memset(buf + N * g.Cr, 0, (g.Np - N) * g.Cr);
        memset(buf + g.Np * g.Cr + N * 2 * g.G, 0, (g.Np - N) * 2 * g.G);
    }
    for (int l = 0; l < relayout_levels(g.R); ++l)   // step A
        for (int64_t i = 0; i < ((int64_t)1 << l); ++i) {
            int64_t a, b;
            relayout_node(g.R, l, i, a, b);
            if (b - a < 2) continue;
            const int64_t m = (a + b) / 2;
            const int64_t base = (a * g.T + (m - a) * g.C) / 16, nx = (b - m) * g.C / 16, ny = (m - a) * g.S / 16;
            reverse_u128_host(buf, base, nx);
            reverse_u128_host(buf, base + nx, ny);
            reverse_u128_host(buf, base, nx + ny);
        }
    return MBQ_OK;
}

int relayout_inplace(int bits, int64_t N, int64_t K, void *buf, int n_cu, hipStream_t s, hipError_t *hip_err) {
    auto hip_fail = [&](hipError_t e) {
        *hip_err = e;
        return MBQ_ERR_HIP;
    };
    const RelayoutGeom g = relayout_geom(bits, N, K);
    if (!relayout_schedule_ok(g)) return MBQ_ERR_SHAPE;
    const int tile = bits == 4 ? Layout<4>::kTileBytes : Layout<6>::kTileBytes;
    const int per_wg = (int)(151552 / tile);
    const int64_t rb_per_batch = (int64_t)n_cu * per_wg / g.G;
    if (rb_per_batch < 1) return MBQ_ERR_SHAPE;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    uint32_t *sync = relayout_sync_ptr(dev);
    if (!sync) return hip_fail(hipErrorInvalidSymbol);
    uint8_t *b = static_cast<uint8_t *>(buf);
    auto blocks = [](int64_t work) { return (unsigned)std::min<int64_t>(std::max<int64_t>((work + 255) / 256, 1), 4096); };
    if (g.Np > N) {   // step P
        const int64_t x = N * 2 * g.G, y = (g.Np - N) * g.Cr, st = N * g.Cr;
        uint16_t *b16 = reinterpret_cast<uint16_t *>(b);
        reverse_u16_kernel<<<blocks(x / 4), 256, 0, s>>>(b16, st / 2, x / 2);
        reverse_u16_kernel<<<blocks(y / 4), 256, 0, s>>>(b16, (st + x) / 2, y / 2);
        reverse_u16_kernel<<<blocks((x + y) / 4), 256, 0, s>>>(b16, st / 2, (x + y) / 2);
        zero_bytes_kernel<<<blocks((g.Np - N) * g.Cr), 256, 0, s>>>(b, N * g.Cr, (g.Np - N) * g.Cr);
        zero_bytes_kernel<<<blocks((g.Np - N) * 2 * g.G), 256, 0, s>>>(b, g.Np * g.Cr + N * 2 * g.G,
                                                                         (g.Np - N) * 2 * g.G);
        if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e);
    }
    for (int l = 0; l < relayout_levels(g.R); ++l) {   // step A
        const unsigned nodes = 1u << l;
        const unsigned bx = std::max(1u, std::min(256u, (unsigned)((g.R * g.T / 16 / nodes + 511) / 512)));
        for (int which = 0; which < 3; ++which)
            interleave_level_kernel<<<dim3(bx, nodes), 256, 0, s>>>(reinterpret_cast<v4i *>(b), g, l, which);
        if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e);
    }
    // step B
    if ((e = hipMemsetAsync(sync, 0, 2 * sizeof(uint32_t), s)) != hipSuccess) return hip_fail(e);
    void *args[] = {(void *)&b, (void *)&g, (void *)&per_wg, (void *)&rb_per_batch, (void *)&sync};
    const void *fn = bits == 4 ? reinterpret_cast<const void *>(&relayout_tiles_kernel<4>)
                               : reinterpret_cast<const void *>(&relayout_tiles_kernel<6>);
    e = hipLaunchCooperativeKernel(fn, dim3(n_cu), dim3(256), args, (unsigned)(per_wg * tile), s);
    if (e != hipSuccess) return hip_fail(e);
    uint32_t flags[2] = {0, 0};
    if ((e = hipMemcpyAsync(flags, sync, sizeof(flags), hipMemcpyDeviceToHost, s)) != hipSuccess) return hip_fail(e);
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e);
    return flags[1] ? MBQ_ERR_TIMEOUT : MBQ_OK;
}

}  // namespace mbq
