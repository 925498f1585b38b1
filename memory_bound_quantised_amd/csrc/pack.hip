// Weight re-layout: canonical (checkpoint-order) codes + fp16 group scales <->
// the kernel-order tiles described in mbq_internal.h.  Runs once per matrix at
// load time ("Optimizing the Linear Kernel": the re-layout is done once per
// model load).  One block per tile; every thread moves 16 B (W4) or 12 B (W6).
#include "mbq_internal.h"
#include "mbq_kernels.h"

namespace mbq {

namespace {

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
    if (n < N) {
        const int4 c = *reinterpret_cast<const int4 *>(canon + n * (K / 2) + g * 64 + (l >> 4) * 16);
        const uint32_t cw[4] = {(uint32_t)c.x, (uint32_t)c.y, (uint32_t)c.z, (uint32_t)c.w};
        // canonical code e (0..31) = nibble (e & 1) of canonical byte e >> 1
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
    if (n < N) {
        const uint32_t *src = reinterpret_cast<const uint32_t *>(canon + n * (3 * K / 4) + koff);
        const uint32_t b0 = src[0], b1 = src[1], b2 = src[2];
        // 24-bit little-endian words p = 0..3 of the 12 bytes, 4 codes each
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

}  // namespace mbq
