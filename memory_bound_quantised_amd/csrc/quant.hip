// Per-row int8 activation quantisation, optionally preceded by the prologue it
// absorbs ("Optimizing the Linear Kernel": the quantisation absorbs the
// RMSNorm or SwiGLU that precedes it).  One block of 256 threads per row; the
// arithmetic is quant_row (quant_rows.h), shared with the linear that runs
// the prologue itself.
#include "quant_rows.h"
#include "mbq_kernels.h"

namespace mbq {

namespace {

constexpr int kThreads = 256;

template <int PRO>
__global__ __launch_bounds__(kThreads) void prologue_quant_kernel(const uint16_t *__restrict__ x, int64_t x_stride,
                                                                  const uint16_t *__restrict__ u, int64_t u_stride,
                                                                  const uint16_t *__restrict__ w,
                                                                  uint16_t *__restrict__ h, int64_t K,
                                                                  int8_t *__restrict__ q, float *__restrict__ s) {
    __shared__ double red_d[kThreads / 64];
    __shared__ float red_f[kThreads / 64];
    const int64_t m = blockIdx.x;
    const uint16_t *xr = x + m * x_stride;
    const uint16_t *ur = u ? u + m * u_stride : nullptr;
    const auto put = [&](int64_t c, uint32_t lo, uint32_t hi) {
        *reinterpret_cast<uint2 *>(q + m * K + 8 * c) = make_uint2(lo, hi);
    };
    const auto put_h = [&](int64_t c, const float (&t)[8]) {
        uint32_t hp[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hp[i] = f32_to_bf16_bits(t[2 * i]) | (f32_to_bf16_bits(t[2 * i + 1]) << 16);
        *reinterpret_cast<uint4 *>(h + m * K + 8 * c) = make_uint4(hp[0], hp[1], hp[2], hp[3]);
    };
    float sc;
    if (PRO == MBQ_PRO_SWIGLU_QUANT && h)
        sc = quant_row<PRO, kThreads, true>(xr, ur, w, K, red_d, red_f, put, put_h);
    else
        sc = quant_row<PRO, kThreads, false>(xr, ur, w, K, red_d, red_f, put, put_h);
    if (threadIdx.x == 0) s[m] = sc;
}

}  // namespace

hipError_t launch_prologue_quant(int pro, int64_t M, int64_t K, const void *x, int64_t x_stride,
                                 const void *u, int64_t u_stride, const void *w, void *h, int8_t *q,
                                 float *s, hipStream_t st) {
    const dim3 grid((unsigned)M), block(kThreads);
    const uint16_t *xs = (const uint16_t *)x, *us = (const uint16_t *)u, *ws = (const uint16_t *)w;
    uint16_t *hs = (uint16_t *)h;
    switch (pro) {
        case MBQ_PRO_RMSNORM_QUANT:
            prologue_quant_kernel<MBQ_PRO_RMSNORM_QUANT><<<grid, block, 0, st>>>(xs, x_stride, us, u_stride, ws, hs, K, q, s);
            break;
        case MBQ_PRO_WRMSNORM_QUANT:
            prologue_quant_kernel<MBQ_PRO_WRMSNORM_QUANT><<<grid, block, 0, st>>>(xs, x_stride, us, u_stride, ws, hs, K, q, s);
            break;
        case MBQ_PRO_SWIGLU_QUANT:
            prologue_quant_kernel<MBQ_PRO_SWIGLU_QUANT><<<grid, block, 0, st>>>(xs, x_stride, us, u_stride, ws, hs, K, q, s);
            break;
        default:
            prologue_quant_kernel<MBQ_PRO_QUANT><<<grid, block, 0, st>>>(xs, x_stride, us, u_stride, ws, hs, K, q, s);
            break;
    }
    return hipGetLastError();
}

}  // namespace mbq
