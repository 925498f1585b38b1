// HBM stream-read ceiling: the rate at which this GPU delivers a plain
// sequential read of device memory, the reference the weight stream's own
// rate is judged against ("What is the bottleneck?" on the page "Doubling LLM
// token rates in ComfyUI": decode speed is set by how fast the GPU reads the
// model from VRAM).
//
// Two workgroups of four waves per CU; each wave reads one contiguous range of
// whole 1 KiB chunks (one non-temporal 16-byte load per lane, the same load
// the weight stream uses) with two batches of kBatch chunks in flight, and
// folds what it read into a digest so the loads cannot be dropped.
#include "mbq_internal.h"
#include "mbq_kernels.h"

namespace mbq {

namespace {

constexpr int kBatch = 8;

__global__ __launch_bounds__(256) void stream_read_kernel(const v4i *__restrict__ buf, int64_t chunks,
                                                          uint32_t *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nw = (int64_t)gridDim.x * 4;
    const int64_t c1 = chunks * (w + 1) / nw;
    int64_t c = chunks * w / nw;
    v4i acc = {0, 0, 0, 0};
    if (c + kBatch <= c1) {
        v4i a[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) a[u] = load_stream(buf + (c + u) * 64 + lane);
        for (; c + 2 * kBatch <= c1; c += kBatch) {
            v4i b[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) b[u] = load_stream(buf + (c + kBatch + u) * 64 + lane);
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                acc ^= a[u];
                a[u] = b[u];
            }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) acc ^= a[u];
        c += kBatch;
    }
    for (; c < c1; ++c) acc ^= load_stream(buf + c * 64 + lane);
    const uint32_t d = (uint32_t)(acc.x ^ acc.y ^ acc.z ^ acc.w);
    // one store per wave, only when the digest has one particular value: the
    // loads stay live and the store traffic is nil
    if (d == 0x9E3779B9u) *gptr(sink) = d;
}

}  // namespace

hipError_t launch_stream_read(const void *buf, int64_t bytes, uint32_t *sink, int n_cu, hipStream_t st) {
    stream_read_kernel<<<dim3((unsigned)(2 * n_cu)), dim3(256), 0, st>>>((const v4i *)buf, bytes / kSlab, sink);
    return hipGetLastError();
}

}  // namespace mbq
