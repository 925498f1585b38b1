// The skinny linear for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc): the same
// kernels as mbq_w4a8_linear / mbq_w6a8_linear, with the split-K counters and
// fp32 partials in a file-scope device array instead of a caller workspace.
//
// The array lives in the library's code object, so each GPU the library runs
// on holds its own copy until the process ends.  Host code never passes the
// array's name to a kernel (in host code it is only a stand-in symbol): at the
// first call on a device, with that device current, its address is looked up
// with hipGetSymbolAddress and kept per device, and its counter region is
// zeroed by a fill kernel on the caller's stream.  The linear kernel leaves
// every counter it uses at zero again when it completes, so later calls need
// no clearing.  All calls on one GPU share the array: calls that overlap in
// time on one GPU (different streams, not synchronised) race.
#include <mutex>

#include "../../include/mbq.h"
#include "mbq_internal.h"
#include "mbq_kernels.h"

namespace mbq {

namespace {

// Counters (64 KiB) plus the partials of the largest split-K plan: plan_linear
// keeps (row blocks x splits) below 4096 (a split only where the matrix has
// fewer than 2048 row blocks, at most ceil(2048 / row blocks) of them), each
// holding M x 64 floats, M <= 8.
constexpr int64_t kScratchBytes = kCounterBytes + (int64_t)4096 * kMaxM * 64 * 4;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ void zero_words(uint32_t *p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void *g_scratch[kMaxDevices];   // device address of `scratch` per device, once set up

// Device address of this device's array, setting it up on first use (with
// `dev` current): symbol lookup, then the counter region zeroed on `st`.
hipError_t scratch_of(int dev, hipStream_t st, void **out) {
    std::lock_guard<std::mutex> g(g_lock);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        zero_words<<<64, 256, 0, st>>>((uint32_t *)ptr, kCounterBytes / 4);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

int64_t noalloc_scratch_bytes() { return kScratchBytes; }

// Status or MBQ_OK; *hip_err receives the failing HIP call's error.
int linear_noalloc(int bits, int64_t M, int64_t N, int64_t K, const int8_t *q, const float *s,
                   const void *packed, void *y, hipStream_t st, hipError_t *hip_err) {
    const LinearPlan plan = plan_linear(bits, M, N, K);
    if (plan.ws_bytes > kScratchBytes) return MBQ_ERR_WORKSPACE;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) return MBQ_ERR_DEVICE;
    void *ws = nullptr;
    if (e == hipSuccess) e = scratch_of(dev, st, &ws);
    if (e == hipSuccess) e = launch_linear(bits, M, N, K, q, s, packed, y, N, ws, plan, st);
    if (e != hipSuccess) {
        *hip_err = e;
        return MBQ_ERR_HIP;
    }
    return MBQ_OK;
}

}  // namespace mbq
