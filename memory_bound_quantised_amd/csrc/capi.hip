// C ABI of libmbq (declared in include/mbq.h): argument validation, workspace
// sizing and dispatch.  Every check runs before the first HIP call, so a call
// that returns an error has enqueued nothing.
#include <string.h>

#include <atomic>
#include <vector>

#include "../../include/mbq.h"
#include "mbq_internal.h"
#include "mbq_kernels.h"

using namespace mbq;

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
    g_last_hip_error = (int)e;
    return MBQ_ERR_HIP;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
bool bits_ok(int bits) { return bits == 4 || bits == 6; }
bool k_ok(int64_t K) { return K >= kGroup && K % kGroup == 0 && K <= (int64_t)1 << 24; }
bool n_ok(int64_t N) { return N >= 1 && N <= kMaxN; }
bool m_ok(int64_t M) { return M >= 1 && M <= kMaxM; }

// 0 = unknown, 1 = gfx950, -1 = other; cached per device ordinal.
std::atomic<int> g_dev_ok[64];

int check_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= 64) return MBQ_ERR_DEVICE;
    int st = g_dev_ok[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail(e);
        st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        g_dev_ok[dev].store(st, std::memory_order_relaxed);
    }
    return st == 1 ? MBQ_OK : MBQ_ERR_DEVICE;
}

int linear_common(int bits, int64_t M, int64_t N, int64_t K, const int8_t *q, const float *s,
                  const void *packed, void *y, void *ws, int64_t ws_bytes, void *stream) {
    if (!q || !s || !packed || !y) return MBQ_ERR_NULL;
    if (!m_ok(M) || !n_ok(N) || !k_ok(K)) return MBQ_ERR_SHAPE;
    if (!aligned(packed, 256) || !aligned(q, 16) || !aligned(s, 4) || !aligned(y, 16))
        return MBQ_ERR_ALIGN;
    const LinearPlan plan = plan_linear(bits, M, N, K);
    if (!ws || ws_bytes < plan.ws_bytes) return MBQ_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return MBQ_ERR_ALIGN;
    int st = check_device();
    if (st) return st;
    hipError_t e = launch_linear(bits, M, N, K, q, s, packed, y, N, ws, plan, (hipStream_t)stream);
    return e == hipSuccess ? MBQ_OK : hip_fail(e);
}

// ------------------------------------------------------------------ layer sequence

struct Phase {
    int32_t first, count;   // ops [first, first + count)
};

int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }

// Validates the op list and splits it into phases; returns the workspace size
// or a negative status.
int64_t analyse_program(const mbq_op *ops, int32_t n_ops, const int64_t *widths, int32_t n_bufs,
                        int64_t M, std::vector<Phase> *phases) {
    if (!ops || !widths) return MBQ_ERR_NULL;
    if (n_ops < 1 || n_bufs < 1) return MBQ_ERR_PROGRAM;
    if (!m_ok(M)) return MBQ_ERR_SHAPE;
    for (int32_t b = 0; b < n_bufs; ++b)
        if (widths[b] < 8 || widths[b] % 8 || widths[b] > kMaxN) return MBQ_ERR_PROGRAM;
    int64_t k_max = 0, lin_ws = 0;
    std::vector<Phase> ph;
    for (int32_t i = 0; i < n_ops; ++i) {
        const mbq_op &o = ops[i];
        if (!bits_ok(o.bits)) return MBQ_ERR_BITS;
        if (!o.packed) return MBQ_ERR_NULL;
        if (!aligned(o.packed, 256)) return MBQ_ERR_ALIGN;
        if (o.prologue < MBQ_PRO_QUANT || o.prologue > MBQ_PRO_SWIGLU_QUANT) return MBQ_ERR_PROGRAM;
        if (!k_ok(o.K) || !n_ok(o.N)) return MBQ_ERR_SHAPE;
        if (o.in_buf < 0 || o.in_buf >= n_bufs || o.out_buf < 0 || o.out_buf >= n_bufs)
            return MBQ_ERR_PROGRAM;
        if (o.out_buf == o.in_buf) return MBQ_ERR_PROGRAM;
        if (o.K > widths[o.in_buf] || o.N != widths[o.out_buf]) return MBQ_ERR_PROGRAM;
        const bool swiglu = o.prologue == MBQ_PRO_SWIGLU_QUANT, wnorm = o.prologue == MBQ_PRO_WRMSNORM_QUANT;
        if (swiglu && (o.in_buf2 < 0 || o.in_buf2 >= n_bufs || o.in_buf2 == o.out_buf ||
                       o.in_buf2 == o.in_buf || o.K > widths[o.in_buf2]))
            return MBQ_ERR_PROGRAM;
        if (wnorm && !o.norm_w) return MBQ_ERR_NULL;
        if (wnorm && !aligned(o.norm_w, 16)) return MBQ_ERR_ALIGN;
        const mbq_op &f = ops[ph.empty() ? i : ph.back().first];
        const bool joins = !ph.empty() && f.in_buf == o.in_buf && f.prologue == o.prologue && f.K == o.K &&
                           (!swiglu || f.in_buf2 == o.in_buf2) && (!wnorm || f.norm_w == o.norm_w);
        if (joins) {
            for (int32_t j = ph.back().first; j < i; ++j)
                if (ops[j].out_buf == o.out_buf) return MBQ_ERR_PROGRAM;
            ph.back().count++;
        } else {
            ph.push_back(Phase{i, 1});
        }
        if (o.K > k_max) k_max = o.K;
        const LinearPlan p = plan_linear(o.bits, M, o.N, o.K);
        if (p.ws_bytes > lin_ws) lin_ws = p.ws_bytes;
    }
    if (phases) *phases = ph;
    // [q int8 M x k_max][s fp32 x 4][linear workspace]
    return align256(M * k_max) + 256 + align256(lin_ws);
}

}  // namespace

extern "C" {

const char *mbq_status_string(int status) {
    switch (status) {
        case MBQ_OK: return "ok";
        case MBQ_ERR_NULL: return "null pointer";
        case MBQ_ERR_SHAPE: return "unsupported shape (M in 1..8, K multiple of 128, 1 <= N <= 2^20)";
        case MBQ_ERR_BITS: return "bits must be 4 or 6";
        case MBQ_ERR_ALIGN: return "misaligned pointer";
        case MBQ_ERR_WORKSPACE: return "workspace missing or too small";
        case MBQ_ERR_PROGRAM: return "malformed op list";
        case MBQ_ERR_HIP: return "HIP runtime error";
        case MBQ_ERR_DEVICE: return "current device is not gfx950";
        case MBQ_ERR_TIMEOUT: return "a wait inside the fused walk gave up";
        default: return "unknown status";
    }
}

int mbq_last_hip_error(void) { return g_last_hip_error; }

const char *mbq_version(void) { return "mbq 0.1 (gfx950)"; }

int64_t mbq_packed_bytes(int bits, int64_t N, int64_t K) {
    if (!bits_ok(bits)) return MBQ_ERR_BITS;
    if (!n_ok(N) || !k_ok(K)) return MBQ_ERR_SHAPE;
    return row_blocks(N) * (K / kGroup) * tile_bytes(bits);
}

int mbq_pack_weights(int bits, int64_t N, int64_t K, const void *w_canon, const void *scales_f16,
                     void *packed, void *stream) {
    if (!bits_ok(bits)) return MBQ_ERR_BITS;
    if (!w_canon || !scales_f16 || !packed) return MBQ_ERR_NULL;
    if (!n_ok(N) || !k_ok(K)) return MBQ_ERR_SHAPE;
    if (!aligned(w_canon, 16) || !aligned(scales_f16, 2) || !aligned(packed, 256)) return MBQ_ERR_ALIGN;
    int st = check_device();
    if (st) return st;
    hipError_t e = launch_pack(bits, N, K, w_canon, scales_f16, packed, (hipStream_t)stream);
    return e == hipSuccess ? MBQ_OK : hip_fail(e);
}

int mbq_unpack_weights(int bits, int64_t N, int64_t K, const void *packed, void *w_canon,
                       void *scales_f16, void *stream) {
    if (!bits_ok(bits)) return MBQ_ERR_BITS;
    if (!w_canon || !scales_f16 || !packed) return MBQ_ERR_NULL;
    if (!n_ok(N) || !k_ok(K)) return MBQ_ERR_SHAPE;
    if (!aligned(w_canon, 16) || !aligned(scales_f16, 2) || !aligned(packed, 256)) return MBQ_ERR_ALIGN;
    int st = check_device();
    if (st) return st;
    hipError_t e = launch_unpack(bits, N, K, packed, w_canon, scales_f16, (hipStream_t)stream);
    return e == hipSuccess ? MBQ_OK : hip_fail(e);
}

static int quant_common(int pro, int64_t M, int64_t K, const void *x, const void *u, const void *w, void *h,
                        int8_t *q, float *s, void *stream) {
    if (!x || !q || !s) return MBQ_ERR_NULL;
    if ((pro == MBQ_PRO_SWIGLU_QUANT && !u) || (pro == MBQ_PRO_WRMSNORM_QUANT && !w)) return MBQ_ERR_NULL;
    if (!m_ok(M) || !k_ok(K)) return MBQ_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4)) return MBQ_ERR_ALIGN;
    if ((u && !aligned(u, 16)) || (w && !aligned(w, 16)) || (h && !aligned(h, 16))) return MBQ_ERR_ALIGN;
    int st = check_device();
    if (st) return st;
    hipError_t e = launch_prologue_quant(pro, M, K, x, K, u, K, w, h, q, s, (hipStream_t)stream);
    return e == hipSuccess ? MBQ_OK : hip_fail(e);
}

int mbq_quantize_act(int64_t M, int64_t K, const void *x_bf16, int8_t *q, float *s, void *stream) {
    return quant_common(MBQ_PRO_QUANT, M, K, x_bf16, nullptr, nullptr, nullptr, q, s, stream);
}

int mbq_rmsnorm_quantize_act(int64_t M, int64_t K, const void *x_bf16, int8_t *q, float *s,
                             void *stream) {
    return quant_common(MBQ_PRO_RMSNORM_QUANT, M, K, x_bf16, nullptr, nullptr, nullptr, q, s, stream);
}

int mbq_wrmsnorm_quantize_act(int64_t M, int64_t K, const void *x_bf16, const void *w_bf16, int8_t *q,
                              float *s, void *stream) {
    return quant_common(MBQ_PRO_WRMSNORM_QUANT, M, K, x_bf16, nullptr, w_bf16, nullptr, q, s, stream);
}

int mbq_swiglu_quantize_act(int64_t M, int64_t K, const void *g_bf16, const void *u_bf16, void *h_bf16,
                            int8_t *q, float *s, void *stream) {
    return quant_common(MBQ_PRO_SWIGLU_QUANT, M, K, g_bf16, u_bf16, nullptr, h_bf16, q, s, stream);
}

int64_t mbq_linear_workspace_bytes(int bits, int64_t M, int64_t N, int64_t K) {
    if (!bits_ok(bits)) return MBQ_ERR_BITS;
    if (!m_ok(M) || !n_ok(N) || !k_ok(K)) return MBQ_ERR_SHAPE;
    return plan_linear(bits, M, N, K).ws_bytes;
}

int mbq_w4a8_linear(int64_t M, int64_t N, int64_t K, const int8_t *q, const float *s,
                    const void *packed, void *y_bf16, void *ws, int64_t ws_bytes, void *stream) {
    return linear_common(4, M, N, K, q, s, packed, y_bf16, ws, ws_bytes, stream);
}

int mbq_w6a8_linear(int64_t M, int64_t N, int64_t K, const int8_t *q, const float *s,
                    const void *packed, void *y_bf16, void *ws, int64_t ws_bytes, void *stream) {
    return linear_common(6, M, N, K, q, s, packed, y_bf16, ws, ws_bytes, stream);
}

int64_t mbq_linear_prologue_workspace_bytes(int bits, int64_t M, int64_t N, int64_t K) {
    if (!bits_ok(bits)) return MBQ_ERR_BITS;
    if (!m_ok(M) || !n_ok(N) || !k_ok(K)) return MBQ_ERR_SHAPE;
    return linear_prologue_ws_bytes(bits, M, N, K);
}

int mbq_linear_prologue(int bits, int prologue, int64_t M, int64_t N, int64_t K, const void *x_bf16,
                        const void *u_bf16, const void *w_bf16, const void *packed, void *y_bf16, void *ws,
                        int64_t ws_bytes, void *stream) {
    if (!bits_ok(bits)) return MBQ_ERR_BITS;
    if (prologue < MBQ_PRO_QUANT || prologue > MBQ_PRO_SWIGLU_QUANT) return MBQ_ERR_PROGRAM;
    if (!x_bf16 || !packed || !y_bf16) return MBQ_ERR_NULL;
    if (prologue == MBQ_PRO_SWIGLU_QUANT && !u_bf16) return MBQ_ERR_NULL;
    if (prologue == MBQ_PRO_WRMSNORM_QUANT && !w_bf16) return MBQ_ERR_NULL;
    if (!m_ok(M) || !n_ok(N) || !k_ok(K)) return MBQ_ERR_SHAPE;
    if (!aligned(packed, 256) || !aligned(x_bf16, 16) || !aligned(y_bf16, 16) ||
        (u_bf16 && !aligned(u_bf16, 16)) || (w_bf16 && !aligned(w_bf16, 16)))
        return MBQ_ERR_ALIGN;
    if (!ws || ws_bytes < linear_prologue_ws_bytes(bits, M, N, K)) return MBQ_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return MBQ_ERR_ALIGN;
    int st = check_device();
    if (st) return st;
    const void *u = prologue == MBQ_PRO_SWIGLU_QUANT ? u_bf16 : nullptr;
    const void *w = prologue == MBQ_PRO_WRMSNORM_QUANT ? w_bf16 : nullptr;
    hipError_t e = launch_linear_prologue(bits, prologue, M, N, K, x_bf16, u, w, packed, y_bf16, ws,
                                          (hipStream_t)stream);
    return e == hipSuccess ? MBQ_OK : hip_fail(e);
}

int mbq_linear_noalloc(int bits, int64_t M, int64_t N, int64_t K, const int8_t *q, const float *s,
                       const void *packed, void *y_bf16, void *stream) {
    if (!bits_ok(bits)) return MBQ_ERR_BITS;
    if (!q || !s || !packed || !y_bf16) return MBQ_ERR_NULL;
    if (!m_ok(M) || !n_ok(N) || !k_ok(K)) return MBQ_ERR_SHAPE;
    if (!aligned(packed, 256) || !aligned(q, 16) || !aligned(s, 4) || !aligned(y_bf16, 16)) return MBQ_ERR_ALIGN;
    if (plan_linear(bits, M, N, K).ws_bytes > noalloc_scratch_bytes()) return MBQ_ERR_WORKSPACE;
    int st = check_device();
    if (st) return st;
    hipError_t he = hipSuccess;
    st = linear_noalloc(bits, M, N, K, q, s, packed, y_bf16, (hipStream_t)stream, &he);
    return st == MBQ_ERR_HIP ? hip_fail(he) : st;
}

int mbq_linear_group_acc(int bits, int form, int64_t M, int64_t N, int64_t K, const int8_t *q,
                         const void *packed, int32_t *acc, void *stream) {
    if (!bits_ok(bits)) return MBQ_ERR_BITS;
    if (form != MBQ_FORM_DOT4 && form != MBQ_FORM_MFMA && form != MBQ_FORM_ROWSET) return MBQ_ERR_SHAPE;
    if (!q || !packed || !acc) return MBQ_ERR_NULL;
    if (!m_ok(M) || !n_ok(N) || !k_ok(K)) return MBQ_ERR_SHAPE;
    if (!aligned(packed, 256) || !aligned(q, 16) || !aligned(acc, 4)) return MBQ_ERR_ALIGN;
    int st = check_device();
    if (st) return st;
    hipError_t e = launch_group_acc(bits, form, M, N, K, q, packed, acc, (hipStream_t)stream);
    return e == hipSuccess ? MBQ_OK : hip_fail(e);
}

static int device_cus(int *n_cu) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    return e == hipSuccess ? MBQ_OK : hip_fail(e);
}

int mbq_stream_read(const void *buf, int64_t bytes, uint32_t *sink, void *stream) {
    if (!buf || !sink) return MBQ_ERR_NULL;
    if (bytes < kSlab || bytes % kSlab) return MBQ_ERR_SHAPE;
    if (!aligned(buf, 256) || !aligned(sink, 4)) return MBQ_ERR_ALIGN;
    int st = check_device();
    if (st) return st;
    int n_cu = 0;
    st = device_cus(&n_cu);
    if (st) return st;
    hipError_t e = launch_stream_read(buf, bytes, sink, n_cu, (hipStream_t)stream);
    return e == hipSuccess ? MBQ_OK : hip_fail(e);
}

int mbq_pack_weights_inplace(int bits, int64_t N, int64_t K, void *buf, int64_t buf_bytes, void *stream) {
    if (!bits_ok(bits)) return MBQ_ERR_BITS;
    if (!buf) return MBQ_ERR_NULL;
    if (!n_ok(N) || !k_ok(K)) return MBQ_ERR_SHAPE;
    if (!aligned(buf, 256)) return MBQ_ERR_ALIGN;
    if (buf_bytes < mbq_packed_bytes(bits, N, K)) return MBQ_ERR_WORKSPACE;
    int st = check_device();
    if (st) return st;
    int n_cu = 0;
    st = device_cus(&n_cu);
    if (st) return st;
    hipError_t he = hipSuccess;
    st = relayout_inplace(bits, N, K, buf, n_cu, (hipStream_t)stream, &he);
    return st == MBQ_ERR_HIP ? hip_fail(he) : st;
}

int mbq_relayout_interleave_host(int bits, int64_t N, int64_t K, void *host_buf, int64_t buf_bytes) {
    if (!bits_ok(bits)) return MBQ_ERR_BITS;
    if (!host_buf) return MBQ_ERR_NULL;
    if (!n_ok(N) || !k_ok(K)) return MBQ_ERR_SHAPE;
    if (buf_bytes < mbq_packed_bytes(bits, N, K)) return MBQ_ERR_WORKSPACE;
    return relayout_interleave_host(bits, N, K, (uint8_t *)host_buf);
}

static bool attn_shape_ok(int64_t M, int64_t n_q, int64_t n_kv, int64_t D, int64_t P) {
    return m_ok(M) && n_kv >= 1 && n_q >= n_kv && n_q % n_kv == 0 && n_q <= 4096 && (n_q / n_kv) * M <= 64 &&
           (D == 64 || D == 128 || D == 256) && P >= 0 && P + M <= ((int64_t)1 << 30);
}

static int attn_cus(int *n_cu) {
    int n = 0;
    if (hipGetDeviceCount(&n) == hipSuccess && n > 0 && device_cus(n_cu) == MBQ_OK) return MBQ_OK;
    *n_cu = 256;   // without a device: the MI355X's CU count
    return MBQ_OK;
}

int64_t mbq_attention_workspace_bytes(int64_t M, int64_t n_q, int64_t n_kv, int64_t D, int64_t P) {
    if (!attn_shape_ok(M, n_q, n_kv, D, P)) return MBQ_ERR_SHAPE;
    int n_cu = 256;
    attn_cus(&n_cu);
    return plan_attention(M, n_q, n_kv, D, P, n_cu).ws_bytes;
}

int mbq_decode_attention(int64_t M, int64_t n_q, int64_t n_kv, int64_t D, int64_t P, int64_t L, const void *q,
                         const void *k_cache, const void *v_cache, void *o, void *ws, int64_t ws_bytes,
                         void *stream) {
    if (!q || !k_cache || !v_cache || !o) return MBQ_ERR_NULL;
    if (!attn_shape_ok(M, n_q, n_kv, D, P) || L < P + M) return MBQ_ERR_SHAPE;
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 2)) return MBQ_ERR_ALIGN;
    if (!ws) return MBQ_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return MBQ_ERR_ALIGN;
    int st = check_device();
    if (st) return st;
    int n_cu = 0;
    st = device_cus(&n_cu);
    if (st) return st;
    const AttnPlan pl = plan_attention(M, n_q, n_kv, D, P, n_cu);
    if (ws_bytes < pl.ws_bytes) return MBQ_ERR_WORKSPACE;
    hipError_t e = launch_attention(pl, M, n_q, n_kv, D, P, L, q, k_cache, v_cache, o, ws, (hipStream_t)stream);
    return e == hipSuccess ? MBQ_OK : hip_fail(e);
}

// CUs the fused walk's plan is sized for: the current device's, or the
// MI355X's 256 when no device is visible (sizing queries work without one).
static int plan_cus() {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return 256;
    int n_cu = 0;
    return device_cus(&n_cu) == MBQ_OK && n_cu > 0 ? n_cu : 256;
}

// The sequence workspace holds two disjoint regions: the fused walk's (plan,
// statistics, tagged copies, partials; none when the fused walk rejects the
// list) and after it the unfused form's (quantised activations, scales and
// the linears' self-clearing counters).  Either form can therefore run on a
// workspace the other has used.
static int64_t fused_region_bytes(const mbq_op *ops, int32_t n_ops, const int64_t *widths, int32_t n_bufs,
                                  int64_t M) {
    const int64_t f = build_sequence_plan(ops, n_ops, nullptr, widths, n_bufs, M, plan_cus(), nullptr, nullptr);
    return f > 0 ? align256(f) : 0;
}

int64_t mbq_sequence_workspace_bytes(const mbq_op *ops, int32_t n_ops, const int64_t *buf_widths,
                                     int32_t n_bufs, int64_t M) {
    const int64_t unfused = analyse_program(ops, n_ops, buf_widths, n_bufs, M, nullptr);
    if (unfused < 0) return unfused;
    return fused_region_bytes(ops, n_ops, buf_widths, n_bufs, M) + unfused;
}

int mbq_sequence_prepare(const mbq_op *ops, int32_t n_ops, void *const *bufs, const int64_t *buf_widths,
                         int32_t n_bufs, int64_t M, void *ws, int64_t ws_bytes, void *stream,
                         mbq_sequence_info *info) {
    if (!bufs || !info) return MBQ_ERR_NULL;
    const int64_t unfused = analyse_program(ops, n_ops, buf_widths, n_bufs, M, nullptr);
    if (unfused < 0) return (int)unfused;
    for (int32_t b = 0; b < n_bufs; ++b) {
        if (!bufs[b]) return MBQ_ERR_NULL;
        if (!aligned(bufs[b], 16)) return MBQ_ERR_ALIGN;
    }
    if (!ws) return MBQ_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return MBQ_ERR_ALIGN;
    // lists the fused walk rejects are refused before anything touches the device
    const int64_t pre = build_sequence_plan(ops, n_ops, nullptr, buf_widths, n_bufs, M, 256, nullptr, nullptr);
    if (pre < 0) return (int)pre;
    int st = check_device();
    if (st) return st;
    const int n_cu = plan_cus();
    SeqBuild b;
    const int64_t need = build_sequence_plan(ops, n_ops, bufs, buf_widths, n_bufs, M, n_cu, (uint8_t *)ws, &b);
    if (need < 0) return (int)need;
    if (ws_bytes < need) return MBQ_ERR_WORKSPACE;
    hipStream_t hs = (hipStream_t)stream;
    hipError_t e = hipMemsetAsync(ws, 0, 128, hs);   // the error word's line; the walk epoch after it stays
    if (e == hipSuccess)
        e = hipMemcpyAsync((char *)ws + b.plan_offset, b.blob.data(), b.blob.size(), hipMemcpyHostToDevice, hs);
    if (e == hipSuccess) e = hipStreamSynchronize(hs);
    if (e != hipSuccess) return hip_fail(e);
    memset(info, 0, sizeof(*info));
    info->magic = 0x6d62712d73657131ull;
    info->bits = b.bits;
    info->M = (int32_t)M;
    info->grid = b.grid;
    info->lds_bytes = b.lds_bytes;
    info->ws_bytes = need;
    info->plan_offset = b.plan_offset;
    info->full = b.full ? 1 : 0;
    return MBQ_OK;
}

int mbq_sequence_run(const mbq_sequence_info *info, void *ws, void *stream) {
    if (!info || !ws) return MBQ_ERR_NULL;
    if (info->magic != 0x6d62712d73657131ull || (info->bits != 4 && info->bits != 6) || info->M < 1 ||
        info->M > kMaxM || info->grid < 1)
        return MBQ_ERR_PROGRAM;
    if (!aligned(ws, 256)) return MBQ_ERR_ALIGN;
    hipError_t e = launch_sequence(info->bits, info->M, info->full != 0, info->grid, info->lds_bytes,
                                   (const char *)ws + info->plan_offset, (uint32_t *)ws, (hipStream_t)stream);
    return e == hipSuccess ? MBQ_OK : hip_fail(e);
}

int mbq_sequence_check(void *ws, void *stream) {
    if (!ws) return MBQ_ERR_NULL;
    uint32_t word = 0;
    hipStream_t hs = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(&word, ws, 4, hipMemcpyDeviceToHost, hs);
    if (e == hipSuccess) e = hipStreamSynchronize(hs);
    if (e != hipSuccess) return hip_fail(e);
    if (word == 0) return MBQ_OK;
    e = hipMemsetAsync(ws, 0, 4, hs);
    if (e == hipSuccess) e = hipStreamSynchronize(hs);
    if (e != hipSuccess) return hip_fail(e);
    return word == 2 ? MBQ_ERR_PROGRAM : MBQ_ERR_TIMEOUT;
}

int mbq_layer_sequence(const mbq_op *ops, int32_t n_ops, void *const *bufs, const int64_t *buf_widths,
                       int32_t n_bufs, int64_t M, void *ws, int64_t ws_bytes, void *stream) {
    mbq_sequence_info info;
    int st = mbq_sequence_prepare(ops, n_ops, bufs, buf_widths, n_bufs, M, ws, ws_bytes, stream, &info);
    if (st) return st;
    return mbq_sequence_run(&info, ws, stream);
}

int mbq_layer_sequence_unfused(const mbq_op *ops, int32_t n_ops, void *const *bufs,
                               const int64_t *buf_widths, int32_t n_bufs, int64_t M, void *ws,
                               int64_t ws_bytes, void *stream) {
    if (!bufs) return MBQ_ERR_NULL;
    std::vector<Phase> phases;
    const int64_t unfused = analyse_program(ops, n_ops, buf_widths, n_bufs, M, &phases);
    if (unfused < 0) return (int)unfused;
    const int64_t base = fused_region_bytes(ops, n_ops, buf_widths, n_bufs, M);
    const int64_t need = base + unfused;
    for (int32_t b = 0; b < n_bufs; ++b) {
        if (!bufs[b]) return MBQ_ERR_NULL;
        if (!aligned(bufs[b], 16)) return MBQ_ERR_ALIGN;
    }
    if (!ws || ws_bytes < need) return MBQ_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return MBQ_ERR_ALIGN;
    int st = check_device();
    if (st) return st;
    hipStream_t hs = (hipStream_t)stream;
    int64_t k_max = 0;
    for (int32_t i = 0; i < n_ops; ++i) k_max = ops[i].K > k_max ? ops[i].K : k_max;
    char *region = (char *)ws + base;
    int8_t *q = (int8_t *)region;
    float *s = (float *)(region + align256(M * k_max));
    void *lin_ws = region + align256(M * k_max) + 256;
    for (const Phase &p : phases) {
        const mbq_op &o0 = ops[p.first];
        const bool swiglu = o0.prologue == MBQ_PRO_SWIGLU_QUANT;
        hipError_t e = launch_prologue_quant(o0.prologue, M, o0.K, bufs[o0.in_buf], buf_widths[o0.in_buf],
                                             swiglu ? bufs[o0.in_buf2] : nullptr,
                                             swiglu ? buf_widths[o0.in_buf2] : 0,
                                             o0.prologue == MBQ_PRO_WRMSNORM_QUANT ? o0.norm_w : nullptr, nullptr,
                                             q, s, hs);
        if (e != hipSuccess) return hip_fail(e);
        for (int32_t i = p.first; i < p.first + p.count; ++i) {
            const mbq_op &o = ops[i];
            const LinearPlan plan = plan_linear(o.bits, M, o.N, o.K);
            e = launch_linear(o.bits, M, o.N, o.K, q, s, o.packed, bufs[o.out_buf], o.N, lin_ws, plan, hs);
            if (e != hipSuccess) return hip_fail(e);
        }
    }
    return MBQ_OK;
}

}  // extern "C"
