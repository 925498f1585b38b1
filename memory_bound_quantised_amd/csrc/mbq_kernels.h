// Host-side launchers of the libmbq kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

struct mbq_op;

namespace mbq {

// In-place re-layout (pack.hip).  Byte geometry of a matrix: canonical codes
// (Cr bytes per row, pc per row and group), padded row count Np = 64 R, and
// per row block C code bytes, S scale bytes, T = C + S (= G packed tiles).
struct RelayoutGeom {
    int64_t N, K, G, R, Np, Cr, pc, C, S, T, canon_bytes, packed_bytes;
};
__host__ __device__ inline RelayoutGeom relayout_geom(int bits, int64_t N, int64_t K) {
    RelayoutGeom g;
    g.N = N;
    g.K = K;
    g.G = K / 128;
    g.R = (N + 63) / 64;
    g.Np = 64 * g.R;
    g.Cr = K * bits / 8;
    g.pc = 128 * bits / 8;
    g.C = 64 * g.Cr;
    g.S = 64 * 2 * g.G;
    g.T = g.C + g.S;
    g.canon_bytes = N * (g.Cr + 2 * g.G);
    g.packed_bytes = g.R * g.T;
    return g;
}
// Interval [a, b) of row blocks at node i of recursion level `level` of step
// A: the root is [0, R), and a node [a, b) splits at (a + b) / 2, the bits of
// i choosing left or right from the top level down.
__host__ __device__ inline void relayout_node(int64_t R, int level, int64_t i, int64_t &a, int64_t &b) {
    a = 0;
    b = R;
    for (int d = level - 1; d >= 0; --d) {
        const int64_t m = (a + b) / 2;
        if ((i >> d) & 1) a = m;
        else b = m;
    }
}
// Steps P and A of the re-layout on a host buffer (tests of the schedule).
int relayout_interleave_host(int bits, int64_t N, int64_t K, uint8_t *buf);
// The whole re-layout on the device, in place; waits for the stream.  On
// MBQ_ERR_HIP, *hip_err holds the failing call's error.
int relayout_inplace(int bits, int64_t N, int64_t K, void *buf, int n_cu, hipStream_t s, hipError_t *hip_err);

// Split-prefix decode attention (attn.hip).
struct AttnPlan {
    // blocks_per_split: blocks of each split; the last (n_blocks mod n_split) splits take one more
    int64_t n_blocks = 0, blocks_per_split = 0, n_split = 0, rows = 0;
    int64_t block = 64;      // positions per block
    int64_t merge_tpq = 1;   // merge lanes per four outputs
    bool two_per_cu = false; // two workgroups per CU (the split kernel's register-capped form)
    int64_t off_cnt = 0, off_ml = 0, off_o = 0, ws_bytes = 0;
    int lds_bytes = 0;
    bool merge_inline = false;   // merge the splits at the end of the split launch
};
AttnPlan plan_attention(int64_t M, int64_t n_q, int64_t n_kv, int64_t D, int64_t P, int n_cu);
hipError_t launch_attention(const AttnPlan &pl, int64_t M, int64_t n_q, int64_t n_kv, int64_t D, int64_t P,
                            int64_t L, const void *q, const void *k, const void *v, void *o, void *ws,
                            hipStream_t st);

hipError_t launch_pack(int bits, int64_t N, int64_t K, const void *canon, const void *scales,
                       void *packed, hipStream_t s);
hipError_t launch_unpack(int bits, int64_t N, int64_t K, const void *packed, void *canon,
                         void *scales, hipStream_t s);

// Per-row quantisation of columns [0, K) of x (bf16, row stride x_stride
// elements) after prologue `pro` (an MBQ_PRO_* value): w is the weighted
// norm's bf16 [K] weights; u (row stride u_stride) the SwiGLU up rows, h an
// optional bf16 [M][K] copy of the SwiGLU output.
hipError_t launch_prologue_quant(int pro, int64_t M, int64_t K, const void *x, int64_t x_stride,
                                 const void *u, int64_t u_stride, const void *w, void *h, int8_t *q,
                                 float *s, hipStream_t st);

// Per-op skinny linear: work split, workspace size and launch.
struct LinearPlan {
    int64_t n_rb;      // row blocks of 64
    int64_t groups;    // K / 128
    int64_t splits;    // waves per row block (k ranges)
    int64_t ws_bytes;  // counters + fp32 partials
    bool rb_form;      // one workgroup per row block, no partials (splits unused)
    bool rs_form;      // with rb_form: four workgroups per row block, one per row set
};
LinearPlan plan_linear(int bits, int64_t M, int64_t N, int64_t K);
hipError_t launch_linear(int bits, int64_t M, int64_t N, int64_t K, const int8_t *q, const float *s,
                         const void *packed, void *y, int64_t y_stride, void *ws, const LinearPlan &plan,
                         hipStream_t st);
// The linear with its prologue and quantisation run inside it where the
// row-block form applies, else as a prologue launch into the workspace first.
int64_t linear_prologue_ws_bytes(int bits, int64_t M, int64_t N, int64_t K);
hipError_t launch_linear_prologue(int bits, int pro, int64_t M, int64_t N, int64_t K, const void *x, const void *u,
                                  const void *w, const void *packed, void *y, void *ws, hipStream_t st);
// The linear on the library's own device scratch (noalloc.hip): status or MBQ_OK.
int64_t noalloc_scratch_bytes();
int linear_noalloc(int bits, int64_t M, int64_t N, int64_t K, const int8_t *q, const float *s,
                   const void *packed, void *y, hipStream_t st, hipError_t *hip_err);
// Exact int32 group sums through the matrix-core (mfma) or v_dot4 tile form.
hipError_t launch_group_acc(int bits, int form, int64_t M, int64_t N, int64_t K, const int8_t *q,
                            const void *packed, int32_t *acc, hipStream_t st);

// HBM stream-read ceiling (ceiling.hip): one pass over bytes (a multiple of 1 KiB).
hipError_t launch_stream_read(const void *buf, int64_t bytes, uint32_t *sink, int n_cu, hipStream_t st);

// Fused decode-step walk (persistent kernel).
struct SeqBuild {
    int64_t ws_bytes = 0;
    int64_t plan_offset = 0;
    int grid = 0;
    int lds_bytes = 0;
    int bits = 0;
    bool full = false;           // the walk needs the weighted-norm / SwiGLU form of the kernel
    std::vector<uint8_t> blob;   // plan bytes to copy to ws + plan_offset
};
// Validates the op list and lays out the workspace; with ws and bufs also fills
// out->blob with the device plan.  Returns the workspace bytes or a negative status.
int64_t build_sequence_plan(const struct mbq_op *ops, int32_t n_ops, void *const *bufs,
                            const int64_t *widths, int32_t n_bufs, int64_t M, int n_cu, uint8_t *ws,
                            SeqBuild *out);
// The walk kernel of each form for (bits, M): the plain form (prologues 0 and
// 1 only) and the full one (also weighted RMSNorms and SwiGLU inputs).
const void *seq_kernel_plain(int bits, int64_t M);
const void *seq_kernel_full(int bits, int64_t M);
hipError_t launch_sequence(int bits, int64_t M, bool full, int grid, int lds_bytes, const void *plan, uint32_t *err, hipStream_t st);

}  // namespace mbq
