/*
 * mbq.h -- C ABI of libmbq: memory-bound quantised skinny linears for MI355X (gfx950).
 *
 * The hot path of batch-of-one LLM token generation as described on the page
 * "Doubling LLM token rates in ComfyUI" (blog.comfy.org):
 *   - section "What is the bottleneck?": a dense, often square weight matrix
 *     times one activation row (M = 1) or a thin block (M = 2..8) for a
 *     multi-token-prediction verify step; every weight is read once per step
 *     for about one operation, so HBM read speed bounds the step;
 *   - section "Optimizing the Linear Kernel": W4A8 / W6A8 weights (4- or 6-bit
 *     integer codes with per-group scales), the activation quantised to 8 bits,
 *     an integer matrix-vector kernel, weights and their group scales
 *     re-laid out once per model load in the order the kernel consumes them,
 *     and the activation quantisation fused with the RMSNorm before it.
 *
 * Definitions used by every entry point (the pages state the operations but
 * not their formulas; these are the readings the library implements):
 *   canonical W4   u8[N][K/2]: two's-complement int4 codes in [-8, 7], even k in
 *                  the low nibble of byte k/2.
 *   canonical W6   u8[N][3K/4]: int6 codes in [-32, 31]; codes 4j..4j+3 form the
 *                  little-endian 24-bit word of bytes 3j..3j+2, code 4j+i at bits 6i.
 *   scales         IEEE fp16 S[N][K/128]: one scale per 128 consecutive k of a row.
 *   quantisation   per row m: amax = max_k |x[m][k]|, s[m] = amax / 127 (fp32, IEEE
 *                  divide); q[m][k] = clamp(round_half_even(x[m][k] / s[m]), -127, 127);
 *                  an all-zero row gives s = 0 and q = 0.
 *   linear         acc[m][n][g] = sum_{k in group g} q[m][k] * w[n][k]  (exact int32);
 *                  y[m][n] = bf16_round_nearest_even(s[m] * sum_g S[n][g] * acc[m][n][g])
 *                  with the group sum taken in fp32 (so y matches the exact value
 *                  to within fp32 summation error before the bf16 rounding).
 *   RMSNorm        (weightless, optional before a quantisation): ss = sum_k x^2 in
 *                  fp64, r = 1 / sqrtf((float)(ss / K) + 1e-6f) in fp32,
 *                  t = bf16_round(x * r); then the quantisation runs on t.
 *
 * Conventions for every call:
 *   - Pointers marked "device" are caller-owned device memory of the current
 *     HIP device; "host" pointers are ordinary host memory read during the
 *     call only.  The library never allocates or frees memory.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls validate
 *     their arguments, enqueue work on `stream` and return without waiting;
 *     device faults surface at the caller's next synchronisation.
 *   - Return value: MBQ_OK (0) or a negative mbq_status.  On any non-zero
 *     status nothing has been enqueued, except MBQ_ERR_HIP, which reports a
 *     launch failure (the HIP error code is then in mbq_last_hip_error()).
 *   - Shapes: M in [1, 8]; K a positive multiple of 128 (at most 2^24);
 *     1 <= N <= 2^20; bits 4 or 6.
 *   - Alignment: packed weights 256-byte aligned; activation, q and y
 *     pointers 16-byte aligned; workspaces 256-byte aligned.
 *   - Workspaces: caller-owned device memory of at least the queried size,
 *     zero-filled before its first use (e.g. allocated with zeros).  A linear
 *     that runs to completion leaves its workspace's counters zero again, so
 *     the same workspace serves any later linear of any shape.  A walk's
 *     workspace (mbq_sequence_workspace_bytes) holds two disjoint regions, the
 *     fused walk's and the unfused form's, so both forms may share it; the
 *     fused region keeps the prepared plan and tagged data between steps and
 *     must not be handed to other calls while the plan is in use.  Calls that
 *     share a workspace must not overlap in time (same stream, or synchronised).
 */
#ifndef MBQ_H
#define MBQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MBQ_OK = 0,
    MBQ_ERR_NULL = -1,      /* a required pointer is NULL */
    MBQ_ERR_SHAPE = -2,     /* M, N or K outside the supported set */
    MBQ_ERR_BITS = -3,      /* bits is not 4 or 6 */
    MBQ_ERR_ALIGN = -4,     /* a pointer violates the alignment rules */
    MBQ_ERR_WORKSPACE = -5, /* workspace NULL or smaller than required */
    MBQ_ERR_PROGRAM = -6,   /* malformed layer-sequence op list */
    MBQ_ERR_HIP = -7,       /* a HIP runtime call failed */
    MBQ_ERR_DEVICE = -8,    /* the current device is not a gfx950 */
    MBQ_ERR_TIMEOUT = -9    /* a bounded wait inside the fused walk gave up */
} mbq_status;

/* Human-readable name of a status code (static string, never NULL). */
const char *mbq_status_string(int status);

/* hipError_t behind the last MBQ_ERR_HIP returned on this thread (0 if none). */
int mbq_last_hip_error(void);

/* Library version string (static). */
const char *mbq_version(void);

/* ---------------------------------------------------------------- weight layout
 * Kernel-order layout ("Optimizing the Linear Kernel": weights and their
 * per-group scales interleaved in the order the kernel consumes them, laid out
 * once per model load).  Rows are cut into blocks of 64; each (row block,
 * 128-wide k group) tile holds the 64 rows' codes followed by their 64 fp16
 * scales, and tiles follow each other row block by row block, k group by k
 * group.  Rows past N are zero-filled.  The layout is opaque to callers: its
 * size comes from mbq_packed_bytes and it is produced by mbq_pack_weights.
 */

/* Bytes of the packed layout for an N x K matrix of `bits`-bit codes, or a
 * negative mbq_status for invalid arguments. */
int64_t mbq_packed_bytes(int bits, int64_t N, int64_t K);

/* Re-lay a canonical matrix (w_canon: device u8, scales_f16: device fp16
 * [N][K/128]) into `packed` (device, mbq_packed_bytes bytes).  Lossless. */
int mbq_pack_weights(int bits, int64_t N, int64_t K, const void *w_canon,
                     const void *scales_f16, void *packed, void *stream);

/* Inverse of mbq_pack_weights (device pointers); for tests and tooling. */
int mbq_unpack_weights(int bits, int64_t N, int64_t K, const void *packed,
                       void *w_canon, void *scales_f16, void *stream);

/* The same re-layout done in place ("Optimizing the Linear Kernel": the
 * kernel-order re-layout happens in VRAM, in place, once per load, with no
 * extra RAM or VRAM).  buf (device, 256-byte aligned, buf_bytes >=
 * mbq_packed_bytes(bits, N, K)) holds on entry the canonical codes of the N
 * rows (row stride K * bits / 8 bytes, as mbq_pack_weights reads them)
 * immediately followed by the fp16 scales [N][K/128]; bytes past those are
 * ignored.  On return it holds exactly what mbq_pack_weights would write
 * (padding rows zero).  No workspace: the bytes move inside buf (block
 * rotations, then a grid-wide pass that stages whole row blocks in LDS).
 * Waits for `stream`; a set-up call.  Calls on one device must not overlap
 * (they share one grid-barrier word).  Returns MBQ_ERR_WORKSPACE if buf_bytes
 * is too small, MBQ_ERR_SHAPE if K / 128 exceeds the tiles the device can
 * stage at once (about 9000 groups at W4, 6000 at W6), MBQ_ERR_TIMEOUT if the
 * grid barrier gave up (buf is then undefined). */
int mbq_pack_weights_inplace(int bits, int64_t N, int64_t K, void *buf, int64_t buf_bytes, void *stream);

/* Test helper, host only: the first two steps of the in-place re-layout
 * (padding rows, then row blocks interleaved as [codes of rows 64b..64b+63]
 * [their scales] for b = 0, 1, ..) on a host buffer of buf_bytes >=
 * mbq_packed_bytes(bits, N, K) holding the canonical codes and scales. */
int mbq_relayout_interleave_host(int bits, int64_t N, int64_t K, void *host_buf, int64_t buf_bytes);

/* ---------------------------------------------------------------- activation quantisation
 * "Optimizing the Linear Kernel": quantise the activation to 8 bits before
 * the integer linear.  x_bf16: device bf16 [M][K] (row stride K);
 * q: device int8 [M][K]; s: device fp32 [M]. */
int mbq_quantize_act(int64_t M, int64_t K, const void *x_bf16, int8_t *q, float *s,
                     void *stream);

/* Same, preceded by the weightless RMSNorm of each row (the prologue fusion
 * of "Optimizing the Linear Kernel").  Arguments as mbq_quantize_act. */
int mbq_rmsnorm_quantize_act(int64_t M, int64_t K, const void *x_bf16, int8_t *q, float *s,
                             void *stream);

/* Same, preceded by the weighted RMSNorm of each row: r = 1/sqrt(mean(x^2) +
 * 1e-6) (sum of squares in fp64, r in fp32), t = bf16(fp32(x * w * r)) where
 * the product x * w of two bf16 values is exact.  w_bf16: device bf16 [K]
 * norm weights, 16-byte aligned.  Other arguments as mbq_quantize_act. */
int mbq_wrmsnorm_quantize_act(int64_t M, int64_t K, const void *x_bf16, const void *w_bf16,
                              int8_t *q, float *s, void *stream);

/* Same, preceded by the SwiGLU gate in front of a down projection (the
 * prologue fusion of "Optimizing the Linear Kernel"): h = bf16(silu(g) * u)
 * with silu(g) = g / (1 + exp(-g)) in fp32.  g_bf16, u_bf16: device bf16
 * [M][K]; h_bf16: device bf16 [M][K] receiving h, or null.  Other arguments
 * as mbq_quantize_act. */
int mbq_swiglu_quantize_act(int64_t M, int64_t K, const void *g_bf16, const void *u_bf16,
                            void *h_bf16, int8_t *q, float *s, void *stream);

/* ---------------------------------------------------------------- the skinny linear
 * "What is the bottleneck?" / "Optimizing the Linear Kernel": y = rescale(q x W^T).
 * q: device int8 [M][K]; s: device fp32 [M]; packed: device, from
 * mbq_pack_weights with the matching bits; y_bf16: device bf16 [M][N];
 * ws: device workspace of mbq_linear_workspace_bytes bytes (see conventions). */
int64_t mbq_linear_workspace_bytes(int bits, int64_t M, int64_t N, int64_t K);

int mbq_w4a8_linear(int64_t M, int64_t N, int64_t K, const int8_t *q, const float *s,
                    const void *packed, void *y_bf16, void *ws, int64_t ws_bytes,
                    void *stream);

int mbq_w6a8_linear(int64_t M, int64_t N, int64_t K, const int8_t *q, const float *s,
                    const void *packed, void *y_bf16, void *ws, int64_t ws_bytes,
                    void *stream);

/* The linear with the quantisation, and the prologue before it, inside it
 * (page "Doubling LLM token rates in ComfyUI", "Optimizing the Linear
 * Kernel": the quantisation absorbs the RMSNorm or SwiGLU in front of it, so
 * the intermediate is never written).  y = the linear of (q, s), where (q, s)
 * is what mbq_quantize_act, mbq_rmsnorm_quantize_act,
 * mbq_wrmsnorm_quantize_act or mbq_swiglu_quantize_act gives for the rows.
 *   bits      4 or 6.
 *   prologue  MBQ_PRO_QUANT: the rows x themselves; MBQ_PRO_RMSNORM_QUANT:
 *             the weightless RMSNorm of x; MBQ_PRO_WRMSNORM_QUANT: the
 *             RMSNorm of x weighted by w; MBQ_PRO_SWIGLU_QUANT: silu(x) * u,
 *             x being the gate rows and u the up rows.
 *   x_bf16, u_bf16  bf16 [M][K], row-major, 16-byte aligned; u_bf16 null
 *             unless the prologue is SwiGLU.
 *   w_bf16    bf16 [K] norm weights, 16-byte aligned; null unless weighted.
 *   packed, y_bf16, stream  as mbq_w4a8_linear.
 *   ws        device workspace, 256-byte aligned, of
 *             mbq_linear_prologue_workspace_bytes(bits, M, N, K) bytes,
 *             zero-filled before its first use (as for the linear).
 * Where the linear's one-workgroup-per-row-block form applies (up to 512
 * row blocks of 64 rows, and K up to 6144 or at least 48 row blocks and K up
 * to 20480) and M x K is at most 143360, every workgroup runs the prologue and the
 * quantisation on the rows into its LDS and reads its activation codes from
 * there: one launch, nothing written but y.  Other shapes run the prologue
 * and quantisation as a launch of their own into the workspace first.  The
 * codes and scales are computed by the same routine as the quantisation
 * calls', so y equals those calls followed by the linear bit for bit (a
 * block of another size sums the fp64 squares of a norm in another order,
 * which could move r only where the mean square lies within a few units of
 * 2^-40 of an fp32 rounding boundary).
 * Returns MBQ_ERR_PROGRAM for an unknown prologue, MBQ_ERR_NULL for a
 * missing pointer the prologue needs, and otherwise as mbq_w4a8_linear. */
int64_t mbq_linear_prologue_workspace_bytes(int bits, int64_t M, int64_t N, int64_t K);
int mbq_linear_prologue(int bits, int prologue, int64_t M, int64_t N, int64_t K, const void *x_bf16,
                        const void *u_bf16, const void *w_bf16, const void *packed, void *y_bf16, void *ws,
                        int64_t ws_bytes, void *stream);

/* The same linear for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): no
 * workspace argument.  Its split-K counters and partials live in an array of
 * 8 MiB + 64 KiB inside the library's device code (one per GPU it runs on,
 * held until the process ends), which holds the scratch of every supported
 * shape; the first call on a device looks up that array and zeroes its
 * counters with a small kernel on `stream`, and every completed call leaves
 * them zero again.  The call itself allocates nothing.  All calls on one GPU
 * share the array, so calls that overlap in time on one GPU (different
 * streams, not synchronised) race.  bits is 4 or 6; other arguments and
 * results as mbq_w4a8_linear.  Returns MBQ_ERR_WORKSPACE if a shape ever
 * needed more scratch than the array holds. */
int mbq_linear_noalloc(int bits, int64_t M, int64_t N, int64_t K, const int8_t *q, const float *s,
                       const void *packed, void *y_bf16, void *stream);

/* The exact int32 group sums acc[m][n][g] (device int32 [M][N][K/128]) that the
 * linears rescale, for tests.  `form` picks the tile code that produces them,
 * each being the very functions the product runs:
 *   MBQ_FORM_MFMA    the whole-tile matrix-core code (v_mfma_i32_16x16x64_i8,
 *                    activation rows padded to 16): the linear's split and
 *                    row-block forms and the fused walk, at every M;
 *   MBQ_FORM_ROWSET  the row-set code of the linear's row-set form (the tile's
 *                    four sets of 16 rows loaded, unpacked and multiplied one
 *                    set at a time);
 *   MBQ_FORM_DOT4    the v_dot4 tile with its four 32-k slice sums added in
 *                    int32 (a second form, not on the product's path).
 * Returns MBQ_ERR_SHAPE for any other form. */
enum { MBQ_FORM_DOT4 = 0, MBQ_FORM_MFMA = 1, MBQ_FORM_ROWSET = 2 };
int mbq_linear_group_acc(int bits, int form, int64_t M, int64_t N, int64_t K, const int8_t *q,
                         const void *packed, int32_t *acc, void *stream);

/* ---------------------------------------------------------------- decode attention
 * "Paying attention to the attention!": the grouped-query attention of a decode
 * step for a short query -- the committed token, or it and the MTP draft rows
 * with their causal verification -- without a materialised mask.  The cached
 * prefix is split across many workgroups, and a second kernel on the same
 * stream combines their partial softmax results (none when one split covers
 * it).  With MBQ_ATTN_COMBINE=inline in the environment at the call, the
 * splits of each key/value head combine them at the end of the same launch
 * instead: the launch is cooperative (every split resident), and each split
 * merges a share of its head's outputs once all have published.  Where the
 * device will not take that grid at once, the second kernel combines them.
 * The in-launch combine is the slower of the two here: the cooperative launch
 * costs more than the second kernel.
 *
 * q: device bf16 [M][n_q][D]; k_cache, v_cache: device bf16 [n_kv][L][D]
 * (row stride D, head stride L * D) holding the M new tokens' keys and values
 * at positions P .. P+M-1; o: device bf16 [M][n_q][D].  Token i attends to
 * positions 0 .. P+i; query head h reads key/value head h / (n_q / n_kv);
 * scores are scaled by 1/sqrt(D); softmax and sums in fp32.
 * Shapes: M in 1..8, D in {64, 128, 256}, n_q a multiple of n_kv with
 * (n_q / n_kv) * M <= 64, L >= P + M.  q and the caches 16-byte aligned.
 * ws: device, 256-byte aligned, >= mbq_attention_workspace_bytes(...) bytes:
 * the partial results (scratch) and, at its start, the in-launch combine's
 * per-head counters.  Any contents for the default combine; for the in-launch
 * one, zero-filled before its first use (every completed call leaves the
 * counters at zero, so one workspace serves calls of any shape in turn).
 * Calls sharing a workspace must not overlap.  Enqueued on `stream`. */
int64_t mbq_attention_workspace_bytes(int64_t M, int64_t n_q, int64_t n_kv, int64_t D, int64_t P);
int mbq_decode_attention(int64_t M, int64_t n_q, int64_t n_kv, int64_t D, int64_t P, int64_t L, const void *q,
                         const void *k_cache, const void *v_cache, void *o, void *ws, int64_t ws_bytes,
                         void *stream);

/* ---------------------------------------------------------------- measurement
 * HBM stream-read ceiling ("What is the bottleneck?": token generation is
 * bound by how fast the GPU reads the model from VRAM): one pass over `bytes`
 * bytes of device memory at buf (256-byte aligned; bytes a positive multiple
 * of 1024) with the same 16-byte non-temporal loads the weight stream uses,
 * spread over every CU.  The bytes read are folded into a digest; *sink
 * (device uint32, 4-byte aligned) is written only for one particular digest
 * value, so the call leaves it untouched in practice.  The achieved rate of
 * this call is the measured ceiling the weight stream is judged against. */
int mbq_stream_read(const void *buf, int64_t bytes, uint32_t *sink, void *stream);

/* ---------------------------------------------------------------- decode-step walk
 * "What is the bottleneck?": one decode step reads every weight matrix of the
 * model once.  An op list describes the walk: op i quantises columns [0, K) of
 * buffer in_buf after its prologue (none, the weightless or weighted RMSNorm,
 * or the SwiGLU gate of in_buf and in_buf2, as in the quantisation calls
 * above), multiplies by its packed matrix and writes all N columns of buffer
 * out_buf.  Consecutive ops with the same inputs, prologue, norm_w pointer and
 * K share one quantisation (a phase, e.g. q/k/v or gate/up).  Semantics
 * are those of running the ops one after the other.  Buffers are device bf16
 * [M][width] with row stride width. */
enum { MBQ_PRO_QUANT = 0, MBQ_PRO_RMSNORM_QUANT = 1, MBQ_PRO_WRMSNORM_QUANT = 2, MBQ_PRO_SWIGLU_QUANT = 3 };

typedef struct mbq_op {
    int32_t bits;        /* 4 or 6 */
    int32_t prologue;    /* MBQ_PRO_* */
    int64_t N;           /* output columns; must equal the width of out_buf */
    int64_t K;           /* input columns read; multiple of 128, <= width of in_buf */
    const void *packed;  /* device, from mbq_pack_weights(bits, N, K) */
    int32_t in_buf;      /* index into bufs (the gate for MBQ_PRO_SWIGLU_QUANT) */
    int32_t out_buf;     /* index into bufs; differs from the inputs and from the
                            out_buf of every other op of the same phase */
    int32_t in_buf2;     /* MBQ_PRO_SWIGLU_QUANT: the up buffer; otherwise ignored */
    int32_t reserved;    /* 0 */
    const void *norm_w;  /* MBQ_PRO_WRMSNORM_QUANT: device bf16 [K] norm weights,
                            16-byte aligned; otherwise ignored */
} mbq_op;

/* Workspace bytes for the walk: the fused walk's region (none when the fused
 * walk rejects the list, see mbq_sequence_prepare) followed by the unfused
 * form's, or a negative mbq_status (MBQ_ERR_PROGRAM for a malformed op list).
 * ops, buf_widths: host. */
int64_t mbq_sequence_workspace_bytes(const mbq_op *ops, int32_t n_ops,
                                     const int64_t *buf_widths, int32_t n_bufs, int64_t M);

/* Launch parameters of a prepared walk (filled by mbq_sequence_prepare; host memory). */
typedef struct mbq_sequence_info {
    uint64_t magic;
    int32_t bits, M;
    int32_t grid, lds_bytes;
    int64_t ws_bytes;
    int64_t plan_offset;
    int32_t full;        /* 1: the walk uses the weighted-RMSNorm or SwiGLU prologue */
    int32_t reserved;
} mbq_sequence_info;

/* Validate the walk and write its execution plan into ws (device), then wait
 * for `stream` to drain (a set-up call, not for the per-step loop).  ops,
 * bufs (device pointers) and buf_widths (elements per row, multiples of 8)
 * are host arrays.  All ops must share one bit width.  Returns
 * MBQ_ERR_PROGRAM if an op reads a buffer index out of range, N != width of
 * out_buf, K > width of in_buf, a phase writes its own input or the same
 * buffer twice, the bit widths differ, or one op's output is read with two
 * different K.  The fused walk also returns MBQ_ERR_PROGRAM (the unfused call
 * takes such lists) when the consumers of one op's output disagree on the norm
 * weights, or use a weighted RMSNorm and no weights, or when a SwiGLU op's
 * gate and up buffers are not either both written before the walk or both
 * written by ops of one phase with equal N whose outputs nothing else in the
 * walk reads; when an op overwrites a buffer that an earlier phase read as
 * an input written before the walk; and when one buffer is written by several
 * ops whose row blocks are finalised by different workgroups (the walk
 * orders neither case; the same op layout repeated layer after layer is
 * fine).  The plan stays valid while ws, bufs, the packed weights and the
 * norm weights stay where they are. */
int mbq_sequence_prepare(const mbq_op *ops, int32_t n_ops, void *const *bufs,
                         const int64_t *buf_widths, int32_t n_bufs, int64_t M, void *ws,
                         int64_t ws_bytes, void *stream, mbq_sequence_info *info);

/* One decode step: a single persistent-kernel launch that runs every op of
 * the prepared walk with all its quantisations fused in, keeping the weight
 * stream going across op boundaries.  Enqueued on `stream`; does not wait.
 * Needs every workgroup of its grid resident at once (cooperative launch);
 * nothing else may run on the device in parallel with it.  May be captured
 * in a HIP graph and replayed: each launch reads the workspace's launch
 * count on the device and tags the words it hands between workgroups with
 * it, so a replay never takes a word an earlier launch left. */
int mbq_sequence_run(const mbq_sequence_info *info, void *ws, void *stream);

/* Wait for `stream`, then report whether the last walks run on ws completed
 * normally: MBQ_OK, MBQ_ERR_TIMEOUT (a bounded wait gave up: outputs are not
 * valid) or MBQ_ERR_PROGRAM (ws held no prepared plan).  Clears the report. */
int mbq_sequence_check(void *ws, void *stream);

/* mbq_sequence_prepare + mbq_sequence_run. */
int mbq_layer_sequence(const mbq_op *ops, int32_t n_ops, void *const *bufs,
                       const int64_t *buf_widths, int32_t n_bufs, int64_t M, void *ws,
                       int64_t ws_bytes, void *stream);

/* The same walk as one quantisation launch plus one linear launch per op
 * (mixed bit widths allowed).  Same results within the linear's tolerance;
 * kept as the unfused baseline.  Does not wait. */
int mbq_layer_sequence_unfused(const mbq_op *ops, int32_t n_ops, void *const *bufs,
                               const int64_t *buf_widths, int32_t n_bufs, int64_t M, void *ws,
                               int64_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MBQ_H */
