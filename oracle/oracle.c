/*
 * CPU oracle for the skinny W4A8 / W6A8 linear of batch-of-one LLM decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU baseline
 * do.  It shares no code, header, table or constant with the HIP library.
 *
 * Source: "Doubling LLM token rates in ComfyUI" (blog.comfy.org), sections
 * "What is the bottleneck?" (a dense weight matrix times one activation row,
 * or a thin block of a few rows for an MTP verify step) and "Optimizing the
 * Linear Kernel" (W4A8 / W6A8 checkpoints, per-group weight scales, quantise
 * the activation to 8 bits, then an integer matrix-vector product; the kernel
 * rewrite keeps the result of the model unchanged).  The pages state no
 * formulas; the readings used here are:
 *   - weight codes are two's-complement integers, int4 in [-8,7] two per
 *     byte with even k in the low nibble, int6 in [-32,31] four per three
 *     bytes read as a little-endian 24-bit word (k%4 selects bits 6*(k%4));
 *     rows are n-major (N x K), one fp16 scale per 128 consecutive k of a row;
 *   - activations are quantised per row: amax = max|x|, s = amax/127 (IEEE
 *     fp32 divide), q = clamp(round_half_even(x/s), -127, 127); an all-zero
 *     row gives s = 0 and q = 0.  These quantisation decisions are taken in
 *     fp32, the precision the GPU kernel uses, so both sides agree bit for bit;
 *   - acc[m][n][g] = sum over the 128 k of group g of q[m][k]*w[n][k], exact
 *     in 32-bit integers;
 *   - y[m][n] = bf16_round_nearest_even( s[m] * sum_g S[n][g] * acc[m][n][g] ),
 *     with the sum taken in fp64 here;
 *   - the optional weightless RMSNorm in front of a quantisation (the page's
 *     prologue fusion absorbs the RMSNorm that precedes the quantisation):
 *     ss = sum_k x^2 in fp64, r = 1/sqrtf(f32(ss/K) + 1e-6f) in fp32,
 *     t = bf16_round(f32(x) * r);
 *   - the weighted RMSNorm (same section; a norm with a learned per-column
 *     weight w, bf16): the same ss and r, then t = bf16_round(f32((x*w) * r)),
 *     where x*w of two bf16 values is exact in fp32, so t carries a single
 *     fp32 rounding before the bf16 one (the pages fix no order; this one makes
 *     max|t| = bf16_round(f32(max|x*w| * r)), since both roundings are monotone);
 *   - the SwiGLU gate in front of the down projection (same section: the
 *     quantisation absorbs the SwiGLU that precedes it): h = bf16_round(
 *     g / (1 + exp(-g)) * u) for bf16 g (gate) and u (up), evaluated in fp64
 *     here; the GPU's fp32 evaluation may land one bf16 step away where the
 *     value sits next to a rounding boundary.
 * Every loop below is the plain definition: no blocking, no reordering.
 */
#include <math.h>
#include <stdlib.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>

#define GROUP 128

/* ---- number formats ---------------------------------------------------- */

static float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* IEEE binary16 -> double, straight from the format's definition. */
static double f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);      /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Nearest bf16 (8 significant bits), ties to even, straight from a double.
 * Values beyond the largest finite bf16 round to infinity. */
static uint16_t f64_to_bf16(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                                   /* a = f * 2^e, f in [0.5, 1) */
    int qexp = e - 8;                               /* spacing of 8-bit significands */
    if (qexp < -133) qexp = -133;                   /* bf16 subnormal spacing 2^-133 */
    double r = nearbyint(ldexp(a, -qexp));          /* default mode: nearest even */
    r = ldexp(r, qexp);
    if (r > 0x1.FEp127) return sign | 0x7F80;       /* overflow -> inf */
    float f = (float)r;                             /* exact: r has <= 8 bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return sign | (uint16_t)(u >> 16);
}

static uint16_t f32_to_bf16(float f) { return f64_to_bf16((double)f); }

/* ---- weight codes -------------------------------------------------------- */

int oracle_w4_code(const uint8_t *row, int64_t k) {
    int nib = (row[k / 2] >> (4 * (k % 2))) & 0xF;
    return nib >= 8 ? nib - 16 : nib;
}

int oracle_w6_code(const uint8_t *row, int64_t k) {
    int64_t j = k / 4;
    uint32_t t = (uint32_t)row[3 * j] | ((uint32_t)row[3 * j + 1] << 8) |
                 ((uint32_t)row[3 * j + 2] << 16);
    int c = (int)((t >> (6 * (k % 4))) & 0x3F);
    return c >= 32 ? c - 64 : c;
}

static int64_t row_bytes(int bits, int64_t K) { return K * bits / 8; }

static int code_at(int bits, const uint8_t *row, int64_t k) {
    return bits == 4 ? oracle_w4_code(row, k) : oracle_w6_code(row, k);
}

/* w[n][k] as int8, for tests that want the decoded matrix. */
int oracle_decode(int bits, int64_t N, int64_t K, const uint8_t *canon, int8_t *w) {
    if (bits != 4 && bits != 6) return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            w[n * K + k] = (int8_t)code_at(bits, canon + n * row_bytes(bits, K), k);
    return 0;
}

/* ---- activation quantisation ------------------------------------------- */

int oracle_quantize_act(int64_t M, int64_t K, const uint16_t *x, int8_t *q, float *s) {
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *xr = x + m * K;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(bf16_to_f32(xr[k]));
            if (a > amax) amax = a;
        }
        if (amax == 0.0f) {
            s[m] = 0.0f;
            for (int64_t k = 0; k < K; ++k) q[m * K + k] = 0;
            continue;
        }
        float sc = amax / 127.0f;
        s[m] = sc;
        for (int64_t k = 0; k < K; ++k) {
            float r = rintf(bf16_to_f32(xr[k]) / sc);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            q[m * K + k] = (int8_t)r;
        }
    }
    return 0;
}

/* ---- weightless RMSNorm (prologue of the first quantisation of a layer) -- */

int oracle_rmsnorm_bf16(int64_t M, int64_t K, const uint16_t *x, uint16_t *t) {
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *xr = x + m * K;
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double v = (double)bf16_to_f32(xr[k]);
            ss += v * v;
        }
        float ms = (float)(ss / (double)K);
        float r = 1.0f / sqrtf(ms + 1e-6f);
        for (int64_t k = 0; k < K; ++k) t[m * K + k] = f32_to_bf16(bf16_to_f32(xr[k]) * r);
    }
    return 0;
}

/* ---- weighted RMSNorm (w: bf16 [K], one weight per input column) --------- */

int oracle_wrmsnorm_bf16(int64_t M, int64_t K, const uint16_t *x, const uint16_t *w, uint16_t *t) {
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *xr = x + m * K;
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double v = (double)bf16_to_f32(xr[k]);
            ss += v * v;
        }
        float ms = (float)(ss / (double)K);
        float r = 1.0f / sqrtf(ms + 1e-6f);
        for (int64_t k = 0; k < K; ++k) {
            float a = bf16_to_f32(xr[k]) * bf16_to_f32(w[k]);   /* exact */
            t[m * K + k] = f32_to_bf16(a * r);
        }
    }
    return 0;
}

/* ---- SwiGLU: h = silu(g) * u, rounded to bf16 ----------------------------- */

int oracle_swiglu_bf16(int64_t n, const uint16_t *g, const uint16_t *u, uint16_t *h) {
    for (int64_t i = 0; i < n; ++i) {
        double gv = (double)bf16_to_f32(g[i]);
        double uv = (double)bf16_to_f32(u[i]);
        h[i] = f64_to_bf16(gv / (1.0 + exp(-gv)) * uv);
    }
    return 0;
}

/* ---- integer group dot products ------------------------------------------ */

int oracle_group_acc(int bits, int64_t M, int64_t N, int64_t K, const int8_t *q,
                     const uint8_t *canon, int32_t *acc) {
    if ((bits != 4 && bits != 6) || K % GROUP) return -1;
    int64_t G = K / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t *row = canon + n * row_bytes(bits, K);
        for (int64_t m = 0; m < M; ++m)
            for (int64_t g = 0; g < G; ++g) {
                int32_t a = 0;
                for (int64_t k = g * GROUP; k < (g + 1) * GROUP; ++k)
                    a += (int32_t)q[m * K + k] * (int32_t)code_at(bits, row, k);
                acc[(m * N + n) * G + g] = a;
            }
    }
    return 0;
}

/* ---- the linear: quantised activation x packed weights -> bf16 ---------- */

int oracle_linear(int bits, int64_t M, int64_t N, int64_t K, const int8_t *q, const float *s,
                  const uint8_t *canon, const uint16_t *scales, double *ypre, uint16_t *y) {
    if ((bits != 4 && bits != 6) || K % GROUP) return -1;
    int64_t G = K / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t *row = canon + n * row_bytes(bits, K);
        for (int64_t m = 0; m < M; ++m) {
            double tot = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                int32_t a = 0;
                for (int64_t k = g * GROUP; k < (g + 1) * GROUP; ++k)
                    a += (int32_t)q[m * K + k] * (int32_t)code_at(bits, row, k);
                tot += f16_to_f64(scales[n * G + g]) * (double)a;
            }
            double v = (double)s[m] * tot;
            if (ypre) ypre[m * N + n] = v;
            if (y) y[m * N + n] = f64_to_bf16(v);
        }
    }
    return 0;
}

/* ---- split-prefix decode attention ---------------------------------------
 *
 * "Doubling LLM token rates in ComfyUI", section "Paying attention to the
 * attention!": the decode attention of the grouped-query layers takes a short
 * query -- one token, or the committed token and the MTP draft rows with their
 * causal verification -- without a materialised mask.  What it computes is
 * ordinary scaled dot-product attention; the readings used here:
 *   - M new tokens sit at cache positions P .. P+M-1 (their keys and values
 *     are already in the cache); token i attends to positions 0 .. P+i;
 *   - query head h reads key/value head h / (n_q / n_kv);
 *   - score = (q . k) / sqrt(D), softmax over the attended positions, output
 *     = sum of softmax weight times v, rounded once to bf16 (nearest even);
 *     everything here in fp64 from the bf16 inputs.
 * Layouts: q and o [M][n_q][D]; k and v caches [n_kv][L][D] (L >= P+M). */
int oracle_decode_attention(int64_t M, int64_t n_q, int64_t n_kv, int64_t D, int64_t P, int64_t L,
                            const uint16_t *q, const uint16_t *kc, const uint16_t *vc, uint16_t *o) {
    if (n_kv < 1 || n_q % n_kv || P + M > L) return -1;
    const int64_t qpg = n_q / n_kv;
    const double scale = 1.0 / sqrt((double)D);
#pragma omp parallel for schedule(dynamic)
    for (int64_t r = 0; r < M * n_q; ++r) {
        const int64_t i = r / n_q, h = r % n_q, g = h / qpg;
        const int64_t n = P + i + 1;                   /* attended positions */
        const uint16_t *qr = q + r * D;
        const uint16_t *kg = kc + g * L * D, *vg = vc + g * L * D;
        double *s = (double *)malloc((size_t)n * sizeof(double));
        double *acc = (double *)calloc((size_t)D, sizeof(double));
        double mx = -INFINITY;
        for (int64_t p = 0; p < n; ++p) {
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d) dot += (double)bf16_to_f32(qr[d]) * (double)bf16_to_f32(kg[p * D + d]);
            s[p] = dot * scale;
            if (s[p] > mx) mx = s[p];
        }
        double den = 0.0;
        for (int64_t p = 0; p < n; ++p) {
            const double w = exp(s[p] - mx);
            den += w;
            for (int64_t d = 0; d < D; ++d) acc[d] += w * (double)bf16_to_f32(vg[p * D + d]);
        }
        for (int64_t d = 0; d < D; ++d) o[r * D + d] = f64_to_bf16(acc[d] / den);
        free(s);
        free(acc);
    }
    return 0;
}

/* Threads the OpenMP loops above use (reported with CPU timings). */
int oracle_num_threads(void) { return omp_get_max_threads(); }

/* Threads for later calls (the CPU-baseline timing runs on all cores and on one). */
void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

/* Exposed for the tests of the number formats. */
uint16_t oracle_f64_to_bf16(double v) { return f64_to_bf16(v); }
double oracle_f16_to_f64(uint16_t h) { return f16_to_f64(h); }
