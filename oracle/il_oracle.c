/*
 * il_oracle.c -- TEST INFRASTRUCTURE, not part of the product.
 *
 * A plain, slow, obviously correct CPU implementation of the accelerator
 * linear layer: a batch of matmuls over one shared f32 input,
 *
 *     y[t][n_out] = x[t][n_in] * W^T                       (1)
 *
 * as stated in the doc comment of `struct Job` on the oxinfer 0.0.0
 * `src/gpu.rs` page, with every weight W `[n_out, n_in]` row-major in one of
 * the three storage formats of `enum WeightRef` on the same page (Bf16 as raw
 * u16 bits, Q8, Q4).
 *
 * Only the test suite, the package's smoke check and the benchmark's CPU
 * baseline leg may load this file's library.  Nothing in the product path
 * links, imports or calls it, and it shares no source with the GPU path.
 *
 * Method: dequantise, then multiply.  Each weight element is decoded to the
 * f32 value it denotes; each output is the sum over k of the exact f64
 * products x*w in increasing k, rounded once to f32.  Beside it, the bound
 * sum_k |x*w| (f64) that the tolerance check scales with.
 *
 * Host formats (the pages import QMatrix / Q4Matrix without showing their
 * layout; these are this library's readings, listed with the others in the
 * design notes):
 *   BF16: uint16_t[n_out][n_in], raw bfloat16 bits.
 *   Q8  : n_out * (n_in/32) packed 36-byte blocks, row-major by (row, block),
 *         each { float32 scale (little-endian); int8 q[32]; };
 *         w = (float)q * scale   -- one f32 multiply, round-to-nearest-even.
 *   Q4  : n_out * (n_in/32) packed 18-byte blocks, row-major by (row, block),
 *         each { uint16 f16 scale bits (little-endian); uint8 qs[16]; },
 *         qs[j] holds element 2j in its low nibble, element 2j+1 in its high;
 *         w = (code - 8) * f16(scale)  -- exact in f32.
 *
 * Built with plain `gcc -O2` (no -ffast-math, no intrinsics).  OpenMP, when
 * enabled, splits rows between threads; every output is still summed
 * serially, so the result does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_BF16 = 0, ORC_Q8 = 1, ORC_Q4 = 2 };
enum { ORC_BLOCK = 32, ORC_Q8_BLOCK_BYTES = 36, ORC_Q4_BLOCK_BYTES = 18 };

/* bfloat16 -> double, from the format's definition: 1 sign bit, 8 exponent
 * bits (bias 127), 7 fraction bits; exponent 0 is subnormal (f * 2^-133),
 * exponent 255 is Inf (f == 0) or NaN. */
double orc_bf16_value(uint16_t bits)
{
    int sign = bits >> 15;
    int e = (bits >> 7) & 0xFF;
    int f = bits & 0x7F;
    double v;
    if (e == 0)
        v = ldexp((double)f, -126 - 7);
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 127 - 7);
    return sign ? -v : v;
}

/* IEEE 754 binary16 -> double, from its definition: 1 sign bit, 5 exponent
 * bits (bias 15), 10 fraction bits; exponent 0 is subnormal (f * 2^-24),
 * exponent 31 is Inf (f == 0) or NaN. */
double orc_f16_value(uint16_t bits)
{
    int sign = bits >> 15;
    int e = (bits >> 10) & 0x1F;
    int f = bits & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 15 - 10);
    return sign ? -v : v;
}

static uint16_t rd_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

static float rd_f32(const uint8_t *p)
{
    uint32_t u = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) |
                 ((uint32_t)p[3] << 24);
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Size in bytes of one weight in its host format (the storage that
 * `WeightRef::bytes` counts); -1 on a bad format or shape. */
int64_t orc_weight_bytes(int fmt, int64_t n_out, int64_t n_in)
{
    if (n_out <= 0 || n_in <= 0) return -1;
    if (fmt == ORC_BF16) return n_out * n_in * 2;
    if (n_in % ORC_BLOCK) return -1;
    if (fmt == ORC_Q8) return n_out * (n_in / ORC_BLOCK) * ORC_Q8_BLOCK_BYTES;
    if (fmt == ORC_Q4) return n_out * (n_in / ORC_BLOCK) * ORC_Q4_BLOCK_BYTES;
    return -1;
}

/* Decode row `r` of a host-format weight to f32 values w[0..n_in). */
int orc_dequant_row(const void *weight, int fmt, int64_t n_in, int64_t r, float *w)
{
    const uint8_t *base = (const uint8_t *)weight;
    if (fmt == ORC_BF16) {
        const uint8_t *row = base + (size_t)r * (size_t)n_in * 2;
        for (int64_t k = 0; k < n_in; ++k)
            w[k] = (float)orc_bf16_value(rd_u16(row + 2 * k));
        return 0;
    }
    if (n_in % ORC_BLOCK) return -1;
    int64_t nb = n_in / ORC_BLOCK;
    if (fmt == ORC_Q8) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = base + ((size_t)r * (size_t)nb + (size_t)b) * ORC_Q8_BLOCK_BYTES;
            float scale = rd_f32(blk);
            for (int e = 0; e < ORC_BLOCK; ++e) {
                float q = (float)(int8_t)blk[4 + e];
                w[b * ORC_BLOCK + e] = q * scale; /* one f32 multiply */
            }
        }
        return 0;
    }
    if (fmt == ORC_Q4) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = base + ((size_t)r * (size_t)nb + (size_t)b) * ORC_Q4_BLOCK_BYTES;
            double scale = orc_f16_value(rd_u16(blk));
            for (int e = 0; e < ORC_BLOCK; ++e) {
                uint8_t byte = blk[2 + e / 2];
                int code = (e % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
                w[b * ORC_BLOCK + e] = (float)((double)(code - 8) * scale);
            }
        }
        return 0;
    }
    return -1;
}

/* ------------------------------------------------------------- quantiser
 * The upload quantiser: the step before the matmul that builds the Q8 / Q4
 * blocks from full-precision weights.  The pages import QMatrix / Q4Matrix
 * without printing how they are built, so the rule is this library's
 * reading: symmetric absmax scaling per 32-element block of a row.  With
 * amax = max_e |w_e| over the block,
 *   Q8: s = amax / 127 (one f32 division); q_e = rint(w_e / s) clamped to
 *       [-127, 127]; the block stores s as f32;
 *   Q4: s = the f32 quotient amax / 7 rounded to the nearest binary16 (ties
 *       to even) and saturated at 65504, the largest finite binary16;
 *       code_e = rint(w_e / s) clamped to [-8, 7], plus 8, with s the stored
 *       binary16 scale read back as f32 -- so codes are chosen against the
 *       scale the dequantisation will use;
 *   a zero scale (amax == 0, or a quotient that rounds to 0) stores scale 0
 *   and all-zero values (Q8 code 0, Q4 code 8).
 * Every division is one correctly rounded f32 division and rint rounds half
 * to even (the default rounding mode).  Inputs must be finite. */

/* f32 -> binary16 bits, round to nearest even, from the format definition:
 * bias 15, 10 fraction bits, subnormal quantum 2^-24; magnitudes from 65520
 * (halfway between 65504 and 2^16) up round to Inf; NaN -> a quiet NaN. */
uint16_t orc_f16_bits(float v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs((double)v);
    if (isnan(v)) return 0x7E00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal or zero: a count of 2^-24 quanta (a count of 1024 is the
         * smallest normal number, whose bits are exactly 1024) */
        double q = nearbyint(a * ldexp(1.0, 24));
        return (uint16_t)(sign | (uint16_t)q);
    }
    int e;
    double m = frexp(a, &e); /* a = m * 2^e, m in [0.5, 1): a = (1 + f/1024) * 2^(e-1) */
    double f = nearbyint((2.0 * m - 1.0) * 1024.0);
    int be = e - 1 + 15;
    if (f == 1024.0) {
        f = 0.0;
        ++be;
    }
    if (be >= 31) return sign | 0x7C00; /* rounded past 65504: Inf */
    return (uint16_t)(sign | (uint16_t)(be << 10) | (uint16_t)f);
}

void orc_f16_bits_array(const float *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_bits(v[i]);
}

static void wr_f32(uint8_t *p, float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    p[0] = (uint8_t)u;
    p[1] = (uint8_t)(u >> 8);
    p[2] = (uint8_t)(u >> 16);
    p[3] = (uint8_t)(u >> 24);
}

/* f32 weights [n_out][n_in] -> host-format Q8 or Q4 blocks in `out`
 * (orc_weight_bytes(fmt, n_out, n_in) bytes).  Returns 0, or -1 on a bad
 * format (bf16 is not a quantised format) or shape. */
int orc_quantize(const float *w, int fmt, int64_t n_out, int64_t n_in, uint8_t *out)
{
    if (fmt != ORC_Q8 && fmt != ORC_Q4) return -1;
    if (orc_weight_bytes(fmt, n_out, n_in) < 0) return -1;
    int64_t nb = n_in / ORC_BLOCK;
    for (int64_t r = 0; r < n_out; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const float *src = w + (size_t)r * (size_t)n_in + (size_t)b * ORC_BLOCK;
            float amax = 0.0f;
            for (int e = 0; e < ORC_BLOCK; ++e)
                if (fabsf(src[e]) > amax) amax = fabsf(src[e]);
            if (fmt == ORC_Q8) {
                uint8_t *blk = out + ((size_t)r * (size_t)nb + (size_t)b) * ORC_Q8_BLOCK_BYTES;
                float s = amax / 127.0f;
                wr_f32(blk, s);
                for (int e = 0; e < ORC_BLOCK; ++e) {
                    float q = 0.0f;
                    if (s != 0.0f) {
                        q = rintf(src[e] / s);
                        if (q > 127.0f) q = 127.0f;
                        if (q < -127.0f) q = -127.0f;
                    }
                    blk[4 + e] = (uint8_t)(int8_t)q;
                }
            } else {
                uint8_t *blk = out + ((size_t)r * (size_t)nb + (size_t)b) * ORC_Q4_BLOCK_BYTES;
                uint16_t sb = orc_f16_bits(amax / 7.0f);
                if (sb == 0x7C00) sb = 0x7BFF; /* saturate at 65504 */
                float s = (float)orc_f16_value(sb);
                blk[0] = (uint8_t)sb;
                blk[1] = (uint8_t)(sb >> 8);
                memset(blk + 2, 0, 16);
                for (int e = 0; e < ORC_BLOCK; ++e) {
                    int code = 8;
                    if (s != 0.0f) {
                        float q = rintf(src[e] / s);
                        if (q > 7.0f) q = 7.0f;
                        if (q < -8.0f) q = -8.0f;
                        code = (int)q + 8;
                    }
                    blk[2 + e / 2] |= (uint8_t)((e % 2 == 0) ? code : code << 4);
                }
            }
        }
    }
    return 0;
}

/* Equation (1) for output rows [r0, r1) of one weight.  y and bound are
 * [t][r1 - r0] row-major: y[i][j] = (float) sum_k x[i][k] * w[r0 + j][k] with
 * f64 products and an f64 running sum in increasing k; bound[i][j] =
 * sum_k |x[i][k] * w[r0 + j][k]| in f64.  Returns 0, or -1 on bad arguments. */
int orc_matmul_rows(const float *x, int64_t t, int64_t n_in, const void *weight, int fmt,
                    int64_t n_out, int64_t r0, int64_t r1, float *y, double *bound,
                    int nthreads)
{
    if (t < 0 || n_in <= 0 || r0 < 0 || r1 > n_out || r0 > r1) return -1;
    if (orc_weight_bytes(fmt, n_out, n_in) < 0) return -1;
    int64_t nr = r1 - r0;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : failed)
#endif
    {
        float *w = (float *)malloc((size_t)n_in * sizeof(float));
        if (!w) {
            failed = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
            for (int64_t j = 0; j < nr; ++j) {
                if (orc_dequant_row(weight, fmt, n_in, r0 + j, w)) {
                    failed = 1;
                    continue;
                }
                for (int64_t i = 0; i < t; ++i) {
                    const float *xi = x + (size_t)i * (size_t)n_in;
                    double acc = 0.0, mag = 0.0;
                    for (int64_t k = 0; k < n_in; ++k) {
                        double p = (double)xi[k] * (double)w[k];
                        acc += p;
                        mag += fabs(p);
                    }
                    y[(size_t)i * (size_t)nr + (size_t)j] = (float)acc;
                    bound[(size_t)i * (size_t)nr + (size_t)j] = mag;
                }
            }
            free(w);
        }
    }
    (void)nthreads;
    return failed ? -1 : 0;
}

/* Equation (1) at chosen points only: y[p] = output (ii[p], rr[p]).  Used to
 * check full-size GPU results on a sample the oracle computes one by one. */
int orc_matmul_points(const float *x, int64_t t, int64_t n_in, const void *weight, int fmt,
                      int64_t n_out, int64_t n_pts, const int64_t *ii, const int64_t *rr,
                      float *y, double *bound, int nthreads)
{
    if (t < 0 || n_in <= 0 || n_pts < 0) return -1;
    if (orc_weight_bytes(fmt, n_out, n_in) < 0) return -1;
    for (int64_t p = 0; p < n_pts; ++p)
        if (ii[p] < 0 || ii[p] >= t || rr[p] < 0 || rr[p] >= n_out) return -1;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : failed)
#endif
    {
        float *w = (float *)malloc((size_t)n_in * sizeof(float));
        if (!w) {
            failed = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
            for (int64_t p = 0; p < n_pts; ++p) {
                if (orc_dequant_row(weight, fmt, n_in, rr[p], w)) {
                    failed = 1;
                    continue;
                }
                const float *xi = x + (size_t)ii[p] * (size_t)n_in;
                double acc = 0.0, mag = 0.0;
                for (int64_t k = 0; k < n_in; ++k) {
                    double prod = (double)xi[k] * (double)w[k];
                    acc += prod;
                    mag += fabs(prod);
                }
                y[p] = (float)acc;
                bound[p] = mag;
            }
            free(w);
        }
    }
    (void)nthreads;
    return failed ? -1 : 0;
}

/* ------------------------------------------------ fused gate/up + GELU
 * The feed-forward step of the drafter page (oxinfer 0.0.1 src/drafter.rs,
 * `Drafter::step`): gate and up projections of the same input, then
 * `gelu_mul(&mut g, &u)`, i.e. g <- GELU(g) * u element-wise.  The page calls
 * gelu_mul without printing it; the reading taken is the plain GELU,
 *     GELU(v) = v * Phi(v) = 0.5 * v * (1 + erf(v / sqrt(2))),
 * Phi the standard normal CDF (erf from the C library, in double).
 *
 * For output rows [r0, r1) of the two weights (same format and shape):
 *   G, U = the f64 sums of (1) for the gate and up rows (as orc_matmul_rows),
 *   y    = (float)(GELU(G) * U),
 *   bound such that 4e-3 * bound is the error a product of two matmuls each
 *   within 4e-3 * sum|x*w| of its exact value may carry:
 *     |GELU(g) u - GELU(G) U| <= L tau Bg (|U| + tau Bu) + |GELU(G)| tau Bu
 *   with tau = 4e-3, Bg / Bu the sum |x*w| of each row and L = 1.13 >= the
 *   largest slope of GELU (Phi(v) + v phi(v) peaks at 1.1289 at v = sqrt 2);
 *   plus 2^-20 |y| for the rounding of the final product, divided by tau. */
double orc_gelu(double v) { return 0.5 * v * (1.0 + erf(v / sqrt(2.0))); }

int orc_gelu_mul_rows(const float *x, int64_t t, int64_t n_in, const void *gate, const void *up, int fmt,
                      int64_t n_out, int64_t r0, int64_t r1, float *y, double *bound, int nthreads)
{
    if (t < 0 || n_in <= 0 || r0 < 0 || r1 > n_out || r0 > r1) return -1;
    if (orc_weight_bytes(fmt, n_out, n_in) < 0) return -1;
    const double tau = 4e-3, lip = 1.13;
    int64_t nr = r1 - r0;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : failed)
#endif
    {
        float *wg = (float *)malloc((size_t)n_in * sizeof(float));
        float *wu = (float *)malloc((size_t)n_in * sizeof(float));
        if (!wg || !wu) {
            failed = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
            for (int64_t j = 0; j < nr; ++j) {
                if (orc_dequant_row(gate, fmt, n_in, r0 + j, wg) || orc_dequant_row(up, fmt, n_in, r0 + j, wu)) {
                    failed = 1;
                    continue;
                }
                for (int64_t i = 0; i < t; ++i) {
                    const float *xrow = x + (size_t)i * (size_t)n_in;
                    double g = 0.0, u = 0.0, bg = 0.0, bu = 0.0;
                    for (int64_t k = 0; k < n_in; ++k) {
                        double gk = (double)xrow[k] * (double)wg[k];
                        double uk = (double)xrow[k] * (double)wu[k];
                        g += gk;
                        u += uk;
                        bg += fabs(gk);
                        bu += fabs(uk);
                    }
                    double gl = orc_gelu(g);
                    double v = gl * u;
                    double allow = lip * tau * bg * (fabs(u) + tau * bu) + fabs(gl) * tau * bu +
                                   ldexp(fabs(v), -20);
                    y[(size_t)i * (size_t)nr + (size_t)j] = (float)v;
                    bound[(size_t)i * (size_t)nr + (size_t)j] = allow / tau;
                }
            }
        }
        free(wg);
        free(wu);
    }
    (void)nthreads;
    return failed ? -1 : 0;
}

/* ------------------------------------------- centroid-masked LM head
 * The end of `Drafter::step` on the oxinfer 0.0.1 src/drafter.rs page: for
 * each row x (length h) of a batch,
 *   1. centroid logits cl[c] = centroids[c] . x for the C centroids (bf16
 *      rows, [C, h]);
 *   2. the k centroids with the largest logits;
 *   3. for each chosen cluster c and j < per = V / C, the token
 *      ordering[c * per + j] and its score embed[token] . x (bf16 rows of
 *      the [V, h] embedding);
 *   4. the token of the largest score, the first one met winning ties, the
 *      clusters visited in the order of step 2 and tokens in j order.
 * The page selects with select_nth_unstable, which leaves the order of the k
 * clusters (and the choice among equal logits at the k-th place) open; the
 * reading taken here: clusters ordered by decreasing logit, equal logits by
 * increasing cluster index.  Logits and scores are exact f64 sums of the f64
 * products, and each decision is taken on them rounded once to f32 (the
 * precision the page computes them in).
 * Outputs per row: the token, the k clusters in visiting order, the f32
 * score of the token, and for the checks the f64 logits and their bounds
 * sum |x * w| (cl, cl_bound: [t][C]). */
static double orc_bf16_dot(const uint16_t *w, const float *x, int64_t h, double *mag)
{
    double acc = 0.0, m = 0.0;
    for (int64_t e = 0; e < h; ++e) {
        double p = orc_bf16_value(w[e]) * (double)x[e];
        acc += p;
        m += fabs(p);
    }
    if (mag) *mag = m;
    return acc;
}

int orc_centroid_argmax(const float *x, int64_t t, int64_t h, const uint16_t *centroids, int64_t n_c,
                        const uint16_t *embed, int64_t vocab, const uint32_t *ordering, int64_t k,
                        int32_t *token, int32_t *clusters, float *score, double *cl, double *cl_bound)
{
    if (t < 0 || h <= 0 || n_c <= 0 || k < 1 || vocab < n_c || vocab % n_c) return -1;
    if (k > n_c) k = n_c; /* the page takes top_k_centroids.min(num_centroids) */
    const int64_t per = vocab / n_c;
    for (int64_t v = 0; v < vocab; ++v)
        if (ordering[v] >= (uint64_t)vocab) return -1;
    int64_t *idx = (int64_t *)malloc((size_t)n_c * sizeof(int64_t));
    float *clf = (float *)malloc((size_t)n_c * sizeof(float));
    if (!idx || !clf) {
        free(idx);
        free(clf);
        return -1;
    }
    for (int64_t i = 0; i < t; ++i) {
        const float *xi = x + (size_t)i * (size_t)h;
        double *cli = cl + (size_t)i * (size_t)n_c;
        double *cbi = cl_bound + (size_t)i * (size_t)n_c;
        for (int64_t c = 0; c < n_c; ++c) {
            cli[c] = orc_bf16_dot(centroids + (size_t)c * (size_t)h, xi, h, &cbi[c]);
            clf[c] = (float)cli[c];
            idx[c] = c;
        }
        /* the k largest f32 logits, equal logits by increasing index: a
         * selection sort over the first k places */
        for (int64_t a = 0; a < k; ++a) {
            int64_t best = a;
            for (int64_t b = a + 1; b < n_c; ++b) {
                float vb = clf[idx[b]], vbest = clf[idx[best]];
                if (vb > vbest || (vb == vbest && idx[b] < idx[best])) best = b;
            }
            int64_t tmp = idx[a];
            idx[a] = idx[best];
            idx[best] = tmp;
        }
        float best_s = -INFINITY;
        int32_t best_tok = -1;
        for (int64_t a = 0; a < k; ++a) {
            const int64_t c = idx[a];
            clusters[(size_t)i * (size_t)k + (size_t)a] = (int32_t)c;
            for (int64_t j = 0; j < per; ++j) {
                const uint32_t tok = ordering[c * per + j];
                float sc = (float)orc_bf16_dot(embed + (size_t)tok * (size_t)h, xi, h, NULL);
                if (best_tok < 0 || sc > best_s) {
                    best_s = sc;
                    best_tok = (int32_t)tok;
                }
            }
        }
        token[i] = best_tok;
        score[i] = best_s;
    }
    free(idx);
    free(clf);
    return 0;
}

/* Exact score (f64) and its bound of one token for row x: embed[tok] . x. */
double orc_token_score(const float *x, int64_t h, const uint16_t *embed, int64_t tok, double *bound)
{
    return orc_bf16_dot(embed + (size_t)tok * (size_t)h, x, h, bound);
}

/* The acceptance test on n outputs: |y - y_ref| <= tol * bound, element by
 * element; a NaN or Inf in y always fails, and bound == 0 demands y == y_ref.
 * Returns the number of failing elements; *first_bad is the first failing
 * index (-1 if none) and *worst the largest |y - y_ref| / bound seen (an
 * element with bound == 0 and y != y_ref counts as +Inf). */
int64_t orc_check(const float *y, const float *y_ref, const double *bound, int64_t n,
                  double tol, int64_t *first_bad, double *worst)
{
    int64_t bad = 0;
    double wmax = 0.0;
    if (first_bad) *first_bad = -1;
    for (int64_t e = 0; e < n; ++e) {
        double got = (double)y[e];
        double want = (double)y_ref[e];
        double err = fabs(got - want);
        double ratio;
        int ok;
        if (isnan(got) || isinf(got)) {
            ok = 0;
            ratio = INFINITY;
        } else if (bound[e] == 0.0) {
            ok = (err == 0.0);
            ratio = ok ? 0.0 : INFINITY;
        } else {
            ratio = err / bound[e];
            ok = (err <= tol * bound[e]);
        }
        if (!(ratio <= wmax)) wmax = ratio;
        if (!ok) {
            if (bad == 0 && first_bad) *first_bad = e;
            ++bad;
        }
    }
    if (worst) *worst = wmax;
    return bad;
}
