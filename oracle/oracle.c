/*
 * oracle.c -- plain, slow, obviously-correct CPU reference for the quantized
 * mixture-of-experts expert matmul (Q4_0 weights x Q8_1 activations).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or constant
 * with the HIP library.
 *
 * What is computed (sources):
 *   - The hot path: for every flat (token, top-k) pair p = t*top_k + j, take
 *     the expert e = topk_ids[t][j], and dot each Q4_0 weight row of expert e
 *     with token t's Q8_1 activation row; one output row per pair.
 *     [FreeToken PR #185 "fix(kernel): launch GGUF MoE GEMV token axis on
 *      grid.x, not grid.z", sections Problem and Fix: the MoE GEMV runs one
 *      grid entry per flat (token, top-k) index with Q8_1 activations]
 *   - Expert ids outside [0, E) give an all-zero output row (the masking of
 *     non-local experts described in "Current Bug: CuTeDSLMoERunner", Bug 8).
 *   - The second layer of an expert FFN takes one activation row per pair
 *     (what the first layer produced for that pair, "Current Bug:
 *     CuTeDSLMoERunner", Bug 6): the same matmul with activation row p instead
 *     of t.  Its outputs are combined per token as the router-weighted sum
 *     out[t][n] = sum_j gates[t][j] * y[t*top_k + j][n] (the usual top-k MoE
 *     combine; the pages do not print it).
 *   - The first layer's output feeds a gated activation: the matmul output of
 *     a pair holds the gate in columns [0, I) and the up projection in
 *     [I, 2I), and the layer's output is act(gate) * up, [rows][I].  The
 *     activations are the tanh-approximated GELU that follows the GEMV in
 *     FreeToken PR #185 (Problem) and SiLU ("Current Bug: CuTeDSLMoERunner",
 *     Bug 6).  The [gate | up] order of the halves is a reading; the pages
 *     print no layout.
 *   - The byte layouts are the GGUF Q4_0 / Q8_1 blocks the FreeToken page
 *     serves ("Tested on": a Q4_0 .gguf checkpoint).  The pages name the
 *     formats but do not print them; the readings used here are:
 *       Q4_0 block (18 B) = fp16 d, then 16 bytes; byte i holds element i in
 *         its low nibble and element i+16 in its high nibble; value = (q-8)*d.
 *       Q8_1 block (36 B) = fp16 d, fp16 s, then 32 int8 q; value = q*d,
 *         s = d * sum(q) (stored, not used by the matmul).
 *   - Quantisers (data preparation): Q8_1: d = amax/127, q = round(x/d)
 *     (half away from zero), q = 0 when amax = 0.  Q4_0: m = the element of
 *     largest magnitude (first on ties), d = m / -8, q = clamp(round(x/d)+8,
 *     0, 15), q = 8 when d = 0.  Both decisions are taken in fp32, the
 *     precision the kernels use.
 *
 * Precision: integer partials are exact int32; every floating-point output of
 * the matmul is computed in fp64.  Each block term P*d4*d8 is exact in fp64
 * (at most 15+11+11 significant bits); only the fp64 sum over blocks rounds.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no intrinsics).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define QK 32           /* values per block */
#define Q4_0_BYTES 18   /* fp16 d + 16 nibble bytes */
#define Q8_1_BYTES 36   /* fp16 d + fp16 s + 32 int8 */

/* ------------------------------------------------------------------------ */
/* IEEE binary16 conversions, written from the format definition:           */
/* 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0 holds */
/* subnormals (fraction * 2^-24), exponent 31 holds inf / NaN.               */
/* ------------------------------------------------------------------------ */

float oracle_fp16_to_fp32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int exp = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (exp == 0) {
        v = ldexp((double)frac, -24);                 /* subnormal or zero */
    } else if (exp == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + frac), exp - 25);   /* (1.frac) * 2^(exp-15) */
    }
    return (float)(sign ? -v : v);
}

/* Round to nearest, ties to even; subnormals kept; overflow -> inf. */
uint16_t oracle_fp32_to_fp16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    double v = fabs((double)f);
    if (isnan(f)) return (uint16_t)(sign | 0x7e00);
    if (isinf(f)) return (uint16_t)(sign | 0x7c00);
    if (v == 0.0) return sign;

    /* spacing of binary16 values around v */
    int ex;
    frexp(v, &ex);               /* v = fr * 2^ex, fr in [0.5, 1) */
    int e = ex - 1;              /* v in [2^e, 2^(e+1)) */
    if (e < -14) e = -14;        /* subnormal range shares the 2^-24 spacing */
    double ulp = ldexp(1.0, e - 10);
    double r = nearbyint(v / ulp);   /* exact division by a power of two; ties-to-even */
    double u = r * ulp;              /* the rounded magnitude, exact */

    if (u > 65504.0) return (uint16_t)(sign | 0x7c00);
    if (u < ldexp(1.0, -14)) {
        return (uint16_t)(sign | (uint16_t)(u / ldexp(1.0, -24)));  /* subnormal */
    }
    frexp(u, &ex);
    e = ex - 1;
    int frac = (int)(u / ldexp(1.0, e - 10)) - 1024;
    return (uint16_t)(sign | ((e + 15) << 10) | frac);
}

/* Array forms, so the conversions can be checked exhaustively from Python. */
void oracle_fp16_to_fp32_array(const uint16_t* h, int64_t n, float* f)
{
    for (int64_t i = 0; i < n; ++i) f[i] = oracle_fp16_to_fp32(h[i]);
}

void oracle_fp32_to_fp16_array(const float* f, int64_t n, uint16_t* h)
{
    for (int64_t i = 0; i < n; ++i) h[i] = oracle_fp32_to_fp16(f[i]);
}

/* ------------------------------------------------------------------------ */
/* Quantisers.                                                              */
/* ------------------------------------------------------------------------ */

static void put_u16(uint8_t* p, uint16_t v) { p[0] = (uint8_t)(v & 0xff); p[1] = (uint8_t)(v >> 8); }
static uint16_t get_u16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* x: fp32 [rows][K] row-major, K % 32 == 0.  y: [rows][K/32] Q8_1 blocks. */
void oracle_quantize_q8_1(const float* x, int64_t rows, int64_t K, uint8_t* y)
{
    int64_t nb = K / QK;
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const float* xb = x + r * K + b * QK;
            uint8_t* yb = y + (r * nb + b) * Q8_1_BYTES;
            float amax = 0.0f;
            for (int i = 0; i < QK; ++i) {
                float m = fabsf(xb[i]);
                if (m > amax) amax = m;
            }
            float d = amax / 127.0f;
            int sum = 0;
            for (int i = 0; i < QK; ++i) {
                int q = (amax == 0.0f) ? 0 : (int)roundf(xb[i] / d);
                yb[4 + i] = (uint8_t)(int8_t)q;
                sum += q;
            }
            float s = d * (float)sum;
            put_u16(yb + 0, oracle_fp32_to_fp16(d));
            put_u16(yb + 2, oracle_fp32_to_fp16(s));
        }
    }
}

/* w: fp32 [rows][K] row-major.  y: [rows][K/32] Q4_0 blocks. */
void oracle_quantize_q4_0(const float* w, int64_t rows, int64_t K, uint8_t* y)
{
    int64_t nb = K / QK;
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const float* xb = w + r * K + b * QK;
            uint8_t* yb = y + (r * nb + b) * Q4_0_BYTES;
            float m = 0.0f, amax = 0.0f;
            for (int i = 0; i < QK; ++i) {
                if (fabsf(xb[i]) > amax) { amax = fabsf(xb[i]); m = xb[i]; }
            }
            float d = m / -8.0f;
            int q[QK];
            for (int i = 0; i < QK; ++i) {
                if (d == 0.0f) { q[i] = 8; continue; }
                int v = (int)roundf(xb[i] / d) + 8;
                q[i] = v < 0 ? 0 : (v > 15 ? 15 : v);
            }
            put_u16(yb, oracle_fp32_to_fp16(d));
            for (int i = 0; i < QK / 2; ++i) {
                yb[2 + i] = (uint8_t)(q[i] | (q[i + QK / 2] << 4));
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Block decoding.                                                          */
/* ------------------------------------------------------------------------ */

/* Weight code of element i (0..31) of a Q4_0 block, already minus 8. */
static int q4_value(const uint8_t* blk, int i)
{
    uint8_t byte = blk[2 + (i % 16)];
    int nib = (i < 16) ? (byte & 0x0f) : (byte >> 4);
    return nib - 8;
}

static int q8_value(const uint8_t* blk, int i)
{
    return (int)(int8_t)blk[4 + i];
}

/* Integer dot product of one Q4_0 block with one Q8_1 block: exact. */
static int32_t block_partial(const uint8_t* wblk, const uint8_t* ablk)
{
    int32_t p = 0;
    for (int i = 0; i < QK; ++i) p += q4_value(wblk, i) * q8_value(ablk, i);
    return p;
}

static const uint8_t* weight_block(const uint8_t* w, int64_t e, int64_t n, int64_t b, int64_t N, int64_t nb)
{
    return w + ((e * N + n) * nb + b) * Q4_0_BYTES;
}

static const uint8_t* act_block(const uint8_t* a, int64_t t, int64_t b, int64_t nb)
{
    return a + (t * nb + b) * Q8_1_BYTES;
}

/* ------------------------------------------------------------------------ */
/* The MoE expert matmul.                                                   */
/* ------------------------------------------------------------------------ */

/* One output row: out[n] = sum_b P[n][b] * d4[n][b] * d8[b] in fp64.
 * abssum (nullable) gets sum_b |term| for error bounds. */
static void one_pair(const uint8_t* w, const uint8_t* a, int64_t e, int64_t t,
                     int64_t E, int64_t N, int64_t nb, double* out, double* abssum)
{
    for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0, aabs = 0.0;
        if (e >= 0 && e < E) {
            for (int64_t b = 0; b < nb; ++b) {
                const uint8_t* wb = weight_block(w, e, n, b, N, nb);
                const uint8_t* ab = act_block(a, t, b, nb);
                double d4 = (double)oracle_fp16_to_fp32(get_u16(wb));
                double d8 = (double)oracle_fp16_to_fp32(get_u16(ab));
                double term = (double)block_partial(wb, ab) * d4 * d8;
                acc += term;
                aabs += fabs(term);
            }
        }
        out[n] = acc;
        if (abssum) abssum[n] = aabs;
    }
}

/* w: [E][N][K/32] Q4_0; ids: [T][top_k] int32; out: [T*top_k][N] fp64;
 * abssum: same shape or NULL.  a: Q8_1 rows; pair p reads row p / act_div
 * (act_div = top_k: a is [T][K/32], one row per token; act_div = 1: a is
 * [T*top_k][K/32], one row per pair). */
void oracle_moe_ex(const uint8_t* w, const uint8_t* a, const int32_t* ids,
                   int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k, int64_t act_div,
                   double* out, double* abssum)
{
    int64_t nb = K / QK;
    int64_t p;
#pragma omp parallel for schedule(dynamic, 1)
    for (p = 0; p < T * top_k; ++p) {
        int64_t row = p / act_div;
        one_pair(w, a, (int64_t)ids[p], row, E, N, nb, out + p * N, abssum ? abssum + p * N : NULL);
    }
}

void oracle_moe(const uint8_t* w, const uint8_t* a, const int32_t* ids,
                int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k,
                double* out, double* abssum)
{
    oracle_moe_ex(w, a, ids, E, N, K, T, top_k, top_k, out, abssum);
}

/* The same for a chosen list of pairs: out row i belongs to pair pairs[i]. */
void oracle_moe_pairs_ex(const uint8_t* w, const uint8_t* a, const int32_t* ids,
                         int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k, int64_t act_div,
                         const int64_t* pairs, int64_t npairs, double* out, double* abssum)
{
    int64_t nb = K / QK;
    int64_t i;
    (void)T;
    (void)top_k;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < npairs; ++i) {
        int64_t p = pairs[i];
        one_pair(w, a, (int64_t)ids[p], p / act_div, E, N, nb, out + i * N, abssum ? abssum + i * N : NULL);
    }
}

void oracle_moe_pairs(const uint8_t* w, const uint8_t* a, const int32_t* ids,
                      int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k,
                      const int64_t* pairs, int64_t npairs, double* out, double* abssum)
{
    oracle_moe_pairs_ex(w, a, ids, E, N, K, T, top_k, top_k, pairs, npairs, out, abssum);
}

/* Integer partials P[p][n][b]; masked pairs give zeros; pair p reads
 * activation row p / act_div. */
void oracle_moe_partials_ex(const uint8_t* w, const uint8_t* a, const int32_t* ids,
                            int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k, int64_t act_div,
                            int32_t* partials)
{
    int64_t nb = K / QK;
    int64_t p;
#pragma omp parallel for schedule(dynamic, 1)
    for (p = 0; p < T * top_k; ++p) {
        int64_t t = p / act_div;
        int64_t e = ids[p];
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t b = 0; b < nb; ++b) {
                int32_t v = 0;
                if (e >= 0 && e < E)
                    v = block_partial(weight_block(w, e, n, b, N, nb), act_block(a, t, b, nb));
                partials[(p * N + n) * nb + b] = v;
            }
        }
    }
}

void oracle_moe_partials(const uint8_t* w, const uint8_t* a, const int32_t* ids,
                         int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k,
                         int32_t* partials)
{
    oracle_moe_partials_ex(w, a, ids, E, N, K, T, top_k, top_k, partials);
}

/* Top-k combine in fp64: out[t][n] = sum_j gates[t][j] * y[t*top_k + j][n],
 * abssum[t][n] = sum_j |gates[t][j] * y[t*top_k + j][n]| (nullable).
 * y: [T*top_k][N] fp64; gates: [T][top_k] fp32; out: [T][N] fp64. */
void oracle_combine_topk(const double* y, const float* gates, int64_t T, int64_t top_k, int64_t N,
                         double* out, double* abssum)
{
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < T; ++t) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, aabs = 0.0;
            for (int64_t j = 0; j < top_k; ++j) {
                double term = (double)gates[t * top_k + j] * y[(t * top_k + j) * N + n];
                acc += term;
                aabs += fabs(term);
            }
            out[t * N + n] = acc;
            if (abssum) abssum[t * N + n] = aabs;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Sibling GGUF weight formats against Q8_1 activations.                    */
/* ------------------------------------------------------------------------ */
/* FreeToken PR #185 (Problem) counts launchers for the other GGUF block
 * types sharing the GEMV's geometry; the pages print none of their layouts.
 * Reading: the GGUF layouts, type ids as in GGUF files:
 *   Q4_1 (3, 20 B): fp16 d, fp16 m, 16 nibble bytes    w = q d + m,    q in 0..15
 *   Q5_0 (6, 22 B): fp16 d, 32-bit qh, 16 nibble bytes w = (q - 16) d, q in 0..31
 *   Q5_1 (7, 24 B): fp16 d, fp16 m, qh, 16 nibble bytes w = q d + m,   q in 0..31
 *   Q8_0 (8, 34 B): fp16 d, 32 int8                      w = q d
 * (Q4_0 is type 2.)  Nibble byte i holds element i (low) and i + 16 (high);
 * bit i of qh (little-endian) is bit 4 of element i.  The matmul is the dot
 * product of the dequantised weights and the dequantised Q8_1 activations;
 * per block that is d d8 sum((q - z) q8) + m d8 sum(q8), z the format's zero
 * point (8, 16 or 0), exact in fp64.  The Q8_1 s field is not used. */

int oracle_w_block_bytes(int type)
{
    switch (type) {
    case 2: return 18;
    case 3: return 20;
    case 6: return 22;
    case 7: return 24;
    case 8: return 34;
    default: return 0;
    }
}

/* codes q[32], zero point, scale, offset of one block */
static void w_decode(int type, const uint8_t* blk, int q[32], int* zero, double* d, double* m)
{
    *d = (double)oracle_fp16_to_fp32(get_u16(blk));
    *m = 0.0;
    *zero = 0;
    const uint8_t* nib = NULL;
    uint32_t qh = 0;
    switch (type) {
    case 2: nib = blk + 2; *zero = 8; break;
    case 3: *m = (double)oracle_fp16_to_fp32(get_u16(blk + 2)); nib = blk + 4; break;
    case 6:
        qh = (uint32_t)blk[2] | ((uint32_t)blk[3] << 8) | ((uint32_t)blk[4] << 16) | ((uint32_t)blk[5] << 24);
        nib = blk + 6; *zero = 16; break;
    case 7:
        *m = (double)oracle_fp16_to_fp32(get_u16(blk + 2));
        qh = (uint32_t)blk[4] | ((uint32_t)blk[5] << 8) | ((uint32_t)blk[6] << 16) | ((uint32_t)blk[7] << 24);
        nib = blk + 8; break;
    case 8:
        for (int i = 0; i < QK; ++i) q[i] = (int)(int8_t)blk[2 + i];
        return;
    default: return;
    }
    for (int i = 0; i < QK; ++i) {
        int v = (i < 16) ? (nib[i] & 0x0f) : (nib[i - 16] >> 4);
        if (type == 6 || type == 7) v |= (int)((qh >> i) & 1u) << 4;
        q[i] = v;
    }
}

static void w_encode(int type, const int q[32], float d, float m, uint8_t* blk)
{
    put_u16(blk, oracle_fp32_to_fp16(d));
    if (type == 8) {
        for (int i = 0; i < QK; ++i) blk[2 + i] = (uint8_t)(int8_t)q[i];
        return;
    }
    uint8_t* nib = blk + 2;
    uint32_t qh = 0;
    for (int i = 0; i < QK; ++i) qh |= (uint32_t)((q[i] >> 4) & 1) << i;
    if (type == 3 || type == 7) { put_u16(blk + 2, oracle_fp32_to_fp16(m)); nib = blk + 4; }
    if (type == 6 || type == 7) {
        uint8_t* h = (type == 6) ? blk + 2 : blk + 4;
        for (int k = 0; k < 4; ++k) h[k] = (uint8_t)(qh >> (8 * k));
        nib = h + 4;
    }
    for (int i = 0; i < QK / 2; ++i) nib[i] = (uint8_t)((q[i] & 0x0f) | ((q[i + 16] & 0x0f) << 4));
}

/* Quantise fp32 rows [rows][K] into blocks of `type` (test input generation):
 * symmetric formats scale by the element of largest magnitude (Q5_0: d =
 * that element / -16, Q8_0: d = max|x| / 127), offset formats by the range
 * (d = (max - min) / levels, m = min); codes round to nearest and clamp. */
void oracle_quantize_w(int type, const float* w, int64_t rows, int64_t K, uint8_t* y)
{
    const int64_t nb = K / QK;
    const int bytes = oracle_w_block_bytes(type);
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const float* xb = w + r * K + b * QK;
            uint8_t* yb = y + (r * nb + b) * bytes;
            float mn = xb[0], mx = xb[0], amax = 0.0f, sgn = 0.0f;
            for (int i = 0; i < QK; ++i) {
                if (xb[i] < mn) mn = xb[i];
                if (xb[i] > mx) mx = xb[i];
                if (fabsf(xb[i]) > amax) { amax = fabsf(xb[i]); sgn = xb[i]; }
            }
            int q[QK];
            float d = 0.0f, m = 0.0f;
            if (type == 2 || type == 6) {
                const int half = (type == 2) ? 8 : 16;
                d = sgn / (float)-half;
                for (int i = 0; i < QK; ++i) {
                    int v = d == 0.0f ? half : (int)roundf(xb[i] / d) + half;
                    q[i] = v < 0 ? 0 : (v > 2 * half - 1 ? 2 * half - 1 : v);
                }
            } else if (type == 8) {
                d = amax / 127.0f;
                for (int i = 0; i < QK; ++i) q[i] = d == 0.0f ? 0 : (int)roundf(xb[i] / d);
            } else {
                const int levels = (type == 3) ? 15 : 31;
                d = (mx - mn) / (float)levels;
                m = mn;
                for (int i = 0; i < QK; ++i) {
                    int v = d == 0.0f ? 0 : (int)roundf((xb[i] - mn) / d);
                    q[i] = v < 0 ? 0 : (v > levels ? levels : v);
                }
            }
            if (type == 2) {   /* the Q4_0 layout */
                put_u16(yb, oracle_fp32_to_fp16(d));
                for (int i = 0; i < QK / 2; ++i) yb[2 + i] = (uint8_t)(q[i] | (q[i + QK / 2] << 4));
            } else {
                w_encode(type, q, d, m, yb);
            }
        }
    }
}

/* One block: integer part P = sum (q - z) q8, the activation sum S = sum q8,
 * and the fp64 term d d8 P + m d8 S with the sum of the absolute parts. */
static void w_block(int type, const uint8_t* wb, const uint8_t* ab, int32_t* P, double* term, double* absterm)
{
    int q[QK], z;
    double d, m;
    w_decode(type, wb, q, &z, &d, &m);
    const double d8 = (double)oracle_fp16_to_fp32(get_u16(ab));
    int32_t p = 0, sum = 0;
    for (int i = 0; i < QK; ++i) {
        const int a = q8_value(ab, i);
        p += (q[i] - z) * a;
        sum += a;
    }
    *P = p;
    const double t1 = d * d8 * (double)p, t2 = m * d8 * (double)sum;
    *term = t1 + t2;
    *absterm = fabs(t1) + fabs(t2);
}

static void w_pair(int type, const uint8_t* w, const uint8_t* a, int64_t e, int64_t row,
                   int64_t E, int64_t N, int64_t nb, double* out, double* abssum)
{
    const int bytes = oracle_w_block_bytes(type);
    for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0, aabs = 0.0;
        if (e >= 0 && e < E) {
            for (int64_t b = 0; b < nb; ++b) {
                int32_t P;
                double t, at;
                w_block(type, w + ((e * N + n) * nb + b) * bytes, act_block(a, row, b, nb), &P, &t, &at);
                acc += t;
                aabs += at;
            }
        }
        out[n] = acc;
        if (abssum) abssum[n] = aabs;
    }
}

/* The matmul for weights of `type`: as oracle_moe_pairs_ex (pair p reads
 * activation row p / act_div; out row i belongs to pair pairs[i]). */
void oracle_moe_w_pairs(int type, const uint8_t* w, const uint8_t* a, const int32_t* ids,
                        int64_t E, int64_t N, int64_t K, int64_t act_div,
                        const int64_t* pairs, int64_t npairs, double* out, double* abssum)
{
    const int64_t nb = K / QK;
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < npairs; ++i) {
        const int64_t p = pairs[i];
        w_pair(type, w, a, (int64_t)ids[p], p / act_div, E, N, nb, out + i * N, abssum ? abssum + i * N : NULL);
    }
}

/* Integer parts P[p][n][b] = sum (q - z) q8 for weights of `type` (zeros for masked pairs). */
void oracle_moe_w_partials(int type, const uint8_t* w, const uint8_t* a, const int32_t* ids,
                           int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k, int64_t act_div,
                           int32_t* partials)
{
    const int64_t nb = K / QK;
    const int bytes = oracle_w_block_bytes(type);
    int64_t p;
#pragma omp parallel for schedule(dynamic, 1)
    for (p = 0; p < T * top_k; ++p) {
        const int64_t e = ids[p];
        for (int64_t n = 0; n < N; ++n)
            for (int64_t b = 0; b < nb; ++b) {
                int32_t P = 0;
                double t, at;
                if (e >= 0 && e < E)
                    w_block(type, w + ((e * N + n) * nb + b) * bytes, act_block(a, p / act_div, b, nb), &P, &t, &at);
                partials[(p * N + n) * nb + b] = P;
            }
    }
}

/* Gated activations in fp64 (libm exp and tanh):
 *   act 1, SiLU:      x / (1 + exp(-x))
 *   act 2, GELU-tanh: x / 2 * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3))) */
double oracle_act(int act, double x)
{
    if (act == 1) return x / (1.0 + exp(-x));
    if (act == 2) {
        const double k = sqrt(2.0 / 3.14159265358979323846);
        return 0.5 * x * (1.0 + tanh(k * (x + 0.044715 * x * x * x)));
    }
    return NAN;
}

/* y: [rows][2 I] fp64, gate in columns [0, I), up in [I, 2 I);
 * out[r][c] = act(y[r][c]) * y[r][I + c], out: [rows][I]. */
void oracle_act_and_mul(const double* y, int64_t rows, int64_t I, int act, double* out)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r)
        for (int64_t c = 0; c < I; ++c)
            out[r * I + c] = oracle_act(act, y[r * 2 * I + c]) * y[r * 2 * I + I + c];
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
