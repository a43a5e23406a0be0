/*
 * CPU oracle for block-quantized decode GEMV — TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this code.  It shares nothing with the HIP library: no headers, no
 * helpers, no tables.  It is deliberately plain: every weight is decoded to
 * fp64, every product is formed in fp64 and the sum runs over k in ascending
 * order, one output at a time.
 *
 * What it computes (the definition, not an approximation):
 *
 *   Q8G64  (int8 codes, one fp16 scale per 64 consecutive k of a row)
 *     w[n][k] = q[n][k] * scale[n][k/64]
 *   Q4G32  (4-bit codes 0..15, two per byte, fp16 scale and fp16 min per
 *           32 consecutive k of a row)
 *     c[n][k] = nibble k of row n (even k in the low nibble of byte k/2)
 *     w[n][k] = c[n][k] * scale[n][k/32] + min[n][k/32]
 *   both
 *     y[i][n] = sum_k w[n][k] * x[i][k]          (x is bf16)
 *     a[i][n] = sum_k |w[n][k] * x[i][k]|        (the tolerance scale)
 *
 * Further formats (same structure, same plain loops):
 *   Q8G128 w[n][k] = q[n][k] * scale[n][k/128]          (fp16 scale)
 *   Q8PC   w[n][k] = q[n][k] * scale[n]                  (fp32 scale per row)
 *
 * Sources.  The W8 reading (signed int8 weight codes, bf16 activations,
 * weights consumed in their quantized form and widened only inside the dot
 * product) follows the "Qwen3-14B TP4 W8A16 Decode" section of the Qwen3 C++
 * Reference Runtime README (MetaInfer-cpp) and the "W8 direct read" section
 * of the zLLM GLM-5.3 ROCm decode post on juejin.  The dequantize-in-register
 * GEMV with activations kept in bf16 is the W4A16 reading in the commit log
 * of vllm.cpp pull request #1936 ("perf(GFX1100-TG200)").  The byte layout of
 * the two formats (group sizes, fp16 scale/min, w = code*scale + min, nibble
 * order) is not printed on those pages; the readings used here are listed in
 * the design notes of this repository.
 *
 * Parity status: every function here is pinned by tests that do not re-type
 * it (hand-worked examples, closed forms, invariants, library special cases).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

/* IEEE-754 binary16 bit pattern -> exact double.
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double half_bits_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24);               /* zero or subnormal */
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + frac), expo - 25); /* (1.f) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* bfloat16 bit pattern (the high half of an IEEE binary32) -> exact double.
 * 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
static double bf16_bits_to_double(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int expo = (b >> 7) & 0xff;
    int frac = b & 0x7f;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -133);               /* zero or subnormal */
    } else if (expo == 255) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(128 + frac), expo - 134); /* (1.f) * 2^(e-127) */
    }
    return sign ? -v : v;
}

/* Exposed so the tests can pin the two decoders against numpy on their own. */
double oracle_half_to_double(uint16_t h) { return half_bits_to_double(h); }
double oracle_bf16_to_double(uint16_t b) { return bf16_bits_to_double(b); }

/* Q8G64 decode GEMV for output rows n0 <= n < n1.
 *   q      [N][K] int8, row-major
 *   scale  [N][K/64] fp16 bit patterns, row-major
 *   x      m rows of bf16 bit patterns, row i starts at x + i*ldx
 *   y, a   m rows of doubles, row i starts at y + i*ldy (a likewise)
 * Returns 0, or -1 if the shape is not a whole number of groups. */
int oracle_q8g64(const int8_t *q, const uint16_t *scale, int64_t N, int64_t K,
                 const uint16_t *x, int64_t m, int64_t ldx,
                 int64_t n0, int64_t n1, double *y, double *a, int64_t ldy)
{
    if (K % 64 != 0 || n0 < 0 || n1 > N || n0 > n1) return -1;
    const int64_t groups = K / 64;
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t n = n0; n < n1; ++n) {
            double sum = 0.0, abs_sum = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double code = (double)q[n * K + k];
                double s = half_bits_to_double(scale[n * groups + k / 64]);
                double w = code * s;
                double xv = bf16_bits_to_double(x[i * ldx + k]);
                sum += w * xv;
                abs_sum += fabs(w * xv);
            }
            y[i * ldy + n] = sum;
            a[i * ldy + n] = abs_sum;
        }
    }
    return 0;
}

/* Q4G32 decode GEMV for output rows n0 <= n < n1.
 *   codes  [N][K/2] bytes; element k of a row is the low nibble of byte k/2
 *          when k is even and the high nibble when k is odd
 *   scale, minv  [N][K/32] fp16 bit patterns, row-major
 *   x, y, a as for oracle_q8g64. */
int oracle_q4g32(const uint8_t *codes, const uint16_t *scale, const uint16_t *minv,
                 int64_t N, int64_t K,
                 const uint16_t *x, int64_t m, int64_t ldx,
                 int64_t n0, int64_t n1, double *y, double *a, int64_t ldy)
{
    if (K % 32 != 0 || n0 < 0 || n1 > N || n0 > n1) return -1;
    const int64_t groups = K / 32;
    const int64_t row_bytes = K / 2;
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t n = n0; n < n1; ++n) {
            double sum = 0.0, abs_sum = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                uint8_t byte = codes[n * row_bytes + k / 2];
                int c = (k % 2 == 0) ? (byte & 0x0f) : (byte >> 4);
                double s = half_bits_to_double(scale[n * groups + k / 32]);
                double mn = half_bits_to_double(minv[n * groups + k / 32]);
                double w = (double)c * s + mn;
                double xv = bf16_bits_to_double(x[i * ldx + k]);
                sum += w * xv;
                abs_sum += fabs(w * xv);
            }
            y[i * ldy + n] = sum;
            a[i * ldy + n] = abs_sum;
        }
    }
    return 0;
}

/* IEEE-754 binary32 bit pattern -> exact double.
 * 1 sign bit, 8 exponent bits (bias 127), 23 fraction bits. */
static double f32_bits_to_double(uint32_t f)
{
    int sign = (f >> 31) & 1;
    int expo = (f >> 23) & 0xff;
    uint32_t frac = f & 0x7fffffu;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -149);                      /* zero or subnormal */
    } else if (expo == 255) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(0x800000u + frac), expo - 150);  /* (1.f) * 2^(e-127) */
    }
    return sign ? -v : v;
}

double oracle_f32_to_double(uint32_t f) { return f32_bits_to_double(f); }

/* Q8G128 decode GEMV: int8 codes, one fp16 scale per 128 consecutive k of a
 * row (the LM-head format of the per-operator format map in the zLLM
 * GLM-5.3 ROCm decode post).  Arguments as for oracle_q8g64, with
 * scale [N][K/128]. */
int oracle_q8g128(const int8_t *q, const uint16_t *scale, int64_t N, int64_t K,
                  const uint16_t *x, int64_t m, int64_t ldx,
                  int64_t n0, int64_t n1, double *y, double *a, int64_t ldy)
{
    if (K % 128 != 0 || n0 < 0 || n1 > N || n0 > n1) return -1;
    const int64_t groups = K / 128;
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t n = n0; n < n1; ++n) {
            double sum = 0.0, abs_sum = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double code = (double)q[n * K + k];
                double s = half_bits_to_double(scale[n * groups + k / 128]);
                double w = code * s;
                double xv = bf16_bits_to_double(x[i * ldx + k]);
                sum += w * xv;
                abs_sum += fabs(w * xv);
            }
            y[i * ldy + n] = sum;
            a[i * ldy + n] = abs_sum;
        }
    }
    return 0;
}

/* Q8 per output channel (W8A16 of the "Qwen3-14B TP4 W8A16 Decode" section
 * of the Qwen3 C++ Reference Runtime README): int8 codes, one fp32 scale per
 * output row, bf16 activations.  scale is [N] binary32 bit patterns. */
int oracle_q8pc(const int8_t *q, const uint32_t *scale, int64_t N, int64_t K,
                const uint16_t *x, int64_t m, int64_t ldx,
                int64_t n0, int64_t n1, double *y, double *a, int64_t ldy)
{
    if (n0 < 0 || n1 > N || n0 > n1) return -1;
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t n = n0; n < n1; ++n) {
            double s = f32_bits_to_double(scale[n]);
            double sum = 0.0, abs_sum = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double w = (double)q[n * K + k] * s;
                double xv = bf16_bits_to_double(x[i * ldx + k]);
                sum += w * xv;
                abs_sum += fabs(w * xv);
            }
            y[i * ldy + n] = sum;
            a[i * ldy + n] = abs_sum;
        }
    }
    return 0;
}

/* Greedy token choice over fp32 logits: for each row i < m, the index of the
 * largest of x[i*ldx + 0 .. N-1], the lowest such index on ties.  This is
 * the (value, lower index) rule of the split argmax in the commit log of
 * vllm.cpp pull request #1936, which makes the choice independent of how a
 * row is split.  Values are compared as the real numbers the fp32 bit
 * patterns denote, so -0 and +0 tie.  A NaN counts as larger than every
 * number, and the first NaN of a row wins (numpy.argmax does the same).
 * A plain left-to-right scan, one row at a time. */
int oracle_argmax_f32(const uint32_t *x, int64_t m, int64_t N, int64_t ldx, int64_t *out)
{
    if (m < 0 || N < 1 || ldx < N) return -1;
    for (int64_t i = 0; i < m; ++i) {
        int64_t best = 0;
        double best_v = f32_bits_to_double(x[i * ldx]);
        int best_nan = isnan(best_v);
        for (int64_t n = 1; n < N && !best_nan; ++n) {
            double v = f32_bits_to_double(x[i * ldx + n]);
            if (isnan(v)) {
                best = n;
                best_nan = 1;
            } else if (v > best_v) {
                best = n;
                best_v = v;
            }
        }
        out[i] = best;
    }
    return 0;
}
