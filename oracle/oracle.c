/*
 * Reference oracle for the last-axis row normalizations.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plainly written CPU
 * definition that the HIP kernels are checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header, table or helper with the HIP library, and includes no HIP
 * header.  Every floating-point step is done in IEEE double.
 *
 * Sources (the pages the method is described on):
 *  - "Fused transformer kernels on Emily" notebook, Part 1, the composed
 *    RMSNorm cell: square, mean over the last axis, add eps, square root,
 *    divide, multiply by the weight.
 *  - Emily.Fast API docs, section `rms_norm`: x * rsqrt(mean(x^2, last axis)
 *    + eps) * weight, weight of shape {width} broadcast over leading dims.
 *  - Emily.Fast API docs, section `layer_norm`: mean and variance of the last
 *    axis, then (x - mean) / sqrt(var + eps) * weight + bias.
 *  - mlx-c-rust `compile/norm_fusion.rs`, module docs and the dual head-norm
 *    graph builder: two independent RMS norms (queries with the query scale
 *    weight, keys with the key scale weight), one shared eps, outputs in the
 *    order queries then keys.
 *
 * Readings taken where the pages are silent:
 *  - The variance divides by the width (population variance), matching a
 *    Welford accumulator's M2 / n.
 *  - eps is used exactly as the fp32 value the caller passes, widened to
 *    double.
 *  - No intermediate rounding: the result is the exact-as-double value; the
 *    comparison with a bf16 or fp32 output happens in the tests.
 *  - A NULL bias means a zero bias.
 *
 * Rotary position embedding (Emily.Fast docs, sections `rope` and
 * `rope_with_freqs`), applied after the dual head RMSNorm:
 *  - angle of pair i of a head vector at position p:
 *      theta_i = p * scale * inv_freq_i,  inv_freq_i = base^(-2i/dims)
 *    (the geometric-progression schedule), or inv_freq_i = freqs[i] when an
 *    inverse-frequency table of dims/2 entries is given;
 *  - p = offset + token index (the scalar offset of the docs);
 *  - pairs: split-half (i, i + dims/2) by default, paired-interleave
 *    (2i, 2i + 1) when `traditional`; a pair (a, b) becomes
 *      (a cos - b sin, b cos + a sin);
 *  - only the first `dims` features of a head vector rotate, the rest pass
 *    through (the docs' "trailing dims" read as the rotated feature count
 *    of the last axis).
 *
 * RMSNorm with a SwiGLU-style gate epilogue (mlx-c-rust
 * `compile/norm_fusion.rs`, module docs: the output RMS normalization of the
 * gated-delta block chained into its "precise SwiGLU" epilogue).  The page
 * names the chain but does not define SwiGLU; the reading taken:
 *  - y_j = RMSNorm(x, w)_j * SiLU(g_j), SiLU(g) = g * sigmoid(g)
 *    = g / (1 + exp(-g)) (the Swish-1 gate of the GLU variants), applied to
 *    a gate tensor g of x's shape; the normalization itself is unchanged;
 *  - "precise": no rounding between the norm and the gate; one rounding of
 *    the final value (in the tests).
 *
 * Element types: 0 = IEEE binary32, 1 = bfloat16 (the upper 16 bits of a
 * binary32), 2 = IEEE binary16.  All widen to double without rounding.
 *
 * parity pins: every function here is pinned by the CPU tests (closed-form
 * hand cases, exact rational brute force, invariants, special cases).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F16 2

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits; exponent 0 holds zeros and subnormals (fraction * 2^-24), exponent
 * 31 holds infinities (fraction 0) and NaNs. */
static double half_to_double(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int exponent = (h >> 10) & 0x1f;
    const int fraction = h & 0x3ff;
    double v;
    if (exponent == 0)
        v = ldexp((double)fraction, -24);
    else if (exponent == 31)
        v = fraction ? NAN : INFINITY;
    else
        v = ldexp((double)(fraction | 0x400), exponent - 25);
    return sign ? -v : v;
}

/* Widen element i of a buffer of the given element type to double. */
static double widen(const void *p, int dtype, int64_t i)
{
    if (dtype == ORACLE_F32) {
        const float *f = (const float *)p;
        return (double)f[i];
    }
    if (dtype == ORACLE_F16)
        return half_to_double(((const uint16_t *)p)[i]);
    /* bfloat16: the stored 16 bits are the high half of a binary32. */
    const uint16_t *h = (const uint16_t *)p;
    uint32_t bits = ((uint32_t)h[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/*
 * RMSNorm of each row (Emily.Fast docs, `rms_norm`; Emily notebook, Part 1):
 *   ms  = (sum_j x_j^2) / N
 *   y_j = x_j / sqrt(ms + eps) * w_j
 * x: rows*width elements, w: width elements, y: rows*width doubles.
 */
void oracle_rms(const void *x, const void *w, int dtype, int64_t rows,
                int64_t width, float eps, double *y)
{
    const double e = (double)eps;
    for (int64_t r = 0; r < rows; ++r) {
        double sum_sq = 0.0;
        for (int64_t j = 0; j < width; ++j) {
            double v = widen(x, dtype, r * width + j);
            sum_sq += v * v;
        }
        double mean_sq = sum_sq / (double)width;
        double root = sqrt(mean_sq + e);
        for (int64_t j = 0; j < width; ++j) {
            double v = widen(x, dtype, r * width + j);
            y[r * width + j] = v / root * widen(w, dtype, j);
        }
    }
}

/*
 * LayerNorm of each row (Emily.Fast docs, `layer_norm`):
 *   mean = (sum_j x_j) / N
 *   var  = (sum_j (x_j - mean)^2) / N
 *   y_j  = (x_j - mean) / sqrt(var + eps) * w_j + b_j
 * The variance is taken in a second pass over the row, around the mean of
 * the first pass.  b may be NULL, which means zeros.
 */
void oracle_layer(const void *x, const void *w, const void *b, int dtype,
                  int64_t rows, int64_t width, float eps, double *y)
{
    const double e = (double)eps;
    for (int64_t r = 0; r < rows; ++r) {
        double sum = 0.0;
        for (int64_t j = 0; j < width; ++j)
            sum += widen(x, dtype, r * width + j);
        double mean = sum / (double)width;

        double sum_dev_sq = 0.0;
        for (int64_t j = 0; j < width; ++j) {
            double d = widen(x, dtype, r * width + j) - mean;
            sum_dev_sq += d * d;
        }
        double var = sum_dev_sq / (double)width;
        double root = sqrt(var + e);

        for (int64_t j = 0; j < width; ++j) {
            double d = widen(x, dtype, r * width + j) - mean;
            double bias = b ? widen(b, dtype, j) : 0.0;
            y[r * width + j] = d / root * widen(w, dtype, j) + bias;
        }
    }
}

/*
 * Dual-output query/key head RMSNorm (mlx-c-rust `compile/norm_fusion.rs`):
 * the queries, viewed as q_rows head vectors of head_dim, are RMS-normalized
 * with the query scale weight; the keys, k_rows head vectors, with the key
 * scale weight; both with the same eps.  Outputs: queries into qy, keys into
 * ky.
 */
void oracle_dual_head_rms(const void *q, const void *k, const void *qw,
                          const void *kw, int dtype, int64_t q_rows,
                          int64_t k_rows, int64_t head_dim, float eps,
                          double *qy, double *ky)
{
    oracle_rms(q, qw, dtype, q_rows, head_dim, eps, qy);
    oracle_rms(k, kw, dtype, k_rows, head_dim, eps, ky);
}

/*
 * Rotary position embedding of fp64 head vectors, in place (Emily.Fast docs,
 * `rope` / `rope_with_freqs`).  v holds rows = tokens * heads vectors of
 * head_dim; row r belongs to token r / heads.  freqs (dims/2 fp32 inverse
 * frequencies) may be NULL, then base gives the schedule.
 */
void oracle_rope_rows(double *v, int64_t rows, int64_t heads, int64_t head_dim,
                      int64_t dims, int traditional, float base, float scale,
                      int64_t offset, const float *freqs)
{
    const int64_t half = dims / 2;
    for (int64_t r = 0; r < rows; ++r) {
        const double pos = (double)(offset + r / heads);
        double *x = v + r * head_dim;
        for (int64_t i = 0; i < half; ++i) {
            double inv_freq = freqs ? (double)freqs[i]
                                    : pow((double)base, -2.0 * (double)i / (double)dims);
            double theta = pos * (double)scale * inv_freq;
            double c = cos(theta), s = sin(theta);
            int64_t a = traditional ? 2 * i : i;
            int64_t b = traditional ? 2 * i + 1 : i + half;
            double xa = x[a], xb = x[b];
            x[a] = xa * c - xb * s;
            x[b] = xb * c + xa * s;
        }
    }
}

/*
 * The dual head RMSNorm followed by the rotary embedding of both outputs:
 * queries q [tokens, q_heads, head_dim], keys k [tokens, k_heads, head_dim],
 * the same positions for both (mlx-c-rust `compile/norm_fusion.rs` for the
 * dual norm; Emily.Fast `rope` for the rotation).
 */
void oracle_dual_head_rms_rope(const void *q, const void *k, const void *qw,
                               const void *kw, int dtype, int64_t tokens,
                               int64_t q_heads, int64_t k_heads, int64_t head_dim,
                               float eps, int64_t dims, int traditional, float base,
                               float scale, int64_t offset, const float *freqs,
                               double *qy, double *ky)
{
    oracle_dual_head_rms(q, k, qw, kw, dtype, tokens * q_heads, tokens * k_heads,
                         head_dim, eps, qy, ky);
    oracle_rope_rows(qy, tokens * q_heads, q_heads, head_dim, dims, traditional, base,
                     scale, offset, freqs);
    oracle_rope_rows(ky, tokens * k_heads, k_heads, head_dim, dims, traditional, base,
                     scale, offset, freqs);
}

/*
 * RMSNorm followed by the SiLU-gate epilogue, each row:
 *   y_j = x_j / sqrt(ms + eps) * w_j * g_j / (1 + exp(-g_j))
 * x, g: rows*width elements; w: width elements; y: rows*width doubles.
 */
void oracle_rms_swiglu(const void *x, const void *g, const void *w, int dtype,
                       int64_t rows, int64_t width, float eps, double *y)
{
    oracle_rms(x, w, dtype, rows, width, eps, y);
    for (int64_t i = 0; i < rows * width; ++i) {
        double gate = widen(g, dtype, i);
        double silu = gate / (1.0 + exp(-gate));
        y[i] = y[i] * silu;
    }
}
