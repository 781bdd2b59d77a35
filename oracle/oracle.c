/*
 * oracle.c -- CPU oracle for row-wise RMSNorm and fused RMSNorm + rotate-half
 * RoPE over bf16 activations.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg load this library.  It shares no
 * code, header, table or helper with the HIP library: it is plain C (libc and
 * libm only), built with gcc, and computes in IEEE double, rounding once at
 * the very end (double -> binary32 -> bf16, round-to-nearest-even each time).
 *
 * What it computes, and where that comes from
 * -------------------------------------------
 *  - RMSNorm.  The Hugging Face "cuda-kernels" skill page ("CUDA Kernels for
 *    Diffusers & Transformers", section "Kernel-Specific Guidelines", item
 *    RMSNorm) fixes the layout [..., hidden_size] (the normalised dimension is
 *    the innermost, contiguous one), the default epsilon 1e-6, and that the
 *    weight may be absent (section "Diffusers Critical Pitfalls", item 1: an
 *    absent weight behaves as a weight of ones).  The page prints no formula;
 *    this oracle takes the standard definition
 *        y[r, j] = x[r, j] / sqrt( (1/H) * sum_k x[r, k]^2 + eps ) * w[j]
 *    with eps added to the mean of squares inside the square root.
 *  - RMSNorm + RoPE.  The LTX-2 "ltx-kernels" README (introduction, the list
 *    of fused element ops in the ops_cpp extension) names rms_norm_rope but
 *    gives no formula.  The skill page (section "Kernel-Specific Guidelines",
 *    item RoPE) fixes the 1D layout [batch, seq, heads, head_dim].  This
 *    oracle takes the plainest reading: RMSNorm over the whole hidden row
 *    (heads * head_dim), then, per head, the rotate-half rotation pairing
 *    element i with element i + head_dim/2:
 *        out[i]          = y[i] * cos[p, i] - y[i + d/2] * sin[p, i]
 *        out[i + d/2]    = y[i + d/2] * cos[p, i] + y[i] * sin[p, i]
 *    i.e. out = y * [cos, cos] + rotate_half(y) * [sin, sin] with
 *    rotate_half([y1, y2]) = [-y2, y1].  Row r sits at position p = r mod
 *    seq_len; the cos/sin tables are inputs, binary32 [seq_len, d/2].
 *    The rotation acts on the un-rounded normalised value (one rounding).
 *  - RMSNorm + interleaved RoPE.  The README's sibling op name
 *    (rms_norm_split_rope) implies a second pairing; the pages define
 *    neither.  The other standard pairing rotates adjacent elements:
 *        out[2i]     = y[2i] * cos[p, i] - y[2i + 1] * sin[p, i]
 *        out[2i + 1] = y[2i + 1] * cos[p, i] + y[2i] * sin[p, i]
 *    with the same [seq_len, head_dim/2] tables and row positions.
 *
 *  - RMSNorm with adaptive modulation (AdaLN).  The skill page (section
 *    "Kernel-Specific Guidelines", item AdaLN) gives the formula
 *    norm(x) * weight * (1 + scale) + shift, used in DiT blocks for
 *    conditioning.  Read with per-sample scale and shift rows: row r of x
 *    belongs to sample b = r / rows_per_sample and uses scale[b, :] and
 *    shift[b, :]; norm(x) * weight is the RMSNorm above.  One rounding.
 *
 * Data format
 * -----------
 *  bf16 values travel as uint16_t bit patterns (the upper half of an IEEE
 *  binary32).  All outputs are double; oracle_round() turns them into the
 *  binary32 "reference" and its bf16 rounding.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* A bf16 is the upper 16 bits of an IEEE binary32, so widening is a shift
 * and is exact. */
static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* binary32 -> bf16, round to nearest, ties to even (IEEE 754 default mode).
 * The 16 dropped bits decide: above one half of a bf16 ulp rounds away from
 * zero in magnitude, below rounds toward zero, exactly one half rounds to the
 * even neighbour.  A carry out of the mantissa correctly bumps the exponent
 * (and the largest finite values round up to infinity).  NaN stays NaN and
 * is made quiet, so a payload living only in the dropped bits is not lost. */
uint16_t oracle_bf16_from_f32(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xffffu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        kept += 1u;
    return (uint16_t)kept;
}

/* Array form of oracle_bf16_from_f32 (bit patterns in, bit patterns out). */
void oracle_bf16_array(const float *f, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_from_f32(f[i]);
}

/* Round n doubles to binary32 (ref32) and then to bf16 (ref16).  Either
 * output may be NULL. */
void oracle_round(const double *y, int64_t n, float *ref32, uint16_t *ref16)
{
    for (int64_t i = 0; i < n; ++i) {
        float f = (float)y[i];
        if (ref32)
            ref32[i] = f;
        if (ref16)
            ref16[i] = oracle_bf16_from_f32(f);
    }
}

/* Normalise one row: z[j] = x[j] * rstd * w[j] with
 * rstd = 1 / sqrt(sum_j x[j]^2 / H + eps).  Each bf16 square is exact in
 * double and the row sum carries a relative error below H * 2^-53.  eps is
 * the binary32 value the caller passes (1e-6 becomes 9.99999997e-7), widened
 * exactly.  With eps = 0 and an all-zero row, rstd is +inf and every output
 * is 0 * inf = NaN, as IEEE arithmetic gives. */
static void normalise_row(double *z, const uint16_t *x, const uint16_t *w,
                          int64_t hidden, float eps)
{
    double sum_sq = 0.0;
    for (int64_t j = 0; j < hidden; ++j) {
        double v = bf16_value(x[j]);
        sum_sq += v * v;
    }
    double mean_sq = sum_sq / (double)hidden;
    double rstd = 1.0 / sqrt(mean_sq + (double)eps);
    for (int64_t j = 0; j < hidden; ++j) {
        double wj = w ? bf16_value(w[j]) : 1.0;
        z[j] = bf16_value(x[j]) * rstd * wj;
    }
}

/* Row-wise RMSNorm.
 *   y      out, double [rows * hidden]
 *   x      in,  bf16 bits [rows * hidden], row-major, hidden innermost
 *   w      in,  bf16 bits [hidden], or NULL for a weight of ones
 * Returns 0, or -1 on a bad shape or NULL pointer. */
int oracle_rmsnorm(double *y, const uint16_t *x, const uint16_t *w,
                   int64_t rows, int64_t hidden, float eps)
{
    if (!y || !x || rows < 0 || hidden <= 0)
        return -1;
    for (int64_t r = 0; r < rows; ++r)
        normalise_row(y + r * hidden, x + r * hidden, w, hidden, eps);
    return 0;
}

/* Fused RMSNorm over the whole hidden row, then rotate-half RoPE per head.
 *   y        out, double [rows * hidden]
 *   mag      out (may be NULL), double [rows * hidden]: for each output the
 *            sum of the magnitudes of its two products, |a*c| + |b*s| for a
 *            first-half element and |b*c| + |a*s| for a second-half one.  It
 *            bounds the cancellation in that output and sets the tolerance
 *            floor used when comparing against binary32 kernels.
 *   cos_tab, sin_tab  in, binary32 [seq_len, head_dim/2], row-major, shared
 *            by all heads; row r of x uses table row r mod seq_len.
 * Requires hidden == heads * head_dim and an even head_dim.
 * Returns 0, or -1 on a bad shape or NULL pointer. */
int oracle_rmsnorm_rope(double *y, double *mag, const uint16_t *x,
                        const uint16_t *w, const float *cos_tab,
                        const float *sin_tab, int64_t rows, int64_t hidden,
                        int32_t heads, int32_t head_dim, int64_t seq_len,
                        float eps)
{
    if (!y || !x || !cos_tab || !sin_tab || rows < 0 || hidden <= 0 ||
        heads <= 0 || head_dim <= 0 || head_dim % 2 != 0 ||
        (int64_t)heads * head_dim != hidden || seq_len <= 0)
        return -1;
    const int32_t half = head_dim / 2;
    for (int64_t r = 0; r < rows; ++r) {
        double *yr = y + r * hidden;
        normalise_row(yr, x + r * hidden, w, hidden, eps);
        const int64_t p = r % seq_len;
        const float *cp = cos_tab + p * half;
        const float *sp = sin_tab + p * half;
        for (int32_t h = 0; h < heads; ++h) {
            double *head = yr + (int64_t)h * head_dim;
            for (int32_t i = 0; i < half; ++i) {
                double a = head[i];        /* first half  */
                double b = head[i + half]; /* second half */
                double c = (double)cp[i];
                double s = (double)sp[i];
                head[i] = a * c - b * s;
                head[i + half] = b * c + a * s;
                if (mag) {
                    double *m = mag + r * hidden + (int64_t)h * head_dim;
                    m[i] = fabs(a * c) + fabs(b * s);
                    m[i + half] = fabs(b * c) + fabs(a * s);
                }
            }
        }
    }
    return 0;
}

/* Fused RMSNorm over the whole hidden row, then RoPE per head on adjacent
 * pairs (2i, 2i + 1), both rotated by table column i.  Arguments and return
 * value as for oracle_rmsnorm_rope; mag as there (|a c| + |b s| for the
 * even element, |b c| + |a s| for the odd one). */
int oracle_rmsnorm_rope_interleaved(double *y, double *mag, const uint16_t *x,
                                    const uint16_t *w, const float *cos_tab,
                                    const float *sin_tab, int64_t rows,
                                    int64_t hidden, int32_t heads,
                                    int32_t head_dim, int64_t seq_len,
                                    float eps)
{
    if (!y || !x || !cos_tab || !sin_tab || rows < 0 || hidden <= 0 ||
        heads <= 0 || head_dim <= 0 || head_dim % 2 != 0 ||
        (int64_t)heads * head_dim != hidden || seq_len <= 0)
        return -1;
    const int32_t half = head_dim / 2;
    for (int64_t r = 0; r < rows; ++r) {
        double *yr = y + r * hidden;
        normalise_row(yr, x + r * hidden, w, hidden, eps);
        const int64_t p = r % seq_len;
        const float *cp = cos_tab + p * half;
        const float *sp = sin_tab + p * half;
        for (int32_t h = 0; h < heads; ++h) {
            double *head = yr + (int64_t)h * head_dim;
            for (int32_t i = 0; i < half; ++i) {
                double a = head[2 * i];     /* even element */
                double b = head[2 * i + 1]; /* odd element  */
                double c = (double)cp[i];
                double s = (double)sp[i];
                head[2 * i] = a * c - b * s;
                head[2 * i + 1] = b * c + a * s;
                if (mag) {
                    double *m = mag + r * hidden + (int64_t)h * head_dim;
                    m[2 * i] = fabs(a * c) + fabs(b * s);
                    m[2 * i + 1] = fabs(b * c) + fabs(a * s);
                }
            }
        }
    }
    return 0;
}

/* RMSNorm followed by per-sample modulation:
 *   y[r, j] = x[r, j] * rstd_r * w[j] * (1 + scale[b, j]) + shift[b, j],
 *   b = r / rows_per_sample.
 *   mag    out (may be NULL), double [rows * hidden]: |n * (1 + scale)| +
 *          |shift| for each output (n the normalised value), which bounds
 *          the cancellation of the final sum.
 *   scale, shift  in, bf16 bits [ceil(rows / rows_per_sample), hidden], or
 *                 NULL for zeros.
 * Returns 0, or -1 on a bad shape or NULL pointer. */
int oracle_rmsnorm_adaln(double *y, double *mag, const uint16_t *x, const uint16_t *w,
                         const uint16_t *scale, const uint16_t *shift,
                         int64_t rows, int64_t hidden, int64_t rows_per_sample,
                         float eps)
{
    if (!y || !x || rows < 0 || hidden <= 0 || rows_per_sample <= 0)
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        double *yr = y + r * hidden;
        normalise_row(yr, x + r * hidden, w, hidden, eps);
        const int64_t b = r / rows_per_sample;
        for (int64_t j = 0; j < hidden; ++j) {
            double sc = scale ? bf16_value(scale[b * hidden + j]) : 0.0;
            double sh = shift ? bf16_value(shift[b * hidden + j]) : 0.0;
            double modulated = yr[j] * (1.0 + sc);
            yr[j] = modulated + sh;
            if (mag)
                mag[r * hidden + j] = fabs(modulated) + fabs(sh);
        }
    }
    return 0;
}
