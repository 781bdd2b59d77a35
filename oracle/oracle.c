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
 *    norm(x) * weight * (1 + scale) + shift, the conditioning step of a
 *    DiT block.  Read with per-sample scale and shift rows: row r of x
 *    belongs to sample b = r / rows_per_sample and uses scale[b, :] and
 *    shift[b, :]; norm(x) * weight is the RMSNorm above.  One rounding.
 *
 * Data format
 * -----------
 *  Inputs are bf16 (uint16_t bit patterns, the upper half of an IEEE
 *  binary32), IEEE binary16 (uint16_t bit patterns) or IEEE binary32, the
 *  three precisions the skill page lists ("Supported Data Types"); the `_dt`
 *  functions take the type, the others are bf16.  All outputs are double;
 *  oracle_round_dt() turns them into the binary32 "reference" and its
 *  rounding to the output type.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_BF16 = 0, ORACLE_F16 = 1, ORACLE_F32 = 2 };

/* A bf16 is the upper 16 bits of an IEEE binary32, so widening is a shift
 * and is exact. */
static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE binary16 -> value: sign, 5-bit exponent (bias 15), 10-bit fraction;
 * exponent 0 is zero or subnormal (fraction * 2^-24), 31 is inf or NaN. */
static double f16_value(uint16_t bits)
{
    int sign = bits >> 15;
    int exponent = (bits >> 10) & 0x1f;
    int fraction = bits & 0x3ff;
    double v;
    if (exponent == 0)
        v = ldexp((double)fraction, -24);
    else if (exponent == 31)
        v = fraction ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + fraction), exponent - 25);
    return sign ? -v : v;
}

/* Element i of an array of the given type, as a double (exact). */
static double value_at(const void *base, int64_t i, int dtype)
{
    if (dtype == ORACLE_BF16)
        return bf16_value(((const uint16_t *)base)[i]);
    if (dtype == ORACLE_F16)
        return f16_value(((const uint16_t *)base)[i]);
    return (double)((const float *)base)[i];
}

/* Decode n elements of the given type to doubles (exact). */
void oracle_decode(const void *x, int64_t n, int dtype, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = value_at(x, i, dtype);
}

/* binary32 -> IEEE binary16, round to nearest, ties to even.  The value is
 * scaled to units of the binary16 quantum of its binade (2^(e-10) for
 * normal e, 2^-24 for subnormals), rounded to an integer with nearbyint in
 * the default round-to-nearest-even mode, and reassembled; a carry to 2048
 * units moves to the next binade.  Magnitudes from 65520 (half way past the
 * largest finite 65504) round to infinity.  NaN stays NaN and is quiet. */
uint16_t oracle_f16_from_f32(float f)
{
    double v = (double)f;
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isnan(v))
        return (uint16_t)(sign | 0x7e00u);
    if (a >= 65520.0)
        return (uint16_t)(sign | 0x7c00u);
    int e;
    frexp(a, &e); /* a = m * 2^e with m in [0.5, 1): the binade is 2^(e-1) */
    e -= 1;
    if (a == 0.0 || e < -14)
        e = -14;  /* subnormal range: fixed quantum 2^-24 */
    double units = nearbyint(ldexp(a, 10 - e)); /* a / 2^(e-10), exact scaling */
    uint32_t u = (uint32_t)units;
    if (e == -14 && u < 1024)
        return (uint16_t)(sign | u);               /* subnormal (or zero) */
    /* biased exponent field plus fraction; u == 2048 carries into e + 1 */
    return (uint16_t)(sign | ((((uint32_t)(e + 15)) << 10) + (u - 1024)));
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

/* Array form of oracle_f16_from_f32. */
void oracle_f16_array(const float *f, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f16_from_f32(f[i]);
}

/* Round n doubles to binary32 (ref32) and then to the output type (ref_out:
 * bf16 or binary16 bit patterns, or binary32 values).  Either output may be
 * NULL. */
void oracle_round_dt(const double *y, int64_t n, float *ref32, void *ref_out, int dtype)
{
    for (int64_t i = 0; i < n; ++i) {
        float f = (float)y[i];
        if (ref32)
            ref32[i] = f;
        if (!ref_out)
            continue;
        if (dtype == ORACLE_BF16)
            ((uint16_t *)ref_out)[i] = oracle_bf16_from_f32(f);
        else if (dtype == ORACLE_F16)
            ((uint16_t *)ref_out)[i] = oracle_f16_from_f32(f);
        else
            ((float *)ref_out)[i] = f;
    }
}

/* bf16 form of oracle_round_dt. */
void oracle_round(const double *y, int64_t n, float *ref32, uint16_t *ref16)
{
    oracle_round_dt(y, n, ref32, ref16, ORACLE_BF16);
}

/* Normalise one row: z[j] = x[j] * rstd * w[j] with
 * rstd = 1 / sqrt(sum_j x[j]^2 / H + eps).  Each bf16 square is exact in
 * double and the row sum carries a relative error below H * 2^-53.  eps is
 * the binary32 value the caller passes (1e-6 becomes 9.99999997e-7), widened
 * exactly.  With eps = 0 and an all-zero row, rstd is +inf and every output
 * is 0 * inf = NaN, as IEEE arithmetic gives. */
static void normalise_row(double *z, const void *x, int64_t row, const void *w,
                          int64_t hidden, float eps, int dtype)
{
    double sum_sq = 0.0;
    for (int64_t j = 0; j < hidden; ++j) {
        double v = value_at(x, row * hidden + j, dtype);
        sum_sq += v * v;
    }
    double mean_sq = sum_sq / (double)hidden;
    double rstd = 1.0 / sqrt(mean_sq + (double)eps);
    for (int64_t j = 0; j < hidden; ++j) {
        double wj = w ? value_at(w, j, dtype) : 1.0;
        z[j] = value_at(x, row * hidden + j, dtype) * rstd * wj;
    }
}

static int known_dtype(int dtype)
{
    return dtype == ORACLE_BF16 || dtype == ORACLE_F16 || dtype == ORACLE_F32;
}

/* Row-wise RMSNorm.
 *   y      out, double [rows * hidden]
 *   x      in,  bf16 bits [rows * hidden], row-major, hidden innermost
 *   w      in,  bf16 bits [hidden], or NULL for a weight of ones
 * Returns 0, or -1 on a bad shape or NULL pointer. */
int oracle_rmsnorm_dt(double *y, const void *x, const void *w, int64_t rows,
                      int64_t hidden, float eps, int dtype)
{
    if (!y || !x || rows < 0 || hidden <= 0 || !known_dtype(dtype))
        return -1;
    for (int64_t r = 0; r < rows; ++r)
        normalise_row(y + r * hidden, x, r, w, hidden, eps, dtype);
    return 0;
}

int oracle_rmsnorm(double *y, const uint16_t *x, const uint16_t *w,
                   int64_t rows, int64_t hidden, float eps)
{
    return oracle_rmsnorm_dt(y, x, w, rows, hidden, eps, ORACLE_BF16);
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
int oracle_rmsnorm_rope_dt(double *y, double *mag, const void *x,
                           const void *w, const float *cos_tab,
                           const float *sin_tab, int64_t rows, int64_t hidden,
                           int32_t heads, int32_t head_dim, int64_t seq_len,
                           float eps, int dtype)
{
    if (!y || !x || !cos_tab || !sin_tab || rows < 0 || hidden <= 0 ||
        heads <= 0 || head_dim <= 0 || head_dim % 2 != 0 ||
        (int64_t)heads * head_dim != hidden || seq_len <= 0 || !known_dtype(dtype))
        return -1;
    const int32_t half = head_dim / 2;
    for (int64_t r = 0; r < rows; ++r) {
        double *yr = y + r * hidden;
        normalise_row(yr, x, r, w, hidden, eps, dtype);
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

int oracle_rmsnorm_rope(double *y, double *mag, const uint16_t *x,
                        const uint16_t *w, const float *cos_tab,
                        const float *sin_tab, int64_t rows, int64_t hidden,
                        int32_t heads, int32_t head_dim, int64_t seq_len,
                        float eps)
{
    return oracle_rmsnorm_rope_dt(y, mag, x, w, cos_tab, sin_tab, rows, hidden,
                                  heads, head_dim, seq_len, eps, ORACLE_BF16);
}

/* Fused RMSNorm over the whole hidden row, then RoPE per head on adjacent
 * pairs (2i, 2i + 1), both rotated by table column i.  Arguments and return
 * value as for oracle_rmsnorm_rope; mag as there (|a c| + |b s| for the
 * even element, |b c| + |a s| for the odd one). */
int oracle_rmsnorm_rope_interleaved_dt(double *y, double *mag, const void *x,
                                       const void *w, const float *cos_tab,
                                       const float *sin_tab, int64_t rows,
                                       int64_t hidden, int32_t heads,
                                       int32_t head_dim, int64_t seq_len,
                                       float eps, int dtype)
{
    if (!y || !x || !cos_tab || !sin_tab || rows < 0 || hidden <= 0 ||
        heads <= 0 || head_dim <= 0 || head_dim % 2 != 0 ||
        (int64_t)heads * head_dim != hidden || seq_len <= 0 || !known_dtype(dtype))
        return -1;
    const int32_t half = head_dim / 2;
    for (int64_t r = 0; r < rows; ++r) {
        double *yr = y + r * hidden;
        normalise_row(yr, x, r, w, hidden, eps, dtype);
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

int oracle_rmsnorm_rope_interleaved(double *y, double *mag, const uint16_t *x,
                                    const uint16_t *w, const float *cos_tab,
                                    const float *sin_tab, int64_t rows,
                                    int64_t hidden, int32_t heads,
                                    int32_t head_dim, int64_t seq_len,
                                    float eps)
{
    return oracle_rmsnorm_rope_interleaved_dt(y, mag, x, w, cos_tab, sin_tab, rows,
                                              hidden, heads, head_dim, seq_len,
                                              eps, ORACLE_BF16);
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
int oracle_rmsnorm_adaln_dt(double *y, double *mag, const void *x, const void *w,
                            const void *scale, const void *shift,
                            int64_t rows, int64_t hidden, int64_t rows_per_sample,
                            float eps, int dtype)
{
    if (!y || !x || rows < 0 || hidden <= 0 || rows_per_sample <= 0 || !known_dtype(dtype))
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        double *yr = y + r * hidden;
        normalise_row(yr, x, r, w, hidden, eps, dtype);
        const int64_t b = r / rows_per_sample;
        for (int64_t j = 0; j < hidden; ++j) {
            double sc = scale ? value_at(scale, b * hidden + j, dtype) : 0.0;
            double sh = shift ? value_at(shift, b * hidden + j, dtype) : 0.0;
            double modulated = yr[j] * (1.0 + sc);
            yr[j] = modulated + sh;
            if (mag)
                mag[r * hidden + j] = fabs(modulated) + fabs(sh);
        }
    }
    return 0;
}

int oracle_rmsnorm_adaln(double *y, double *mag, const uint16_t *x, const uint16_t *w,
                         const uint16_t *scale, const uint16_t *shift,
                         int64_t rows, int64_t hidden, int64_t rows_per_sample,
                         float eps)
{
    return oracle_rmsnorm_adaln_dt(y, mag, x, w, scale, shift, rows, hidden,
                                   rows_per_sample, eps, ORACLE_BF16);
}
