/*
 * ltxnorm.h -- C ABI of libltxnorm.so: row-wise RMSNorm, fused RMSNorm + RoPE
 * (rotate-half and interleaved pairs) and AdaLN-modulated RMSNorm over bf16,
 * fp16 or fp32 activations, as HIP kernels for gfx950 (MI355X).
 *
 * Operations
 *   RMSNorm over the innermost dimension of [..., hidden] activations, with
 *   epsilon (default 1e-6) and a weight that may be absent: Hugging Face
 *   "cuda-kernels" skill page ("CUDA Kernels for Diffusers & Transformers"),
 *   section "Kernel-Specific Guidelines", RMSNorm; an absent weight acts as a
 *   weight of ones (same page, "Diffusers Critical Pitfalls", item 1).  The
 *   page prints no formula; the library computes the standard definition
 *       y[r, j] = x[r, j] * rsqrt( (1/H) * sum_k x[r, k]^2 + eps ) * w[j]
 *   with the sum of squares accumulated in binary32 and one rounding to bf16
 *   (round-to-nearest-even) at the output.
 *
 *   Fused RMSNorm followed by rotary position embedding: the rms_norm_rope op
 *   listed among the fused element ops of the LTX-2 ltx-kernels README
 *   (introduction).  The row is normalised over the full hidden size, then
 *   each head of head_dim elements (1D layout [batch, seq, heads, head_dim],
 *   skill page, section "Kernel-Specific Guidelines", RoPE) is rotated
 *   rotate-half style: element i pairs with element i + head_dim/2 and
 *       out[i]          = y[i] * c - y[i + d/2] * s
 *       out[i + d/2]    = y[i + d/2] * c + y[i] * s
 *   with c = cos_tab[p, i], s = sin_tab[p, i], p = row mod seq_len, applied
 *   to the un-rounded binary32 y, then rounded once to bf16.
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers (HIP device memory, or memory the device
 *     can access) unless stated otherwise.  bf16 tensors are arrays of 16-bit
 *     IEEE bfloat16 values, row-major, contiguous, hidden innermost.
 *   - Ownership: the caller allocates and frees every buffer.  The library
 *     allocates nothing and never synchronises; work is enqueued on `stream`
 *     (0 = the null stream) and runs asynchronously.  Faults inside a kernel
 *     surface at the caller's next synchronisation.
 *   - The destination comes first, as in an out-variant op.
 *   - Arguments are validated on the host before any HIP call; a rejected
 *     call enqueues nothing.  No C++ exception crosses this boundary.
 *   - Calls are thread-safe and reentrant.  The only state the library keeps
 *     is a mutex-guarded table of how many workgroups of a kernel instance
 *     the device holds at once (queried from HIP on first use and never
 *     changed), which sizes the grid of the kernel for rows of any length.
 *   - Each operation has a bf16 entry point and a `_dt` twin taking the I/O
 *     dtype (the skill page, "Supported Data Types", lists FP16, BF16 and
 *     FP32); x, out, weight, scale and shift all use that dtype, the
 *     rotation tables are always binary32, and arithmetic is binary32 with
 *     one rounding to the output type (round to nearest even; NaN stays NaN;
 *     fp16 overflows to infinity).
 */
#ifndef LTXNORM_H
#define LTXNORM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LTXNORM_ABI_VERSION 4

#define LTXNORM_API __attribute__((visibility("default")))

/* Largest supported hidden size, every dtype.  Rows of up to 65536 bf16/fp16
 * or 32768 fp32 elements are held in registers and read from HBM once;
 * longer rows are read twice (once for the sum of squares, once to
 * normalise).  Out of place, a call of a few hundred such rows of many
 * chunks may cut them into chunks over many workgroups in three launches
 * (ltxnorm_describe_launch names the choice), and between the first and the
 * last of them the start of each row's output holds binary32 partial sums: a
 * reader of out sees the results only after the call's work on the stream is
 * done, as for every call. */
#define LTXNORM_MAX_HIDDEN (1 << 24)

typedef enum ltxnorm_dtype {
    LTXNORM_BF16 = 0,  /* bfloat16 (8 values per 16-byte vector) */
    LTXNORM_F16 = 1,   /* IEEE binary16 (8 per vector)           */
    LTXNORM_F32 = 2    /* IEEE binary32 (4 per vector)           */
} ltxnorm_dtype;

typedef enum ltxnorm_status {
    LTXNORM_OK = 0,
    LTXNORM_ERR_NULL = 1,        /* a required pointer is NULL                       */
    LTXNORM_ERR_SHAPE = 2,       /* rows < 0, hidden <= 0, size overflow, or a RoPE
                                    shape that does not fit (see below)             */
    LTXNORM_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned                 */
    LTXNORM_ERR_UNSUPPORTED = 4, /* unknown dtype, or hidden > LTXNORM_MAX_HIDDEN    */
    LTXNORM_ERR_ALIAS = 5,       /* out partially overlaps x, or overlaps an input
                                    that is only read (weight, tables)              */
    LTXNORM_ERR_VALUE = 6,       /* eps negative, infinite or NaN                    */
    LTXNORM_ERR_HIP = 7          /* the HIP runtime refused the launch               */
} ltxnorm_status;

/*
 * Row-wise RMSNorm, bf16 in / bf16 out, binary32 arithmetic.
 *
 *   out     bf16 [rows, hidden], written.  May equal x exactly (in place);
 *           any other overlap with x, or overlap with weight, is ERR_ALIAS.
 *   x       bf16 [rows, hidden], read.
 *   weight  bf16 [hidden], read; NULL means a weight of ones (bit-identical
 *           to passing ones).
 *   rows    number of rows (B*S); 0 returns LTXNORM_OK and enqueues nothing
 *           (pointers may then be NULL).
 *   hidden  row length H, 1 <= H <= LTXNORM_MAX_HIDDEN.  Rows of a whole
 *           number of 16-byte vectors (H a multiple of 8 for bf16/fp16, of 4
 *           for fp32) take the fastest kernels; any other H is supported.
 *   eps     added to the mean of squares inside the root; finite, >= 0.
 *           With eps = 0 an all-zero row gives NaN (0 * inf), as IEEE does.
 *   stream  HIP stream to enqueue on.
 * out, x and weight must be 16-byte aligned.
 */
LTXNORM_API ltxnorm_status ltxnorm_rmsnorm_fwd(void *out, const void *x, const void *weight,
                                               int64_t rows, int64_t hidden, float eps,
                                               hipStream_t stream);

/* ltxnorm_rmsnorm_fwd for any ltxnorm_dtype. */
LTXNORM_API ltxnorm_status ltxnorm_rmsnorm_fwd_dt(void *out, const void *x, const void *weight,
                                                  int64_t rows, int64_t hidden, float eps,
                                                  ltxnorm_dtype dtype, hipStream_t stream);

/*
 * Fused RMSNorm over the full row, then rotate-half RoPE per head.
 *
 *   out, x, weight, rows, eps, stream   as for ltxnorm_rmsnorm_fwd.
 *   cos_tab, sin_tab  binary32 [seq_len, head_dim/2], row-major, read; shared
 *           by all heads; row r of x uses table row (r mod seq_len).  A caller
 *           with other positions (a sequence shard, flattened t*h*w video
 *           positions) passes tables holding one row per position it needs.
 *           Both must be 16-byte aligned and must not overlap out.
 *   hidden  must equal heads * head_dim.
 *   heads   number of heads, >= 1.
 *   head_dim  even, >= 2.  A head_dim that is a multiple of 16 (bf16/fp16)
 *           or 8 (fp32), with hidden a whole number of 16-byte vectors, takes
 *           the vector kernels; other even head_dims pair through LDS (rows
 *           up to 16320 elements held in registers) or, for longer rows,
 *           through the two-pass path.
 *   seq_len number of table rows, >= 1.
 * Shape errors (hidden != heads*head_dim, head_dim odd or < 2, seq_len < 1)
 * give LTXNORM_ERR_SHAPE.
 */
LTXNORM_API ltxnorm_status ltxnorm_rmsnorm_rope_fwd(void *out, const void *x, const void *weight,
                                                    const float *cos_tab, const float *sin_tab,
                                                    int64_t rows, int64_t hidden, int32_t heads,
                                                    int32_t head_dim, int64_t seq_len, float eps,
                                                    hipStream_t stream);

/* ltxnorm_rmsnorm_rope_fwd for any ltxnorm_dtype. */
LTXNORM_API ltxnorm_status ltxnorm_rmsnorm_rope_fwd_dt(void *out, const void *x,
                                                       const void *weight, const float *cos_tab,
                                                       const float *sin_tab, int64_t rows,
                                                       int64_t hidden, int32_t heads,
                                                       int32_t head_dim, int64_t seq_len,
                                                       float eps, ltxnorm_dtype dtype,
                                                       hipStream_t stream);

/*
 * Fused RMSNorm over the full row, then RoPE per head on adjacent pairs.
 *
 * The LTX-2 ltx-kernels README (introduction) lists a sibling op,
 * rms_norm_split_rope, next to rms_norm_rope, without defining either; the
 * two standard pairings are rotate-half (ltxnorm_rmsnorm_rope_fwd) and the
 * interleaved one computed here:
 *     out[2i]     = y[2i] * c - y[2i + 1] * s
 *     out[2i + 1] = y[2i + 1] * c + y[2i] * s
 * with c = cos_tab[p, i], s = sin_tab[p, i] for i < head_dim/2 within each
 * head, p = row mod seq_len, on the un-rounded binary32 y.
 *
 * Arguments, layouts, ownership and errors as for ltxnorm_rmsnorm_rope_fwd
 * (head_dim even; multiples of 8 bf16/fp16 or 4 fp32 with hidden a whole
 * number of vectors take the vector kernel).
 */
LTXNORM_API ltxnorm_status ltxnorm_rmsnorm_rope_interleaved_fwd(
    void *out, const void *x, const void *weight, const float *cos_tab, const float *sin_tab,
    int64_t rows, int64_t hidden, int32_t heads, int32_t head_dim, int64_t seq_len, float eps,
    hipStream_t stream);

/* ltxnorm_rmsnorm_rope_interleaved_fwd for any ltxnorm_dtype. */
LTXNORM_API ltxnorm_status ltxnorm_rmsnorm_rope_interleaved_fwd_dt(
    void *out, const void *x, const void *weight, const float *cos_tab, const float *sin_tab,
    int64_t rows, int64_t hidden, int32_t heads, int32_t head_dim, int64_t seq_len, float eps,
    ltxnorm_dtype dtype, hipStream_t stream);

/*
 * RMSNorm with per-sample adaptive modulation (AdaLN, the conditioning step
 * of a DiT block): Hugging Face cuda-kernels skill page, section
 * "Kernel-Specific Guidelines", AdaLN, gives norm(x) * weight * (1 + scale)
 * + shift.  Computed as
 *     y[r, j] = ((x[r, j] * rstd_r) * w[j]) * (1 + scale[b, j]) + shift[b, j]
 * with b = r / rows_per_sample (integer division), binary32 arithmetic and
 * one rounding to bf16.
 *
 *   out, x, weight, rows, hidden, eps, stream   as for ltxnorm_rmsnorm_fwd.
 *   scale, shift  bf16 [ceil(rows / rows_per_sample), hidden], row-major,
 *           read; NULL means zeros.  With both NULL the call runs
 *           ltxnorm_rmsnorm_fwd's kernel and row split, and the result
 *           equals it bit for bit.  16-byte aligned; must not overlap out.
 *   rows_per_sample  rows sharing one modulation row (S for [B, S, H] x);
 *           >= 1, else LTXNORM_ERR_SHAPE.
 */
LTXNORM_API ltxnorm_status ltxnorm_rmsnorm_adaln_fwd(void *out, const void *x,
                                                     const void *weight, const void *scale,
                                                     const void *shift, int64_t rows,
                                                     int64_t hidden, int64_t rows_per_sample,
                                                     float eps, hipStream_t stream);

/* ltxnorm_rmsnorm_adaln_fwd for any ltxnorm_dtype (scale and shift in the
 * same dtype as x). */
LTXNORM_API ltxnorm_status ltxnorm_rmsnorm_adaln_fwd_dt(void *out, const void *x,
                                                        const void *weight, const void *scale,
                                                        const void *shift, int64_t rows,
                                                        int64_t hidden, int64_t rows_per_sample,
                                                        float eps, ltxnorm_dtype dtype,
                                                        hipStream_t stream);

/* The operations, for ltxnorm_describe_launch. */
typedef enum ltxnorm_op {
    LTXNORM_OP_RMSNORM = 0,           /* ltxnorm_rmsnorm_fwd                   */
    LTXNORM_OP_ROPE = 1,              /* ltxnorm_rmsnorm_rope_fwd (rotate-half) */
    LTXNORM_OP_ROPE_INTERLEAVED = 2,  /* ltxnorm_rmsnorm_rope_interleaved_fwd  */
    LTXNORM_OP_ADALN = 3              /* ltxnorm_rmsnorm_adaln_fwd             */
} ltxnorm_op;

/*
 * Which kernel, and which launch shape, a call of operation `op` with these
 * shapes would use.  It is written as one NUL-terminated line of text into
 * buf, truncated to len bytes, for example
 *     "rmsnorm_kernel wavefronts_per_row=3 vectors_per_lane=2 rows_per_block=2
 *      threads=384 lds_bytes=0 load_priority=always"
 * (the kernel names are those a profiler shows; lds_bytes is the dynamic
 * LDS the launch requests per workgroup, not the kernels' fixed LDS for
 * cross-wavefront sums, table rows or a staged weight).  load_priority
 * says when the kernel's wavefronts raise their priority while a row's
 * loads issue: "always", "never", or "one_wave": only when the launch's
 * whole grid is resident on the device at once (decided at launch from the
 * device's occupancy for that instance; rotate-half and head-packed RoPE
 * then may hold their weight, and AdaLN does hold it, in 4 KB of LDS per
 * workgroup instead of registers, so that more rows fit; such launches of
 * head-packed and whole-row rotate-half RoPE show as
 * rmsnorm_rope_packed_wl_kernel and rmsnorm_rope_xor_wl_kernel).  It changes timing only, never a
 * result bit.  An RMSNorm line of 3 or 4 wavefronts x 2 vectors ends in
 * "one_wave_vectors_per_lane=6" (or 8): when the whole grid then fits on the
 * device at once, one wavefront takes each row with that many vectors per
 * lane instead, adding the squares in the same order, so the result bits
 * do not depend on which of the two a call takes.  Rows of up to 160
 * vectors may share wavefronts instead, in segments of a few lanes:
 *     "rmsnorm_short_kernel lanes_per_row=8 vectors_per_lane=2
 *      rows_per_wavefront=8 rows_per_block=32 threads=256 lds_bytes=0
 *      load_priority=one_wave"
 * The general kernel's line ends in "load_priority=always grid=resident":
 * its grid is capped at the number of workgroups the device holds at once,
 * each workgroup looping over rows; every other kernel takes one workgroup
 * per group of rows.
 * Rows past the register budget take two passes in one workgroup per row,
 *     "rmsnorm_long_kernel passes=2 rows_per_block=1 threads=1024 lds_bytes=0"
 * or, for a few hundred rows of many chunks, the split kernels:
 *     "rmsnorm_split_kernels launches=3 chunks_per_row=64
 *      vectors_per_chunk=2048 slots_per_row=64 threads=256 lds_bytes=0
 *      in_place=rmsnorm_long_kernel"
 * where in_place names the kernel a call with out == x takes instead (the
 * split stages partial sums in out, which must not be x).  heads and
 * head_dim are read for the RoPE operations only.  LTXNORM_OP_ADALN describes a call
 * with modulation rows (one with neither runs LTXNORM_OP_RMSNORM's kernel).
 *
 * The row split fixes the order in which a row's squares are added, so two
 * operations give bit-identical normalised values only when they take the
 * same split: RoPE at position 0 (cos 1, sin 0) equals RMSNorm bit for bit
 * where both take the same split, and within the rounding of the sum
 * elsewhere.
 *
 * Shapes are validated as the entry point validates them.  No pointer
 * other than buf is involved: the call enqueues nothing and needs no GPU.
 * Returns the status the entry point would return for the shapes,
 * LTXNORM_ERR_NULL for a NULL buf with len > 0, or LTXNORM_ERR_UNSUPPORTED
 * for an unknown op.  rows == 0 describes as "none".
 */
LTXNORM_API ltxnorm_status ltxnorm_describe_launch(ltxnorm_op op, int64_t rows, int64_t hidden,
                                                   int32_t heads, int32_t head_dim,
                                                   ltxnorm_dtype dtype, char *buf, size_t len);

/* Static, never-NULL description of a status code (unknown codes included). */
LTXNORM_API const char *ltxnorm_status_str(ltxnorm_status s);

/* LTXNORM_ABI_VERSION of the built library. */
LTXNORM_API int ltxnorm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LTXNORM_H */
