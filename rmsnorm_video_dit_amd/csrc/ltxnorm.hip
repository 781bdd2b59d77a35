// ltxnorm.hip -- C ABI of libltxnorm.so (declared in include/ltxnorm.h):
// host-side validation of every argument before any HIP call, then dispatch
// to the kernels of the I/O dtype (ltxnorm_bf16.hip, ltxnorm_f16.hip,
// ltxnorm_f32.hip; the kernels themselves are in ltxnorm_kernels.h and
// ltxnorm_general.h).
//
// Operations: RMSNorm over [..., hidden] with optional weight and eps (Hugging
// Face cuda-kernels skill page, "Kernel-Specific Guidelines", RMSNorm); the
// fused RMSNorm + RoPE op rms_norm_rope of the LTX-2 ltx-kernels README
// (introduction), with rotate-half or interleaved pairs; AdaLN modulation
// (skill page, "Kernel-Specific Guidelines", AdaLN); in the three precisions
// the skill page lists ("Supported Data Types").

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>

#include "ltxnorm.h"
#include "ltxnorm_launch.h"

using ltxnorm_detail::Op;
using ltxnorm_detail::Request;

namespace {

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Half-open byte ranges [a, a + na) and [b, b + nb) overlap.
bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

// Shape checks shared by every entry point, in order: dtype, shape, scalar
// value.
ltxnorm_status check_shape(int64_t rows, int64_t hidden, float eps, ltxnorm_dtype dtype) {
    if (ltxnorm_detail::elems_per_vec(dtype) == 0) return LTXNORM_ERR_UNSUPPORTED;
    const int eb = ltxnorm_detail::elem_bytes(dtype);
    if (rows < 0 || hidden <= 0) return LTXNORM_ERR_SHAPE;
    if (hidden > LTXNORM_MAX_HIDDEN) return LTXNORM_ERR_UNSUPPORTED;
    if (rows > INT64_MAX / (hidden * eb)) return LTXNORM_ERR_SHAPE;
    if (!std::isfinite(eps) || eps < 0.0f) return LTXNORM_ERR_VALUE;
    return LTXNORM_OK;
}

// The RoPE entry points' extra shape checks: rotation pairs need an even
// head_dim, and the heads must tile the row.
ltxnorm_status check_rope_shape(int64_t hidden, int32_t heads, int32_t head_dim, int64_t seq_len) {
    if (heads < 1 || head_dim < 2 || head_dim % 2 != 0 || seq_len < 1 ||
        (int64_t)heads * head_dim != hidden)
        return LTXNORM_ERR_SHAPE;
    if (seq_len > INT64_MAX / ((int64_t)head_dim * 4)) return LTXNORM_ERR_SHAPE;
    return LTXNORM_OK;
}

// Checks shared by every entry point, in order: dtype, shape, scalar value,
// empty, pointers, alignment, aliasing.  Returns OK with *empty set when
// there is nothing to launch.
ltxnorm_status check_common(void* out, const void* x, const void* weight, int64_t rows,
                            int64_t hidden, float eps, ltxnorm_dtype dtype, bool* empty) {
    *empty = false;
    const ltxnorm_status st = check_shape(rows, hidden, eps, dtype);
    if (st != LTXNORM_OK) return st;
    const int eb = ltxnorm_detail::elem_bytes(dtype);
    if (rows == 0) {
        *empty = true;
        return LTXNORM_OK;
    }
    if (out == nullptr || x == nullptr) return LTXNORM_ERR_NULL;
    if (misaligned(out) || misaligned(x) || (weight && misaligned(weight))) return LTXNORM_ERR_ALIGN;
    const int64_t nbytes = rows * hidden * eb;
    if (out != x && overlap(out, nbytes, x, nbytes)) return LTXNORM_ERR_ALIAS;
    if (weight && overlap(out, nbytes, weight, hidden * eb)) return LTXNORM_ERR_ALIAS;
    return LTXNORM_OK;
}

// Validation shared by the RoPE entry points.
ltxnorm_status check_rope(void* out, const void* x, const void* weight, const float* cos_tab,
                          const float* sin_tab, int64_t rows, int64_t hidden, int32_t heads,
                          int32_t head_dim, int64_t seq_len, float eps, ltxnorm_dtype dtype,
                          bool* empty) {
    if (ltxnorm_detail::elems_per_vec(dtype) == 0) return LTXNORM_ERR_UNSUPPORTED;
    ltxnorm_status st = check_rope_shape(hidden, heads, head_dim, seq_len);
    if (st != LTXNORM_OK) return st;
    st = check_common(out, x, weight, rows, hidden, eps, dtype, empty);
    if (st != LTXNORM_OK || *empty) return st;
    if (cos_tab == nullptr || sin_tab == nullptr) return LTXNORM_ERR_NULL;
    if (misaligned(cos_tab) || misaligned(sin_tab)) return LTXNORM_ERR_ALIGN;
    const int64_t nbytes = rows * hidden * ltxnorm_detail::elem_bytes(dtype);
    const int64_t tbytes = seq_len * (head_dim / 2) * 4;
    if (overlap(out, nbytes, cos_tab, tbytes) || overlap(out, nbytes, sin_tab, tbytes))
        return LTXNORM_ERR_ALIAS;
    return LTXNORM_OK;
}

ltxnorm_status dispatch(Op op, const Request& r, ltxnorm_dtype dtype, hipStream_t stream) {
    switch (dtype) {
        case LTXNORM_BF16: return ltxnorm_detail::launch_bf16(op, r, stream);
        case LTXNORM_F16: return ltxnorm_detail::launch_f16(op, r, stream);
        case LTXNORM_F32: return ltxnorm_detail::launch_f32(op, r, stream);
    }
    return LTXNORM_ERR_UNSUPPORTED;
}

ltxnorm_status rope(Op op, void* out, const void* x, const void* weight, const float* cos_tab,
                    const float* sin_tab, int64_t rows, int64_t hidden, int32_t heads,
                    int32_t head_dim, int64_t seq_len, float eps, ltxnorm_dtype dtype,
                    hipStream_t stream) {
    bool empty = false;
    ltxnorm_status st = check_rope(out, x, weight, cos_tab, sin_tab, rows, hidden, heads, head_dim,
                                   seq_len, eps, dtype, &empty);
    if (st != LTXNORM_OK || empty) return st;
    const Request r{out, x, weight, cos_tab, sin_tab, nullptr, nullptr, rows, hidden,
                    seq_len, 1, head_dim, eps};
    return dispatch(op, r, dtype, stream);
}

}  // namespace

extern "C" {

LTXNORM_API ltxnorm_status ltxnorm_rmsnorm_fwd_dt(void* out, const void* x, const void* weight,
                                                  int64_t rows, int64_t hidden, float eps,
                                                  ltxnorm_dtype dtype, hipStream_t stream) {
    bool empty = false;
    ltxnorm_status st = check_common(out, x, weight, rows, hidden, eps, dtype, &empty);
    if (st != LTXNORM_OK || empty) return st;
    const Request r{out, x, weight, nullptr, nullptr, nullptr, nullptr, rows, hidden, 1, 1, 0, eps};
    return dispatch(Op::kRmsNorm, r, dtype, stream);
}

LTXNORM_API ltxnorm_status ltxnorm_rmsnorm_fwd(void* out, const void* x, const void* weight,
                                               int64_t rows, int64_t hidden, float eps,
                                               hipStream_t stream) {
    return ltxnorm_rmsnorm_fwd_dt(out, x, weight, rows, hidden, eps, LTXNORM_BF16, stream);
}

LTXNORM_API ltxnorm_status ltxnorm_rmsnorm_rope_fwd_dt(void* out, const void* x, const void* weight,
                                                       const float* cos_tab, const float* sin_tab,
                                                       int64_t rows, int64_t hidden, int32_t heads,
                                                       int32_t head_dim, int64_t seq_len, float eps,
                                                       ltxnorm_dtype dtype, hipStream_t stream) {
    return rope(Op::kRopeRotateHalf, out, x, weight, cos_tab, sin_tab, rows, hidden, heads,
                head_dim, seq_len, eps, dtype, stream);
}

LTXNORM_API ltxnorm_status ltxnorm_rmsnorm_rope_fwd(void* out, const void* x, const void* weight,
                                                    const float* cos_tab, const float* sin_tab,
                                                    int64_t rows, int64_t hidden, int32_t heads,
                                                    int32_t head_dim, int64_t seq_len, float eps,
                                                    hipStream_t stream) {
    return rope(Op::kRopeRotateHalf, out, x, weight, cos_tab, sin_tab, rows, hidden, heads,
                head_dim, seq_len, eps, LTXNORM_BF16, stream);
}

LTXNORM_API ltxnorm_status ltxnorm_rmsnorm_rope_interleaved_fwd_dt(
    void* out, const void* x, const void* weight, const float* cos_tab, const float* sin_tab,
    int64_t rows, int64_t hidden, int32_t heads, int32_t head_dim, int64_t seq_len, float eps,
    ltxnorm_dtype dtype, hipStream_t stream) {
    return rope(Op::kRopeInterleaved, out, x, weight, cos_tab, sin_tab, rows, hidden, heads,
                head_dim, seq_len, eps, dtype, stream);
}

LTXNORM_API ltxnorm_status ltxnorm_rmsnorm_rope_interleaved_fwd(
    void* out, const void* x, const void* weight, const float* cos_tab, const float* sin_tab,
    int64_t rows, int64_t hidden, int32_t heads, int32_t head_dim, int64_t seq_len, float eps,
    hipStream_t stream) {
    return rope(Op::kRopeInterleaved, out, x, weight, cos_tab, sin_tab, rows, hidden, heads,
                head_dim, seq_len, eps, LTXNORM_BF16, stream);
}

LTXNORM_API ltxnorm_status ltxnorm_rmsnorm_adaln_fwd_dt(void* out, const void* x, const void* weight,
                                                        const void* scale, const void* shift,
                                                        int64_t rows, int64_t hidden,
                                                        int64_t rows_per_sample, float eps,
                                                        ltxnorm_dtype dtype, hipStream_t stream) {
    if (ltxnorm_detail::elems_per_vec(dtype) == 0) return LTXNORM_ERR_UNSUPPORTED;
    if (rows_per_sample < 1) return LTXNORM_ERR_SHAPE;
    bool empty = false;
    ltxnorm_status st = check_common(out, x, weight, rows, hidden, eps, dtype, &empty);
    if (st != LTXNORM_OK || empty) return st;
    if ((scale && misaligned(scale)) || (shift && misaligned(shift))) return LTXNORM_ERR_ALIGN;
    const int eb = ltxnorm_detail::elem_bytes(dtype);
    const int64_t samples = ltxnorm_detail::sample_count(rows, rows_per_sample);
    const int64_t nbytes = rows * hidden * eb;
    const int64_t mbytes = samples * hidden * eb;
    if ((scale && overlap(out, nbytes, scale, mbytes)) || (shift && overlap(out, nbytes, shift, mbytes)))
        return LTXNORM_ERR_ALIAS;
    const Request r{out, x, weight, nullptr, nullptr, scale, shift, rows, hidden, 1,
                    rows_per_sample, 0, eps};
    // Without modulation rows the operation is RMSNorm.  RMSNorm's kernel and
    // row split then serve it: the split fixes the order in which a row's
    // squares are added, so the result equals ltxnorm_rmsnorm_fwd bit for
    // bit, and the modulation arithmetic is skipped.
    return dispatch(scale == nullptr && shift == nullptr ? Op::kRmsNorm : Op::kAdaLN, r, dtype,
                    stream);
}

LTXNORM_API ltxnorm_status ltxnorm_rmsnorm_adaln_fwd(void* out, const void* x, const void* weight,
                                                     const void* scale, const void* shift,
                                                     int64_t rows, int64_t hidden,
                                                     int64_t rows_per_sample, float eps,
                                                     hipStream_t stream) {
    return ltxnorm_rmsnorm_adaln_fwd_dt(out, x, weight, scale, shift, rows, hidden,
                                        rows_per_sample, eps, LTXNORM_BF16, stream);
}

LTXNORM_API ltxnorm_status ltxnorm_describe_launch(ltxnorm_op op, int64_t rows, int64_t hidden,
                                                   int32_t heads, int32_t head_dim,
                                                   ltxnorm_dtype dtype, char* buf, size_t len) {
    if (buf == nullptr && len > 0) return LTXNORM_ERR_NULL;
    const int epv = ltxnorm_detail::elems_per_vec(dtype);
    if (epv == 0) return LTXNORM_ERR_UNSUPPORTED;
    Op kop;
    switch (op) {
        case LTXNORM_OP_RMSNORM: kop = Op::kRmsNorm; break;
        case LTXNORM_OP_ROPE: kop = Op::kRopeRotateHalf; break;
        case LTXNORM_OP_ROPE_INTERLEAVED: kop = Op::kRopeInterleaved; break;
        case LTXNORM_OP_ADALN: kop = Op::kAdaLN; break;
        default: return LTXNORM_ERR_UNSUPPORTED;
    }
    // the entry points' shape checks (in their order)
    const bool rope = kop == Op::kRopeRotateHalf || kop == Op::kRopeInterleaved;
    ltxnorm_status st = rope ? check_rope_shape(hidden, heads, head_dim, 1) : LTXNORM_OK;
    if (st == LTXNORM_OK) st = check_shape(rows, hidden, 1e-6f, dtype);
    if (st != LTXNORM_OK) return st;
    const Request r{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, rows,
                    hidden, 1, 1, rope ? head_dim : 0, 1e-6f};
    const ltxnorm_detail::Choice c = ltxnorm_detail::choose(kop, r, epv);
    using ltxnorm_detail::Kernel;
    const char* name = ltxnorm_detail::kernel_name(c.kernel);
    if (len == 0) return LTXNORM_OK;
    if (c.kernel == Kernel::kNone) {
        std::snprintf(buf, len, "none");
    } else if (c.kernel == Kernel::kShort) {
        const int per_wave = ltxnorm_detail::kWave / c.lanes_per_row;
        std::snprintf(buf, len, "%s lanes_per_row=%d vectors_per_lane=%d rows_per_wavefront=%d rows_per_block=%d threads=%d lds_bytes=0 load_priority=one_wave",
                      name, c.lanes_per_row, c.plan.per, per_wave, ltxnorm_detail::kShortWavesPerBlock * per_wave,
                      ltxnorm_detail::kWave * ltxnorm_detail::kShortWavesPerBlock);
    } else if (c.kernel == Kernel::kLong) {
        std::snprintf(buf, len, "%s passes=2 rows_per_block=1 threads=%d lds_bytes=0", name,
                      ltxnorm_detail::kLongThreads);
    } else if (c.kernel == Kernel::kSplit) {
        std::snprintf(buf, len, "%s launches=3 chunks_per_row=%d vectors_per_chunk=%d slots_per_row=%d threads=256 lds_bytes=0 in_place=rmsnorm_long_kernel",
                      name, c.chunks, ltxnorm_detail::kSplitChunkVectors, ltxnorm_detail::split_slots(c.chunks));
    } else {
        const int rpb = ltxnorm_detail::rows_per_block(c.plan.wpr);
        // wave priority for the loads: always, when the grid is resident at
        // once (one-wavefront instances), or never (the dispatch's rule)
        const bool always = c.kernel == Kernel::kGeneral ||
                            ((c.kernel == Kernel::kRmsNorm || c.kernel == Kernel::kAdaLN) && c.plan.wpr > 1);
        const bool one_wave = c.plan.wpr == 1 && c.kernel != Kernel::kGeneral && c.kernel != Kernel::kRopePair;
        // rows of a few wavefronts: one wavefront of that many vectors per
        // lane when the whole grid is resident at once
        const int regroup = ltxnorm_detail::regroup_vectors(c.kernel, c.plan, rope ? (int)(head_dim / epv) : 0);
        char tail[64] = "";
        if (c.kernel == Kernel::kGeneral)
            std::snprintf(tail, sizeof(tail), " grid=resident");
        else if (regroup)
            std::snprintf(tail, sizeof(tail), " one_wave_vectors_per_lane=%d", regroup);
        std::snprintf(buf, len, "%s wavefronts_per_row=%d %s=%d rows_per_block=%d threads=%d lds_bytes=%lld load_priority=%s%s",
                      name, c.plan.wpr, c.kernel == Kernel::kRopePair ? "pairs_per_lane" : "vectors_per_lane",
                      c.plan.per, rpb, ltxnorm_detail::kWave * c.plan.wpr * rpb,
                      (long long)(c.lds_per_row * rpb), always ? "always" : (one_wave ? "one_wave" : "never"), tail);
    }
    return LTXNORM_OK;
}

LTXNORM_API const char* ltxnorm_status_str(ltxnorm_status s) {
    switch (s) {
        case LTXNORM_OK: return "ok";
        case LTXNORM_ERR_NULL: return "a required pointer is NULL";
        case LTXNORM_ERR_SHAPE:
            return "invalid shape (rows, hidden, heads, head_dim, seq_len or rows_per_sample)";
        case LTXNORM_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case LTXNORM_ERR_UNSUPPORTED: return "unsupported dtype, or hidden above LTXNORM_MAX_HIDDEN";
        case LTXNORM_ERR_ALIAS: return "out overlaps an input other than exactly x";
        case LTXNORM_ERR_VALUE: return "eps must be finite and non-negative";
        case LTXNORM_ERR_HIP: return "the HIP runtime rejected the kernel launch";
    }
    return "unknown ltxnorm status";
}

LTXNORM_API int ltxnorm_version(void) { return LTXNORM_ABI_VERSION; }

}  // extern "C"
