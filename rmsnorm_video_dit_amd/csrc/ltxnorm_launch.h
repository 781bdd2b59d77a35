// ltxnorm_launch.h -- internal interface between the C-ABI layer
// (ltxnorm.hip) and the per-dtype kernel translation units
// (ltxnorm_bf16.hip, ltxnorm_f16.hip, ltxnorm_f32.hip).  Not installed.
#pragma once

#include <cstdint>

#include "ltxnorm.h"

namespace ltxnorm_detail {

// Which fused operation to run on validated arguments.
enum class Op {
    kRmsNorm,          // RMSNorm
    kRopeRotateHalf,   // RMSNorm + RoPE, pairs (i, i + head_dim/2)
    kRopeInterleaved,  // RMSNorm + RoPE, pairs (2i, 2i + 1)
    kAdaLN,            // RMSNorm * (1 + scale[b]) + shift[b]
};

// Arguments after host-side validation.  Pointers are device pointers;
// unused ones are null.  Shapes are in elements.
struct Request {
    void* out;
    const void* x;
    const void* w;
    const float* cos_tab;
    const float* sin_tab;
    const void* scale;
    const void* shift;
    int64_t rows;
    int64_t hidden;
    int64_t seq_len;
    int64_t rows_per_sample;
    int32_t head_dim;
    float eps;
};

// Elements per 16-byte vector for an I/O dtype (8 for 16-bit types, 4 for
// binary32), or 0 for an unknown dtype.
inline int elems_per_vec(ltxnorm_dtype d) {
    switch (d) {
        case LTXNORM_BF16:
        case LTXNORM_F16: return 8;
        case LTXNORM_F32: return 4;
    }
    return 0;
}

inline int elem_bytes(ltxnorm_dtype d) { return d == LTXNORM_F32 ? 4 : 2; }

// Enqueue one operation; the request has passed validation for this dtype.
ltxnorm_status launch_bf16(Op op, const Request& r, hipStream_t stream);
ltxnorm_status launch_f16(Op op, const Request& r, hipStream_t stream);
ltxnorm_status launch_f32(Op op, const Request& r, hipStream_t stream);

}  // namespace ltxnorm_detail
