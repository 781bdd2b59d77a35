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

// Launch geometry shared by the host-side choice below and the kernels.
constexpr int kWave = 64;                 // lanes per wavefront
constexpr int kMaxVecPerLane = 8;         // register budget for one row slice
constexpr int kMaxWavesPerRow = 16;       // 1024-thread workgroup
constexpr int64_t kMaxGrid = 1 << 30;     // rows beyond grid * rows-per-block loop
// Register budget of the one-pass kernels, in 16-byte vectors per row.
constexpr int64_t kMaxRowVectors = (int64_t)kMaxWavesPerRow * kWave * kMaxVecPerLane;
// The general kernel also holds two weight chunks per vector: at most five
// vectors per lane (more spill at 16 wavefronts); longer rows take the
// two-pass kernel.
constexpr int kMaxGeneralVecPerLane = 5;
constexpr int64_t kMaxGeneralRowVectors = (int64_t)kMaxWavesPerRow * kWave * kMaxGeneralVecPerLane;
// Dynamic LDS the rotate-half general kernel may take per workgroup.
constexpr int64_t kMaxExchangeLds = 64 * 1024 - 256;
constexpr int kLongThreads = 1024;        // two-pass kernel: one row per workgroup
// Split kernels (rows beyond the register budget, out of place): chunks of
// kSplitChunkVectors vectors of a row, one 256-thread workgroup each, at most
// kSplitMaxChunkCount chunks per row (the partials a wavefront reads at once).
// The two-pass kernel gives a row one 1024-thread workgroup, one at a time
// per CU: rows go in rounds of 256, and a round that is not full still lasts
// about as long as one workgroup's stream (about 35 GB/s).  Rows of at least
// kSplitMinChunks chunks take the split below kSplitMaxRows rows (bf16 rows
// of 262144, us, two passes -> split: 96 rows 44.5 -> 35.6; 160 53.5 ->
// 50.7; 288 99.2 -> 83.0; 384 118.9 -> 103.0; 512 144.6 -> 130.4; 576
// 169.9 -> 156.5; 608 173.4 -> 170.2; but 256 rows 69.7 -> 71.9, 640 174.2
// -> 178.4, 768 210.1 -> 212.1).  With fewer chunks the split's three
// launches cost more than they gain (128 rows of 65544, five chunks: 16.5 ->
// 23.4 us; 1200 rows of 131072, eight chunks: 154.7 -> 165.0 us).
constexpr int kSplitChunkVectors = 2048;
constexpr int kSplitMaxChunkCount = 2048;
constexpr int kSplitMinChunks = 16;
constexpr int64_t kSplitMaxRows = 623;
// Workgroup slots per row in the split's second launch (every chunk).
// Workgroups are dealt to the 8 XCDs in turn, so with the slot count a
// multiple of 8 chunk c of every row runs on the same XCD and that XCD's L2
// keeps its weight chunk: 64 rows of 2^20 fetched the 2 MB weight about 25
// times when a chunk fell on a different XCD for every row, and ran 79.3 ->
// 75.5 us with one XCD per chunk.  Padding a count leaves one XCD with fewer
// chunks per row (15 chunks padded to 16: 2 on seven XCDs, 1 on the eighth;
// 160 rows of 262144 ran 50.7 -> 52.3 us), so a count is padded only where
// that costs at most 2 %.
constexpr __host__ __device__ int split_slots(int chunks) {
    const int padded = (chunks + 7) & ~7;
    return padded * 50 <= chunks * 51 ? padded : chunks;
}

// Samples (modulation rows) for `rows` rows of `rows_per_sample` each, the
// last possibly partial: ceil(rows / rows_per_sample) without overflow for
// any rows >= 0 and rows_per_sample >= 1 (a caller may pass a huge
// rows_per_sample to mean one sample).
inline int64_t sample_count(int64_t rows, int64_t rows_per_sample) {
    return rows / rows_per_sample + (rows % rows_per_sample != 0 ? 1 : 0);
}

// How a row is split over lanes.
struct Plan {
    int wpr;    // wavefronts per row
    int per;    // vectors (or pair units) per lane
    bool full;  // no masking needed
};

// How a row is split.  `items` are 16-byte vectors, or pair units of two
// vectors.  A single wavefront takes the row while each lane holds at most
// `one_wave_max` items; longer rows are spread over enough wavefronts (up to
// 16) that each lane holds about `spread` items, and past 16 wavefronts the
// lanes take more, up to the register budget.  Measured at [16384 x 3072]
// bf16 (384 vectors per row): 3 wavefronts x 2 vectors reached 6.08 TB/s,
// 2 x 3 6.02, 1 x 6 5.98, 6 x 1 5.46; at hidden 2048 one wavefront x 4
// vectors was best (6.11 TB/s) and 4 x 1 the worst.
inline Plan plan_for(int64_t items, int one_wave_max, int spread) {
    int wpr = 1;
    if (items > (int64_t)kWave * one_wave_max) {
        const int64_t w = (items + (int64_t)kWave * spread - 1) / ((int64_t)kWave * spread);
        wpr = (int)(w < kMaxWavesPerRow ? w : kMaxWavesPerRow);
    }
    const int64_t lanes = (int64_t)kWave * wpr;
    const int per = (int)((items + lanes - 1) / lanes);
    return Plan{wpr, per, items == (int64_t)per * lanes};
}

// The split for AdaLN and the fused RoPE kernels, which read more than x and
// the weight per vector (modulation rows, table slices) or exchange values
// between lanes: rows of 257..768 vectors go over two or three wavefronts
// with 3-4 vectors per lane instead of 3-6 wavefronts with 2.  Measured at
// about 200 MB per launch, bf16 (% of 8 TB/s, plan_for's split -> this one):
// AdaLN 55.6 -> 67.0 at hidden 2304, 59.8 -> 68.4 at 2560, 66.4 -> 67.6 at
// 3072, 63.3 -> 65.2 at 5120, 63.7 -> 65.0 at 6144, even at 4096; rotate-half
// RoPE (heads of 128) 65.5 -> 73.8 at 2304, 69.2 -> 74.5 at 2560, 73.5 ->
// 74.8 at 3072, 72.6 -> 74.1 at 3584.  At 8192 (1024 vectors) AdaLN keeps
// plan_for's 8 x 2 (65.3 against 62.1 for 4 x 4).
constexpr int64_t kWideMin = (int64_t)kWave * 4 + 1;
constexpr int64_t kWideMax = (int64_t)kWave * 4 * 3;
constexpr int64_t kWideIlMax = (int64_t)kWave * 5;
inline Plan plan_wide(int64_t items) {
    if (items < kWideMin || items > kWideMax) return plan_for(items, 4, 2);
    return plan_for(items, 4, 4);
}

// Rotate-half RoPE takes plan_wide's split up to 512 vectors, 3 vectors per
// lane over three or four wavefronts for 513..768 (hidden 5120, heads of
// 128: 71.9 -> 73.2 %; 6144: 72.0 -> 73.8 %; up to 512 vectors that split
// would be 3 x 3, which measured 2-3 points below plan_wide's), and 4 vectors
// per lane past 768 (against plan_for's 2, heads of 128: hidden 6656 68.3 ->
// 71.8 %, 8192 70.3 -> 71.7 %, 12288 66.2 -> 69.8 %, 16384 65.3 -> 68.8 %;
// at 24576 the two tie, and past 4096 vectors both are 16 wavefronts).
inline Plan plan_wide_xor(int64_t items) {
    if (items < kWideMin) return plan_for(items, 4, 2);
    if (items > kWideMax) return plan_for(items, 4, 4);
    if (items <= (int64_t)kWave * 4 * 2) return plan_wide(items);
    return plan_for(items, 4, 3);
}

// Rows per workgroup: four single-wavefront rows, two rows of 2-3
// wavefronts, one row of 4-16 wavefronts.
constexpr int rows_per_block(int wpr) { return wpr == 1 ? 4 : (wpr <= 3 ? 2 : 1); }

// The kernel that serves a request.
enum class Kernel {
    kNone,                   // nothing to launch (no rows)
    kRmsNorm,                // rmsnorm_kernel
    kAdaLN,                  // rmsnorm_adaln_kernel
    kRopeXor,                // rmsnorm_rope_xor_kernel (power-of-two half heads)
    kRopePacked,             // rmsnorm_rope_packed_kernel, half heads of whole vectors
    kRopePackedOdd,          // rmsnorm_rope_packed_kernel, half heads of odd 4-element groups
    kRopePair,               // rmsnorm_rope_pair_kernel
    kRopeInterleaved,        // rmsnorm_rope_interleaved_kernel, table slice per slot
    kRopeInterleavedShared,  // rmsnorm_rope_interleaved_kernel, one table slice per row
    kShort,                  // rmsnorm_short_kernel (rows in segments of at most 32 lanes)
    kGeneral,                // rmsnorm_general_kernel (any row length)
    kLong,                   // rmsnorm_long_kernel (two passes, one workgroup per row)
    kSplit,                  // rmsnorm_split_* kernels (long rows in chunks, three launches)
};

// Rows of at most kMaxShortVectors vectors can always take one vector per
// lane on the power of two at or above their vector count (64 / lanes rows
// per wavefront): the layout rotate-half falls back to when two vectors per
// lane would put a vector's partner outside the row's segment.  Segmented
// rows take four wavefronts per workgroup.
constexpr int kMaxShortVectors = 32;
constexpr int kShortWavesPerBlock = 4;

struct Choice {
    Kernel kernel;
    Plan plan;            // one-pass kernels: row split; segmented rows: per = vectors per lane
    int64_t lds_per_row;  // dynamic LDS bytes per row slot (general rotate-half)
    int lanes_per_row;    // segmented rows: lanes per row (a power of two <= 32)
    int chunks = 0;       // split kernels: chunks per row
};

inline int pow2_at_least(int64_t n) {
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

// Rows of at most 160 vectors in segments of S lanes (a power of two up to
// 32) with V vectors per lane, 64 / S rows per wavefront; {0, 0} leaves the
// row to one wavefront per row with ceil(n / 64) vectors per lane.
//  * n <= 8: one vector per lane on the power of two at or above n (two
//    vectors on half the lanes measured 47 % against 75 % at hidden 32, 61
//    against 75 % at 64: a load then reads half of each 128-byte line).
//  * 9 <= n <= 64: two vectors per lane on the power of two at or above n / 2
//    lanes (16 x 3 for 33..48, which needs fewer slots).
//    Against one vector per lane on the power of two at or above n, or one
//    wavefront per row (bf16, about 200 MB per launch, % of 8 TB/s): hidden
//    128 (8 x 2) RMSNorm 70-75 -> 76.7, AdaLN 65-68 -> 73.6, rotate-half
//    64 -> 69, interleaved 63 -> 68; 256 (16 x 2) 74 -> 77, 66 -> 73.7, 64.5
//    -> 70.3, 63.5 -> 72.2; 512 (32 x 2) 73 -> 76.6, 69 -> 73.1, 66 -> 70.5,
//    70 -> 73.  Four vectors per lane measured lower at 16 and 32 vectors.
//  * 65..160: 16 x 5, 32 x 3 or, with `with_32x5`, 32 x 5 where it covers
//    the row in fewer slots than one wavefront per row (fewest slots wins):
//    AdaLN at hidden 576 (16 x 5) 59 -> 69.5 %, 704 (32 x 3) 65.5 -> 70 %,
//    1152 (32 x 5) 67.1 -> 68.7 %; rotate-half RoPE (heads of 64) at 576 55
//    -> 68.7 %, 1152 67.4 -> 70.4 %; interleaved at 576 60 -> 67 %.  32 x 5
//    lost for interleaved RoPE (1152: 68 -> 66 %) and RMSNorm (75.9 -> 75.5
//    %), which keep one wavefront; so does every row of 97..128 vectors (one
//    wavefront with 2 vectors per lane beat 32 x 4 by 1-5 points for the
//    fused operations at hidden 1024).
struct Segments {
    int lanes, per;
};
inline Segments segments_for(int64_t n, bool with_32x5) {
    if (n < 1 || n > 160) return Segments{0, 0};
    if (n <= 8) return Segments{pow2_at_least(n), 1};
    if (n <= 64) {
        if (n > 32 && n <= 48) return Segments{16, 3};
        return Segments{pow2_at_least((n + 1) / 2), 2};
    }
    static constexpr Segments kShapes[] = {{16, 5}, {32, 3}, {32, 5}};
    const int64_t one_wave = (int64_t)kWave * ((n + kWave - 1) / kWave);
    Segments best{0, 0};
    for (const Segments& c : kShapes) {
        if (c.lanes == 32 && c.per == 5 && !with_32x5) continue;
        const int64_t slots = (int64_t)c.lanes * c.per;
        if (slots >= n && slots < one_wave && (best.lanes == 0 || slots < (int64_t)best.lanes * best.per))
            best = c;
    }
    return best;
}

// The kernel and row split for a validated request with E elements per
// 16-byte vector.  Rows of whole vectors within the register budget take
// the vector kernels (and heads those kernels can pair); other rows that fit
// take the general one-pass kernel; longer rows the two-pass kernel.
inline Choice choose(Op op, const Request& r, int E) {
    const int64_t H = r.hidden;
    if (r.rows == 0) return Choice{Kernel::kNone, Plan{0, 0, false}, 0, 0};
    const bool whole = H % E == 0;
    // most vectors one row touches (a row that starts inside a vector
    // touches up to two more than H / E)
    const int64_t touched = whole ? H / E : (H + 2 * E - 2) / E;
    const bool fits = touched <= kMaxRowVectors;
    const bool gfits = touched <= kMaxGeneralRowVectors;
    const Plan gp = plan_for(touched, 4, 2);
    const Choice general{Kernel::kGeneral, gp, 0, 0};
    // rows past the budget: two passes in one workgroup per row, or, for a
    // few rows of many chunks, in chunks over many workgroups when the call
    // is out of place (the partial sums are staged in the row's own output)
    // and the operation is element-wise after the norm
    const bool in_place = r.out != nullptr && r.out == r.x;
    const int64_t chunks = (touched + kSplitChunkVectors - 1) / kSplitChunkVectors;
    const bool split = !in_place && op != Op::kRopeRotateHalf && r.rows <= kSplitMaxRows &&
                       chunks >= kSplitMinChunks && chunks <= kSplitMaxChunkCount;
    const Choice two_pass = split ? Choice{Kernel::kSplit, Plan{4, kSplitChunkVectors / 256, false}, 0, 0, (int)chunks}
                                  : Choice{Kernel::kLong, Plan{kLongThreads / kWave, 0, false}, 0, 0};
    const int64_t nvec = H / E;
    const bool short_row = whole && nvec <= kMaxShortVectors;
    const Choice short_rows{Kernel::kShort, Plan{1, 1, false}, 0, short_row ? pow2_at_least(nvec) : 0};
    const bool wide_op = op == Op::kAdaLN || op == Op::kRopeRotateHalf;
    const Segments sg = whole ? segments_for(nvec, wide_op) : Segments{0, 0};
    const Choice segmented{Kernel::kShort, Plan{1, sg.per, false}, 0, sg.lanes};
    switch (op) {
        case Op::kRmsNorm:
            if (sg.lanes) return segmented;
            if (whole && fits) return Choice{Kernel::kRmsNorm, plan_for(nvec, 4, 2), 0, 0};
            return gfits ? general : two_pass;
        case Op::kAdaLN:
            if (sg.lanes) return segmented;
            if (whole && fits) return Choice{Kernel::kAdaLN, plan_wide(nvec), 0, 0};
            return gfits ? general : two_pass;
        case Op::kRopeRotateHalf: {
            const int d = r.head_dim;
            const bool even = d % (2 * E) == 0;                 // half heads of whole vectors
            const bool odd = E == 8 && d % E == 0 && !even;     // ... of 4-element groups
            if (whole && fits && even) {
                const int P = d / (2 * E);
                if ((P & (P - 1)) == 0 && P <= kWave / 2) {  // partner lanes within one wavefront
                    // partner l ^ P inside the row's lanes, or the lane's
                    // other slot (two vectors per lane, P == lanes)
                    if (sg.lanes && (2 * P <= sg.lanes || (sg.per == 2 && P == sg.lanes))) return segmented;
                    if (short_row) return short_rows;     // one vector per lane
                    return Choice{Kernel::kRopeXor, plan_wide_xor(nvec), 0, 0};
                }
            }
            const int vph = d / E;
            if (whole && fits && (even || odd) && vph <= kWave / 2) {
                // heads packed into wavefronts (lw of 64 lanes used); the
                // wide split for 257..768 lane slots' worth of vectors, as
                // for the other fused kernels (bf16, about 200 MB per launch:
                // 32 x 72 57 -> 70.6 %, 40 x 72 65 -> 72 %, 32 x 80 61 -> 71 %,
                // 32 x 96 66.5 -> 71 %)
                const int lw = kWave - kWave % vph;
                Plan p = plan_wide((nvec * kWave + lw - 1) / lw);
                p.per = (int)((nvec + (int64_t)lw * p.wpr - 1) / ((int64_t)lw * p.wpr));
                p.full = false;
                if (p.per <= kMaxVecPerLane)
                    return Choice{odd ? Kernel::kRopePackedOdd : Kernel::kRopePacked, p, 0, 0};
            }
            if (whole && fits && even) return Choice{Kernel::kRopePair, plan_for(H / (2 * E), 2, 1), 0, 0};
            const int64_t lds_row = H * (int64_t)sizeof(float);
            if (gfits && lds_row * rows_per_block(gp.wpr) <= kMaxExchangeLds)
                return Choice{Kernel::kGeneral, gp, lds_row, 0};
            return two_pass;
        }
        case Op::kRopeInterleaved: {
            if (whole && fits && r.head_dim % E == 0) {
                if (sg.lanes) return segmented;
                // The wide split only where plan_for's 3 x 2 leaves a sixth
                // or more of its slots idle: hidden 2304 (bf16, heads of
                // 128) 68.8 -> 74.0 %, 2560 71.0 -> 74.0 %; from 384 vectors
                // on, plan_for's split measured 1-4 points better (3072,
                // 3584, 4096, 6144, 8192).
                const Plan p = nvec <= kWideIlMax ? plan_wide(nvec) : plan_for(nvec, 4, 2);
                const int vph = r.head_dim / E;
                return Choice{(kWave * p.wpr) % vph == 0 ? Kernel::kRopeInterleavedShared
                                                         : Kernel::kRopeInterleaved,
                              p, 0, 0};
            }
            return gfits ? general : two_pass;
        }
    }
    return Choice{Kernel::kNone, Plan{0, 0, false}, 0, 0};
}

// Rows of W wavefronts x P vectors per lane that a launch may regroup into
// one wavefront of W * P vectors per lane when that grid is resident at
// once (adding the squares in the W-wavefront order, so the bits do not
// change): the vectors per lane of that form, or 0.  Per kernel, the splits
// its plans produce that have such instances: RMSNorm 3 x 2 and 4 x 2,
// AdaLN and rotate-half RoPE 2 x 3 and 2 x 4, interleaved RoPE with one
// table slice per row 2 x 3, 3 x 2 and 4 x 2 when a head's vectors
// (vec_per_head) divide one wavefront's lanes, so the slice stays shared.
inline int regroup_vectors(Kernel k, const Plan& p, int vec_per_head) {
    const int W = p.wpr, P = p.per;
    bool ok = false;
    switch (k) {
        case Kernel::kRmsNorm: ok = P == 2 && (W == 3 || W == 4); break;
        case Kernel::kAdaLN:
        case Kernel::kRopeXor: ok = W == 2 && (P == 3 || P == 4); break;
        case Kernel::kRopeInterleavedShared:
            ok = ((W == 2 && P == 3) || (P == 2 && (W == 3 || W == 4))) && vec_per_head > 0 &&
                 kWave % vec_per_head == 0;
            break;
        default: break;
    }
    return ok ? W * P : 0;
}

inline const char* kernel_name(Kernel k) {
    switch (k) {
        case Kernel::kNone: return "none";
        case Kernel::kRmsNorm: return "rmsnorm_kernel";
        case Kernel::kAdaLN: return "rmsnorm_adaln_kernel";
        case Kernel::kRopeXor: return "rmsnorm_rope_xor_kernel";
        case Kernel::kRopePacked: return "rmsnorm_rope_packed_kernel";
        case Kernel::kRopePackedOdd: return "rmsnorm_rope_packed_kernel(odd)";
        case Kernel::kRopePair: return "rmsnorm_rope_pair_kernel";
        case Kernel::kRopeInterleaved: return "rmsnorm_rope_interleaved_kernel";
        case Kernel::kRopeInterleavedShared: return "rmsnorm_rope_interleaved_kernel(shared)";
        case Kernel::kShort: return "rmsnorm_short_kernel";
        case Kernel::kGeneral: return "rmsnorm_general_kernel";
        case Kernel::kLong: return "rmsnorm_long_kernel";
        case Kernel::kSplit: return "rmsnorm_split_kernels";
    }
    return "?";
}

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
