// ltxnorm_dispatch.h -- host side: how a row is split over lanes and
// wavefronts, which kernel instance serves a request, and the launch.
// Included once per I/O dtype; not a public header.
#pragma once

#include "ltxnorm_kernels.h"
#include "ltxnorm_general.h"

namespace ltxnorm_detail {
namespace {

// ---------------------------------------------------------------------------
// Host side: row split, per-plan dispatch, launch.
// ---------------------------------------------------------------------------

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

inline ltxnorm_status launch(const void* fn, int threads, int rows_per_block, const KArgs& args,
                             size_t lds_bytes, hipStream_t stream) {
    // One workgroup per group of rows: a grid-stride loop capped at the
    // resident capacity measured 3-4% slower than letting the dispatcher
    // stream fresh workgroups, which keeps every CU busy to the last rows.
    const int64_t need = (args.rows + rows_per_block - 1) / rows_per_block;
    const unsigned grid = (unsigned)(need < kMaxGrid ? need : kMaxGrid);
    KArgs copy = args;
    void* params[] = {&copy};
    const hipError_t e =
        hipLaunchKernel(fn, dim3(grid), dim3(threads), params, (unsigned)lds_bytes, stream);
    return e == hipSuccess ? LTXNORM_OK : LTXNORM_ERR_HIP;
}

// One launcher per kernel family: fn<WPR, PER, FULL>() picks the instance.
template <typename IO>
struct RmsL {
    template <int WPR, int PER, bool FULL>
    static const void* fn() { return (const void*)&rmsnorm_kernel<IO, PER, WPR, FULL>; }
};
template <typename IO>
struct RopeXorL {
    template <int WPR, int PER, bool FULL>
    static const void* fn() { return (const void*)&rmsnorm_rope_xor_kernel<IO, PER, WPR, FULL>; }
};
template <typename IO>
struct RopePairL {
    template <int WPR, int PER, bool FULL>
    static const void* fn() { return (const void*)&rmsnorm_rope_pair_kernel<IO, PER, WPR, FULL>; }
};
template <typename IO, bool SHARED>
struct RopeIlL {
    template <int WPR, int PER, bool FULL>
    static const void* fn() {
        return (const void*)&rmsnorm_rope_interleaved_kernel<IO, PER, WPR, FULL, SHARED>;
    }
};
template <typename IO>
struct AdaL {
    template <int WPR, int PER, bool FULL>
    static const void* fn() { return (const void*)&rmsnorm_adaln_kernel<IO, PER, WPR, FULL>; }
};
template <typename IO, bool ODD>
struct RopePackedL {
    template <int WPR, int PER, bool FULL>
    static const void* fn() { return (const void*)&rmsnorm_rope_packed_kernel<IO, PER, WPR, ODD>; }
};
// The general kernel masks every row itself: FULL does not select anything.
template <typename IO, GOp OP>
struct GeneralL {
    template <int WPR, int PER, bool FULL>
    static const void* fn() { return (const void*)&rmsnorm_general_kernel<IO, OP, PER, WPR>; }
};

template <typename LN, int WPR, int LO, int HI>
ltxnorm_status by_per(const Plan& p, const KArgs& a, size_t lds_per_row, hipStream_t s) {
    if constexpr (LO > HI) {
        return LTXNORM_ERR_UNSUPPORTED;
    } else {
        if (p.per == LO) {
            const void* fn = p.full ? LN::template fn<WPR, LO, true>() : LN::template fn<WPR, LO, false>();
            return launch(fn, Layout<WPR>::kThreads, Layout<WPR>::kRowsPerBlock, a,
                          lds_per_row * Layout<WPR>::kRowsPerBlock, s);
        }
        return by_per<LN, WPR, LO + 1, HI>(p, a, lds_per_row, s);
    }
}

// Plans that plan_for can produce: one wavefront with 1..ONE items per lane;
// 3..15 wavefronts with exactly SPREAD items per lane (2 wavefronts never
// occur: a row too long for one wavefront needs more than 2 * ONE / SPREAD);
// 16 wavefronts with SPREAD..MAXP items per lane.  lds_per_row: dynamic LDS
// bytes per row slot of the block.
template <typename LN, int ONE, int SPREAD, int MAXP>
ltxnorm_status by_plan(const Plan& p, const KArgs& a, hipStream_t s, size_t lds_per_row = 0) {
    switch (p.wpr) {
        case 1: return by_per<LN, 1, 1, ONE>(p, a, lds_per_row, s);
        case 3: return by_per<LN, 3, SPREAD, SPREAD>(p, a, lds_per_row, s);
        case 4: return by_per<LN, 4, SPREAD, SPREAD>(p, a, lds_per_row, s);
        case 5: return by_per<LN, 5, SPREAD, SPREAD>(p, a, lds_per_row, s);
        case 6: return by_per<LN, 6, SPREAD, SPREAD>(p, a, lds_per_row, s);
        case 7: return by_per<LN, 7, SPREAD, SPREAD>(p, a, lds_per_row, s);
        case 8: return by_per<LN, 8, SPREAD, SPREAD>(p, a, lds_per_row, s);
        case 9: return by_per<LN, 9, SPREAD, SPREAD>(p, a, lds_per_row, s);
        case 10: return by_per<LN, 10, SPREAD, SPREAD>(p, a, lds_per_row, s);
        case 11: return by_per<LN, 11, SPREAD, SPREAD>(p, a, lds_per_row, s);
        case 12: return by_per<LN, 12, SPREAD, SPREAD>(p, a, lds_per_row, s);
        case 13: return by_per<LN, 13, SPREAD, SPREAD>(p, a, lds_per_row, s);
        case 14: return by_per<LN, 14, SPREAD, SPREAD>(p, a, lds_per_row, s);
        case 15: return by_per<LN, 15, SPREAD, SPREAD>(p, a, lds_per_row, s);
        case 16: return by_per<LN, 16, SPREAD, MAXP>(p, a, lds_per_row, s);
        default: return LTXNORM_ERR_UNSUPPORTED;
    }
}

inline int rows_per_block(int wpr) { return wpr == 1 ? 4 : (wpr <= 3 ? 2 : 1); }

// Register budget of the one-pass kernels, in 16-byte vectors per row.
constexpr int64_t kMaxRowVectors = (int64_t)kMaxWavesPerRow * kWave * kMaxVecPerLane;
// The general kernel also holds two weight chunks per vector: at most five
// vectors per lane (more spill at 16 wavefronts); longer rows take the
// two-pass kernel.
constexpr int kMaxGeneralVecPerLane = 5;
constexpr int64_t kMaxGeneralRowVectors = (int64_t)kMaxWavesPerRow * kWave * kMaxGeneralVecPerLane;
// Dynamic LDS the rotate-half general kernel may take per workgroup.
constexpr size_t kMaxExchangeLds = 64 * 1024 - 256;

template <typename IO, GOp OP>
ltxnorm_status launch_long(const KArgs& a, hipStream_t stream) {
    return launch((const void*)&rmsnorm_long_kernel<IO, OP>, kLongThreads, 1, a, 0, stream);
}

// Enqueue `op` for I/O type IO on a validated request.  Rows of whole
// vectors that fit the register budget (and heads the vector kernels can
// pair) take the vector kernels; other rows that fit take the general
// one-pass kernel; longer rows the two-pass kernel.
template <typename IO>
ltxnorm_status launch_op(Op op, const Request& r, hipStream_t stream) {
    constexpr int E = IO::kEpv;
    const int64_t samples = (r.rows + r.rows_per_sample - 1) / r.rows_per_sample;
    KArgs a{r.out, r.x, r.w, r.cos_tab, r.sin_tab, r.scale, r.shift, r.rows, r.seq_len,
            r.rows_per_sample, (int32_t)(r.hidden / E), (int32_t)(r.hidden / (2 * E)),
            r.head_dim / (2 * E), r.head_dim / E, r.head_dim / 2, (int32_t)r.hidden, r.head_dim,
            samples * r.hidden, (float)r.hidden, r.eps};
    const bool whole = r.hidden % E == 0;
    // most vectors one row touches (a row that starts inside a vector touches
    // up to two more than hidden / E)
    const int64_t touched = whole ? r.hidden / E : (r.hidden + 2 * E - 2) / E;
    const bool fits = touched <= kMaxRowVectors;
    const bool gfits = touched <= kMaxGeneralRowVectors;
    const Plan gp = plan_for(touched, 4, 2);
    switch (op) {
        case Op::kRmsNorm:
            if (whole && fits)
                return by_plan<RmsL<IO>, 4, 2, kMaxVecPerLane>(plan_for(a.nvec, 4, 2), a, stream);
            if (gfits) return by_plan<GeneralL<IO, GOp::kRms>, 4, 2, kMaxGeneralVecPerLane>(gp, a, stream);
            return launch_long<IO, GOp::kRms>(a, stream);
        case Op::kAdaLN:
            if (whole && fits)
                return by_plan<AdaL<IO>, 4, 2, kMaxVecPerLane>(plan_for(a.nvec, 4, 2), a, stream);
            if (gfits) return by_plan<GeneralL<IO, GOp::kAda>, 4, 2, kMaxGeneralVecPerLane>(gp, a, stream);
            return launch_long<IO, GOp::kAda>(a, stream);
        case Op::kRopeRotateHalf: {
            const bool even = r.head_dim % (2 * E) == 0;    // half heads of whole vectors
            const bool odd = E == 8 && r.head_dim % E == 0 && !even;  // ... of 4-element groups
            if (whole && fits && even) {
                const int P = a.vec_per_half;
                if ((P & (P - 1)) == 0 && P <= kWave / 2)  // partner lanes within one wavefront
                    return by_plan<RopeXorL<IO>, 4, 2, kMaxVecPerLane>(plan_for(a.nvec, 4, 2), a, stream);
            }
            if (whole && fits && (even || odd) && a.vec_per_head <= kWave / 2) {
                // heads packed into wavefronts (lw of 64 lanes used)
                const int lw = kWave - kWave % a.vec_per_head;
                Plan p = plan_for(((int64_t)a.nvec * kWave + lw - 1) / lw, 4, 2);
                p.per = (int)((a.nvec + (int64_t)lw * p.wpr - 1) / ((int64_t)lw * p.wpr));
                p.full = false;
                if (p.per <= kMaxVecPerLane) {
                    if constexpr (E == 8)
                        if (odd) return by_plan<RopePackedL<IO, true>, 4, 2, kMaxVecPerLane>(p, a, stream);
                    return by_plan<RopePackedL<IO, false>, 4, 2, kMaxVecPerLane>(p, a, stream);
                }
            }
            if (whole && fits && even)
                return by_plan<RopePairL<IO>, 2, 1, kMaxVecPerLane / 2>(plan_for(a.nunits, 2, 1), a,
                                                                        stream);
            const size_t lds_row = (size_t)r.hidden * sizeof(float);
            if (gfits && lds_row * rows_per_block(gp.wpr) <= kMaxExchangeLds)
                return by_plan<GeneralL<IO, GOp::kRopeHalf>, 4, 2, kMaxGeneralVecPerLane>(gp, a, stream,
                                                                                         lds_row);
            return launch_long<IO, GOp::kRopeHalf>(a, stream);
        }
        case Op::kRopeInterleaved: {
            if (whole && fits && r.head_dim % E == 0) {
                const Plan p = plan_for(a.nvec, 4, 2);
                const int vph = r.head_dim / E;
                if ((kWave * p.wpr) % vph == 0)
                    return by_plan<RopeIlL<IO, true>, 4, 2, kMaxVecPerLane>(p, a, stream);
                return by_plan<RopeIlL<IO, false>, 4, 2, kMaxVecPerLane>(p, a, stream);
            }
            if (gfits) return by_plan<GeneralL<IO, GOp::kRopeIl>, 4, 2, kMaxGeneralVecPerLane>(gp, a, stream);
            return launch_long<IO, GOp::kRopeIl>(a, stream);
        }
    }
    return LTXNORM_ERR_UNSUPPORTED;
}

}  // namespace
}  // namespace ltxnorm_detail
