// ltxnorm_dispatch.h -- host side: the kernel instance for the kernel and
// row split that choose() (ltxnorm_launch.h) picks, and the launch.
// Included once per I/O dtype; not a public header.
#pragma once

#include <mutex>

#include "ltxnorm_kernels.h"
#include "ltxnorm_general.h"

namespace ltxnorm_detail {
namespace {

// ---------------------------------------------------------------------------
// Host side: per-plan instance, launch.
// ---------------------------------------------------------------------------

// Workgroups of `fn` (at this size and dynamic LDS) that the stream's device
// holds at once: workgroups per CU times the CU count, or 0 where HIP cannot
// say.  The figure depends only on the device and the kernel instance, so it
// is kept in a table guarded by a mutex (entries are never removed; once the
// table is full, later instances are queried on every launch).
inline int64_t resident_workgroups(const void* fn, int threads, size_t lds_bytes,
                                   hipStream_t stream) {
    struct Entry {
        const void* fn;
        size_t lds;
        int device;
        int64_t n;
    };
    static std::mutex mu;
    static Entry table[512];
    static int used = 0;
    int dev = 0;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess && hipGetDevice(&dev) != hipSuccess) return 0;
    {
        std::lock_guard<std::mutex> lock(mu);
        for (int i = 0; i < used; ++i)
            if (table[i].fn == fn && table[i].lds == lds_bytes && table[i].device == dev) return table[i].n;
    }
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds_bytes) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    const int64_t n = (int64_t)(per_cu > 0 ? per_cu : 0) * (cus > 0 ? cus : 0);
    std::lock_guard<std::mutex> lock(mu);
    if (used < (int)(sizeof(table) / sizeof(table[0]))) table[used++] = Entry{fn, lds_bytes, dev, n};
    return n;
}

// Launch with one workgroup per group of rows.  Most kernels take the full
// grid: a grid-stride loop capped at the resident capacity measured 3-4%
// slower than letting the dispatcher stream fresh workgroups, which keeps
// every CU busy to the last rows.  `resident` caps the grid at the resident
// capacity instead, for kernels that load per-workgroup data worth reusing
// across rows (the general kernel's weight chunks: at hidden 3076, 42.5 ->
// 57.9 % of peak; the cap measured best at one resident wave of workgroups,
// against two, three or four).
inline ltxnorm_status launch(const void* fn, int threads, int rpb, const KArgs& args,
                             size_t lds_bytes, hipStream_t stream, bool resident = false) {
    const int64_t need = (args.rows + rpb - 1) / rpb;
    int64_t grid_rows = need < kMaxGrid ? need : kMaxGrid;
    if (resident) {
        // a multiple of 8 workgroups whenever they loop: the rows a workgroup
        // slot visits then all start at the same offset into a 16-byte vector
        // (the general kernel builds its weight windows once on that basis)
        const int64_t cap = resident_workgroups(fn, threads, lds_bytes, stream) & ~(int64_t)7;
        if (cap > 0 && cap < grid_rows) grid_rows = cap;
    }
    const unsigned grid = (unsigned)grid_rows;
    KArgs copy = args;
    void* params[] = {&copy};
    const hipError_t e =
        hipLaunchKernel(fn, dim3(grid), dim3(threads), params, (unsigned)lds_bytes, stream);
    return e == hipSuccess ? LTXNORM_OK : LTXNORM_ERR_HIP;
}

// One launcher per kernel family: fn<WPR, PER, FULL, PRIO, WL>() picks the
// instance; kResident asks for the grid capped at the resident capacity;
// kOneWavePrio says that the family has one-wavefront instances that raise
// the wave priority for their loads (PRIO), taken when the whole grid is
// resident at once; kOneWaveLds that it also has such instances with the
// weight in LDS (WL), which fit more rows at once.
template <typename IO>
struct RmsL {
    static constexpr bool kResident = false;
    static constexpr bool kOneWavePrio = true;
    static constexpr bool kOneWaveLds = false;
    template <int WPR, int PER, bool FULL, bool PRIO, bool WL = false>
    static const void* fn() { return (const void*)&rmsnorm_kernel<IO, PER, WPR, FULL, PRIO>; }
    // one wavefront of VPL vectors per lane adding in the order of VW
    template <int VPL, bool FULL, int VW>
    static const void* regroup() { return (const void*)&rmsnorm_kernel<IO, VPL, 1, FULL, true, VW>; }
};
template <typename IO>
struct RopeXorL {
    static constexpr bool kResident = false;
    static constexpr bool kOneWavePrio = true;
    static constexpr bool kOneWaveLds = true;
    template <int WPR, int PER, bool FULL, bool PRIO, bool WL = false>
    static const void* fn() {
        if constexpr (WL && FULL) return (const void*)&rmsnorm_rope_xor_wl_kernel<IO, PER>;
        else return (const void*)&rmsnorm_rope_xor_kernel<IO, PER, WPR, FULL, PRIO, WL>;
    }
    template <int VPL, bool FULL, int VW>
    static const void* regroup() { return (const void*)&rmsnorm_rope_xor_kernel<IO, VPL, 1, FULL, true, true, VW>; }
};
template <typename IO>
struct RopePairL {
    static constexpr bool kResident = false;
    static constexpr bool kOneWavePrio = false;
    static constexpr bool kOneWaveLds = false;
    template <int WPR, int PER, bool FULL, bool PRIO, bool WL = false>
    static const void* fn() { return (const void*)&rmsnorm_rope_pair_kernel<IO, PER, WPR, FULL>; }
};
template <typename IO, bool SHARED>
struct RopeIlL {
    static constexpr bool kResident = false;
    static constexpr bool kOneWavePrio = true;
    static constexpr bool kOneWaveLds = !SHARED;
    template <int WPR, int PER, bool FULL, bool PRIO, bool WL = false>
    static const void* fn() {
        return (const void*)&rmsnorm_rope_interleaved_kernel<IO, PER, WPR, FULL, SHARED, PRIO, 1, WL>;
    }
    template <int VPL, bool FULL, int VW>
    static const void* regroup() {
        if constexpr (SHARED) return (const void*)&rmsnorm_rope_interleaved_kernel<IO, VPL, 1, FULL, true, true, VW>;
        return nullptr;
    }
};
template <typename IO>
struct AdaL {
    static constexpr bool kResident = false;
    static constexpr bool kOneWavePrio = true;
    static constexpr bool kOneWaveLds = false;
    template <int WPR, int PER, bool FULL, bool PRIO, bool WL = false>
    static const void* fn() { return (const void*)&rmsnorm_adaln_kernel<IO, PER, WPR, FULL, PRIO>; }
    template <int VPL, bool FULL, int VW>
    static const void* regroup() { return (const void*)&rmsnorm_adaln_kernel<IO, VPL, 1, FULL, true, VW>; }
};
template <typename IO, bool ODD>
struct RopePackedL {
    static constexpr bool kResident = false;
    static constexpr bool kOneWavePrio = true;
    static constexpr bool kOneWaveLds = true;
    template <int WPR, int PER, bool FULL, bool PRIO, bool WL = false>
    static const void* fn() {
        if constexpr (WL) return (const void*)&rmsnorm_rope_packed_wl_kernel<IO, PER, ODD>;
        else return (const void*)&rmsnorm_rope_packed_kernel<IO, PER, WPR, ODD, PRIO>;
    }
};
// The general kernel masks every row itself: FULL does not select anything.
template <typename IO, GOp OP>
struct GeneralL {
    static constexpr bool kResident = true;
    static constexpr bool kOneWavePrio = false;
    static constexpr bool kOneWaveLds = false;
    template <int WPR, int PER, bool FULL, bool PRIO, bool WL = false>
    static const void* fn() { return (const void*)&rmsnorm_general_kernel<IO, OP, PER, WPR>; }
};

// Whether the grid of `rows` rows (rpb per workgroup) is resident at once
// for instance fn, at this size and dynamic LDS.
inline bool fits_one_wave(const void* fn, int threads, int rpb, int64_t rows, size_t lds_bytes,
                          hipStream_t stream) {
    const int64_t need = (rows + rpb - 1) / rpb;
    const int64_t cap = resident_workgroups(fn, threads, lds_bytes, stream);
    return cap > 0 && need <= cap;
}

template <typename LN, int WPR, int LO, int HI>
ltxnorm_status by_per(const Plan& p, const KArgs& a, size_t lds_per_row, hipStream_t s) {
    if constexpr (LO > HI) {
        return LTXNORM_ERR_UNSUPPORTED;
    } else {
        if (p.per == LO) {
            constexpr int kT = Layout<WPR>::kThreads, kRpb = Layout<WPR>::kRowsPerBlock;
            const size_t lds = lds_per_row * kRpb;
            const void* fn = p.full ? LN::template fn<WPR, LO, true, false>()
                                    : LN::template fn<WPR, LO, false, false>();
            if constexpr (WPR == 1 && LN::kOneWavePrio) {
                const void* fp = p.full ? LN::template fn<WPR, LO, true, true>()
                                        : LN::template fn<WPR, LO, false, true>();
                if (fits_one_wave(fp, kT, kRpb, a.rows, lds, s)) {
                    fn = fp;
                } else if constexpr (LN::kOneWaveLds) {
                    const void* fl = p.full ? LN::template fn<WPR, LO, true, true, true>()
                                            : LN::template fn<WPR, LO, false, true, true>();
                    if (fits_one_wave(fl, kT, kRpb, a.rows, lds, s)) fn = fl;
                }
            }
            return launch(fn, kT, kRpb, a, lds, s, LN::kResident);
        }
        return by_per<LN, WPR, LO + 1, HI>(p, a, lds_per_row, s);
    }
}

// One wavefront count W of 4..15: items per lane LO..HI, and ALSO (when
// nonzero) as a single extra instance.
template <typename LN, int W, int LO, int HI, int ALSO>
ltxnorm_status by_per_also(const Plan& p, const KArgs& a, size_t lds_per_row, hipStream_t s) {
    if constexpr (ALSO > 0) {
        if (p.per == ALSO) return by_per<LN, W, ALSO, ALSO>(p, a, lds_per_row, s);
    }
    return by_per<LN, W, LO, HI>(p, a, lds_per_row, s);
}

// Plans that plan_for can produce: one wavefront with 1..ONE items per lane;
// 3..15 wavefronts with exactly SPREAD items per lane (2 wavefronts never
// occur: a row too long for one wavefront needs more than 2 * ONE / SPREAD);
// 16 wavefronts with SPREAD..MAXP items per lane.  WIDE adds plan_wide's
// plans: two or three wavefronts with 3..4 items per lane; PER4 > SPREAD
// adds four wavefronts with SPREAD..PER4 (plan_wide_xor); ALSO4 adds
// ALSO4 items per lane at 4..15 wavefronts (plan_wide_xor past 768
// vectors).  lds_per_row: dynamic LDS bytes per row slot of the block.
// Rows of W wavefronts x P vectors per lane (the splits regroup_vectors
// names for the kernel): the one-wavefront instance of W * P vectors per
// lane that adds the squares in the W-wavefront order (split_order_row_sum),
// raises the wave priority for its loads and keeps the weight in LDS, when
// its whole grid is resident at once; nullptr otherwise.  RMSNorm bf16
// [8192 x 3072] 18.2 -> 17.3 us, [6144 x 3072] 14.5 -> 12.5 us,
// [4096 x 4096] 13.4 -> 11.3 us; launches of more rows keep the split.
template <typename LN, int W, int P>
const void* regroup_instance(bool full) {
    return full ? LN::template regroup<W * P, true, W>() : LN::template regroup<W * P, false, W>();
}
template <typename LN, int W2P3, int W2P4, int W3P2, int W4P2>
const void* one_wave_regroup(int vectors, const Plan& p, const KArgs& a, hipStream_t s) {
    if (vectors == 0) return nullptr;
    const void* fp = nullptr;
    if constexpr (W2P3) if (p.wpr == 2 && p.per == 3) fp = regroup_instance<LN, 2, 3>(p.full);
    if constexpr (W2P4) if (p.wpr == 2 && p.per == 4) fp = regroup_instance<LN, 2, 4>(p.full);
    if constexpr (W3P2) if (p.wpr == 3 && p.per == 2) fp = regroup_instance<LN, 3, 2>(p.full);
    if constexpr (W4P2) if (p.wpr == 4 && p.per == 2) fp = regroup_instance<LN, 4, 2>(p.full);
    if (fp == nullptr) return nullptr;
    return fits_one_wave(fp, Layout<1>::kThreads, Layout<1>::kRowsPerBlock, a.rows, 0, s) ? fp : nullptr;
}

template <typename LN, int ONE, int SPREAD, int MAXP, bool WIDE = false, int PER4 = SPREAD, int ALSO4 = 0>
ltxnorm_status by_plan(const Plan& p, const KArgs& a, hipStream_t s, size_t lds_per_row = 0) {
    switch (p.wpr) {
        case 1: return by_per<LN, 1, 1, ONE>(p, a, lds_per_row, s);
        case 2:
            if constexpr (WIDE) return by_per<LN, 2, 3, 4>(p, a, lds_per_row, s);
            return LTXNORM_ERR_UNSUPPORTED;
        case 3:
            if constexpr (WIDE) return by_per<LN, 3, SPREAD, 4>(p, a, lds_per_row, s);
            return by_per<LN, 3, SPREAD, SPREAD>(p, a, lds_per_row, s);
        case 4: return by_per_also<LN, 4, SPREAD, PER4, (ALSO4 > PER4 ? ALSO4 : 0)>(p, a, lds_per_row, s);
        case 5: return by_per_also<LN, 5, SPREAD, SPREAD, ALSO4>(p, a, lds_per_row, s);
        case 6: return by_per_also<LN, 6, SPREAD, SPREAD, ALSO4>(p, a, lds_per_row, s);
        case 7: return by_per_also<LN, 7, SPREAD, SPREAD, ALSO4>(p, a, lds_per_row, s);
        case 8: return by_per_also<LN, 8, SPREAD, SPREAD, ALSO4>(p, a, lds_per_row, s);
        case 9: return by_per_also<LN, 9, SPREAD, SPREAD, ALSO4>(p, a, lds_per_row, s);
        case 10: return by_per_also<LN, 10, SPREAD, SPREAD, ALSO4>(p, a, lds_per_row, s);
        case 11: return by_per_also<LN, 11, SPREAD, SPREAD, ALSO4>(p, a, lds_per_row, s);
        case 12: return by_per_also<LN, 12, SPREAD, SPREAD, ALSO4>(p, a, lds_per_row, s);
        case 13: return by_per_also<LN, 13, SPREAD, SPREAD, ALSO4>(p, a, lds_per_row, s);
        case 14: return by_per_also<LN, 14, SPREAD, SPREAD, ALSO4>(p, a, lds_per_row, s);
        case 15: return by_per_also<LN, 15, SPREAD, SPREAD, ALSO4>(p, a, lds_per_row, s);
        case 16: return by_per<LN, 16, SPREAD, MAXP>(p, a, lds_per_row, s);
        default: return LTXNORM_ERR_UNSUPPORTED;
    }
}

template <typename IO, GOp OP>
ltxnorm_status launch_long(const KArgs& a, hipStream_t stream) {
    return launch((const void*)&rmsnorm_long_kernel<IO, OP>, kLongThreads, 1, a, 0, stream);
}

// Segmented rows of S lanes x V vectors: the instance that raises the wave
// priority for its loads when the whole grid is resident at once, the plain
// one otherwise (bf16 [16384 x 576] 8.39 -> 7.13 us, [32768 x 256] 7.67 ->
// 7.05 us, AdaLN [8192 x 1152] 9.43 -> 8.94 us; always raised, it had cost
// 4-5 % on grids of several waves).
template <typename IO, GOp OP, int S, int V>
const void* short_instance(const KArgs& a, hipStream_t s) {
    const void* fp = (const void*)&rmsnorm_short_kernel<IO, OP, S, V, true>;
    constexpr int kRpb = kShortWavesPerBlock * (kWave / S);
    if (fits_one_wave(fp, kWave * kShortWavesPerBlock, kRpb, a.rows, 0, s)) return fp;
    return (const void*)&rmsnorm_short_kernel<IO, OP, S, V, false>;
}

// Segmented rows: the instance for the lanes per row and vectors per lane.
template <typename IO, GOp OP>
ltxnorm_status launch_short(int lanes, int per, const KArgs& a, hipStream_t stream) {
    const void* fn = nullptr;
    switch (lanes * 8 + per) {
        case 1 * 8 + 1: fn = short_instance<IO, OP, 1, 1>(a, stream); break;
        case 2 * 8 + 1: fn = short_instance<IO, OP, 2, 1>(a, stream); break;
        case 4 * 8 + 1: fn = short_instance<IO, OP, 4, 1>(a, stream); break;
        case 8 * 8 + 1: fn = short_instance<IO, OP, 8, 1>(a, stream); break;
        case 16 * 8 + 1: fn = short_instance<IO, OP, 16, 1>(a, stream); break;
        case 32 * 8 + 1: fn = short_instance<IO, OP, 32, 1>(a, stream); break;
        case 1 * 8 + 2: fn = short_instance<IO, OP, 1, 2>(a, stream); break;
        case 2 * 8 + 2: fn = short_instance<IO, OP, 2, 2>(a, stream); break;
        case 4 * 8 + 2: fn = short_instance<IO, OP, 4, 2>(a, stream); break;
        case 8 * 8 + 2: fn = short_instance<IO, OP, 8, 2>(a, stream); break;
        case 16 * 8 + 2: fn = short_instance<IO, OP, 16, 2>(a, stream); break;
        case 32 * 8 + 2: fn = short_instance<IO, OP, 32, 2>(a, stream); break;
        case 16 * 8 + 3: fn = short_instance<IO, OP, 16, 3>(a, stream); break;
        case 16 * 8 + 5: fn = short_instance<IO, OP, 16, 5>(a, stream); break;
        case 32 * 8 + 3: fn = short_instance<IO, OP, 32, 3>(a, stream); break;
        case 32 * 8 + 5: fn = short_instance<IO, OP, 32, 5>(a, stream); break;
        default: return LTXNORM_ERR_UNSUPPORTED;
    }
    return launch(fn, kWave * kShortWavesPerBlock, kShortWavesPerBlock * (kWave / lanes), a, 0, stream);
}

// Long rows in chunks: partial sums, then every chunk but the first, then
// the first chunk of every row (whose output holds the staged partials).
template <typename IO, GOp OP>
ltxnorm_status launch_split(const Choice& c, const KArgs& a, hipStream_t stream) {
    if constexpr (OP == GOp::kRopeHalf) {
        return LTXNORM_ERR_UNSUPPORTED;  // not chosen: rotate-half pairs span chunks
    } else {
        KArgs copy = a;
        int chunks = c.chunks;
        void* params[] = {&copy, &chunks};
        const void* fns[3] = {(const void*)&rmsnorm_split_partial_kernel<IO>,
                              (const void*)&rmsnorm_split_apply_kernel<IO, OP, false>,
                              (const void*)&rmsnorm_split_apply_kernel<IO, OP, true>};
        const int64_t grids[3] = {a.rows * chunks, a.rows * split_slots(chunks), a.rows};
        for (int i = 0; i < 3; ++i) {
            const hipError_t e = hipLaunchKernel(fns[i], dim3((unsigned)grids[i]), dim3(kSplitThreads),
                                                 params, 0, stream);
            if (e != hipSuccess) return LTXNORM_ERR_HIP;
        }
        return LTXNORM_OK;
    }
}

template <typename IO, GOp OP>
ltxnorm_status launch_general(const Choice& c, const KArgs& a, hipStream_t stream) {
    if (c.kernel == Kernel::kLong) return launch_long<IO, OP>(a, stream);
    if (c.kernel == Kernel::kSplit) return launch_split<IO, OP>(c, a, stream);
    return by_plan<GeneralL<IO, OP>, 4, 2, kMaxGeneralVecPerLane>(c.plan, a, stream,
                                                                  (size_t)c.lds_per_row);
}

// Enqueue `op` for I/O type IO on a validated request, with the kernel and
// row split that choose() gives.
template <typename IO>
ltxnorm_status launch_op(Op op, const Request& r, hipStream_t stream) {
    constexpr int E = IO::kEpv;
    const Choice c = choose(op, r, E);
    const int regroup = regroup_vectors(c.kernel, c.plan, r.head_dim / E);
    const int64_t samples = sample_count(r.rows, r.rows_per_sample);
    KArgs a{r.out, r.x, r.w, r.cos_tab, r.sin_tab, r.scale, r.shift, r.rows, r.seq_len,
            r.rows_per_sample, (int32_t)(r.hidden / E), (int32_t)(r.hidden / (2 * E)),
            r.head_dim / (2 * E), r.head_dim / E, r.head_dim / 2, (int32_t)r.hidden, r.head_dim,
            samples * r.hidden, (float)r.hidden, r.eps};
    switch (c.kernel) {
        case Kernel::kNone: return LTXNORM_OK;
        case Kernel::kRmsNorm:
            if (const void* fp = one_wave_regroup<RmsL<IO>, 0, 0, 1, 1>(regroup, c.plan, a, stream))
                return launch(fp, Layout<1>::kThreads, Layout<1>::kRowsPerBlock, a, 0, stream);
            return by_plan<RmsL<IO>, 4, 2, kMaxVecPerLane>(c.plan, a, stream);
        case Kernel::kAdaLN:
            if (const void* fp = one_wave_regroup<AdaL<IO>, 1, 1, 0, 0>(regroup, c.plan, a, stream))
                return launch(fp, Layout<1>::kThreads, Layout<1>::kRowsPerBlock, a, 0, stream);
            return by_plan<AdaL<IO>, 4, 2, kMaxVecPerLane, true>(c.plan, a, stream);
        case Kernel::kRopeXor:
            if (const void* fp = one_wave_regroup<RopeXorL<IO>, 1, 1, 0, 0>(regroup, c.plan, a, stream))
                return launch(fp, Layout<1>::kThreads, Layout<1>::kRowsPerBlock, a, 0, stream);
            return by_plan<RopeXorL<IO>, 4, 2, kMaxVecPerLane, true, 3, 4>(c.plan, a, stream);
        case Kernel::kRopePacked:
            return by_plan<RopePackedL<IO, false>, 4, 2, kMaxVecPerLane, true>(c.plan, a, stream);
        case Kernel::kRopePackedOdd:
            if constexpr (E == 8) return by_plan<RopePackedL<IO, true>, 4, 2, kMaxVecPerLane, true>(c.plan, a, stream);
            return LTXNORM_ERR_UNSUPPORTED;  // not chosen for 4-element vectors
        case Kernel::kRopePair:
            return by_plan<RopePairL<IO>, 2, 1, kMaxVecPerLane / 2>(c.plan, a, stream);
        case Kernel::kRopeInterleaved:
            return by_plan<RopeIlL<IO, false>, 4, 2, kMaxVecPerLane, true>(c.plan, a, stream);
        case Kernel::kRopeInterleavedShared:
            if (const void* fp = one_wave_regroup<RopeIlL<IO, true>, 1, 0, 1, 1>(regroup, c.plan, a, stream))
                return launch(fp, Layout<1>::kThreads, Layout<1>::kRowsPerBlock, a, 0, stream);
            return by_plan<RopeIlL<IO, true>, 4, 2, kMaxVecPerLane, true>(c.plan, a, stream);
        case Kernel::kShort:
            switch (op) {
                case Op::kRmsNorm: return launch_short<IO, GOp::kRms>(c.lanes_per_row, c.plan.per, a, stream);
                case Op::kAdaLN: return launch_short<IO, GOp::kAda>(c.lanes_per_row, c.plan.per, a, stream);
                case Op::kRopeRotateHalf: return launch_short<IO, GOp::kRopeHalf>(c.lanes_per_row, c.plan.per, a, stream);
                case Op::kRopeInterleaved: return launch_short<IO, GOp::kRopeIl>(c.lanes_per_row, c.plan.per, a, stream);
            }
            return LTXNORM_ERR_UNSUPPORTED;
        case Kernel::kGeneral:
        case Kernel::kLong:
        case Kernel::kSplit:
            switch (op) {
                case Op::kRmsNorm: return launch_general<IO, GOp::kRms>(c, a, stream);
                case Op::kAdaLN: return launch_general<IO, GOp::kAda>(c, a, stream);
                case Op::kRopeRotateHalf: return launch_general<IO, GOp::kRopeHalf>(c, a, stream);
                case Op::kRopeInterleaved: return launch_general<IO, GOp::kRopeIl>(c, a, stream);
            }
    }
    return LTXNORM_ERR_UNSUPPORTED;
}

}  // namespace
}  // namespace ltxnorm_detail
