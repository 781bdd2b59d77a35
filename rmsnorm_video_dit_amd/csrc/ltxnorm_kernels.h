// ltxnorm_kernels.h -- the register-resident kernels for rows that are whole
// 16-byte vectors: RMSNorm, fused RMSNorm + RoPE (rotate-half and
// interleaved pairs) and AdaLN-modulated RMSNorm.  Device helpers are in
// ltxnorm_device.h; not a public header.
#pragma once

#include "ltxnorm_device.h"

namespace ltxnorm_detail {
namespace {

// ---------------------------------------------------------------------------
// RMSNorm: VPL vectors per lane, WPR wavefronts per row.  FULL means every
// lane's every slot is inside the row (no masking).  Rows of several
// wavefronts raise the wave priority while their loads issue; PRIO does the
// same for one-wavefront rows (the launch asks for it when the whole grid is
// resident at once).  VW > 1 (one-wavefront priority instances of 6 or 8
// vectors per lane) adds the squares in the order of VW wavefronts of
// VPL / VW vectors, the split such rows take otherwise, so the bits do not
// depend on which of the two a launch takes; these instances keep the
// weight in LDS, once per workgroup.
// ---------------------------------------------------------------------------
template <typename IO, int VPL, int WPR, bool FULL, bool PRIO, int VW = 1>
__global__ void __launch_bounds__(Layout<WPR>::kThreads)
rmsnorm_kernel(const KArgs a) {
    static_assert(VW == 1 || (WPR == 1 && PRIO), "split-order sums: one-wavefront priority instances");
    constexpr bool kPrio = WPR > 1 || PRIO;
    constexpr bool kWl = VW > 1;  // weight in LDS
    constexpr int RPB = Layout<WPR>::kRowsPerBlock;
    constexpr int L = Layout<WPR>::kLanesPerRow;
    constexpr int E = IO::kEpv;
    const Lane<WPR> ln;
    if constexpr (kPrio) priority_for_loads();
    __shared__ u32x4 wlds[kWl ? VPL * kWave : 1];
    u32x4 wv[kWl ? 1 : VPL];
    if constexpr (kWl) {
        // every slot of the row's lanes, ones past the row
        for (int v = threadIdx.x; v < VPL * kWave; v += Layout<WPR>::kThreads)
            wlds[v] = (a.w != nullptr && v < a.nvec) ? reinterpret_cast<const u32x4*>(a.w)[v] : splat(IO::kOne);
        __syncthreads();
    } else {
        load_weight<IO, VPL, L, FULL>(wv, a.w, ln.t, a.nvec);
    }

    int parity = 0;
    for (int64_t base = (int64_t)blockIdx.x * RPB; base < a.rows;
         base += (int64_t)gridDim.x * RPB, parity ^= 1) {
        const int64_t row = base + ln.slot;
        const bool active = row < a.rows;
        if (WPR == 1 && !active) continue;  // wave-uniform; no barrier at WPR 1
        const u32x4* xr = reinterpret_cast<const u32x4*>(a.x) + row * a.nvec;
        u32x4* yr = reinterpret_cast<u32x4*>(a.out) + row * a.nvec;

        u32x4 xv[VPL];
        if constexpr (kPrio) priority_for_loads();
        load_row<VPL, L, FULL, WPR>(xv, xr, ln.t, a.nvec, active);
        if constexpr (kPrio) priority_after_loads();
        float sum_sq;
        if constexpr (VW > 1) {
            sum_sq = split_order_row_sum<IO, VPL, VW>(xv);
        } else {
            const float part = sum_squares<IO, VPL>(xv);
            sum_sq = row_sum<WPR>(part, ln.slot, ln.wave_in_row, parity);
        }
        const float rstd = rstd_of(sum_sq, a.hidden_f, a.eps);

#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = k * L + ln.t;
            const bool in = (FULL || v < a.nvec) && (WPR == 1 || active);
            float f[E], g[E];
            keep_packed(xv[k]);
            IO::widen(xv[k], f);
            if constexpr (kWl) {
                u32x4 wk = wlds[v];
                keep_packed(wk);
                IO::widen(wk, g);
            } else {
                keep_packed(wv[k]);
                IO::widen(wv[k], g);
            }
#pragma unroll
            for (int e = 0; e < E; ++e) f[e] = (f[e] * rstd) * g[e];
            if (in) store_stream(yr + v, IO::narrow(f));
        }
    }
}

// ---------------------------------------------------------------------------
// Rows in segments of S lanes (S a power of two up to 32), V vectors per
// lane: lane l of a row's segment holds vectors k*S + l, 64 / S rows per
// wavefront, four wavefronts per workgroup.
//  * Rows of up to 64 vectors (per-head normalisation, small hidden sizes):
//    one wavefront per row would leave most lanes idle (hidden 128 measured
//    28 % of peak that way).  Rows of up to 8 vectors take V = 1 on the power
//    of two at or above the vector count; rows of 9..64 take V = 2 on half
//    as many lanes (16 x 3 for 33..48 vectors), which beat one vector per
//    lane, while segments under 8 lanes (128 bytes of a row per load) lost.
//    Rotate-half partners are lane l ^ P in the same slot (P <= S/2) or, with
//    V = 2 and P == S, the other slot of the same lane.
//  * Rows of 65..160 vectors whose count leaves many of a wavefront's lanes
//    idle take S = 16 or 32 with V = 3 or 5 (72 vectors: 16 x 5; 88: 32 x 3;
//    144: 32 x 5), filling 80-100 % of the slots where one wavefront per row
//    fills 56-75 %.  The choice and its measurements are with segments_for.
// A load instruction covers 64 / S rows' runs of S vectors.  The sum of
// squares is reduced inside each segment by the first log2 S steps of the
// wavefront reduction (and the xor-16 lane swap for S = 32), so every lane of
// a row ends with the same bits.  Partner values move between lanes with DPP
// and the lane swaps (xor_lane), not through the LDS crossbar.  RMSNorm, AdaLN, and RoPE whose partners stay
// inside a row's lanes: rotate-half with power-of-two half heads (partner
// lane l ^ P in the same slot for P <= S/2, the lane's other slot for V = 2
// and P == S) and interleaved pairs.
// ---------------------------------------------------------------------------
template <int S>
__device__ __forceinline__ float segment_sum(float v) {
    if constexpr (S >= 2) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]: xor 1
    if constexpr (S >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]: xor 2
    if constexpr (S >= 8) v += dpp<0x141>(v);   // row_half_mirror: 8 lanes
    if constexpr (S >= 16) v += dpp<0x140>(v);  // row_mirror: 16 lanes
    if constexpr (S >= 32) v += xor_lane<16>(v);  // the other 16 lanes
    return v;
}



template <typename IO, GOp OP, int S, int V, bool PRIO>
__global__ void __launch_bounds__(kWave * kShortWavesPerBlock)
rmsnorm_short_kernel(const KArgs a) {
    constexpr int E = IO::kEpv;
    constexpr int G = kWave / S;           // rows per wavefront
    constexpr int RPB = kShortWavesPerBlock * G;   // rows per workgroup
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int l = lane % S;                // first vector of the lane within the row
    const int seg = lane / S;              // row within the wavefront
    if constexpr (PRIO) priority_for_loads();
    u32x4 wv[V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const int v = k * S + l;
        wv[k] = (a.w != nullptr && v < a.nvec) ? reinterpret_cast<const u32x4*>(a.w)[v] : splat(IO::kOne);
    }

    // rotation constants of this lane: the xor layout of the power-of-two
    // kernel within the row's lanes, whose table slice (v mod P) is the same
    // for every slot, whether S is a multiple of 2P or P == S (then sgn goes
    // unused: the partner is the lane's other slot); or the
    // interleaved table columns of each slot
    int toff[V];
    float sgn = 1.0f;
#pragma unroll
    for (int k = 0; k < V; ++k) toff[k] = 0;
    if constexpr (OP == GOp::kRopeHalf) {
        const int P = a.vec_per_half;
        sgn = (l & P) ? 1.0f : -1.0f;
        toff[0] = (l & (P - 1)) * E;
    } else if constexpr (OP == GOp::kRopeIl) {
#pragma unroll
        for (int k = 0; k < V; ++k) toff[k] = ((k * S + l) % a.vec_per_head) * (E / 2);
    }

    for (int64_t base = (int64_t)blockIdx.x * RPB; base < a.rows; base += (int64_t)gridDim.x * RPB) {
        const int64_t row = base + wave * G + seg;
        const bool rin = row < a.rows;
        const u32x4* xr = reinterpret_cast<const u32x4*>(a.x) + row * a.nvec;
        u32x4* yr = reinterpret_cast<u32x4*>(a.out) + row * a.nvec;
        if constexpr (PRIO) priority_for_loads();
        u32x4 xv[V];
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const int v = k * S + l;
            xv[k] = (rin && v < a.nvec) ? load_stream(xr + v) : u32x4{0u, 0u, 0u, 0u};
        }

        // per-row side inputs, fetched together with x
        u32x4 sv[V], hv[V];
        constexpr int NT = OP == GOp::kRopeIl ? V : 1;   // table slices per row
        constexpr int TW = OP == GOp::kRopeIl ? E / 2 : E;
        float c[NT][TW], sn[NT][TW];
        if constexpr (OP == GOp::kAda) {
            const int64_t sample = rin ? row / a.rows_per_sample : 0;
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const int v = k * S + l;
                const bool in = rin && v < a.nvec;
                sv[k] = (a.scale != nullptr && in) ? reinterpret_cast<const u32x4*>(a.scale)[sample * a.nvec + v]
                                                   : u32x4{0u, 0u, 0u, 0u};
                hv[k] = (a.shift != nullptr && in) ? reinterpret_cast<const u32x4*>(a.shift)[sample * a.nvec + v]
                                                   : splat(IO::kNegZero);
            }
        } else if constexpr (OP == GOp::kRopeHalf || OP == GOp::kRopeIl) {
            const int64_t pos = rin ? row % a.seq_len : 0;
#pragma unroll
            for (int k = 0; k < NT; ++k) {
                load_floats<TW>(a.cos_tab + pos * a.half + toff[k], c[k]);
                load_floats<TW>(a.sin_tab + pos * a.half + toff[k], sn[k]);
            }
        }

        if constexpr (PRIO) priority_after_loads();
        const float part = sum_squares<IO, V>(xv);
        const float rstd = rstd_of(segment_sum<S>(part), a.hidden_f, a.eps);
        if constexpr (OP == GOp::kRopeHalf && V == 2) {
            if (a.vec_per_half >= S) {
                // P == S: the partner of slot k is slot 1 - k of the same
                // lane; slot 0 holds the first half.  Same expression as the
                // exchange below, so the bits do not depend on the path.
                float f0[E], f1[E], g[E];
                keep_packed(xv[0]);
                keep_packed(xv[1]);
                IO::widen(xv[0], f0);
                IO::widen(xv[1], f1);
                keep_packed(wv[0]);
                IO::widen(wv[0], g);
#pragma unroll
                for (int e = 0; e < E; ++e) f0[e] = (f0[e] * rstd) * g[e];
                keep_packed(wv[1]);
                IO::widen(wv[1], g);
#pragma unroll
                for (int e = 0; e < E; ++e) f1[e] = (f1[e] * rstd) * g[e];
                float o0[E], o1[E];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    o0[e] = rot(f0[e], c[0][e], f1[e], sn[0][e] * -1.0f);
                    o1[e] = rot(f1[e], c[0][e], f0[e], sn[0][e] * 1.0f);
                }
                if (rin && l < a.nvec) store_stream(yr + l, IO::narrow(o0));
                if (rin && S + l < a.nvec) store_stream(yr + S + l, IO::narrow(o1));
                continue;
            }
        }
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const int v = k * S + l;
            float f[E], g[E];
            keep_packed(xv[k]);
            IO::widen(xv[k], f);
            keep_packed(wv[k]);
            IO::widen(wv[k], g);
#pragma unroll
            for (int e = 0; e < E; ++e) f[e] = (f[e] * rstd) * g[e];

            float o[E];
            if constexpr (OP == GOp::kAda) {
                float sc[E], sh[E];
                IO::widen(sv[k], sc);
                IO::widen(hv[k], sh);
#pragma unroll
                for (int e = 0; e < E; ++e) o[e] = modulate(f[e], sc[e], sh[e]);
            } else if constexpr (OP == GOp::kRopeHalf) {
                // the partner lane's normalised values; -sin in the first half
                // (P <= S / 2 <= 16 here)
                with_pow2(a.vec_per_half, [&](auto pc) {
                    constexpr int PC = decltype(pc)::value < 16 ? decltype(pc)::value : 16;
#pragma unroll
                    for (int e = 0; e < E; ++e) o[e] = rot(f[e], c[0][e], xor_lane<PC>(f[e]), sn[0][e] * sgn);
                });
            } else if constexpr (OP == GOp::kRopeIl) {
#pragma unroll
                for (int j = 0; j < E / 2; ++j) {
                    o[2 * j] = rot(f[2 * j], c[k][j], -f[2 * j + 1], sn[k][j]);
                    o[2 * j + 1] = rot(f[2 * j + 1], c[k][j], f[2 * j], sn[k][j]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) o[e] = f[e];
            }
            if (rin && v < a.nvec) store_stream(yr + v, IO::narrow(o));
        }
    }
}

// ---------------------------------------------------------------------------
// RMSNorm + rotate-half RoPE with the RMSNorm lane layout, when the number
// of vectors per half head P = head_dim / (2 kEpv) is a power of two up to
// 32.  Lane t holds vectors k*L + t (full 1 KiB lines per load
// instruction); the partner of vector v is v ^ P: the same slot of lane
// t ^ P in the same wavefront.  Each lane normalises its own vector and
// fetches the partner's normalised binary32 values with DPP moves or a lane
// swap (xor_lane), a few VALU cycles each instead of an LDS-crossbar round
// trip per value (exchanging the finished values rather than raw x halves
// the VALU work per vector, which matters because with one row per wavefront
// the whole grid is resident and compute is not hidden behind later loads).  A lane's half
// (bit P of t) and its table slice (floats kEpv * (t mod P) .. + kEpv) do not
// depend on the slot, so each lane reads one table slice per row.  PRIO
// raises the wave priority while a row's loads issue.  WL (one-wavefront
// rows with PRIO only) keeps the weight in LDS, once per workgroup, instead
// of in every wavefront's registers: 4 vectors per lane then take 60 VGPRs
// instead of 75, 8 wavefronts per SIMD instead of 6, so that a launch of
// 8192 rows is resident at once and can take the priority (bf16
// [8192 x 2048] 13.36 -> 12.38 us; where the register-weight instance
// already fits, LDS weight measured 1-3 % slower, so the launch prefers it).
// WL instances also fetch the position's table row into LDS with x
// (TableLds) and take the lane's slice after the reduction, instead of an
// L2 round trip then: 12.42 -> 11.74 us at [8192 x 2048], d = 64.
// ---------------------------------------------------------------------------
template <typename IO, int VPL, int WPR, bool FULL, bool PRIO, bool WL, int VW>
__device__ __forceinline__ void rope_xor_rows(const KArgs& a) {
    static_assert(!WL || (PRIO && WPR == 1), "LDS weight: one-wavefront priority instances only");
    static_assert(VW == 1 || WL, "split-order sums: LDS-weight instances");
    constexpr int RPB = Layout<WPR>::kRowsPerBlock;
    constexpr int L = Layout<WPR>::kLanesPerRow;
    constexpr int E = IO::kEpv;
    const Lane<WPR> ln;
    // one array for every copy of the row loop below (one per P)
    __shared__ u32x4 wlds[WL ? VPL * kWave : 1];
    // one copy of the row loop per partner distance P (a scalar branch at
    // entry): inside it every exchange is straight-line DPP or lane-swap
    // code, and each copy is register-allocated on its own (one loop with a
    // branch per row measured 93 VGPRs against 79)
    with_pow2(a.vec_per_half, [&](auto pc) {
        constexpr int P = decltype(pc)::value;
        const float sgn = (ln.t & P) ? 1.0f : -1.0f;  // second half adds, first subtracts
        const int toff = (ln.t & (P - 1)) * E;

        if constexpr (PRIO) priority_for_loads();
        u32x4 wv[WL ? 1 : VPL];
        if constexpr (WL) {
            // every slot of the row's lanes, ones past the row
            for (int v = threadIdx.x; v < VPL * kWave; v += Layout<WPR>::kThreads)
                wlds[v] = (a.w != nullptr && v < a.nvec) ? reinterpret_cast<const u32x4*>(a.w)[v]
                                                         : splat(IO::kOne);
            __syncthreads();
        } else {
            load_weight<IO, VPL, L, FULL>(wv, a.w, ln.t, a.nvec);
        }

        int parity = 0;
        for (int64_t base = (int64_t)blockIdx.x * RPB; base < a.rows;
             base += (int64_t)gridDim.x * RPB, parity ^= 1) {
            const int64_t row = base + ln.slot;
            const bool active = row < a.rows;
            if (WPR == 1 && !active) continue;
            const int64_t pos = active ? row % a.seq_len : 0;
            const u32x4* xr = reinterpret_cast<const u32x4*>(a.x) + row * a.nvec;
            u32x4* yr = reinterpret_cast<u32x4*>(a.out) + row * a.nvec;

            u32x4 xv[VPL];
            if constexpr (PRIO) priority_for_loads();
            load_row<VPL, L, FULL, WPR>(xv, xr, ln.t, a.nvec, active);
            if constexpr (PRIO) priority_after_loads();
            // The table slice is an L2 hit.  With several wavefronts per row
            // it is fetched together with x, off the critical path behind the
            // row's barrier (H = 3072, d = 128: 69.6 -> 74.1 % of peak;
            // H = 2304: 58.0 -> 64.3 %); with one wavefront per row either
            // order measured the same, and fetching it after the reduction
            // keeps registers free.
            float c[E], ss[E];
            if constexpr (WPR > 1) {
                load_floats<E>(a.cos_tab + pos * a.half + toff, c);
                load_floats<E>(a.sin_tab + pos * a.half + toff, ss);
            }
            TableLds<4, Layout<WPR>::kThreads / kWave, kWave> tabs(ln.slot);
            if constexpr (WL) tabs.fetch(a.cos_tab + pos * a.half, a.sin_tab + pos * a.half, ln.lane, a.half / 4);
            float sum_sq;
            if constexpr (VW > 1) {
                sum_sq = split_order_row_sum<IO, VPL, VW>(xv);
            } else {
                const float part = sum_squares<IO, VPL>(xv);
                sum_sq = row_sum<WPR>(part, ln.slot, ln.wave_in_row, parity);
            }
            const float rstd = rstd_of(sum_sq, a.hidden_f, a.eps);
            if constexpr (WL) {
                tabs.share(ln.lane, a.half / 4);
                tabs.take(toff, c, ss);
                if constexpr (E == 8) tabs.take(toff + 4, c + 4, ss + 4);
            } else if constexpr (WPR == 1) {
                load_floats<E>(a.cos_tab + pos * a.half + toff, c);
                load_floats<E>(a.sin_tab + pos * a.half + toff, ss);
            }
            // the partner term enters with -sin in the first half, +sin in the second
#pragma unroll
            for (int e = 0; e < E; ++e) ss[e] *= sgn;
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                const int v = k * L + ln.t;
                const bool in = (FULL || v < a.nvec) && (WPR == 1 || active);
                keep_packed(xv[k]);
                float own[E], g[E], o[E];
                if constexpr (WL) {
                    u32x4 wk = wlds[v];
                    keep_packed(wk);
                    IO::widen(xv[k], own);
                    IO::widen(wk, g);
                } else {
                    keep_packed(wv[k]);
                    IO::widen(xv[k], own);
                    IO::widen(wv[k], g);
                }
#pragma unroll
                for (int e = 0; e < E; ++e) own[e] = (own[e] * rstd) * g[e];
                // the partner lane's normalised values, exact binary32 bits
#pragma unroll
                for (int e = 0; e < E; ++e) o[e] = rot(own[e], c[e], xor_lane<P>(own[e]), ss[e]);
                if (in) store_stream(yr + v, IO::narrow(o));
            }
        }
    });
}

template <typename IO, int VPL, int WPR, bool FULL, bool PRIO, bool WL, int VW = 1>
__global__ void __launch_bounds__(Layout<WPR>::kThreads)
rmsnorm_rope_xor_kernel(const KArgs a) {
    rope_xor_rows<IO, VPL, WPR, FULL, PRIO, WL, VW>(a);
}

// The WL form of whole-vector rows, its own kernel so that only it carries
// the request for 8 wavefronts per SIMD (fp16, 4 vectors per lane: 66 -> 64
// VGPRs, no spill; masked rows would spill and keep the kernel above).
template <typename IO, int VPL>
__global__ void __launch_bounds__(Layout<1>::kThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
rmsnorm_rope_xor_wl_kernel(const KArgs a) {
    rope_xor_rows<IO, VPL, 1, true, true, true, 1>(a);
}

// ---------------------------------------------------------------------------
// RMSNorm + rotate-half RoPE with head-packed lanes, for heads of vph =
// head_dim / kEpv <= 64 vectors.  Each wavefront uses its first
// lw = 64 - 64 mod vph lanes (the rest idle) for lw consecutive vectors, so
// it always holds whole heads: lane l holds vector l mod vph of a head in
// every slot, and the vector's partner half a head away is in the same
// wavefront.  One load instruction still covers lw * 16 contiguous bytes.
//  * EVEN (head_dim / 2 a multiple of kEpv): the partner is the whole vector
//    of lane l + vph/2 (first half) or l - vph/2 (second half).
//  * ODD (16-bit types, head_dim / 2 an odd multiple of 4): a vector holds
//    two 4-element groups and the half-head offset is an odd number of
//    groups, so group 0's partner is group 1 of some lane and group 1's
//    partner is group 0 of another: two ds_bpermute sources, each fetching a
//    fixed register.
// The lane's table slice (kEpv cos and kEpv sin) does not depend on the slot;
// the wavefront reads the position's table rows once and the lanes take
// their slices through LDS (TableLds).  PRIO raises the wave priority while
// a row's loads issue.  WL (one-wavefront rows with PRIO only) keeps the
// weight in LDS, takes the lane's table slices from LDS per vector instead
// of holding them, and asks for 8 wavefronts per SIMD up to 3 vectors per
// lane (64 VGPRs instead of 76 at d = 72, no spill), so that 8192 rows of
// hidden 1152 are resident at once: 9.84 -> 8.53 us at [8192 x 1152],
// d = 72; where the register-weight instance already fits (4096 and 6144
// rows) this form measured 5 % slower, so the launch prefers that one.
// ---------------------------------------------------------------------------
template <typename IO, int VPL, int WPR, bool ODD, bool PRIO, bool WL>
__device__ __forceinline__ void rope_packed_rows(const KArgs& a) {
    static_assert(!WL || (PRIO && WPR == 1), "LDS weight: one-wavefront priority instances only");
    constexpr int RPB = Layout<WPR>::kRowsPerBlock;
    constexpr int E = IO::kEpv;
    constexpr int G = E / 2;  // elements per group (ODD)
    static_assert(!ODD || E == 8, "the odd layout splits 8-element vectors");
    const Lane<WPR> ln;
    const int vph = a.vec_per_head;
    const int lw = kWave - kWave % vph;
    const int l = ln.lane;
    const int hv = l % vph;                 // vector within its head
    const int head0 = l - hv;               // first lane of the head
    // partner lanes (ds_bpermute byte addresses), signs and table columns
    int src0, src1, col0, col1;
    float sg0, sg1;
    if constexpr (ODD) {
        const int gh = a.half / G;          // groups per half head (odd)
        const int g0 = 2 * hv, g1 = 2 * hv + 1;
        const bool lo0 = g0 < gh, lo1 = g1 < gh;
        const int p0 = lo0 ? g0 + gh : g0 - gh;   // odd: group 1 of its vector
        const int p1 = lo1 ? g1 + gh : g1 - gh;   // even: group 0 of its vector
        src0 = (head0 + (p0 >> 1)) << 2;
        src1 = (head0 + (p1 >> 1)) << 2;
        sg0 = lo0 ? -1.0f : 1.0f;
        sg1 = lo1 ? -1.0f : 1.0f;
        col0 = (lo0 ? g0 : g0 - gh) * G;
        col1 = (lo1 ? g1 : g1 - gh) * G;
    } else {
        const int P = vph / 2;
        const bool lo = hv < P;
        src0 = src1 = (lo ? l + P : l - P) << 2;
        sg0 = sg1 = lo ? -1.0f : 1.0f;
        col0 = (lo ? hv : hv - P) * E;
        col1 = col0 + G;
    }
    auto vec_of = [&](int k) { return (k * WPR + ln.wave_in_row) * lw + l; };

    if constexpr (PRIO) priority_for_loads();
    __shared__ u32x4 wlds[WL ? VPL * kWave : 1];
    u32x4 wv[WL ? 1 : VPL];
    if constexpr (WL) {
        // every slot of the wavefront's lanes, ones past the row
        for (int v = threadIdx.x; v < VPL * kWave; v += Layout<WPR>::kThreads)
            wlds[v] = (a.w != nullptr && v < a.nvec) ? reinterpret_cast<const u32x4*>(a.w)[v] : splat(IO::kOne);
        __syncthreads();
    } else {
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = vec_of(k);
            const bool in = l < lw && v < a.nvec;
            wv[k] = (a.w != nullptr && in) ? reinterpret_cast<const u32x4*>(a.w)[v] : splat(IO::kOne);
        }
    }

    int parity = 0;
    for (int64_t base = (int64_t)blockIdx.x * RPB; base < a.rows;
         base += (int64_t)gridDim.x * RPB, parity ^= 1) {
        const int64_t row = base + ln.slot;
        const bool active = row < a.rows;
        if (WPR == 1 && !active) continue;
        const int64_t pos = active ? row % a.seq_len : 0;
        const u32x4* xr = reinterpret_cast<const u32x4*>(a.x) + row * a.nvec;
        u32x4* yr = reinterpret_cast<u32x4*>(a.out) + row * a.nvec;

        u32x4 xv[VPL];
        if constexpr (PRIO) priority_for_loads();
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = vec_of(k);
            const bool in = l < lw && v < a.nvec && (WPR == 1 || active);
            xv[k] = in ? load_stream(xr + v) : u32x4{0u, 0u, 0u, 0u};
        }
        // the position's table rows, fetched with x by the first vph lanes
        // (vph chunks of G floats per table) and handed out after the
        // reduction: lane l needs the chunks at columns col0 and col1
        float c[E], ss[E];
        // (a.half / G = vph <= 32 chunks per table)
        TableLds<G, Layout<WPR>::kThreads / kWave, kWave / 2> tabs(ln.slot * WPR + ln.wave_in_row);
        tabs.fetch(a.cos_tab + pos * a.half, a.sin_tab + pos * a.half, l, a.half / G);
        if constexpr (PRIO) priority_after_loads();
        const float part = sum_squares<IO, VPL>(xv);
        const float rstd = rstd_of(row_sum<WPR>(part, ln.slot, ln.wave_in_row, parity), a.hidden_f, a.eps);
        tabs.share(l, a.half / G);
        if constexpr (!WL) {
            tabs.take(col0, c, ss);
            tabs.take(col1, c + G, ss + G);
#pragma unroll
            for (int e = 0; e < G; ++e) {
                ss[e] *= sg0;
                ss[e + G] *= sg1;
            }
        }
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = vec_of(k);
            const bool in = l < lw && v < a.nvec && (WPR == 1 || active);
            if constexpr (WL) {  // per vector: fewer registers held
                tabs.take(col0, c, ss);
                tabs.take(col1, c + G, ss + G);
#pragma unroll
                for (int e = 0; e < G; ++e) {
                    ss[e] *= sg0;
                    ss[e + G] *= sg1;
                }
            }
            keep_packed(xv[k]);
            float own[E], g[E], par[E], o[E];
            if constexpr (WL) {
                u32x4 wk = wlds[v];
                keep_packed(wk);
                IO::widen(xv[k], own);
                IO::widen(wk, g);
            } else {
                keep_packed(wv[k]);
                IO::widen(xv[k], own);
                IO::widen(wv[k], g);
            }
#pragma unroll
            for (int e = 0; e < E; ++e) own[e] = (own[e] * rstd) * g[e];
            // group 0 takes the partner lane's second group (ODD) or first
            // group (EVEN); group 1 the other way round
#pragma unroll
            for (int e = 0; e < G; ++e) {
                const int from0 = ODD ? e + G : e;
                const int from1 = ODD ? e : e + G;
                par[e] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src0, __builtin_bit_cast(int, own[from0])));
                par[e + G] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src1, __builtin_bit_cast(int, own[from1])));
            }
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] = rot(own[e], c[e], par[e], ss[e]);
            if (in) store_stream(yr + v, IO::narrow(o));
        }
    }
}

template <typename IO, int VPL, int WPR, bool ODD, bool PRIO>
__global__ void __launch_bounds__(Layout<WPR>::kThreads)
rmsnorm_rope_packed_kernel(const KArgs a) {
    rope_packed_rows<IO, VPL, WPR, ODD, PRIO, false>(a);
}

// The WL form (its own kernel, so that only it carries the occupancy request).
template <typename IO, int VPL, bool ODD>
__global__ void __launch_bounds__(Layout<1>::kThreads) __attribute__((amdgpu_waves_per_eu(VPL <= 3 ? 8 : 1, 8)))
rmsnorm_rope_packed_wl_kernel(const KArgs a) {
    rope_packed_rows<IO, VPL, 1, ODD, true, true>(a);
}

// ---------------------------------------------------------------------------
// RMSNorm + rotate-half RoPE, general head_dim (a multiple of 2 kEpv): UPL
// pair units per lane, each a vector of the first half of a head and its
// partner in the second half, both held by the same lane.  Unit u covers head
// h = u / P, quarter q = u % P (P = head_dim / (2 kEpv)): vectors
// h * 2P + q and that + P, and table floats [kEpv q, kEpv q + kEpv) of the
// row's position.  A load instruction covers half of each cache line (its
// pair covers the other half), so this is the fallback layout.
// ---------------------------------------------------------------------------
template <typename IO, int UPL, int WPR, bool FULL>
__global__ void __launch_bounds__(Layout<WPR>::kThreads)
rmsnorm_rope_pair_kernel(const KArgs a) {
    constexpr int RPB = Layout<WPR>::kRowsPerBlock;
    constexpr int L = Layout<WPR>::kLanesPerRow;
    constexpr int E = IO::kEpv;
    const Lane<WPR> ln;
    const int P = a.vec_per_half;

    int va[UPL], toff[UPL];
    bool uin[UPL];
    u32x4 wa[UPL], wb[UPL];
#pragma unroll
    for (int k = 0; k < UPL; ++k) {
        const int u = k * L + ln.t;
        uin[k] = FULL || u < a.nunits;
        const int h = u / P;
        const int q = u - h * P;
        va[k] = h * 2 * P + q;
        toff[k] = q * E;
        const bool lw = a.w != nullptr && uin[k];
        wa[k] = lw ? reinterpret_cast<const u32x4*>(a.w)[va[k]] : splat(IO::kOne);
        wb[k] = lw ? reinterpret_cast<const u32x4*>(a.w)[va[k] + P] : splat(IO::kOne);
    }

    int parity = 0;
    for (int64_t base = (int64_t)blockIdx.x * RPB; base < a.rows;
         base += (int64_t)gridDim.x * RPB, parity ^= 1) {
        const int64_t row = base + ln.slot;
        const bool active = row < a.rows;
        if (WPR == 1 && !active) continue;
        const int64_t pos = active ? row % a.seq_len : 0;
        const u32x4* xr = reinterpret_cast<const u32x4*>(a.x) + row * a.nvec;
        u32x4* yr = reinterpret_cast<u32x4*>(a.out) + row * a.nvec;
        const float* crow = a.cos_tab + pos * a.half;
        const float* srow = a.sin_tab + pos * a.half;

        u32x4 xa[UPL], xb[UPL];
#pragma unroll
        for (int k = 0; k < UPL; ++k) {
            const bool in = uin[k] && (WPR == 1 || active);
            const u32x4 z = {0u, 0u, 0u, 0u};
            xa[k] = in ? load_stream(xr + va[k]) : z;
            xb[k] = in ? load_stream(xr + va[k] + P) : z;
        }
        const float part = sum_squares<IO, UPL>(xa) + sum_squares<IO, UPL>(xb);
        const float rstd = rstd_of(row_sum<WPR>(part, ln.slot, ln.wave_in_row, parity), a.hidden_f, a.eps);

        // The table slices are L2-resident (every head and batch row shares
        // them); loading them only now keeps registers free while the row's
        // own loads are in flight.
#pragma unroll
        for (int k = 0; k < UPL; ++k) {
            const bool in = uin[k] && (WPR == 1 || active);
            float c[E], s[E];
            if (in) {
                load_floats<E>(crow + toff[k], c);
                load_floats<E>(srow + toff[k], s);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) c[e] = s[e] = 0.0f;
            }
            float ya[E], yb[E], g[E];
            keep_packed(xa[k]);
            keep_packed(xb[k]);
            keep_packed(wa[k]);
            keep_packed(wb[k]);
            IO::widen(xa[k], ya);
            IO::widen(wa[k], g);
#pragma unroll
            for (int e = 0; e < E; ++e) ya[e] = (ya[e] * rstd) * g[e];
            IO::widen(xb[k], yb);
            IO::widen(wb[k], g);
#pragma unroll
            for (int e = 0; e < E; ++e) yb[e] = (yb[e] * rstd) * g[e];
            float o1[E], o2[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                o1[e] = rot(ya[e], c[e], -yb[e], s[e]);
                o2[e] = rot(yb[e], c[e], ya[e], s[e]);
            }
            if (in) {
                store_stream(yr + va[k], IO::narrow(o1));
                store_stream(yr + va[k] + P, IO::narrow(o2));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// RMSNorm + interleaved RoPE: adjacent pairs (2i, 2i + 1) of each head turn
// by table column i.  A pair never straddles a vector, so the RMSNorm lane
// layout needs no exchange at all; vector v of a row covers pairs
// (kEpv / 2) * (v mod (head_dim / kEpv)) .. + kEpv / 2 of its head.  head_dim
// must be a multiple of kEpv (vectors never straddle heads).  SHARED:
// head_dim / kEpv divides the lanes per row (every power-of-two head_dim up
// to 64 kEpv), so all slots of a lane share one table offset and the row
// needs a single table slice per lane.  PRIO raises the wave priority while
// a row's loads issue.  WL (per-slot one-wavefront priority instances) keeps
// the weight in LDS and takes each slot's table slice in turn instead of
// holding them all: 54-62 VGPRs at 3 vectors per lane instead of 78-88, so
// 8192 rows of hidden 1152 fit at once (d = 72: 9.69 -> 8.92 us; d = 24:
// 9.65 -> 8.87 us); the launch prefers the register form where it fits.
// ---------------------------------------------------------------------------
template <typename IO, int VPL, int WPR, bool FULL, bool SHARED, bool PRIO, int VW = 1, bool WL = false>
__global__ void __launch_bounds__(Layout<WPR>::kThreads)
rmsnorm_rope_interleaved_kernel(const KArgs a) {
    static_assert(VW == 1 || (SHARED && PRIO && WPR == 1), "split-order sums: shared-slice priority instances");
    static_assert(!WL || (!SHARED && PRIO && WPR == 1), "LDS weight: per-slot one-wavefront priority instances");
    constexpr bool kWl = VW > 1 || WL;  // weight in LDS
    constexpr int RPB = Layout<WPR>::kRowsPerBlock;
    constexpr int L = Layout<WPR>::kLanesPerRow;
    constexpr int E = IO::kEpv;
    constexpr int NP = E / 2;  // pairs per vector
    const Lane<WPR> ln;
    const int vph = a.vec_per_head;

    if constexpr (PRIO) priority_for_loads();
    __shared__ u32x4 wlds[kWl ? VPL * kWave : 1];
    u32x4 wv[kWl ? 1 : VPL];
    int toff[VPL];
    if constexpr (kWl) {
        for (int v = threadIdx.x; v < VPL * kWave; v += Layout<WPR>::kThreads)
            wlds[v] = (a.w != nullptr && v < a.nvec) ? reinterpret_cast<const u32x4*>(a.w)[v] : splat(IO::kOne);
        __syncthreads();
    } else {
        load_weight<IO, VPL, L, FULL>(wv, a.w, ln.t, a.nvec);
    }
#pragma unroll
    for (int k = 0; k < VPL; ++k) toff[k] = ((k * L + ln.t) % vph) * NP;

    int parity = 0;
    for (int64_t base = (int64_t)blockIdx.x * RPB; base < a.rows;
         base += (int64_t)gridDim.x * RPB, parity ^= 1) {
        const int64_t row = base + ln.slot;
        const bool active = row < a.rows;
        if (WPR == 1 && !active) continue;
        const int64_t pos = active ? row % a.seq_len : 0;
        const u32x4* xr = reinterpret_cast<const u32x4*>(a.x) + row * a.nvec;
        u32x4* yr = reinterpret_cast<u32x4*>(a.out) + row * a.nvec;

        u32x4 xv[VPL];
        if constexpr (PRIO) priority_for_loads();
        load_row<VPL, L, FULL, WPR>(xv, xr, ln.t, a.nvec, active);
        const float* crow = a.cos_tab + pos * a.half;
        const float* srow = a.sin_tab + pos * a.half;
        // Per-slot slices, one wavefront per row, heads of at most 64
        // vectors: the wavefront fetches the position's table rows once, with
        // x (vph chunks of NP floats), and after the reduction each slot takes
        // its slice from the lane holding it (d = 72, 24, 40 at about 200 MB:
        // 66.8 -> 68.8 %, 67.1 -> 68.8 %, 67.3 -> 73.1 % of peak; with one
        // slice per row this measured slower on the [8192 x 2048] workload,
        // and with 16 wavefronts per row it spills registers).  Otherwise, up to four slots fetch their slices at once
        // (one L2 round trip per row, not one per slot: d = 72 and 24 at
        // [43690 x 1152], 64.4 -> 67.2 % and 65.1 -> 67.4 %), with x for
        // several wavefronts per row and after the reduction for one; more
        // slots would spill registers, so there slots 1.. load in turn.
        constexpr bool kAll = !SHARED && VPL <= 4 && !WL;
        constexpr int NT = kAll ? VPL : 1;  // table slices held at once
        float c[NT][NP], sn[NT][NP];
        constexpr bool kGather = !SHARED && WPR == 1;
        const bool gathered = kGather && vph <= kWave;
        TableLds<NP, Layout<WPR>::kThreads / kWave, kWave> tabs(ln.slot * WPR + ln.wave_in_row);
        if constexpr (kGather) {
            if (gathered) tabs.fetch(crow, srow, ln.lane, vph);
        }
        auto load_tables = [&]() {
#pragma unroll
            for (int k = 0; k < NT; ++k) {
                if (gathered) {
                    tabs.take(toff[k], c[k], sn[k]);
                } else {
                    load_floats<NP>(crow + toff[k], c[k]);
                    load_floats<NP>(srow + toff[k], sn[k]);
                }
            }
        };
        if constexpr (WPR > 1) {
            if (!gathered) load_tables();
        }
        if constexpr (PRIO) priority_after_loads();
        float sum_sq;
        if constexpr (VW > 1) {
            sum_sq = split_order_row_sum<IO, VPL, VW>(xv);
        } else {
            const float part = sum_squares<IO, VPL>(xv);
            sum_sq = row_sum<WPR>(part, ln.slot, ln.wave_in_row, parity);
        }
        const float rstd = rstd_of(sum_sq, a.hidden_f, a.eps);
        if constexpr (kGather) {
            if (gathered) tabs.share(ln.lane, vph);
        }
        if (WPR == 1 || gathered) load_tables();
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = k * L + ln.t;
            const bool in = (FULL || v < a.nvec) && (WPR == 1 || active);
            if constexpr (!SHARED && !kAll) {
                if (k > 0) {
                    if (gathered) {
                        tabs.take(toff[k], c[0], sn[0]);
                    } else {
                        load_floats<NP>(crow + toff[k], c[0]);
                        load_floats<NP>(srow + toff[k], sn[0]);
                    }
                }
            }
            const float* ck = c[kAll ? k : 0];
            const float* sk = sn[kAll ? k : 0];
            keep_packed(xv[k]);
            float y[E], g[E], o[E];
            if constexpr (kWl) {
                u32x4 wk = wlds[v];
                keep_packed(wk);
                IO::widen(xv[k], y);
                IO::widen(wk, g);
            } else {
                keep_packed(wv[k]);
                IO::widen(xv[k], y);
                IO::widen(wv[k], g);
            }
#pragma unroll
            for (int e = 0; e < E; ++e) y[e] = (y[e] * rstd) * g[e];
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                o[2 * j] = rot(y[2 * j], ck[j], -y[2 * j + 1], sk[j]);
                o[2 * j + 1] = rot(y[2 * j + 1], ck[j], y[2 * j], sk[j]);
            }
            if (in) store_stream(yr + v, IO::narrow(o));
        }
    }
}

// ---------------------------------------------------------------------------
// RMSNorm with per-sample adaptive modulation (AdaLN, as in DiT blocks):
// y = ((x * rstd) * w) * (1 + scale[b]) + shift[b], b = row / rows_per_sample,
// all in binary32 and rounded once.  The RMSNorm layout and reduction; the
// modulation rows are shared by every row of a sample and come from L2.  A
// null scale reads as +0 (factor exactly 1) and a null shift as -0
// (x + -0 == x for every x, signed zeros included), so with both null the
// result equals plain RMSNorm bit for bit.  Wave priority as for RMSNorm.
// The one-wavefront priority instance (PRIO) keeps the weight in LDS, once
// per workgroup, and fetches the modulation rows after the reduction: 58
// VGPRs at 4 vectors per lane instead of 92, 8 wavefronts per SIMD instead of
// 5, so that 8192 rows of hidden 2048 are resident at once (bf16 14.10 ->
// 12.73 us; 4096 rows 7.91 -> 7.63, 6144 rows 11.52 -> 9.84, fp32 [8192 x
// 1024] 13.86 -> 12.42 us).
// ---------------------------------------------------------------------------
template <typename IO, int VPL, int WPR, bool FULL, bool PRIO, int VW = 1>
__global__ void __launch_bounds__(Layout<WPR>::kThreads)
rmsnorm_adaln_kernel(const KArgs a) {
    static_assert(VW == 1 || (WPR == 1 && PRIO), "split-order sums: one-wavefront priority instances");
    constexpr bool kPrio = WPR > 1 || PRIO;  // as for RMSNorm
    constexpr bool kWl = PRIO && WPR == 1;   // weight in LDS
    constexpr int RPB = Layout<WPR>::kRowsPerBlock;
    constexpr int L = Layout<WPR>::kLanesPerRow;
    constexpr int E = IO::kEpv;
    const Lane<WPR> ln;
    if constexpr (kPrio) priority_for_loads();
    __shared__ u32x4 wlds[kWl ? VPL * kWave : 1];
    u32x4 wv[kWl ? 1 : VPL];
    if constexpr (kWl) {
        // every slot of the row's lanes, ones past the row
        for (int v = threadIdx.x; v < VPL * kWave; v += Layout<WPR>::kThreads)
            wlds[v] = (a.w != nullptr && v < a.nvec) ? reinterpret_cast<const u32x4*>(a.w)[v] : splat(IO::kOne);
        __syncthreads();
    } else {
        load_weight<IO, VPL, L, FULL>(wv, a.w, ln.t, a.nvec);
    }

    int parity = 0;
    for (int64_t base = (int64_t)blockIdx.x * RPB; base < a.rows;
         base += (int64_t)gridDim.x * RPB, parity ^= 1) {
        const int64_t row = base + ln.slot;
        const bool active = row < a.rows;
        if (WPR == 1 && !active) continue;
        const u32x4* xr = reinterpret_cast<const u32x4*>(a.x) + row * a.nvec;
        u32x4* yr = reinterpret_cast<u32x4*>(a.out) + row * a.nvec;
        const int64_t sample = active ? row / a.rows_per_sample : 0;
        const u32x4* sr = reinterpret_cast<const u32x4*>(a.scale) + sample * a.nvec;
        const u32x4* hr = reinterpret_cast<const u32x4*>(a.shift) + sample * a.nvec;

        // The modulation rows are L2 hits.  With one wavefront per row they
        // are fetched together with x, taking their latency off the row's
        // critical path (H = 2048: 15.3 -> 14.0 us at [8192 x 2048]); with
        // several wavefronts per row that cost more than it saved (H = 4096:
        // 26.4 -> 28.1 us), so there they are fetched after the reduction,
        // and so does the priority instance, to hold fewer registers.
        constexpr bool kEarly = WPR == 1 && !kWl;
        auto mod_rows = [&](int k, u32x4& sv, u32x4& hv) {
            const int v = k * L + ln.t;
            const bool in = (FULL || v < a.nvec) && (WPR == 1 || active);
            sv = (a.scale != nullptr && in) ? sr[v] : u32x4{0u, 0u, 0u, 0u};
            hv = (a.shift != nullptr && in) ? hr[v] : splat(IO::kNegZero);
        };
        u32x4 xv[VPL], svv[VPL], hvv[VPL];
        if constexpr (kPrio) priority_for_loads();
        load_row<VPL, L, FULL, WPR>(xv, xr, ln.t, a.nvec, active);
        if constexpr (kEarly) {
#pragma unroll
            for (int k = 0; k < VPL; ++k) mod_rows(k, svv[k], hvv[k]);
        }
        if constexpr (kPrio) priority_after_loads();
        float sum_sq;
        if constexpr (VW > 1) {
            sum_sq = split_order_row_sum<IO, VPL, VW>(xv);
        } else {
            const float part = sum_squares<IO, VPL>(xv);
            sum_sq = row_sum<WPR>(part, ln.slot, ln.wave_in_row, parity);
        }
        const float rstd = rstd_of(sum_sq, a.hidden_f, a.eps);

#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = k * L + ln.t;
            const bool in = (FULL || v < a.nvec) && (WPR == 1 || active);
            u32x4 sv, hv;
            if constexpr (kEarly) {
                sv = svv[k];
                hv = hvv[k];
            } else {
                mod_rows(k, sv, hv);
            }
            keep_packed(xv[k]);
            float f[E], g[E], sc[E], sh[E];
            if constexpr (kWl) {
                u32x4 wk = wlds[v];
                keep_packed(wk);
                IO::widen(xv[k], f);
                IO::widen(wk, g);
            } else {
                keep_packed(wv[k]);
                IO::widen(xv[k], f);
                IO::widen(wv[k], g);
            }
            IO::widen(sv, sc);
            IO::widen(hv, sh);
#pragma unroll
            for (int e = 0; e < E; ++e) f[e] = modulate((f[e] * rstd) * g[e], sc[e], sh[e]);
            if (in) store_stream(yr + v, IO::narrow(f));
        }
    }
}

}  // namespace
}  // namespace ltxnorm_detail
