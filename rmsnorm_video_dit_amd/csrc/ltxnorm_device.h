// ltxnorm_device.h -- device-side building blocks shared by the gfx950
// (MI355X) kernels for row-wise RMSNorm, fused RMSNorm + RoPE (rotate-half
// and interleaved pairs) and AdaLN-modulated RMSNorm, templated on the I/O
// element type: I/O traits, vector access, the wavefront and row reductions,
// kernel arguments.  The kernels are in ltxnorm_kernels.h (rows of whole
// 16-byte vectors) and ltxnorm_general.h (any row length); not a public
// header.
//
// The operations (declared in include/ltxnorm.h):
//  * RMSNorm over the innermost dimension of [..., hidden], eps default 1e-6,
//    optional weight (Hugging Face cuda-kernels skill page, "Kernel-Specific
//    Guidelines", RMSNorm; "Diffusers Critical Pitfalls", item 1 for the
//    absent weight), computed as y = x * rsqrt(mean(x^2) + eps) * w; the
//    three precisions the page lists ("Supported Data Types": FP16, BF16,
//    FP32) as I/O types, binary32 arithmetic throughout.
//  * rms_norm_rope (LTX-2 ltx-kernels README, introduction): that RMSNorm
//    over the full row followed by RoPE per head on the 1D
//    [batch, seq, heads, head_dim] layout (skill page, RoPE), rotate-half or
//    interleaved pairs.
//  * AdaLN (skill page, "Kernel-Specific Guidelines", AdaLN):
//    norm(x) * weight * (1 + scale) + shift with per-sample scale/shift.
//
// Design for gfx950
//  * The ops move 2 (or 4) bytes in and out per element and do a handful of
//    flops: they are bound by HBM bandwidth, so there is no MFMA and the
//    design is about moving each byte once with full-width accesses.
//  * A row is held entirely in VGPRs: HBM is read once and written once.
//    Every access is a 16-byte vector (8 bf16/fp16 or 4 fp32 values);
//    consecutive lanes touch consecutive vectors, so one load instruction
//    covers 1 KiB contiguous.
//  * One wavefront per row while a lane holds at most 4 vectors; longer rows
//    use 3..16 wavefronts (about 2 vectors per lane) whose partial sums meet
//    in LDS.
//  * Sum of squares: per-lane fp32 FMAs in a fixed order, then a fixed DPP
//    butterfly inside each 16-lane row (quad_perm, row_half_mirror,
//    row_mirror) and four readlanes; every lane ends with identical bits and
//    the result is deterministic run to run.
//  * rstd = 1 / sqrt(sum / H + eps) with correctly rounded binary32 divide
//    and square root: it scales exactly under x -> 2^k x, and costs nothing
//    next to the row's memory traffic.
//  * The weight slice (and for RoPE each lane's table offsets) is loaded at
//    the start, in flight together with the row; one workgroup per 1-4 rows.
//  * x is loaded and y stored with the non-temporal hint (streamed once).
//  * Output rounding: binary32 -> bf16 / fp16 round-to-nearest-even
//    (v_cvt_pk_bf16_f32 / v_cvt_f16_f32 under the default rounding mode).
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "ltxnorm_launch.h"

namespace ltxnorm_detail {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));


// ---------------------------------------------------------------------------
// I/O element types.  kEpv values per 16-byte vector; kOne and kNegZero are
// one 32-bit word of the constants 1.0 and -0.0 in the type.
// ---------------------------------------------------------------------------

// bf16 is the upper half of a binary32: widening is exact.  The element at
// the lower address sits in the low 16 bits of each 32-bit word.
struct IoBf16 {
    static constexpr int kEpv = 8;
    static constexpr uint32_t kOne = 0x3F803F80u;
    static constexpr uint32_t kNegZero = 0x80008000u;
    __device__ static __forceinline__ void widen(const u32x4 v, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(v[i] << 16);
            f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
        }
    }
    // nearest, ties to even; NaN stays NaN (v_cvt_pk_bf16_f32)
    __device__ static __forceinline__ u32x4 narrow(const float* f) {
        u32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x2 p = {f[2 * i], f[2 * i + 1]};
            r[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
        }
        return r;
    }
};

// IEEE binary16: widening is exact (v_cvt_f32_f16); narrowing rounds to
// nearest even, overflows to infinity and keeps subnormals.
struct IoF16 {
    static constexpr int kEpv = 8;
    static constexpr uint32_t kOne = 0x3C003C00u;
    static constexpr uint32_t kNegZero = 0x80008000u;
    __device__ static __forceinline__ void widen(const u32x4 v, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // Copy the word out first: this compiler lowers a bit-cast of the
            // vector element v[i] itself to element 0 for every i.
            const uint32_t word = v[i];
            const f16x2 h = __builtin_bit_cast(f16x2, word);
            f[2 * i] = (float)h[0];
            f[2 * i + 1] = (float)h[1];
        }
    }
    __device__ static __forceinline__ u32x4 narrow(const float* f) {
        u32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f16x2 h = {(_Float16)f[2 * i], (_Float16)f[2 * i + 1]};
            r[i] = __builtin_bit_cast(uint32_t, h);
        }
        return r;
    }
};

struct IoF32 {
    static constexpr int kEpv = 4;
    static constexpr uint32_t kOne = 0x3F800000u;
    static constexpr uint32_t kNegZero = 0x80000000u;
    __device__ static __forceinline__ void widen(const u32x4 v, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
    }
    __device__ static __forceinline__ u32x4 narrow(const float* f) {
        return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                     __float_as_uint(f[3])};
    }
};

// Operation of a kernel that serves several: RMSNorm, AdaLN, rotate-half
// RoPE, interleaved RoPE.
enum class GOp { kRms, kAda, kRopeHalf, kRopeIl };

__device__ __forceinline__ u32x4 splat(uint32_t w) { return u32x4{w, w, w, w}; }

// Keep a packed register value opaque to the optimiser, so that it is
// widened where it is used and lives in 4 VGPRs rather than 8.  Without
// this, loop-invariant code motion widens the weight once outside the row
// loop, and common-subexpression elimination keeps the widened row alive
// across the reduction; either doubles the register footprint and halves
// occupancy.  Emits no instruction.
__device__ __forceinline__ void keep_packed(u32x4& v) { asm volatile("" : "+v"(v)); }

// x is read once and y written once: stream both past the caches with the
// non-temporal hint (measured ~3% more HBM throughput than plain accesses on
// a 50/50 read/write stream).  Weights, modulation rows and rotation tables,
// which many rows reuse, use ordinary cached loads.
__device__ __forceinline__ u32x4 load_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_stream(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

// N consecutive binary32 values (N = 2, 4 or 8) from a 16-byte (N >= 4) or
// 8-byte (N = 2) aligned address.
template <int N>
__device__ __forceinline__ void load_floats(const float* p, float* out) {
    if constexpr (N == 2) {
        const f32x2 v = *reinterpret_cast<const f32x2*>(p);
        out[0] = v[0];
        out[1] = v[1];
    } else {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            const f32x4 v = reinterpret_cast<const f32x4*>(p)[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) out[4 * i + j] = v[j];
        }
    }
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                              0xF, 0xF, false));
}

// The value of lane l ^ P, for P a power of two up to 32, without a round
// trip through the LDS crossbar (ds_bpermute): DPP moves inside each 16-lane
// row, the gfx950 lane swaps across rows.  Every lane of the wavefront must
// be active.
//  * P = 1, 2: quad_perm [1,0,3,2] / [2,3,0,1].
//  * P = 4: row_half_mirror (j -> j ^ 7 within the row), then quad_perm
//    [3,2,1,0] (j -> j ^ 3): j ^ 4.
//  * P = 8: row_mirror (j -> j ^ 15), then row_half_mirror (j -> j ^ 7): j ^ 8.
//  * P = 16: v_permlane16_swap of the value with itself swaps the odd rows
//    of the first copy with the even rows of the second, so the first result
//    holds rows (0, 0, 2, 2) and the second rows (1, 1, 3, 3): a lane of an
//    even row takes the second, a lane of an odd row the first.
//  * P = 32: v_permlane32_swap likewise gives halves (lo, lo) and (hi, hi).
template <int P>
__device__ __forceinline__ float xor_lane(float v) {
    static_assert(P == 1 || P == 2 || P == 4 || P == 8 || P == 16 || P == 32, "P: 1..32");
    if constexpr (P == 1) {
        return dpp<0xB1>(v);
    } else if constexpr (P == 2) {
        return dpp<0x4E>(v);
    } else if constexpr (P == 4) {
        return dpp<0x1B>(dpp<0x141>(v));
    } else if constexpr (P == 8) {
        return dpp<0x141>(dpp<0x140>(v));
    } else {
        const uint32_t b = __builtin_bit_cast(uint32_t, v);
        const bool upper = (threadIdx.x & P) != 0;
        if constexpr (P == 16) {
            const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
            return __builtin_bit_cast(float, upper ? r[0] : r[1]);
        } else {
            const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
            return __builtin_bit_cast(float, upper ? r[0] : r[1]);
        }
    }
}

// Call f(std::integral_constant<int, P>{}) for a wave-uniform P in {1, 2,
// 4, 8, 16, 32}: one scalar branch per call, so that what f does for its P
// (every xor_lane<P> of a row) is straight-line code.
template <typename F>
__device__ __forceinline__ void with_pow2(int P, F&& f) {
    switch (P) {
        case 1: f(std::integral_constant<int, 1>{}); break;
        case 2: f(std::integral_constant<int, 2>{}); break;
        case 4: f(std::integral_constant<int, 4>{}); break;
        case 8: f(std::integral_constant<int, 8>{}); break;
        case 16: f(std::integral_constant<int, 16>{}); break;
        default: f(std::integral_constant<int, 32>{}); break;
    }
}

// Sum over the 64 lanes of a fully active wavefront.  Inside each row of 16
// lanes: xor-1 and xor-2 swaps (quad_perm), then the 8-lane and 16-lane
// mirrors; each step adds two equal-shaped partial sums, so all lanes of a
// row hold the same bits.  The four row sums are then combined as
// (r0 + r1) + (r2 + r3) from scalar registers: the result is uniform.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);  // row_half_mirror
    v += dpp<0x140>(v);  // row_mirror
    const int b = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return (r0 + r1) + (r2 + r3);
}

// Rows per workgroup: four single-wavefront rows (256 threads), two rows of
// 2-3 wavefronts, one row of 4-16 wavefronts (256-1024 threads).
template <int WPR>
struct Layout {
    static constexpr int kRowsPerBlock = rows_per_block(WPR);
    static constexpr int kThreads = kWave * WPR * kRowsPerBlock;
    static constexpr int kLanesPerRow = kWave * WPR;
};

// Row total of a per-lane partial: one wavefront per row needs only the
// wave sum; several wavefronts per row publish their sums in LDS (double
// buffered by iteration parity, so one barrier per row suffices) and every
// wavefront adds them in the same order.
template <int WPR>
__device__ __forceinline__ float row_sum(float part, int slot, int wave_in_row, int parity) {
    float s = wave_sum(part);
    if constexpr (WPR > 1) {
        constexpr int RPB = Layout<WPR>::kRowsPerBlock;
        __shared__ float partials[2][RPB][WPR];
        if ((threadIdx.x & (kWave - 1)) == 0) partials[parity][slot][wave_in_row] = s;
        __syncthreads();
        s = 0.0f;
#pragma unroll
        for (int i = 0; i < WPR; ++i) s += partials[parity][slot][i];
    }
    return s;
}

__device__ __forceinline__ float rstd_of(float sum_sq, float hidden_f, float eps) {
    return 1.0f / sqrtf(sum_sq / hidden_f + eps);
}

// Kernel arguments (one layout for every kernel; each reads what it uses).
struct KArgs {
    void* out;
    const void* x;
    const void* w;
    const float* cos_tab;
    const float* sin_tab;
    const void* scale;
    const void* shift;
    int64_t rows;
    int64_t seq_len;
    int64_t rows_per_sample;
    int32_t nvec;           // vectors per row: hidden / kEpv
    int32_t nunits;         // pair units per row (pair-in-lane RoPE): nvec / 2
    int32_t vec_per_half;   // vectors per half head: head_dim / (2 kEpv) (rotate-half)
    int32_t vec_per_head;   // vectors per head: head_dim / kEpv (interleaved)
    int32_t half;           // head_dim / 2: floats per table row
    int32_t hidden;         // row length in elements
    int32_t head_dim;       // elements per head (RoPE)
    int64_t mod_elems;      // elements in each modulation array: samples * hidden
    float hidden_f;
    float eps;
};

// Wave priority around a row's loads: a wavefront raises its priority while
// it issues the loads of its row and drops back as soon as they are in
// flight, so that on a CU where some wavefronts reduce or store and others
// start a row, the new row's requests reach memory first.  Where it is used,
// measured at about 100-200 MB per launch unless stated:
//  * RMSNorm and AdaLN rows of several wavefronts, always (bf16
//    [16384 x 3072] +0.3 %, fp32 +1.0 %, fp32 hidden 4096 +3.8 %; AdaLN
//    hidden 3072 and 4096 +1.3 and +2.1 %), and the general kernel (hidden
//    1028, 2052, 3076 +3.1, +1.9, +0.5 %);
//  * one-wavefront rows of RMSNorm, AdaLN and the RoPE kernels (template flag
//    PRIO) when the whole grid is resident at once: every row's loads then
//    issue before the stores start, instead of reads and writes interleaving
//    (bf16 [8192 x 2048] RMSNorm 13.07 -> 11.33 us, interleaved RoPE 13.30 ->
//    11.56 us; [4096 x 2048] rotate-half RoPE 8.03 -> 7.23 us, AdaLN 8.40 ->
//    7.84 us; [4096 x 2048] RMSNorm 7.89 -> 6.63 us).  On grids of several
//    waves of workgroups the same instances ran 2-9 % slower, and the
//    short-row kernel was slower either way, so those launches do not use it.
//    Rotate-half RoPE also has one-wavefront priority instances with the
//    weight in LDS (flag WL), and AdaLN's priority instances keep theirs
//    there: both fit 8192 rows of hidden 2048 at once.
__device__ __forceinline__ void priority_for_loads() { __builtin_amdgcn_s_setprio(3); }
__device__ __forceinline__ void priority_after_loads() { __builtin_amdgcn_s_setprio(0); }

// One rotation term a * c + b * s in a fixed form: a * c rounded, then
// fused with b * s (b is the partner value, which may still be on its way
// from another lane).  Written out so that the compiler's contraction of
// the plain expression, which may fuse either product and chooses per
// instruction, cannot make two instances or two paths of the same row round
// differently (a - b form passes -b).
__device__ __forceinline__ float rot(float a, float c, float b, float s) { return fmaf(b, s, a * c); }

// AdaLN modulation t * (1 + scale) + shift, fused in one fixed form for
// the same reason.  A null scale (+0) and shift (-0) give t bit for bit.
__device__ __forceinline__ float modulate(float t, float scale, float shift) {
    return fmaf(t, 1.0f + scale, shift);
}

// Common prologue of every kernel: which row slot and lane this thread is.
template <int WPR>
struct Lane {
    int slot, wave_in_row, lane, t;
    __device__ __forceinline__ Lane() {
        // wave-uniform (readfirstlane): row and position arithmetic stays on
        // the scalar unit
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
        slot = wave / WPR;
        wave_in_row = wave % WPR;
        lane = threadIdx.x & (kWave - 1);
        t = wave_in_row * kWave + lane;
    }
};

// Load a row slice (VPL vectors per lane, zeros outside the row).
template <int VPL, int L, bool FULL, int WPR>
__device__ __forceinline__ void load_row(u32x4* xv, const u32x4* xr, int t, int nvec, bool active) {
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int v = k * L + t;
        const bool in = (FULL || v < nvec) && (WPR == 1 || active);
        xv[k] = in ? load_stream(xr + v) : u32x4{0u, 0u, 0u, 0u};
    }
}

// RoPE table slices handed out through LDS, for kernels whose lanes need
// table columns that other lanes fetched.  fetch(): lanes [0, nc) load chunk
// `lane` (W consecutive floats) of the position's cos row and of its sin
// row; the other lanes load nothing.  share(), once those loads have landed:
// the same lanes write their chunks into this wavefront's LDS region.
// take(col): each lane reads the W floats at column col (a multiple of W) of
// both tables, one 8- or 16-byte LDS read per table; lanes reading the same
// chunk read the same address.  Two partial global loads, two LDS writes and
// two LDS reads per chunk a lane needs replace a 16-byte global load per
// table per lane (rows short enough that table reads weigh: hidden 1152,
// heads of 72), and the 2 W ds_bpermute transfers per chunk of an exchange
// between lanes, whose many-to-one reads conflicted in the LDS banks.
// NW wavefronts per workgroup; a wavefront's region holds up to MAXC chunks
// per table.  LDS accesses of one wavefront complete in order, so the reads
// see the writes without a workgroup barrier, and the next row's writes come
// after this row's reads.
template <int W, int NW, int MAXC>
struct TableLds {
    static_assert(W == 2 || W == 4, "chunks of 2 or 4 floats");
    float tc[W], ts[W];
    float* cos_region;
    float* sin_region;
    __device__ __forceinline__ explicit TableLds(int wave) {
        __shared__ __attribute__((aligned(16))) float lds[NW][2][MAXC * W];
        cos_region = &lds[wave][0][0];
        sin_region = &lds[wave][1][0];
    }
    __device__ __forceinline__ void fetch(const float* crow, const float* srow, int lane, int nc) {
#pragma unroll
        for (int j = 0; j < W; ++j) tc[j] = ts[j] = 0.0f;
        if (lane < nc) {
            load_floats<W>(crow + lane * W, tc);
            load_floats<W>(srow + lane * W, ts);
        }
    }
    __device__ __forceinline__ void share(int lane, int nc) {
        if (lane < nc) {
            if constexpr (W == 4) {
                *reinterpret_cast<f32x4*>(cos_region + lane * W) = f32x4{tc[0], tc[1], tc[2], tc[3]};
                *reinterpret_cast<f32x4*>(sin_region + lane * W) = f32x4{ts[0], ts[1], ts[2], ts[3]};
            } else {
                *reinterpret_cast<f32x2*>(cos_region + lane * W) = f32x2{tc[0], tc[1]};
                *reinterpret_cast<f32x2*>(sin_region + lane * W) = f32x2{ts[0], ts[1]};
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    __device__ __forceinline__ void take(int col, float* c, float* s) const {
        if constexpr (W == 4) {
            const f32x4 vc = *reinterpret_cast<const f32x4*>(cos_region + col);
            const f32x4 vs = *reinterpret_cast<const f32x4*>(sin_region + col);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                c[j] = vc[j];
                s[j] = vs[j];
            }
        } else {
            const f32x2 vc = *reinterpret_cast<const f32x2*>(cos_region + col);
            const f32x2 vs = *reinterpret_cast<const f32x2*>(sin_region + col);
            c[0] = vc[0];
            c[1] = vc[1];
            s[0] = vs[0];
            s[1] = vs[1];
        }
    }
};

// Per-lane partial sum of squares of a row slice.
template <typename IO, int VPL>
__device__ __forceinline__ float sum_squares(const u32x4* xv) {
    float part = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        float f[IO::kEpv];
        IO::widen(xv[k], f);
#pragma unroll
        for (int e = 0; e < IO::kEpv; ++e) part = fmaf(f[e], f[e], part);
    }
    return part;
}

// Row total of a row held by one wavefront (VPL vectors per lane, vector
// k * 64 + lane in slot k) in the order in which VW wavefronts of VPL / VW
// vectors per lane would add it: lane l of virtual wavefront j would hold
// vectors (k * VW + j) * 64 + l, k = 0 .. VPL / VW - 1, which are this
// lane's slots k * VW + j.  Each virtual wavefront's partial is the same
// fma chain, reduced by the same wave_sum, and the totals are added in
// row_sum's order, so the result has the bits of the VW-wavefront split.
template <typename IO, int VPL, int VW>
__device__ __forceinline__ float split_order_row_sum(const u32x4* xv) {
    static_assert(VPL % VW == 0, "whole vectors per virtual wavefront");
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < VW; ++j) {
        float part = 0.0f;
#pragma unroll
        for (int k = 0; k < VPL / VW; ++k) {
            float f[IO::kEpv];
            IO::widen(xv[k * VW + j], f);
#pragma unroll
            for (int e = 0; e < IO::kEpv; ++e) part = fmaf(f[e], f[e], part);
        }
        s += wave_sum(part);
    }
    return s;
}

// Weight slice (ones for a null weight).
template <typename IO, int VPL, int L, bool FULL>
__device__ __forceinline__ void load_weight(u32x4* wv, const void* w, int t, int nvec) {
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int v = k * L + t;
        const bool in = FULL || v < nvec;
        wv[k] = (w != nullptr && in) ? reinterpret_cast<const u32x4*>(w)[v] : splat(IO::kOne);
    }
}

}  // namespace
}  // namespace ltxnorm_detail
