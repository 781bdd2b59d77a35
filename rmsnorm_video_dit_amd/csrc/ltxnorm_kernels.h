// ltxnorm_kernels.h -- gfx950 (MI355X) kernels for row-wise RMSNorm, fused
// RMSNorm + RoPE (rotate-half and interleaved pairs) and AdaLN-modulated
// RMSNorm, templated on the I/O element type.  Included once per dtype by
// ltxnorm_bf16.hip / ltxnorm_f16.hip / ltxnorm_f32.hip; not a public header.
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

#include "ltxnorm_launch.h"

namespace ltxnorm_detail {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kMaxVecPerLane = 8;     // register budget for one row slice
constexpr int kMaxWavesPerRow = 16;   // 1024-thread workgroup
constexpr int64_t kMaxGrid = 1 << 30; // rows beyond grid * rows-per-block loop

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
    static constexpr int kRowsPerBlock = WPR == 1 ? 4 : (WPR <= 3 ? 2 : 1);
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
    float hidden_f;
    float eps;
};

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

// ---------------------------------------------------------------------------
// RMSNorm: VPL vectors per lane, WPR wavefronts per row.  FULL means every
// lane's every slot is inside the row (no masking).
// ---------------------------------------------------------------------------
template <typename IO, int VPL, int WPR, bool FULL>
__global__ void __launch_bounds__(Layout<WPR>::kThreads)
rmsnorm_kernel(const KArgs a) {
    constexpr int RPB = Layout<WPR>::kRowsPerBlock;
    constexpr int L = Layout<WPR>::kLanesPerRow;
    constexpr int E = IO::kEpv;
    const Lane<WPR> ln;
    u32x4 wv[VPL];
    load_weight<IO, VPL, L, FULL>(wv, a.w, ln.t, a.nvec);

    int parity = 0;
    for (int64_t base = (int64_t)blockIdx.x * RPB; base < a.rows;
         base += (int64_t)gridDim.x * RPB, parity ^= 1) {
        const int64_t row = base + ln.slot;
        const bool active = row < a.rows;
        if (WPR == 1 && !active) continue;  // wave-uniform; no barrier at WPR 1
        const u32x4* xr = reinterpret_cast<const u32x4*>(a.x) + row * a.nvec;
        u32x4* yr = reinterpret_cast<u32x4*>(a.out) + row * a.nvec;

        u32x4 xv[VPL];
        load_row<VPL, L, FULL, WPR>(xv, xr, ln.t, a.nvec, active);
        const float part = sum_squares<IO, VPL>(xv);
        const float rstd = rstd_of(row_sum<WPR>(part, ln.slot, ln.wave_in_row, parity), a.hidden_f, a.eps);

#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = k * L + ln.t;
            const bool in = (FULL || v < a.nvec) && (WPR == 1 || active);
            float f[E], g[E];
            keep_packed(xv[k]);
            IO::widen(xv[k], f);
            keep_packed(wv[k]);
            IO::widen(wv[k], g);
#pragma unroll
            for (int e = 0; e < E; ++e) f[e] = (f[e] * rstd) * g[e];
            if (in) store_stream(yr + v, IO::narrow(f));
        }
    }
}

// ---------------------------------------------------------------------------
// RMSNorm + rotate-half RoPE with the RMSNorm lane layout, when the number
// of vectors per half head P = head_dim / (2 kEpv) is a power of two up to
// 32.  Lane t holds vectors k*L + t (full 1 KiB lines per load
// instruction); the partner of vector v is v ^ P: the same slot of lane
// t ^ P in the same wavefront.  Each lane normalises its own vector and
// fetches the partner's normalised binary32 values with ds_bpermute
// (exchanging the finished values rather than raw x halves the VALU work per
// vector, which matters because with one row per wavefront the whole grid is
// resident and compute is not hidden behind later loads).  A lane's half
// (bit P of t) and its table slice (floats kEpv * (t mod P) .. + kEpv) do not
// depend on the slot, so each lane reads one table slice per row.
// ---------------------------------------------------------------------------
template <typename IO, int VPL, int WPR, bool FULL>
__global__ void __launch_bounds__(Layout<WPR>::kThreads)
rmsnorm_rope_xor_kernel(const KArgs a) {
    constexpr int RPB = Layout<WPR>::kRowsPerBlock;
    constexpr int L = Layout<WPR>::kLanesPerRow;
    constexpr int E = IO::kEpv;
    const Lane<WPR> ln;
    const int P = a.vec_per_half;
    const int src = ((ln.lane ^ P) & (kWave - 1)) << 2;  // ds_bpermute byte address
    const float sgn = (ln.t & P) ? 1.0f : -1.0f;  // second half adds, first subtracts
    const int toff = (ln.t & (P - 1)) * E;

    u32x4 wv[VPL];
    load_weight<IO, VPL, L, FULL>(wv, a.w, ln.t, a.nvec);

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
        load_row<VPL, L, FULL, WPR>(xv, xr, ln.t, a.nvec, active);
        const float part = sum_squares<IO, VPL>(xv);
        const float rstd = rstd_of(row_sum<WPR>(part, ln.slot, ln.wave_in_row, parity), a.hidden_f, a.eps);

        float c[E], ss[E];
        load_floats<E>(a.cos_tab + pos * a.half + toff, c);
        load_floats<E>(a.sin_tab + pos * a.half + toff, ss);
        // the partner term enters with -sin in the first half, +sin in the second
#pragma unroll
        for (int e = 0; e < E; ++e) ss[e] *= sgn;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = k * L + ln.t;
            const bool in = (FULL || v < a.nvec) && (WPR == 1 || active);
            keep_packed(xv[k]);
            keep_packed(wv[k]);
            float own[E], g[E], par[E], o[E];
            IO::widen(xv[k], own);
            IO::widen(wv[k], g);
#pragma unroll
            for (int e = 0; e < E; ++e) own[e] = (own[e] * rstd) * g[e];
            // the partner lane's normalised values, exact binary32 bits
#pragma unroll
            for (int e = 0; e < E; ++e)
                par[e] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, own[e])));
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] = own[e] * c[e] + par[e] * ss[e];
            if (in) store_stream(yr + v, IO::narrow(o));
        }
    }
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
                o1[e] = ya[e] * c[e] - yb[e] * s[e];
                o2[e] = yb[e] * c[e] + ya[e] * s[e];
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
// needs a single table slice per lane.
// ---------------------------------------------------------------------------
template <typename IO, int VPL, int WPR, bool FULL, bool SHARED>
__global__ void __launch_bounds__(Layout<WPR>::kThreads)
rmsnorm_rope_interleaved_kernel(const KArgs a) {
    constexpr int RPB = Layout<WPR>::kRowsPerBlock;
    constexpr int L = Layout<WPR>::kLanesPerRow;
    constexpr int E = IO::kEpv;
    constexpr int NP = E / 2;  // pairs per vector
    const Lane<WPR> ln;
    const int vph = a.vec_per_head;

    u32x4 wv[VPL];
    int toff[VPL];
    load_weight<IO, VPL, L, FULL>(wv, a.w, ln.t, a.nvec);
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
        load_row<VPL, L, FULL, WPR>(xv, xr, ln.t, a.nvec, active);
        const float part = sum_squares<IO, VPL>(xv);
        const float rstd = rstd_of(row_sum<WPR>(part, ln.slot, ln.wave_in_row, parity), a.hidden_f, a.eps);

        const float* crow = a.cos_tab + pos * a.half;
        const float* srow = a.sin_tab + pos * a.half;
        float c[NP], sn[NP];
        load_floats<NP>(crow + toff[0], c);
        load_floats<NP>(srow + toff[0], sn);
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = k * L + ln.t;
            const bool in = (FULL || v < a.nvec) && (WPR == 1 || active);
            if (!SHARED && k > 0) {
                load_floats<NP>(crow + toff[k], c);
                load_floats<NP>(srow + toff[k], sn);
            }
            keep_packed(xv[k]);
            keep_packed(wv[k]);
            float y[E], g[E], o[E];
            IO::widen(xv[k], y);
            IO::widen(wv[k], g);
#pragma unroll
            for (int e = 0; e < E; ++e) y[e] = (y[e] * rstd) * g[e];
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                o[2 * j] = y[2 * j] * c[j] - y[2 * j + 1] * sn[j];
                o[2 * j + 1] = y[2 * j + 1] * c[j] + y[2 * j] * sn[j];
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
// result equals plain RMSNorm bit for bit.
// ---------------------------------------------------------------------------
template <typename IO, int VPL, int WPR, bool FULL>
__global__ void __launch_bounds__(Layout<WPR>::kThreads)
rmsnorm_adaln_kernel(const KArgs a) {
    constexpr int RPB = Layout<WPR>::kRowsPerBlock;
    constexpr int L = Layout<WPR>::kLanesPerRow;
    constexpr int E = IO::kEpv;
    const Lane<WPR> ln;
    u32x4 wv[VPL];
    load_weight<IO, VPL, L, FULL>(wv, a.w, ln.t, a.nvec);

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
        // 26.4 -> 28.1 us), so there they are fetched after the reduction.
        constexpr bool kEarly = WPR == 1;
        auto mod_rows = [&](int k, u32x4& sv, u32x4& hv) {
            const int v = k * L + ln.t;
            const bool in = (FULL || v < a.nvec) && (WPR == 1 || active);
            sv = (a.scale != nullptr && in) ? sr[v] : u32x4{0u, 0u, 0u, 0u};
            hv = (a.shift != nullptr && in) ? hr[v] : splat(IO::kNegZero);
        };
        u32x4 xv[VPL], svv[VPL], hvv[VPL];
        load_row<VPL, L, FULL, WPR>(xv, xr, ln.t, a.nvec, active);
        if constexpr (kEarly) {
#pragma unroll
            for (int k = 0; k < VPL; ++k) mod_rows(k, svv[k], hvv[k]);
        }
        const float part = sum_squares<IO, VPL>(xv);
        const float rstd = rstd_of(row_sum<WPR>(part, ln.slot, ln.wave_in_row, parity), a.hidden_f, a.eps);

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
            keep_packed(wv[k]);
            float f[E], g[E], sc[E], sh[E];
            IO::widen(xv[k], f);
            IO::widen(wv[k], g);
            IO::widen(sv, sc);
            IO::widen(hv, sh);
#pragma unroll
            for (int e = 0; e < E; ++e) f[e] = ((f[e] * rstd) * g[e]) * (1.0f + sc[e]) + sh[e];
            if (in) store_stream(yr + v, IO::narrow(f));
        }
    }
}

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
                             hipStream_t stream) {
    // One workgroup per group of rows: a grid-stride loop capped at the
    // resident capacity measured 3-4% slower than letting the dispatcher
    // stream fresh workgroups, which keeps every CU busy to the last rows.
    const int64_t need = (args.rows + rows_per_block - 1) / rows_per_block;
    const unsigned grid = (unsigned)(need < kMaxGrid ? need : kMaxGrid);
    KArgs copy = args;
    void* params[] = {&copy};
    const hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(threads), params, 0, stream);
    return e == hipSuccess ? LTXNORM_OK : LTXNORM_ERR_HIP;
}

// One launcher per kernel family: go<WPR, PER, FULL>() picks the instance.
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

template <typename LN, int WPR, int LO, int HI>
ltxnorm_status by_per(const Plan& p, const KArgs& a, hipStream_t s) {
    if constexpr (LO > HI) {
        return LTXNORM_ERR_UNSUPPORTED;
    } else {
        if (p.per == LO) {
            const void* fn = p.full ? LN::template fn<WPR, LO, true>() : LN::template fn<WPR, LO, false>();
            return launch(fn, Layout<WPR>::kThreads, Layout<WPR>::kRowsPerBlock, a, s);
        }
        return by_per<LN, WPR, LO + 1, HI>(p, a, s);
    }
}

// Plans that plan_for can produce: one wavefront with 1..ONE items per lane;
// 3..15 wavefronts with exactly SPREAD items per lane (2 wavefronts never
// occur: a row too long for one wavefront needs more than 2 * ONE / SPREAD);
// 16 wavefronts with SPREAD..MAXP items per lane.
template <typename LN, int ONE, int SPREAD, int MAXP>
ltxnorm_status by_plan(const Plan& p, const KArgs& a, hipStream_t s) {
    switch (p.wpr) {
        case 1: return by_per<LN, 1, 1, ONE>(p, a, s);
        case 3: return by_per<LN, 3, SPREAD, SPREAD>(p, a, s);
        case 4: return by_per<LN, 4, SPREAD, SPREAD>(p, a, s);
        case 5: return by_per<LN, 5, SPREAD, SPREAD>(p, a, s);
        case 6: return by_per<LN, 6, SPREAD, SPREAD>(p, a, s);
        case 7: return by_per<LN, 7, SPREAD, SPREAD>(p, a, s);
        case 8: return by_per<LN, 8, SPREAD, SPREAD>(p, a, s);
        case 9: return by_per<LN, 9, SPREAD, SPREAD>(p, a, s);
        case 10: return by_per<LN, 10, SPREAD, SPREAD>(p, a, s);
        case 11: return by_per<LN, 11, SPREAD, SPREAD>(p, a, s);
        case 12: return by_per<LN, 12, SPREAD, SPREAD>(p, a, s);
        case 13: return by_per<LN, 13, SPREAD, SPREAD>(p, a, s);
        case 14: return by_per<LN, 14, SPREAD, SPREAD>(p, a, s);
        case 15: return by_per<LN, 15, SPREAD, SPREAD>(p, a, s);
        case 16: return by_per<LN, 16, SPREAD, MAXP>(p, a, s);
        default: return LTXNORM_ERR_UNSUPPORTED;
    }
}

// Enqueue `op` for I/O type IO on a validated request.
template <typename IO>
ltxnorm_status launch_op(Op op, const Request& r, hipStream_t stream) {
    constexpr int E = IO::kEpv;
    KArgs a{r.out, r.x, r.w, r.cos_tab, r.sin_tab, r.scale, r.shift, r.rows, r.seq_len,
            r.rows_per_sample, (int32_t)(r.hidden / E), (int32_t)(r.hidden / (2 * E)),
            r.head_dim / (2 * E), r.head_dim / E, r.head_dim / 2, (float)r.hidden, r.eps};
    switch (op) {
        case Op::kRmsNorm:
            return by_plan<RmsL<IO>, 4, 2, kMaxVecPerLane>(plan_for(a.nvec, 4, 2), a, stream);
        case Op::kAdaLN:
            return by_plan<AdaL<IO>, 4, 2, kMaxVecPerLane>(plan_for(a.nvec, 4, 2), a, stream);
        case Op::kRopeRotateHalf: {
            const int P = a.vec_per_half;
            if ((P & (P - 1)) == 0 && P <= kWave / 2)  // partner lanes within one wavefront
                return by_plan<RopeXorL<IO>, 4, 2, kMaxVecPerLane>(plan_for(a.nvec, 4, 2), a, stream);
            return by_plan<RopePairL<IO>, 2, 1, kMaxVecPerLane / 2>(plan_for(a.nunits, 2, 1), a,
                                                                    stream);
        }
        case Op::kRopeInterleaved: {
            const Plan p = plan_for(a.nvec, 4, 2);
            const int vph = r.head_dim / E;
            if ((kWave * p.wpr) % vph == 0)
                return by_plan<RopeIlL<IO, true>, 4, 2, kMaxVecPerLane>(p, a, stream);
            return by_plan<RopeIlL<IO, false>, 4, 2, kMaxVecPerLane>(p, a, stream);
        }
    }
    return LTXNORM_ERR_UNSUPPORTED;
}

}  // namespace
}  // namespace ltxnorm_detail
