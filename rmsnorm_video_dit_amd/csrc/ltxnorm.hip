// ltxnorm.hip -- gfx950 (MI355X) kernels and C-ABI launcher for row-wise
// RMSNorm and fused RMSNorm + rotate-half RoPE over bf16 activations.
//
// The operations (declared in include/ltxnorm.h):
//  * RMSNorm over the innermost dimension of [..., hidden], eps default 1e-6,
//    optional weight (Hugging Face cuda-kernels skill page, "Kernel-Specific
//    Guidelines", RMSNorm; "Diffusers Critical Pitfalls", item 1 for the
//    absent weight), computed as y = x * rsqrt(mean(x^2) + eps) * w.
//  * rms_norm_rope (LTX-2 ltx-kernels README, introduction): that RMSNorm
//    over the full row followed by rotate-half RoPE per head on the 1D
//    [batch, seq, heads, head_dim] layout (skill page, RoPE).
//
// Design for gfx950
//  * The op moves 2 bytes in and 2 bytes out per element and does ~4 flops:
//    it is bound by HBM bandwidth, so there is no MFMA and the whole design
//    is about moving each byte exactly once with full-width accesses.
//  * A row is held entirely in VGPRs: HBM is read once and written once.
//    Every access is a 16-byte bf16x8 vector; consecutive lanes touch
//    consecutive vectors, so one load instruction covers 1 KiB contiguous.
//  * One wavefront per row for hidden <= 2048 (up to 4 vectors per lane),
//    otherwise 3..16 wavefronts per row (about 2 vectors per lane) whose
//    partial sums meet in LDS.
//  * Sum of squares: per-lane fp32 FMAs in a fixed order, then a fixed
//    DPP butterfly inside each 16-lane row (quad_perm, row_half_mirror,
//    row_mirror) and four readlanes; every lane ends with identical bits and
//    the result is deterministic run to run.
//  * rstd = 1 / sqrt(sum / H + eps) with correctly rounded binary32 divide
//    and square root: it scales exactly under x -> 2^k x, and costs nothing
//    next to the row's memory traffic.
//  * The weight slice (and for RoPE each lane's table offsets) is loaded at
//    the start, in flight together with the row; one workgroup per 1-4 rows.
//  * x is loaded and y stored with the non-temporal hint (streamed once).
//  * RoPE pairs element i with i + head_dim/2.  With 8 elements per vector
//    both halves of a pair are whole vectors, head_dim/16 vectors apart, so
//    each lane loads a vector and its partner ("pair unit") and rotates in
//    registers: no cross-lane exchange.  The two load instructions of a pair
//    unit cover complementary halves of the same cache lines and are in
//    flight together.  cos/sin rows (head_dim/2 floats per position) are read
//    through L2; lanes that share a table slice issue the same address.
//  * Output: binary32 -> bf16 round-to-nearest-even via v_cvt_pk_bf16_f32.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "ltxnorm.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kElemsPerVec = 8;       // bf16 values per 16-byte vector
constexpr int kMaxVecPerLane = 8;     // register budget for one row slice
constexpr int kMaxWavesPerRow = 16;   // 1024-thread workgroup
constexpr int64_t kMaxGrid = 1 << 30; // rows beyond grid * rows-per-block loop
constexpr uint32_t kOnesPair = 0x3F803F80u;  // two bf16 1.0

static_assert(LTXNORM_MAX_HIDDEN == kMaxWavesPerRow * kWave * kMaxVecPerLane * kElemsPerVec,
              "cap must match the largest register-resident row");

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

// bf16 is the upper half of a binary32: widening is exact.  The element at
// the lower address sits in the low 16 bits of each 32-bit word.
__device__ __forceinline__ void widen8(const u32x4 v, float f[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(v[i] << 16);
        f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
}

// Round 8 binary32 values to bf16 (nearest, ties to even; NaN stays NaN).
__device__ __forceinline__ u32x4 narrow8(const float f[8]) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f32x2 p = {f[2 * i], f[2 * i + 1]};
        r[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
    }
    return r;
}

// Keep a packed bf16x8 register value opaque to the optimiser, so that it
// is widened where it is used and lives in 4 VGPRs rather than 8.  Without
// this, loop-invariant code motion widens the weight once outside the row
// loop, and common-subexpression elimination keeps the widened row alive
// across the reduction; either doubles the register footprint and halves
// occupancy.  Emits no instruction.
__device__ __forceinline__ void keep_packed(u32x4& v) { asm volatile("" : "+v"(v)); }

// x is read once and y written once: stream both past the caches with the
// non-temporal hint (measured ~3% more HBM throughput than plain accesses on
// a 50/50 read/write stream).  Weights and rotation tables, which every row
// reuses, use ordinary cached loads.
__device__ __forceinline__ u32x4 load_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_stream(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

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

struct RmsArgs {
    uint16_t* out;
    const uint16_t* x;
    const uint16_t* w;
    int64_t rows;
    int32_t nvec;     // hidden / 8
    float hidden_f;
    float eps;
};

// ---------------------------------------------------------------------------
// RMSNorm: VPL vectors per lane, WPR wavefronts per row.  FULL means every
// lane's every slot is inside the row (no masking).
// ---------------------------------------------------------------------------
template <int VPL, int WPR, bool FULL>
__global__ void __launch_bounds__(Layout<WPR>::kThreads)
rmsnorm_kernel(const RmsArgs a) {
    constexpr int RPB = Layout<WPR>::kRowsPerBlock;
    constexpr int L = Layout<WPR>::kLanesPerRow;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform: scalar row math
    const int slot = wave / WPR;
    const int wave_in_row = wave % WPR;
    const int t = wave_in_row * kWave + (threadIdx.x & (kWave - 1));

    u32x4 wv[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int v = k * L + t;
        const bool in = FULL || v < a.nvec;
        wv[k] = (a.w != nullptr && in) ? reinterpret_cast<const u32x4*>(a.w)[v]
                                        : u32x4{kOnesPair, kOnesPair, kOnesPair, kOnesPair};
    }

    int parity = 0;
    for (int64_t base = (int64_t)blockIdx.x * RPB; base < a.rows;
         base += (int64_t)gridDim.x * RPB, parity ^= 1) {
        const int64_t row = base + slot;
        const bool active = row < a.rows;
        if (WPR == 1 && !active) continue;  // wave-uniform; no barrier at WPR 1
        const u32x4* xr = reinterpret_cast<const u32x4*>(a.x) + row * a.nvec;
        u32x4* yr = reinterpret_cast<u32x4*>(a.out) + row * a.nvec;

        u32x4 xv[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = k * L + t;
            const bool in = (FULL || v < a.nvec) && (WPR == 1 || active);
            xv[k] = in ? load_stream(xr + v) : u32x4{0u, 0u, 0u, 0u};
        }

        float part = 0.0f;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            float f[8];
            widen8(xv[k], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) part = fmaf(f[e], f[e], part);
        }
        const float rstd = rstd_of(row_sum<WPR>(part, slot, wave_in_row, parity), a.hidden_f, a.eps);

#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = k * L + t;
            const bool in = (FULL || v < a.nvec) && (WPR == 1 || active);
            float f[8], g[8];
            keep_packed(xv[k]);
            widen8(xv[k], f);
            keep_packed(wv[k]);
            widen8(wv[k], g);
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = (f[e] * rstd) * g[e];
            if (in) store_stream(yr + v, narrow8(f));
        }
    }
}

struct RopeArgs {
    uint16_t* out;
    const uint16_t* x;
    const uint16_t* w;
    const float* cos_tab;
    const float* sin_tab;
    int64_t rows;
    int64_t seq_len;
    int32_t nvec;      // hidden / 8
    int32_t nunits;    // hidden / 16: pair units per row
    int32_t unit_per_head;  // head_dim / 16
    int32_t half;      // head_dim / 2: floats per table row
    float hidden_f;
    float eps;
};

// ---------------------------------------------------------------------------
// RMSNorm + rotate-half RoPE: UPL pair units per lane (2 vectors each).
// Unit u covers head h = u / (d/16), quarter q = u % (d/16): vectors
// h*(d/8) + q (first half of the head) and that + d/16 (second half), and
// table floats [8q, 8q + 8) of the row's position.
// ---------------------------------------------------------------------------
template <int UPL, int WPR, bool FULL>
__global__ void __launch_bounds__(Layout<WPR>::kThreads)
rmsnorm_rope_kernel(const RopeArgs a) {
    constexpr int RPB = Layout<WPR>::kRowsPerBlock;
    constexpr int L = Layout<WPR>::kLanesPerRow;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform: scalar row math
    const int slot = wave / WPR;
    const int wave_in_row = wave % WPR;
    const int t = wave_in_row * kWave + (threadIdx.x & (kWave - 1));

    int va[UPL], toff[UPL];
    bool uin[UPL];
    u32x4 wa[UPL], wb[UPL];
#pragma unroll
    for (int k = 0; k < UPL; ++k) {
        const int u = k * L + t;
        uin[k] = FULL || u < a.nunits;
        const int h = u / a.unit_per_head;
        const int q = u - h * a.unit_per_head;
        va[k] = h * 2 * a.unit_per_head + q;
        toff[k] = q * 8;
        const u32x4 ones = {kOnesPair, kOnesPair, kOnesPair, kOnesPair};
        const bool lw = a.w != nullptr && uin[k];
        wa[k] = lw ? reinterpret_cast<const u32x4*>(a.w)[va[k]] : ones;
        wb[k] = lw ? reinterpret_cast<const u32x4*>(a.w)[va[k] + a.unit_per_head] : ones;
    }

    int parity = 0;
    for (int64_t base = (int64_t)blockIdx.x * RPB; base < a.rows;
         base += (int64_t)gridDim.x * RPB, parity ^= 1) {
        const int64_t row = base + slot;
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
            xb[k] = in ? load_stream(xr + va[k] + a.unit_per_head) : z;
        }

        float part = 0.0f;
#pragma unroll
        for (int k = 0; k < UPL; ++k) {
            float f[8];
            widen8(xa[k], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) part = fmaf(f[e], f[e], part);
            widen8(xb[k], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) part = fmaf(f[e], f[e], part);
        }
        const float rstd = rstd_of(row_sum<WPR>(part, slot, wave_in_row, parity), a.hidden_f, a.eps);

        // The table slices are L2-resident (every head and batch row shares
        // them); loading them only now keeps 16 VGPRs per pair unit free
        // while the row's own loads are in flight.
#pragma unroll
        for (int k = 0; k < UPL; ++k) {
            const bool in = uin[k] && (WPR == 1 || active);
            const f32x4 zf = {0.f, 0.f, 0.f, 0.f};
            const f32x4* cp = reinterpret_cast<const f32x4*>(crow + toff[k]);
            const f32x4* sp = reinterpret_cast<const f32x4*>(srow + toff[k]);
            const f32x4 c0 = in ? cp[0] : zf, c1 = in ? cp[1] : zf;
            const f32x4 s0 = in ? sp[0] : zf, s1 = in ? sp[1] : zf;
            float ya[8], yb[8], g[8];
            keep_packed(xa[k]);
            keep_packed(xb[k]);
            keep_packed(wa[k]);
            keep_packed(wb[k]);
            widen8(xa[k], ya);
            widen8(wa[k], g);
#pragma unroll
            for (int e = 0; e < 8; ++e) ya[e] = (ya[e] * rstd) * g[e];
            widen8(xb[k], yb);
            widen8(wb[k], g);
#pragma unroll
            for (int e = 0; e < 8; ++e) yb[e] = (yb[e] * rstd) * g[e];
            const float c[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
            const float s[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
            float o1[8], o2[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                o1[e] = ya[e] * c[e] - yb[e] * s[e];
                o2[e] = yb[e] * c[e] + ya[e] * s[e];
            }
            if (in) {
                store_stream(yr + va[k], narrow8(o1));
                store_stream(yr + va[k] + a.unit_per_head, narrow8(o2));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// RMSNorm + rotate-half RoPE with the RMSNorm lane layout, for head_dim a
// power of two from 16 to 512.  Lane t holds vectors k*L + t (full 1 KiB
// lines per load instruction).  With P = head_dim / 16 vectors per half
// head, the partner of vector v is v ^ P: the same slot of lane t ^ P in the
// same wavefront.  Each lane normalises its own vector and fetches the
// partner's normalised binary32 values with ds_bpermute (exchanging the
// finished values rather than raw x halves the VALU work per vector, which
// matters because with one row per wavefront the whole grid is resident and
// compute is not hidden behind later loads).  A lane's half (bit P of t) and
// its table slice (floats 8 * (t mod P) .. + 8) do not depend on the slot, so
// each lane reads 8 cos and 8 sin values per row.
// ---------------------------------------------------------------------------
template <int VPL, int WPR, bool FULL>
__global__ void __launch_bounds__(Layout<WPR>::kThreads)
rmsnorm_rope_xor_kernel(const RopeArgs a) {
    constexpr int RPB = Layout<WPR>::kRowsPerBlock;
    constexpr int L = Layout<WPR>::kLanesPerRow;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform: scalar row math
    const int slot = wave / WPR;
    const int wave_in_row = wave % WPR;
    const int lane = threadIdx.x & (kWave - 1);
    const int t = wave_in_row * kWave + lane;
    const int P = a.unit_per_head;
    const int src = ((lane ^ P) & (kWave - 1)) << 2;  // ds_bpermute byte address
    const float sgn = (t & P) ? 1.0f : -1.0f;  // second half adds, first subtracts
    const int toff = (t & (P - 1)) * 8;

    u32x4 wv[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int v = k * L + t;
        const bool in = FULL || v < a.nvec;
        const u32x4 ones = {kOnesPair, kOnesPair, kOnesPair, kOnesPair};
        wv[k] = (a.w != nullptr && in) ? reinterpret_cast<const u32x4*>(a.w)[v] : ones;
    }

    int parity = 0;
    for (int64_t base = (int64_t)blockIdx.x * RPB; base < a.rows;
         base += (int64_t)gridDim.x * RPB, parity ^= 1) {
        const int64_t row = base + slot;
        const bool active = row < a.rows;
        if (WPR == 1 && !active) continue;
        const int64_t pos = active ? row % a.seq_len : 0;
        const u32x4* xr = reinterpret_cast<const u32x4*>(a.x) + row * a.nvec;
        u32x4* yr = reinterpret_cast<u32x4*>(a.out) + row * a.nvec;

        u32x4 xv[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = k * L + t;
            const bool in = (FULL || v < a.nvec) && (WPR == 1 || active);
            xv[k] = in ? load_stream(xr + v) : u32x4{0u, 0u, 0u, 0u};
        }
        float part = 0.0f;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            float f[8];
            widen8(xv[k], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) part = fmaf(f[e], f[e], part);
        }
        const float rstd = rstd_of(row_sum<WPR>(part, slot, wave_in_row, parity), a.hidden_f, a.eps);

        const f32x4* cp = reinterpret_cast<const f32x4*>(a.cos_tab + pos * a.half + toff);
        const f32x4* sp = reinterpret_cast<const f32x4*>(a.sin_tab + pos * a.half + toff);
        const f32x4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
        const float c[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
        // the partner term enters with -sin in the first half, +sin in the second
        const float ss[8] = {sgn * s0[0], sgn * s0[1], sgn * s0[2], sgn * s0[3],
                             sgn * s1[0], sgn * s1[1], sgn * s1[2], sgn * s1[3]};
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = k * L + t;
            const bool in = (FULL || v < a.nvec) && (WPR == 1 || active);
            keep_packed(xv[k]);
            keep_packed(wv[k]);
            float own[8], g[8], par[8], o[8];
            widen8(xv[k], own);
            widen8(wv[k], g);
#pragma unroll
            for (int e = 0; e < 8; ++e) own[e] = (own[e] * rstd) * g[e];
            // the partner lane's normalised values, exact binary32 bits
#pragma unroll
            for (int e = 0; e < 8; ++e)
                par[e] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, own[e])));
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = own[e] * c[e] + par[e] * ss[e];
            if (in) store_stream(yr + v, narrow8(o));
        }
    }
}

// ---------------------------------------------------------------------------
// RMSNorm + interleaved RoPE: adjacent pairs (2i, 2i + 1) of each head turn
// by table column i.  A pair is one 32-bit word of a bf16x8 vector, so the
// RMSNorm lane layout needs no exchange at all; vector v of a row covers
// pairs 4 * (v mod (head_dim / 8)) .. + 4 of its head, i.e. one float4 of cos
// and one of sin.  head_dim must be a multiple of 8 (vectors never straddle
// heads).
// ---------------------------------------------------------------------------
template <int VPL, int WPR, bool FULL, bool SHARED>
__global__ void __launch_bounds__(Layout<WPR>::kThreads)
rmsnorm_rope_interleaved_kernel(const RopeArgs a) {
    constexpr int RPB = Layout<WPR>::kRowsPerBlock;
    constexpr int L = Layout<WPR>::kLanesPerRow;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform: scalar row math
    const int slot = wave / WPR;
    const int wave_in_row = wave % WPR;
    const int t = wave_in_row * kWave + (threadIdx.x & (kWave - 1));
    const int vph = a.half / 4;  // vectors per head = head_dim / 8

    u32x4 wv[VPL];
    int toff[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int v = k * L + t;
        const bool in = FULL || v < a.nvec;
        const u32x4 ones = {kOnesPair, kOnesPair, kOnesPair, kOnesPair};
        wv[k] = (a.w != nullptr && in) ? reinterpret_cast<const u32x4*>(a.w)[v] : ones;
        toff[k] = (v % vph) * 4;
    }

    int parity = 0;
    for (int64_t base = (int64_t)blockIdx.x * RPB; base < a.rows;
         base += (int64_t)gridDim.x * RPB, parity ^= 1) {
        const int64_t row = base + slot;
        const bool active = row < a.rows;
        if (WPR == 1 && !active) continue;
        const int64_t pos = active ? row % a.seq_len : 0;
        const u32x4* xr = reinterpret_cast<const u32x4*>(a.x) + row * a.nvec;
        u32x4* yr = reinterpret_cast<u32x4*>(a.out) + row * a.nvec;

        u32x4 xv[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = k * L + t;
            const bool in = (FULL || v < a.nvec) && (WPR == 1 || active);
            xv[k] = in ? load_stream(xr + v) : u32x4{0u, 0u, 0u, 0u};
        }
        float part = 0.0f;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            float f[8];
            widen8(xv[k], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) part = fmaf(f[e], f[e], part);
        }
        const float rstd = rstd_of(row_sum<WPR>(part, slot, wave_in_row, parity), a.hidden_f, a.eps);

        // SHARED: head_dim / 8 divides the lanes per row (every power-of-two
        // head_dim up to 512), so all slots of a lane share one table offset
        // and the row needs a single float4 of cos and of sin per lane.
        const float* crow = a.cos_tab + pos * a.half;
        const float* srow = a.sin_tab + pos * a.half;
        f32x4 c = *reinterpret_cast<const f32x4*>(crow + toff[0]);
        f32x4 sn = *reinterpret_cast<const f32x4*>(srow + toff[0]);
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = k * L + t;
            const bool in = (FULL || v < a.nvec) && (WPR == 1 || active);
            if (!SHARED && k > 0) {
                c = *reinterpret_cast<const f32x4*>(crow + toff[k]);
                sn = *reinterpret_cast<const f32x4*>(srow + toff[k]);
            }
            keep_packed(xv[k]);
            keep_packed(wv[k]);
            float y[8], g[8], o[8];
            widen8(xv[k], y);
            widen8(wv[k], g);
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = (y[e] * rstd) * g[e];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                o[2 * j] = y[2 * j] * c[j] - y[2 * j + 1] * sn[j];
                o[2 * j + 1] = y[2 * j + 1] * c[j] + y[2 * j] * sn[j];
            }
            if (in) store_stream(yr + v, narrow8(o));
        }
    }
}

struct AdaArgs {
    uint16_t* out;
    const uint16_t* x;
    const uint16_t* w;
    const uint16_t* scale;  // [samples, hidden] or null (zeros)
    const uint16_t* shift;  // [samples, hidden] or null (zeros)
    int64_t rows;
    int64_t rows_per_sample;
    int32_t nvec;
    float hidden_f;
    float eps;
};

// ---------------------------------------------------------------------------
// RMSNorm with per-sample adaptive modulation (AdaLN, as in DiT blocks):
// y = ((x * rstd) * w) * (1 + scale[b]) + shift[b], b = row / rows_per_sample,
// all in binary32 and rounded once.  The RMSNorm layout and reduction; the
// modulation rows are shared by every row of a sample and come from L2 after
// the reduction.  A null scale reads as +0 (factor exactly 1) and a null
// shift as -0 (x + -0 == x for every x, signed zeros included), so with both
// null the result equals plain RMSNorm bit for bit.
// ---------------------------------------------------------------------------
template <int VPL, int WPR, bool FULL>
__global__ void __launch_bounds__(Layout<WPR>::kThreads)
rmsnorm_adaln_kernel(const AdaArgs a) {
    constexpr int RPB = Layout<WPR>::kRowsPerBlock;
    constexpr int L = Layout<WPR>::kLanesPerRow;
    constexpr uint32_t kNegZeroPair = 0x80008000u;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform: scalar row math
    const int slot = wave / WPR;
    const int wave_in_row = wave % WPR;
    const int t = wave_in_row * kWave + (threadIdx.x & (kWave - 1));

    u32x4 wv[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int v = k * L + t;
        const bool in = FULL || v < a.nvec;
        wv[k] = (a.w != nullptr && in) ? reinterpret_cast<const u32x4*>(a.w)[v]
                                        : u32x4{kOnesPair, kOnesPair, kOnesPair, kOnesPair};
    }

    int parity = 0;
    for (int64_t base = (int64_t)blockIdx.x * RPB; base < a.rows;
         base += (int64_t)gridDim.x * RPB, parity ^= 1) {
        const int64_t row = base + slot;
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
            const int v = k * L + t;
            const bool in = (FULL || v < a.nvec) && (WPR == 1 || active);
            sv = (a.scale != nullptr && in) ? sr[v] : u32x4{0u, 0u, 0u, 0u};
            hv = (a.shift != nullptr && in)
                     ? hr[v]
                     : u32x4{kNegZeroPair, kNegZeroPair, kNegZeroPair, kNegZeroPair};
        };
        u32x4 xv[VPL], svv[VPL], hvv[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = k * L + t;
            const bool in = (FULL || v < a.nvec) && (WPR == 1 || active);
            xv[k] = in ? load_stream(xr + v) : u32x4{0u, 0u, 0u, 0u};
        }
        if constexpr (kEarly) {
#pragma unroll
            for (int k = 0; k < VPL; ++k) mod_rows(k, svv[k], hvv[k]);
        }
        float part = 0.0f;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            float f[8];
            widen8(xv[k], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) part = fmaf(f[e], f[e], part);
        }
        const float rstd = rstd_of(row_sum<WPR>(part, slot, wave_in_row, parity), a.hidden_f, a.eps);

#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = k * L + t;
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
            float f[8], g[8], sc[8], sh[8];
            widen8(xv[k], f);
            widen8(wv[k], g);
            widen8(sv, sc);
            widen8(hv, sh);
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = ((f[e] * rstd) * g[e]) * (1.0f + sc[e]) + sh[e];
            if (in) store_stream(yr + v, narrow8(f));
        }
    }
}

// ---------------------------------------------------------------------------
// Host side: validation, per-hidden dispatch, launch.
// ---------------------------------------------------------------------------

struct Plan {
    int wpr;    // wavefronts per row
    int per;    // vectors (RMSNorm) or pair units (RoPE) per lane
    bool full;  // no masking needed
};

// How a row is split.  `items` are 16-byte vectors (RMSNorm) or pair units of
// two vectors (RoPE).  A single wavefront takes the row while each lane holds
// at most `one_wave_max` items; longer rows are spread over enough
// wavefronts (up to 16) that each lane holds about `spread` items, and past
// 16 wavefronts the lanes take more, up to the register budget.  Measured at
// [16384 x 3072] (384 vectors per row): 3 wavefronts x 2 vectors reached
// 6.08 TB/s, 2 x 3 6.02, 1 x 6 5.98, 6 x 1 5.46; at hidden 2048 one
// wavefront x 4 vectors was best (6.11 TB/s) and 4 x 1 the worst.
Plan plan_for(int64_t items, int one_wave_max, int spread) {
    int wpr = 1;
    if (items > (int64_t)kWave * one_wave_max) {
        const int64_t w = (items + (int64_t)kWave * spread - 1) / ((int64_t)kWave * spread);
        wpr = (int)(w < kMaxWavesPerRow ? w : kMaxWavesPerRow);
    }
    const int64_t lanes = (int64_t)kWave * wpr;
    const int per = (int)((items + lanes - 1) / lanes);
    return Plan{wpr, per, items == (int64_t)per * lanes};
}

template <typename Args>
ltxnorm_status launch(const void* fn, int threads, int rows_per_block, int64_t rows, Args args,
                      hipStream_t stream) {
    // One workgroup per group of rows: a grid-stride loop capped at the
    // resident capacity measured 3-4% slower than letting the dispatcher
    // stream fresh workgroups, which keeps every CU busy to the last rows.
    const int64_t need = (rows + rows_per_block - 1) / rows_per_block;
    const unsigned grid = (unsigned)(need < kMaxGrid ? need : kMaxGrid);
    void* params[] = {&args};
    const hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(threads), params, 0, stream);
    return e == hipSuccess ? LTXNORM_OK : LTXNORM_ERR_HIP;
}

template <int WPR, int PER, bool FULL>
ltxnorm_status launch_rms(const RmsArgs& a, hipStream_t s) {
    return launch((const void*)&rmsnorm_kernel<PER, WPR, FULL>, Layout<WPR>::kThreads,
                  Layout<WPR>::kRowsPerBlock, a.rows, a, s);
}

template <int WPR, int PER, bool FULL>
ltxnorm_status launch_rope(const RopeArgs& a, hipStream_t s) {
    return launch((const void*)&rmsnorm_rope_kernel<PER, WPR, FULL>, Layout<WPR>::kThreads,
                  Layout<WPR>::kRowsPerBlock, a.rows, a, s);
}

template <int WPR, int PER, typename Args, typename L>
ltxnorm_status pick_full(const Plan& p, const Args& a, hipStream_t s, L launcher) {
    return p.full ? launcher.template go<WPR, PER, true>(a, s)
                  : launcher.template go<WPR, PER, false>(a, s);
}

struct RmsLauncher {
    template <int WPR, int PER, bool FULL>
    ltxnorm_status go(const RmsArgs& a, hipStream_t s) const { return launch_rms<WPR, PER, FULL>(a, s); }
};
struct RopeLauncher {
    template <int WPR, int PER, bool FULL>
    ltxnorm_status go(const RopeArgs& a, hipStream_t s) const { return launch_rope<WPR, PER, FULL>(a, s); }
};
struct AdaLauncher {
    template <int WPR, int PER, bool FULL>
    ltxnorm_status go(const AdaArgs& a, hipStream_t s) const {
        return launch((const void*)&rmsnorm_adaln_kernel<PER, WPR, FULL>, Layout<WPR>::kThreads,
                      Layout<WPR>::kRowsPerBlock, a.rows, a, s);
    }
};
template <bool SHARED>
struct RopeInterleavedLauncher {
    template <int WPR, int PER, bool FULL>
    ltxnorm_status go(const RopeArgs& a, hipStream_t s) const {
        return launch((const void*)&rmsnorm_rope_interleaved_kernel<PER, WPR, FULL, SHARED>,
                      Layout<WPR>::kThreads, Layout<WPR>::kRowsPerBlock, a.rows, a, s);
    }
};
struct RopeXorLauncher {
    template <int WPR, int PER, bool FULL>
    ltxnorm_status go(const RopeArgs& a, hipStream_t s) const {
        return launch((const void*)&rmsnorm_rope_xor_kernel<PER, WPR, FULL>, Layout<WPR>::kThreads,
                      Layout<WPR>::kRowsPerBlock, a.rows, a, s);
    }
};

template <int WPR, int LO, int HI, typename Args, typename L>
ltxnorm_status by_per(const Plan& p, const Args& a, hipStream_t s, L launcher) {
    if constexpr (LO > HI) {
        return LTXNORM_ERR_UNSUPPORTED;
    } else {
        if (p.per == LO) return pick_full<WPR, LO>(p, a, s, launcher);
        return by_per<WPR, LO + 1, HI>(p, a, s, launcher);
    }
}

// Plans that plan_for can produce: one wavefront with 1..ONE items per lane;
// 3..15 wavefronts with exactly SPREAD items per lane (2 wavefronts never
// occur: a row too long for one wavefront needs more than 2 * ONE / SPREAD);
// 16 wavefronts with SPREAD..MAXP items per lane.
template <int ONE, int SPREAD, int MAXP, typename Args, typename L>
ltxnorm_status by_plan(const Plan& p, const Args& a, hipStream_t s, L launcher) {
    switch (p.wpr) {
        case 1: return by_per<1, 1, ONE>(p, a, s, launcher);
        case 3: return by_per<3, SPREAD, SPREAD>(p, a, s, launcher);
        case 4: return by_per<4, SPREAD, SPREAD>(p, a, s, launcher);
        case 5: return by_per<5, SPREAD, SPREAD>(p, a, s, launcher);
        case 6: return by_per<6, SPREAD, SPREAD>(p, a, s, launcher);
        case 7: return by_per<7, SPREAD, SPREAD>(p, a, s, launcher);
        case 8: return by_per<8, SPREAD, SPREAD>(p, a, s, launcher);
        case 9: return by_per<9, SPREAD, SPREAD>(p, a, s, launcher);
        case 10: return by_per<10, SPREAD, SPREAD>(p, a, s, launcher);
        case 11: return by_per<11, SPREAD, SPREAD>(p, a, s, launcher);
        case 12: return by_per<12, SPREAD, SPREAD>(p, a, s, launcher);
        case 13: return by_per<13, SPREAD, SPREAD>(p, a, s, launcher);
        case 14: return by_per<14, SPREAD, SPREAD>(p, a, s, launcher);
        case 15: return by_per<15, SPREAD, SPREAD>(p, a, s, launcher);
        case 16: return by_per<16, SPREAD, MAXP>(p, a, s, launcher);
        default: return LTXNORM_ERR_UNSUPPORTED;
    }
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Half-open byte ranges [a, a + na) and [b, b + nb) overlap.
bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

// Checks shared by both entry points, in order: shape, scalar value, empty,
// pointers, alignment, aliasing.  Returns OK with *empty set when there is
// nothing to launch.
ltxnorm_status check_common(void* out, const void* x, const void* weight, int64_t rows,
                            int64_t hidden, float eps, bool* empty) {
    *empty = false;
    if (rows < 0 || hidden <= 0) return LTXNORM_ERR_SHAPE;
    if (hidden % kElemsPerVec != 0 || hidden > LTXNORM_MAX_HIDDEN) return LTXNORM_ERR_UNSUPPORTED;
    if (rows > INT64_MAX / (hidden * 2)) return LTXNORM_ERR_SHAPE;
    if (!std::isfinite(eps) || eps < 0.0f) return LTXNORM_ERR_VALUE;
    if (rows == 0) {
        *empty = true;
        return LTXNORM_OK;
    }
    if (out == nullptr || x == nullptr) return LTXNORM_ERR_NULL;
    if (misaligned(out) || misaligned(x) || (weight && misaligned(weight))) return LTXNORM_ERR_ALIGN;
    const int64_t nbytes = rows * hidden * 2;
    if (out != x && overlap(out, nbytes, x, nbytes)) return LTXNORM_ERR_ALIAS;
    if (weight && overlap(out, nbytes, weight, hidden * 2)) return LTXNORM_ERR_ALIAS;
    return LTXNORM_OK;
}

// Validation shared by the RoPE entry points; fills `a` when there is work.
ltxnorm_status check_rope(void* out, const void* x, const void* weight, const float* cos_tab,
                          const float* sin_tab, int64_t rows, int64_t hidden, int32_t heads,
                          int32_t head_dim, int64_t seq_len, float eps, int head_dim_multiple,
                          bool* empty, RopeArgs* a) {
    if (heads < 1 || head_dim < head_dim_multiple || head_dim % head_dim_multiple != 0 ||
        seq_len < 1 || (int64_t)heads * head_dim != hidden)
        return LTXNORM_ERR_SHAPE;
    if (seq_len > INT64_MAX / (head_dim * 4)) return LTXNORM_ERR_SHAPE;
    ltxnorm_status st = check_common(out, x, weight, rows, hidden, eps, empty);
    if (st != LTXNORM_OK || *empty) return st;
    if (cos_tab == nullptr || sin_tab == nullptr) return LTXNORM_ERR_NULL;
    if (misaligned(cos_tab) || misaligned(sin_tab)) return LTXNORM_ERR_ALIGN;
    const int64_t nbytes = rows * hidden * 2;
    const int64_t tbytes = seq_len * (head_dim / 2) * 4;
    if (overlap(out, nbytes, cos_tab, tbytes) || overlap(out, nbytes, sin_tab, tbytes))
        return LTXNORM_ERR_ALIAS;
    *a = RopeArgs{static_cast<uint16_t*>(out), static_cast<const uint16_t*>(x),
                  static_cast<const uint16_t*>(weight), cos_tab, sin_tab, rows, seq_len,
                  (int32_t)(hidden / kElemsPerVec), (int32_t)(hidden / (2 * kElemsPerVec)),
                  head_dim / 16, head_dim / 2, (float)hidden, eps};
    return LTXNORM_OK;
}

}  // namespace

extern "C" {

ltxnorm_status ltxnorm_rmsnorm_fwd(void* out, const void* x, const void* weight, int64_t rows,
                                   int64_t hidden, float eps, hipStream_t stream) {
    bool empty = false;
    ltxnorm_status st = check_common(out, x, weight, rows, hidden, eps, &empty);
    if (st != LTXNORM_OK || empty) return st;
    const int64_t nvec = hidden / kElemsPerVec;
    const Plan p = plan_for(nvec, 4, 2);
    const RmsArgs a{static_cast<uint16_t*>(out), static_cast<const uint16_t*>(x),
                    static_cast<const uint16_t*>(weight), rows, (int32_t)nvec, (float)hidden, eps};
    return by_plan<4, 2, kMaxVecPerLane>(p, a, stream, RmsLauncher{});
}


ltxnorm_status ltxnorm_rmsnorm_rope_fwd(void* out, const void* x, const void* weight,
                                        const float* cos_tab, const float* sin_tab, int64_t rows,
                                        int64_t hidden, int32_t heads, int32_t head_dim,
                                        int64_t seq_len, float eps, hipStream_t stream) {
    bool empty = false;
    RopeArgs a;
    ltxnorm_status st = check_rope(out, x, weight, cos_tab, sin_tab, rows, hidden, heads,
                                   head_dim, seq_len, eps, 16, &empty, &a);
    if (st != LTXNORM_OK || empty) return st;
    if ((head_dim & (head_dim - 1)) == 0 && head_dim <= 16 * 32) {
        // partner lanes lie within one wavefront: the coalesced layout
        const Plan p = plan_for(a.nvec, 4, 2);
        return by_plan<4, 2, kMaxVecPerLane>(p, a, stream, RopeXorLauncher{});
    }
    const Plan p = plan_for(a.nunits, 2, 1);
    return by_plan<2, 1, kMaxVecPerLane / 2>(p, a, stream, RopeLauncher{});
}

ltxnorm_status ltxnorm_rmsnorm_rope_interleaved_fwd(void* out, const void* x, const void* weight,
                                                    const float* cos_tab, const float* sin_tab,
                                                    int64_t rows, int64_t hidden, int32_t heads,
                                                    int32_t head_dim, int64_t seq_len, float eps,
                                                    hipStream_t stream) {
    bool empty = false;
    RopeArgs a;
    ltxnorm_status st = check_rope(out, x, weight, cos_tab, sin_tab, rows, hidden, heads,
                                   head_dim, seq_len, eps, 8, &empty, &a);
    if (st != LTXNORM_OK || empty) return st;
    const Plan p = plan_for(a.nvec, 4, 2);
    const int vph = head_dim / kElemsPerVec;
    if ((kWave * p.wpr) % vph == 0)
        return by_plan<4, 2, kMaxVecPerLane>(p, a, stream, RopeInterleavedLauncher<true>{});
    return by_plan<4, 2, kMaxVecPerLane>(p, a, stream, RopeInterleavedLauncher<false>{});
}

ltxnorm_status ltxnorm_rmsnorm_adaln_fwd(void* out, const void* x, const void* weight,
                                         const void* scale, const void* shift, int64_t rows,
                                         int64_t hidden, int64_t rows_per_sample, float eps,
                                         hipStream_t stream) {
    if (rows_per_sample < 1) return LTXNORM_ERR_SHAPE;
    bool empty = false;
    ltxnorm_status st = check_common(out, x, weight, rows, hidden, eps, &empty);
    if (st != LTXNORM_OK || empty) return st;
    if ((scale && misaligned(scale)) || (shift && misaligned(shift))) return LTXNORM_ERR_ALIGN;
    const int64_t samples = (rows + rows_per_sample - 1) / rows_per_sample;
    const int64_t nbytes = rows * hidden * 2;
    const int64_t mbytes = samples * hidden * 2;
    if ((scale && overlap(out, nbytes, scale, mbytes)) || (shift && overlap(out, nbytes, shift, mbytes)))
        return LTXNORM_ERR_ALIAS;
    const int64_t nvec = hidden / kElemsPerVec;
    const AdaArgs a{static_cast<uint16_t*>(out), static_cast<const uint16_t*>(x),
                    static_cast<const uint16_t*>(weight), static_cast<const uint16_t*>(scale),
                    static_cast<const uint16_t*>(shift), rows, rows_per_sample, (int32_t)nvec,
                    (float)hidden, eps};
    const Plan p = plan_for(nvec, 4, 2);
    return by_plan<4, 2, kMaxVecPerLane>(p, a, stream, AdaLauncher{});
}

const char* ltxnorm_status_str(ltxnorm_status s) {
    switch (s) {
        case LTXNORM_OK: return "ok";
        case LTXNORM_ERR_NULL: return "a required pointer is NULL";
        case LTXNORM_ERR_SHAPE: return "invalid shape (rows, hidden, heads, head_dim or seq_len)";
        case LTXNORM_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case LTXNORM_ERR_UNSUPPORTED: return "hidden must be a multiple of 8 and at most 65536";
        case LTXNORM_ERR_ALIAS: return "out overlaps an input other than exactly x";
        case LTXNORM_ERR_VALUE: return "eps must be finite and non-negative";
        case LTXNORM_ERR_HIP: return "the HIP runtime rejected the kernel launch";
    }
    return "unknown ltxnorm status";
}

int ltxnorm_version(void) { return LTXNORM_ABI_VERSION; }

}  // extern "C"
