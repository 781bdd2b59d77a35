// ltxnorm_general.h -- kernels for rows of any length: hidden sizes that are
// not a whole number of 16-byte vectors, head sizes the vector kernels cannot
// pair, and rows longer than the register budget.  Same operations and the
// same arithmetic as ltxnorm_kernels.h (RMSNorm, Hugging Face cuda-kernels
// skill page, "Kernel-Specific Guidelines", RMSNorm; rms_norm_rope, LTX-2
// ltx-kernels README, introduction; AdaLN, skill page, "Kernel-Specific
// Guidelines", AdaLN); not a public header.
//
// Layout.  When hidden is not a multiple of kEpv, row r starts part-way into
// a 16-byte vector.  The lanes therefore walk the row in the global vector
// grid: lane t of the row takes vectors k * L + t counted from the vector that
// holds the row's first element, so every access inside the row is still an
// aligned 16-byte vector and only the row's first and last vectors, shared
// with the neighbouring rows, are read and written element by element (and
// only the row's own elements).  The weight (and the modulation rows) are then
// misaligned by a row-dependent number of elements: a lane reads the two
// aligned vectors that straddle its window and funnel-shifts them, or element
// by element at the ends of the array.
//
//  * rmsnorm_general_kernel: one pass, the row in registers (as the vector
//    kernels): RMSNorm, AdaLN, and interleaved RoPE, whose pairs
//    (2i, 2i + 1) never straddle a vector because hidden = heads * head_dim
//    is even.  Rotate-half RoPE pairs i with i + head_dim/2, anywhere in the
//    row: the normalised binary32 row goes through LDS (one row of floats per
//    row slot), so in-place calls stay correct.
//  * rmsnorm_long_kernel: rows beyond the register budget.  One 1024-thread
//    workgroup per row reads the row twice: once for the sum of squares, once
//    to normalise and store.  Rotate-half pairs are handled as units of one
//    window of the first half and its partner window in the second half, each
//    read and written by one thread, so that in-place calls stay correct.
#pragma once

#include "ltxnorm_device.h"

namespace ltxnorm_detail {
namespace {

// Operation of a general kernel.
enum class GOp { kRms, kAda, kRopeHalf, kRopeIl };

constexpr int kLongThreads = 1024;                  // one row per workgroup
constexpr int kLongWaves = kLongThreads / kWave;
// vectors in flight per thread (fp32 rows keep two: four spill at 1024 threads)
template <typename IO>
constexpr int kLongUnroll = IO::kEpv == 8 ? 4 : 2;

// Elements base[start + i], i < kEpv, read one by one where lo <= start + i
// < hi, zero elsewhere, packed as one 16-byte vector.
template <typename IO>
__device__ __forceinline__ u32x4 load_elems(const void* base, int64_t start, int64_t lo, int64_t hi) {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if constexpr (IO::kEpv == 8) {
        const uint16_t* p = static_cast<const uint16_t*>(base);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t e = start + i;
            if (e >= lo && e < hi) w[i / 2] |= (uint32_t)p[e] << (16 * (i & 1));
        }
    } else {
        const uint32_t* p = static_cast<const uint32_t*>(base);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t e = start + i;
            if (e >= lo && e < hi) w[i] = p[e];
        }
    }
    return u32x4{w[0], w[1], w[2], w[3]};
}

// Store the elements of v whose index start + i lies in [lo, hi).
template <typename IO>
__device__ __forceinline__ void store_elems(void* base, int64_t start, const u32x4 v, int64_t lo,
                                            int64_t hi) {
    const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
    if constexpr (IO::kEpv == 8) {
        uint16_t* p = static_cast<uint16_t*>(base);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t e = start + i;
            if (e >= lo && e < hi) p[e] = (uint16_t)(w[i / 2] >> (16 * (i & 1)));
        }
    } else {
        uint32_t* p = static_cast<uint32_t*>(base);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t e = start + i;
            if (e >= lo && e < hi) p[e] = w[i];
        }
    }
}

// Elements F .. F + kEpv - 1 of the 2 kEpv elements in words W[0..7].
template <int ELEM_BYTES, int F>
__device__ __forceinline__ u32x4 take(const uint32_t* W) {
    constexpr int kByte = F * ELEM_BYTES;
    constexpr int o = kByte / 4;
    u32x4 r;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        if constexpr (kByte % 4 == 0)
            r[m] = W[o + m];
        else
            r[m] = (W[o + m] >> 16) | (W[o + m + 1] << 16);
    }
    return r;
}

template <typename IO, int F = 1>
__device__ __forceinline__ u32x4 take_at(const uint32_t* W, int f) {
    if constexpr (F >= IO::kEpv) {
        return u32x4{W[0], W[1], W[2], W[3]};
    } else {
        if (f == F) return take<16 / IO::kEpv, F>(W);
        return take_at<IO, F + 1>(W, f);
    }
}

// Elements base[start .. start + kEpv) of an array of n elements, with
// f = start mod kEpv (the same for every lane of a row, so the selection
// below is uniform).  Reads only inside [0, n); elements outside are zero.
template <typename IO>
__device__ __forceinline__ u32x4 load_window(const void* base, int64_t start, int f, int64_t n) {
    constexpr int E = IO::kEpv;
    const u32x4* v = static_cast<const u32x4*>(base);
    const int64_t c = (start - f) / E;  // exact: start - f is a multiple of E
    if (f == 0) {
        if (start >= 0 && start + E <= n) return v[c];
    } else if (c >= 0 && (c + 2) * E <= n) {
        const u32x4 lo = v[c], hi = v[c + 1];
        const uint32_t W[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return take_at<IO>(W, f);
    }
    return load_elems<IO>(base, start, 0, n);
}

// The row's vector q (row-relative elements j0 .. j0 + kEpv, j0 = q kEpv -
// first): whole vectors with the streaming load, the row's end vectors
// element by element (its own elements only).
template <typename IO>
__device__ __forceinline__ u32x4 load_row_vec(const void* x, int64_t s, int64_t g0, int q, int j0,
                                              int hidden) {
    constexpr int E = IO::kEpv;
    if (j0 >= 0 && j0 + E <= hidden) return load_stream(static_cast<const u32x4*>(x) + g0 + q);
    return load_elems<IO>(x, s + j0, s, s + hidden);
}

template <typename IO>
__device__ __forceinline__ void store_row_vec(void* out, int64_t s, int64_t g0, int q, int j0,
                                              int hidden, const u32x4 v) {
    constexpr int E = IO::kEpv;
    if (j0 >= 0 && j0 + E <= hidden)
        store_stream(static_cast<u32x4*>(out) + g0 + q, v);
    else
        store_elems<IO>(out, s + j0, v, s, s + hidden);
}

// Normalise one vector of the row in place: f = (x * rstd) * w, plus the
// AdaLN modulation; fw (fm) = start of the weight (modulation) window mod
// kEpv.  msample = element offset of the row's modulation row.
template <typename IO, GOp OP>
__device__ __forceinline__ void normalise_vec(const KArgs& a, const u32x4 xv, int j0, int fw,
                                              int64_t msample, int fm, float rstd, float* f) {
    constexpr int E = IO::kEpv;
    float g[E];
    IO::widen(xv, f);
    const u32x4 wv = a.w ? load_window<IO>(a.w, j0, fw, a.hidden) : splat(IO::kOne);
    IO::widen(wv, g);
#pragma unroll
    for (int e = 0; e < E; ++e) f[e] = (f[e] * rstd) * g[e];
    if constexpr (OP == GOp::kAda) {
        float sc[E], sh[E];
        const u32x4 sv = a.scale ? load_window<IO>(a.scale, msample + j0, fm, a.mod_elems)
                                 : u32x4{0u, 0u, 0u, 0u};
        const u32x4 hv = a.shift ? load_window<IO>(a.shift, msample + j0, fm, a.mod_elems)
                                 : splat(IO::kNegZero);
        IO::widen(sv, sc);
        IO::widen(hv, sh);
#pragma unroll
        for (int e = 0; e < E; ++e) f[e] = f[e] * (1.0f + sc[e]) + sh[e];
    }
}

// Interleaved RoPE on one normalised vector: pairs (2i, 2i + 1) of a head
// turn by table column i.  j0 is even (hidden even, rows start at even
// element offsets), so pairs never straddle vectors or the row's ends.
template <int E>
__device__ __forceinline__ void rope_interleaved_vec(const KArgs& a, const float* crow,
                                                     const float* srow, int j0, const float* f,
                                                     float* o) {
    const int d = a.head_dim;
    int hd = ((j0 % d) + d) % d;  // position of element 0 in its head
#pragma unroll
    for (int e = 0; e < E; e += 2) {
        const int j = j0 + e;
        if (j >= 0 && j < a.hidden) {
            const float c = crow[hd / 2], sn = srow[hd / 2];
            o[e] = f[e] * c - f[e + 1] * sn;
            o[e + 1] = f[e + 1] * c + f[e] * sn;
        } else {
            o[e] = o[e + 1] = 0.0f;
        }
        hd += 2;
        if (hd == d) hd = 0;
    }
}

// ---------------------------------------------------------------------------
// One-pass kernel for any hidden size that fits the register budget.
// VPL vectors per lane, WPR wavefronts per row, Layout<WPR> rows per block.
// Rotate-half needs Layout<WPR>::kRowsPerBlock * hidden floats of dynamic LDS.
// ---------------------------------------------------------------------------
template <typename IO, GOp OP, int VPL, int WPR>
__global__ void __launch_bounds__(Layout<WPR>::kThreads)
rmsnorm_general_kernel(const KArgs a) {
    constexpr int RPB = Layout<WPR>::kRowsPerBlock;
    constexpr int L = Layout<WPR>::kLanesPerRow;
    constexpr int E = IO::kEpv;
    constexpr bool kExchange = OP == GOp::kRopeHalf;
    extern __shared__ float ybuf[];
    const Lane<WPR> ln;
    const int H = a.hidden;

    int parity = 0;
    for (int64_t base = (int64_t)blockIdx.x * RPB; base < a.rows;
         base += (int64_t)gridDim.x * RPB, parity ^= 1) {
        const int64_t row = base + ln.slot;
        const bool active = row < a.rows;
        // rotate-half reaches block barriers: every wavefront stays
        if (!kExchange && WPR == 1 && !active) continue;
        const int64_t s = active ? row * H : 0;      // the row's first element
        const int first = (int)(s & (E - 1));        // its place in its vector
        const int64_t g0 = s / E;                    // that vector
        const int nch = active ? (first + H + E - 1) / E : 0;  // vectors the row touches
        const int fw = (-first) & (E - 1);           // weight window offset mod E

        u32x4 xv[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int q = k * L + ln.t;
            xv[k] = q < nch ? load_row_vec<IO>(a.x, s, g0, q, q * E - first, H) : u32x4{0u, 0u, 0u, 0u};
        }
        const float part = sum_squares<IO, VPL>(xv);
        const float rstd = rstd_of(row_sum<WPR>(part, ln.slot, ln.wave_in_row, parity), a.hidden_f, a.eps);

        if constexpr (kExchange) {
            float* yrow = ybuf + ln.slot * H;
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                const int q = k * L + ln.t;
                if (q < nch) {
                    const int j0 = q * E - first;
                    float f[E];
                    keep_packed(xv[k]);
                    normalise_vec<IO, OP>(a, xv[k], j0, fw, 0, 0, rstd, f);
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        if (j0 + e >= 0 && j0 + e < H) yrow[j0 + e] = f[e];
                }
            }
            __syncthreads();
            const int64_t pos = active ? row % a.seq_len : 0;
            const float* crow = a.cos_tab + pos * a.half;
            const float* srow = a.sin_tab + pos * a.half;
            const int d = a.head_dim, half = a.half;
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                const int q = k * L + ln.t;
                if (q < nch) {
                    const int j0 = q * E - first;
                    int hd = ((j0 % d) + d) % d;
                    float o[E];
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const int j = j0 + e;
                        if (j >= 0 && j < H) {
                            // first half: a c - b s; second half: b c + a s
                            const bool lo = hd < half;
                            const int col = lo ? hd : hd - half;
                            const float c = crow[col], sn = srow[col];
                            const float par = yrow[lo ? j + half : j - half];
                            o[e] = yrow[j] * c + par * (lo ? -sn : sn);
                        } else {
                            o[e] = 0.0f;
                        }
                        if (++hd == d) hd = 0;
                    }
                    store_row_vec<IO>(a.out, s, g0, q, j0, H, IO::narrow(o));
                }
            }
            __syncthreads();  // the next row reuses the LDS row
        } else {
            const int64_t msample = OP == GOp::kAda && active ? (row / a.rows_per_sample) * H : 0;
            const int fm = (int)((msample - first) & (E - 1));
            const float* crow = nullptr;
            const float* srow = nullptr;
            if constexpr (OP == GOp::kRopeIl) {
                const int64_t pos = active ? row % a.seq_len : 0;
                crow = a.cos_tab + pos * a.half;
                srow = a.sin_tab + pos * a.half;
            }
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                const int q = k * L + ln.t;
                if (q < nch) {
                    const int j0 = q * E - first;
                    float f[E];
                    keep_packed(xv[k]);
                    normalise_vec<IO, OP>(a, xv[k], j0, fw, msample, fm, rstd, f);
                    if constexpr (OP == GOp::kRopeIl) {
                        float o[E];
                        rope_interleaved_vec<E>(a, crow, srow, j0, f, o);
                        store_row_vec<IO>(a.out, s, g0, q, j0, H, IO::narrow(o));
                    } else {
                        store_row_vec<IO>(a.out, s, g0, q, j0, H, IO::narrow(f));
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Two-pass kernel for rows beyond the register budget: one row per
// 1024-thread workgroup.  Pass 1 streams the row for its sum of squares
// (cached loads, so that pass 2 finds much of the row in L2 or the
// Infinity Cache); pass 2 reads it again, normalises and stores.
// ---------------------------------------------------------------------------
template <typename IO, GOp OP>
__global__ void __launch_bounds__(kLongThreads)
rmsnorm_long_kernel(const KArgs a) {
    constexpr int E = IO::kEpv;
    constexpr int T = kLongThreads;
    constexpr int U = kLongUnroll<IO>;
    __shared__ float partials[2][kLongWaves];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int H = a.hidden;

    int parity = 0;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x, parity ^= 1) {
        const int64_t s = row * H;
        const int first = (int)(s & (E - 1));
        const int64_t g0 = s / E;
        const int nch = (first + H + E - 1) / E;
        const int fw = (-first) & (E - 1);

        // pass 1: sum of squares, U vectors in flight per thread
        float part = 0.0f;
        for (int q0 = 0; q0 < nch; q0 += T * U) {
            u32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int q = q0 + u * T + tid;
                const int j0 = q * E - first;
                if (q >= nch)
                    v[u] = u32x4{0u, 0u, 0u, 0u};
                else if (j0 >= 0 && j0 + E <= H)
                    v[u] = static_cast<const u32x4*>(a.x)[g0 + q];
                else
                    v[u] = load_elems<IO>(a.x, s + j0, s, s + H);
            }
            part += sum_squares<IO, U>(v);
        }
        float sum = wave_sum(part);
        if ((tid & (kWave - 1)) == 0) partials[parity][wave] = sum;
        __syncthreads();
        sum = 0.0f;
#pragma unroll
        for (int i = 0; i < kLongWaves; ++i) sum += partials[parity][i];
        const float rstd = rstd_of(sum, a.hidden_f, a.eps);

        const float* crow = nullptr;
        const float* srow = nullptr;
        if constexpr (OP == GOp::kRopeIl || OP == GOp::kRopeHalf) {
            const int64_t pos = row % a.seq_len;
            crow = a.cos_tab + pos * a.half;
            srow = a.sin_tab + pos * a.half;
        }

        if constexpr (OP != GOp::kRopeHalf) {
            // pass 2: vectors in the row's vector grid
            const int64_t msample = OP == GOp::kAda ? (row / a.rows_per_sample) * H : 0;
            const int fm = (int)((msample - first) & (E - 1));
            for (int q0 = 0; q0 < nch; q0 += T * U) {
                u32x4 v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int q = q0 + u * T + tid;
                    v[u] = q < nch ? load_row_vec<IO>(a.x, s, g0, q, q * E - first, H) : u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int q = q0 + u * T + tid;
                    if (q < nch) {
                        const int j0 = q * E - first;
                        float f[E];
                        normalise_vec<IO, OP>(a, v[u], j0, fw, msample, fm, rstd, f);
                        if constexpr (OP == GOp::kRopeIl) {
                            float o[E];
                            rope_interleaved_vec<E>(a, crow, srow, j0, f, o);
                            store_row_vec<IO>(a.out, s, g0, q, j0, H, IO::narrow(o));
                        } else {
                            store_row_vec<IO>(a.out, s, g0, q, j0, H, IO::narrow(f));
                        }
                    }
                }
            }
        } else {
            // pass 2, rotate-half: unit = window of up to E elements of a
            // head's first half (head h, columns i0 .. i0 + cnt) and its
            // partner window half a head later; one thread reads and writes
            // both, so in-place calls stay correct.
            const int d = a.head_dim, half = a.half;
            const int nw = (half + E - 1) / E;  // windows per half head
            const int64_t units = (int64_t)(H / d) * nw;
            const int64_t total = a.rows * (int64_t)H;
            for (int64_t u = tid; u < units; u += T) {
                const int h = (int)(u / nw);
                const int i0 = (int)(u - (int64_t)h * nw) * E;
                const int cnt = half - i0 < E ? half - i0 : E;
                const int ja = h * d + i0, jb = ja + half;
                const int64_t ea = s + ja, eb = s + jb;
                float xa[E], xb[E], ga[E], gb[E];
                IO::widen(load_window<IO>(a.x, ea, (int)(ea & (E - 1)), total), xa);
                IO::widen(load_window<IO>(a.x, eb, (int)(eb & (E - 1)), total), xb);
                IO::widen(a.w ? load_window<IO>(a.w, ja, ja & (E - 1), H) : splat(IO::kOne), ga);
                IO::widen(a.w ? load_window<IO>(a.w, jb, jb & (E - 1), H) : splat(IO::kOne), gb);
                float o1[E], o2[E];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float ya = (xa[e] * rstd) * ga[e];
                    const float yb = (xb[e] * rstd) * gb[e];
                    const float c = e < cnt ? crow[i0 + e] : 0.0f;
                    const float sn = e < cnt ? srow[i0 + e] : 0.0f;
                    o1[e] = ya * c - yb * sn;
                    o2[e] = yb * c + ya * sn;
                }
                if (cnt == E && ((ea | eb) & (E - 1)) == 0) {
                    store_stream(static_cast<u32x4*>(a.out) + ea / E, IO::narrow(o1));
                    store_stream(static_cast<u32x4*>(a.out) + eb / E, IO::narrow(o2));
                } else {
                    store_elems<IO>(a.out, ea, IO::narrow(o1), ea, ea + cnt);
                    store_elems<IO>(a.out, eb, IO::narrow(o2), eb, eb + cnt);
                }
            }
        }
    }
}

}  // namespace
}  // namespace ltxnorm_detail
