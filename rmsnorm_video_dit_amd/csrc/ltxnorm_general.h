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
// aligned 16-byte vector.  The row's first and last vectors are shared with
// the neighbouring rows: they are loaded whole and the other rows' elements
// zeroed in registers, and stored element by element (the row's own elements
// only).  The weight (and the modulation rows) are then misaligned by a
// row-dependent number of elements: a lane funnel-shifts the two aligned
// vectors that straddle its window (held in registers for the weight, loaded
// per row for the modulation), reading element by element only at the ends
// of an array.
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
//  * rmsnorm_split_partial_kernel, rmsnorm_split_apply_kernel: the same rows
//    out of place, cut into chunks over many workgroups in three launches
//    (section below); they add a row's squares in the two-pass kernel's
//    order, so both give the same bits.
#pragma once

#include "ltxnorm_device.h"

namespace ltxnorm_detail {
namespace {

constexpr int kLongWaves = kLongThreads / kWave;     // one row per workgroup
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

// Word I (a compile-time index) of the 8-word concatenation of lo and hi.
template <int I>
__device__ __forceinline__ uint32_t word8(const u32x4 lo, const u32x4 hi) {
    if constexpr (I < 4)
        return lo[I];
    else
        return hi[I - 4];
}

// Elements F .. F + kEpv - 1 of the 2 kEpv elements held in lo and hi.
template <int ELEM_BYTES, int F>
__device__ __forceinline__ u32x4 take(const u32x4 lo, const u32x4 hi) {
    constexpr int kByte = F * ELEM_BYTES;
    constexpr int o = kByte / 4;
    if constexpr (kByte % 4 == 0) {
        return u32x4{word8<o>(lo, hi), word8<o + 1>(lo, hi), word8<o + 2>(lo, hi), word8<o + 3>(lo, hi)};
    } else {
        return u32x4{(word8<o>(lo, hi) >> 16) | (word8<o + 1>(lo, hi) << 16),
                     (word8<o + 1>(lo, hi) >> 16) | (word8<o + 2>(lo, hi) << 16),
                     (word8<o + 2>(lo, hi) >> 16) | (word8<o + 3>(lo, hi) << 16),
                     (word8<o + 3>(lo, hi) >> 16) | (word8<o + 4>(lo, hi) << 16)};
    }
}

// The same for a shift f known only at run time but uniform across the
// wavefront: a chain of uniform branches, each with compile-time word
// indices and its result kept opaque (keep_packed), so that the optimiser
// cannot merge the branches into one read of a runtime-indexed array, which
// lands in private (scratch) memory: a select over the words written that
// way measured 12 points of peak slower, and the merge also happened by
// itself to the branch chain over a word array for binary32 rows.
template <typename IO, int F = 1>
__device__ __forceinline__ u32x4 take_at(const u32x4 lo, const u32x4 hi, int f) {
    if constexpr (F >= IO::kEpv) {
        return lo;
    } else {
        if (f == F) {
            u32x4 r = take<16 / IO::kEpv, F>(lo, hi);
            keep_packed(r);
            return r;
        }
        return take_at<IO, F + 1>(lo, hi, f);
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
        return take_at<IO>(v[c], v[c + 1], f);
    }
    return load_elems<IO>(base, start, 0, n);
}

// Store elements lo .. hi - 1 (0 <= lo < hi <= kEpv) of the aligned vector
// at p as naturally aligned pieces: up from byte lo * size in pieces of 2, 4
// and 8 bytes while the start is misaligned, then down in pieces of 8, 4 and
// 2 bytes (at most four stores).  Where a row boundary falls on a 4-byte
// boundary, no store is narrower than 4 bytes: a 2-byte store leaves a
// partially written 4-byte word in the cache, and rows of hidden 3076 took
// 41 % of peak with one 2-byte store per element at their end vectors.
template <typename IO>
__device__ __forceinline__ void store_vec_range(u32x4* p, const u32x4 v, int lo, int hi) {
    constexpr int ES = 16 / IO::kEpv;  // bytes per element
    char* base = reinterpret_cast<char*>(p);
    int b0 = lo * ES;
    const int b1 = hi * ES;
    // word i of v for a lane-varying i, as selects (no indexed array)
    auto word = [&](int i) { return i == 0 ? v[0] : (i == 1 ? v[1] : (i == 2 ? v[2] : v[3])); };
    auto put2 = [&](int b) {
        __builtin_nontemporal_store((uint16_t)(word(b >> 2) >> (8 * (b & 3))),
                                    reinterpret_cast<uint16_t*>(base + b));
    };
    auto put4 = [&](int b) { __builtin_nontemporal_store(word(b >> 2), reinterpret_cast<uint32_t*>(base + b)); };
    if (b1 - b0 == 16) {
        store_stream(p, v);
        return;
    }
    if constexpr (ES == 2) {
        if ((b0 & 2) && b0 + 2 <= b1) {
            put2(b0);
            b0 += 2;
        }
    }
    if ((b0 & 4) && b0 + 4 <= b1) {
        put4(b0);
        b0 += 4;
    }
    if ((b0 & 8) && b0 + 8 <= b1) {  // bytes 8 .. 15
        __builtin_nontemporal_store(u32x2{v[2], v[3]}, reinterpret_cast<u32x2*>(base + 8));
        b0 += 8;
    }
    if (b1 - b0 >= 8) {  // bytes 0 .. 7 (b0 is 0 here)
        __builtin_nontemporal_store(u32x2{v[0], v[1]}, reinterpret_cast<u32x2*>(base));
        b0 += 8;
    }
    if (b1 - b0 >= 4) {
        put4(b0);
        b0 += 4;
    }
    if constexpr (ES == 2) {
        if (b1 - b0 >= 2) put2(b0);
    }
}

// Store a row's vector q (row-relative elements j0 .. j0 + kEpv): whole
// vectors with the streaming store, the row's end vectors as aligned pieces
// holding the row's own elements only.
template <typename IO>
__device__ __forceinline__ void store_row_vec(void* out, int64_t g0, int q, int j0, int hidden,
                                              const u32x4 v) {
    constexpr int E = IO::kEpv;
    u32x4* p = static_cast<u32x4*>(out) + g0 + q;
    if (j0 >= 0 && j0 + E <= hidden)
        store_stream(p, v);
    else
        store_vec_range<IO>(p, v, j0 < 0 ? -j0 : 0, hidden - j0 < E ? hidden - j0 : E);
}

// Zero the elements of v outside positions [lo, hi) of the vector
// (0 <= lo, hi <= kEpv): the parts of a row's end vectors that belong to the
// neighbouring rows.
template <typename IO>
__device__ __forceinline__ u32x4 keep_range(u32x4 v, int lo, int hi) {
    const uint32_t keep = ((1u << hi) - 1u) & ~((1u << lo) - 1u);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        uint32_t mk;
        if constexpr (IO::kEpv == 8)
            mk = ((keep >> (2 * m)) & 1u ? 0x0000FFFFu : 0u) | ((keep >> (2 * m + 1)) & 1u ? 0xFFFF0000u : 0u);
        else
            mk = (keep >> m) & 1u ? 0xFFFFFFFFu : 0u;
        v[m] &= mk;
    }
    return v;
}

// Chunk c of the weight (elements c kEpv .. + kEpv), zero outside [0, H);
// ones for a null weight.
template <typename IO>
__device__ __forceinline__ u32x4 weight_chunk(const void* w, int c, int hidden) {
    constexpr int E = IO::kEpv;
    if (w == nullptr) return splat(IO::kOne);
    if (c < 0) return u32x4{0u, 0u, 0u, 0u};
    if ((c + 1) * E <= hidden) return static_cast<const u32x4*>(w)[c];
    return load_elems<IO>(w, (int64_t)c * E, 0, hidden);
}

// Chunk c of the weight when it is whole (ones for a null weight, zero
// otherwise): a load on one side only, so it issues without waiting; the
// weight's partial last chunk is fetched separately.
template <typename IO>
__device__ __forceinline__ u32x4 whole_weight_chunk(const void* w, int c, int hidden) {
    constexpr int E = IO::kEpv;
    if (w == nullptr) return splat(IO::kOne);
    return (c >= 0 && (c + 1) * E <= hidden) ? static_cast<const u32x4*>(w)[c] : u32x4{0u, 0u, 0u, 0u};
}

// The weight window of a row's vector q from the lane's two resident chunks
// q - 1 and q: f = window start mod kEpv, the same for the whole row.
template <typename IO>
__device__ __forceinline__ u32x4 weight_window(u32x4 lo, u32x4 hi, int f) {
    if (f == 0) return hi;
    keep_packed(lo);
    keep_packed(hi);
    return take_at<IO>(lo, hi, f);
}

// Interleaved RoPE on one normalised vector: pairs (2i, 2i + 1) of a head
// turn by table column i.  j0 is even (hidden even, rows start at even
// element offsets), so pairs never straddle vectors or the row's ends.  The
// column is computed for every pair, valid or not, so that all table reads
// are in range and issue together.
template <int E>
__device__ __forceinline__ void rope_interleaved_vec(const KArgs& a, const float* crow,
                                                     const float* srow, int j0, const float* f,
                                                     float* o) {
    const int d = a.head_dim;
    int hd = ((j0 % d) + d) % d;  // position of element 0 in its head
    float c[E / 2], sn[E / 2];
#pragma unroll
    for (int p = 0; p < E / 2; ++p) {
        c[p] = crow[hd / 2];
        sn[p] = srow[hd / 2];
        hd += 2;
        if (hd == d) hd = 0;
    }
#pragma unroll
    for (int p = 0; p < E / 2; ++p) {
        o[2 * p] = rot(f[2 * p], c[p], -f[2 * p + 1], sn[p]);
        o[2 * p + 1] = rot(f[2 * p + 1], c[p], f[2 * p], sn[p]);
    }
}

// ---------------------------------------------------------------------------
// One-pass kernel for any hidden size that fits the register budget.
// VPL vectors per lane, WPR wavefronts per row, Layout<WPR> rows per block.
// Rotate-half needs Layout<WPR>::kRowsPerBlock * hidden floats of dynamic LDS.
//
// Every lane issues all its row loads before using any: an if/else with a
// load on each side makes the compiler wait for every outstanding load at the
// join, which serialised the loads of a row (H = 3076 measured 41 % of peak
// that way).  So whole vectors are loaded unconditionally, the tensor's final
// partial vector (if any) is fetched afterwards under a uniform branch, and
// the neighbouring rows' elements in a row's end vectors are zeroed in
// registers.  Each lane's weight windows are built once per workgroup: the
// launch keeps every row of a workgroup slot at the same offset into its
// first vector.
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
    const int64_t total = a.rows * (int64_t)H;
    const int64_t whole = total / E;  // whole vectors in x

    // The weight window of every slot, built once.  A row starts
    // (row * H) mod E elements into its first vector; the launch makes the
    // grid-stride step (gridDim.x * RPB rows) a multiple of 8 whenever a
    // workgroup loops, so every row this slot visits has its first row's
    // offset and the same window (from chunks q - 1 and q).
    priority_for_loads();
    u32x4 wwin[VPL];
    {
        const int64_t row0 = (int64_t)blockIdx.x * RPB + ln.slot;
        const int fw0 = (int)((-(row0 * (int64_t)H)) & (E - 1));
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int q = k * L + ln.t;
            wwin[k] = weight_window<IO>(weight_chunk<IO>(a.w, q - 1, H), weight_chunk<IO>(a.w, q, H), fw0);
        }
    }

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

        u32x4 xv[VPL];
        priority_for_loads();
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int q = k * L + ln.t;
            const bool in = q < nch && g0 + q < whole;
            xv[k] = in ? load_stream(static_cast<const u32x4*>(a.x) + g0 + q) : u32x4{0u, 0u, 0u, 0u};
        }
        if (active && s + H > whole * E) {  // the tensor's final, partial vector
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                const int q = k * L + ln.t;
                if (q < nch && g0 + q >= whole) xv[k] = load_elems<IO>(a.x, (g0 + q) * E, s, s + H);
            }
        }
        priority_after_loads();
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int j0 = (k * L + ln.t) * E - first;
            const int lo = j0 < 0 ? -j0 : 0;
            const int hi = H - j0 >= E ? E : (H - j0 > 0 ? H - j0 : 0);
            xv[k] = keep_range<IO>(xv[k], lo, hi);
        }
        const float part = sum_squares<IO, VPL>(xv);
        const float rstd = rstd_of(row_sum<WPR>(part, ln.slot, ln.wave_in_row, parity), a.hidden_f, a.eps);

        auto normalise = [&](int k, float* f) {
            float g[E];
            keep_packed(xv[k]);
            IO::widen(xv[k], f);
            keep_packed(wwin[k]);
            IO::widen(wwin[k], g);
#pragma unroll
            for (int e = 0; e < E; ++e) f[e] = (f[e] * rstd) * g[e];
        };

        if constexpr (kExchange) {
            float* yrow = ybuf + ln.slot * H;
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                const int q = k * L + ln.t;
                if (q < nch) {
                    const int j0 = q * E - first;
                    float f[E];
                    normalise(k, f);
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
                    float c[E], sn[E];
#pragma unroll
                    for (int e = 0; e < E; ++e) {  // columns in range for every element
                        const int col = hd < half ? hd : hd - half;
                        c[e] = crow[col];
                        sn[e] = hd < half ? -srow[col] : srow[col];
                        if (++hd == d) hd = 0;
                    }
                    hd = ((j0 % d) + d) % d;
                    float o[E];
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        // first half: a c - b s; second half: b c + a s
                        const int j = j0 + e;
                        const bool valid = j >= 0 && j < H;
                        // indices clamped into the row: every LDS read is in range
                        const int jj = valid ? j : 0;
                        const int pj = valid ? (hd < half ? j + half : j - half) : 0;
                        o[e] = rot(yrow[jj], c[e], yrow[pj], sn[e]);
                        if (++hd == d) hd = 0;
                    }
                    store_row_vec<IO>(a.out, g0, q, j0, H, IO::narrow(o));
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
                    normalise(k, f);
                    if constexpr (OP == GOp::kAda) {
                        float sc[E], sh[E];
                        const u32x4 sv = a.scale ? load_window<IO>(a.scale, msample + j0, fm, a.mod_elems)
                                                 : u32x4{0u, 0u, 0u, 0u};
                        const u32x4 hv = a.shift ? load_window<IO>(a.shift, msample + j0, fm, a.mod_elems)
                                                 : splat(IO::kNegZero);
                        IO::widen(sv, sc);
                        IO::widen(hv, sh);
#pragma unroll
                        for (int e = 0; e < E; ++e) f[e] = modulate(f[e], sc[e], sh[e]);
                    }
                    if constexpr (OP == GOp::kRopeIl) {
                        float o[E];
                        rope_interleaved_vec<E>(a, crow, srow, j0, f, o);
                        store_row_vec<IO>(a.out, g0, q, j0, H, IO::narrow(o));
                    } else {
                        store_row_vec<IO>(a.out, g0, q, j0, H, IO::narrow(f));
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Rows beyond the register budget: helpers shared by the two-pass kernel and
// the split kernels.
// ---------------------------------------------------------------------------

// A row's place in the global vector grid of x (and of out).
template <int E>
struct RowSpan {
    int64_t s;  // the row's first element
    int first;  // its place in its vector
    int64_t g0; // that vector
    int nch;    // vectors the row touches
    int fw;     // (-first) mod E: the shift of the row's weight windows
    __device__ __forceinline__ RowSpan(int64_t row, int H)
        : s(row * H), first((int)(s & (E - 1))), g0(s / E), nch((first + H + E - 1) / E),
          fw((-first) & (E - 1)) {}
};

// U vectors of a row, row-relative vectors q0 + u * stride + t: loads issued
// before any use (the pattern of the one-pass kernel), whole vectors first,
// then the tensor's final partial vector under a uniform branch, then the
// neighbouring rows' elements zeroed.  Vectors past the row are zero.
template <typename IO, int U>
__device__ __forceinline__ void load_span(const KArgs& a, const RowSpan<IO::kEpv>& r, int64_t whole,
                                          int q0, int stride, int t, u32x4* v) {
    constexpr int E = IO::kEpv;
    const int H = a.hidden;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int q = q0 + u * stride + t;
        const bool in = q < r.nch && r.g0 + q < whole;
        const u32x4* p = static_cast<const u32x4*>(a.x) + r.g0 + q;
        v[u] = in ? *p : u32x4{0u, 0u, 0u, 0u};
    }
    if (r.s + H > whole * E) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int q = q0 + u * stride + t;
            if (q < r.nch && r.g0 + q >= whole) v[u] = load_elems<IO>(a.x, (r.g0 + q) * E, r.s, r.s + H);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int j0 = (q0 + u * stride + t) * E - r.first;
        const int lo = j0 < 0 ? -j0 : 0;
        const int hi = H - j0 >= E ? E : (H - j0 > 0 ? H - j0 : 0);
        v[u] = keep_range<IO>(v[u], lo, hi);
    }
}

// Normalise U vectors of row `row` (as load_span places them), apply the
// AdaLN modulation or the interleaved rotation, and store them, except the
// row-relative vectors [skip_lo, skip_hi): every operation but rotate-half,
// whose pairs are half a head apart.
template <typename IO, GOp OP, int U>
__device__ __forceinline__ void apply_span(const KArgs& a, const RowSpan<IO::kEpv>& r, int64_t row,
                                           int64_t whole, int q0, int stride, int t, float rstd,
                                           int skip_lo = 0, int skip_hi = 0) {
    static_assert(OP != GOp::kRopeHalf, "rotate-half pairs are not element-wise");
    constexpr int E = IO::kEpv;
    const int H = a.hidden;
    const int64_t msample = OP == GOp::kAda ? (row / a.rows_per_sample) * H : 0;
    const int fm = (int)((msample - r.first) & (E - 1));
    const float* crow = nullptr;
    const float* srow = nullptr;
    if constexpr (OP == GOp::kRopeIl) {
        const int64_t pos = row % a.seq_len;
        crow = a.cos_tab + pos * a.half;
        srow = a.sin_tab + pos * a.half;
    }
    const int wfull = H / E;  // whole weight chunks
    u32x4 v[U], wl[U], wh[U];
    load_span<IO, U>(a, r, whole, q0, stride, t, v);
#pragma unroll
    for (int u = 0; u < U; ++u) wh[u] = whole_weight_chunk<IO>(a.w, q0 + u * stride + t, H);
    // A row that starts on a vector boundary (every row, when hidden is a
    // whole number of vectors) takes its weight windows whole: chunk q - 1
    // is loaded, and read, only for shifted windows (a uniform branch).
    if (r.fw != 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) wl[u] = whole_weight_chunk<IO>(a.w, q0 + u * stride + t - 1, H);
    }
    if (a.w != nullptr && wfull * E != H && q0 + stride * (U - 1) + stride > wfull) {
        // windows reaching the weight's partial last chunk
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int q = q0 + u * stride + t;
            if (q - 1 == wfull) wl[u] = load_elems<IO>(a.w, (int64_t)wfull * E, 0, H);
            if (q == wfull) wh[u] = load_elems<IO>(a.w, (int64_t)wfull * E, 0, H);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int q = q0 + u * stride + t;
        if (q < r.nch && (q < skip_lo || q >= skip_hi)) {
            const int j0 = q * E - r.first;
            float f[E], g[E];
            IO::widen(v[u], f);
            IO::widen(r.fw == 0 ? wh[u] : weight_window<IO>(wl[u], wh[u], r.fw), g);
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
                for (int e = 0; e < E; ++e) f[e] = modulate(f[e], sc[e], sh[e]);
            }
            if constexpr (OP == GOp::kRopeIl) {
                float o[E];
                rope_interleaved_vec<E>(a, crow, srow, j0, f, o);
                store_row_vec<IO>(a.out, r.g0, q, j0, H, IO::narrow(o));
            } else {
                store_row_vec<IO>(a.out, r.g0, q, j0, H, IO::narrow(f));
            }
        }
    }
}

// Long rows are summed in chunks of kSplitChunk vectors, the same way by the
// two-pass kernel and the split kernels, so a row's rstd has the same bits
// whichever of them a call takes (in place or not).  A chunk: 256 threads,
// thread t adds the squares of vectors k * 256 + t (k = 0..7, in order), then
// the wavefront tree, then the 4 wavefronts' sums in order.  The row: lane l
// adds chunk sums l, l + 64, l + 128, ... in order, then the wavefront tree.
// At most 8 terms per lane chain, 33 per partial chain, two 6-level trees.
constexpr int kSplitThreads = 256;
constexpr int kSplitVpt = 8;                                // vectors per thread and chunk
constexpr int kSplitChunk = kSplitThreads * kSplitVpt;      // vectors per chunk
constexpr int kSplitMaxChunks = kSplitMaxChunkCount;        // partials a wavefront reads at once
static_assert(kSplitChunk == kSplitChunkVectors, "chunk size shared with the host");
// chunks of the longest row (2^24 elements, 4 per vector, starting inside a vector)
constexpr int kLongMaxChunks = ((1 << 22) + 1 + kSplitChunk - 1) / kSplitChunk;
constexpr int kLongGroups = kLongThreads / kSplitThreads;  // chunks summed at once

// ---------------------------------------------------------------------------
// Two-pass kernel for rows beyond the register budget: one row per
// 1024-thread workgroup.  Pass 1 streams the row for its sum of squares, four
// chunks at a time (one per group of 256 threads); pass 2 reads it again,
// normalises and stores.  Both passes load x through the caches: at
// [256 x 262144] bf16, pass 2 with non-temporal loads measured 69.8 us
// against 68.1 us cached, and non-temporal loads in both passes 75.9 us.
// The library takes it for calls in place and for rotate-half pairs; the
// split kernels below take the other long rows.
// ---------------------------------------------------------------------------
template <typename IO, GOp OP>
__global__ void __launch_bounds__(kLongThreads)
rmsnorm_long_kernel(const KArgs a) {
    constexpr int E = IO::kEpv;
    constexpr int T = kLongThreads;
    constexpr int U = kLongUnroll<IO>;
    __shared__ float wsums[2][kLongWaves];
    __shared__ float chunk_sums[kLongMaxChunks];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int group = wave / (kSplitThreads / kWave), gt = tid % kSplitThreads;
    const int lane = tid & (kWave - 1);
    const int H = a.hidden;
    const int64_t whole = a.rows * (int64_t)H / E;  // whole vectors in x

    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const RowSpan<E> r(row, H);

        // pass 1: the chunk sums, four chunks at a time (a group's chunk past
        // the row is all zeros and is not recorded)
        const int chunks = (r.nch + kSplitChunk - 1) / kSplitChunk;
        for (int c0 = 0, it = 0; c0 < chunks; c0 += kLongGroups, ++it) {
            const int c = c0 + group;
            u32x4 v[kSplitVpt];
            load_span<IO, kSplitVpt>(a, r, whole, c * kSplitChunk, kSplitThreads, gt, v);
            const float s = wave_sum(sum_squares<IO, kSplitVpt>(v));
            if (lane == 0) wsums[it & 1][wave] = s;
            __syncthreads();
            if (gt == 0 && c < chunks) {
                float t = 0.0f;
#pragma unroll
                for (int i = 0; i < kSplitThreads / kWave; ++i) t += wsums[it & 1][group * (kSplitThreads / kWave) + i];
                chunk_sums[c] = t;
            }
        }
        __syncthreads();
        // the row total, as the split kernels add it
        float t = 0.0f;
        for (int i = lane; i < chunks; i += kWave) t += chunk_sums[i];
        const float rstd = rstd_of(wave_sum(t), a.hidden_f, a.eps);

        if constexpr (OP != GOp::kRopeHalf) {
            // pass 2: vectors in the row's vector grid
            for (int q0 = 0; q0 < r.nch; q0 += T * U) apply_span<IO, OP, U>(a, r, row, whole, q0, T, tid, rstd);
        } else {
            // pass 2, rotate-half: unit = window of up to E elements of a
            // head's first half (head h, columns i0 .. i0 + cnt) and its
            // partner window half a head later; one thread reads and writes
            // both, so in-place calls stay correct.
            const int64_t pos = row % a.seq_len;
            const float* crow = a.cos_tab + pos * a.half;
            const float* srow = a.sin_tab + pos * a.half;
            const int d = a.head_dim, half = a.half;
            const int nw = (half + E - 1) / E;  // windows per half head
            const int64_t units = (int64_t)(H / d) * nw;
            const int64_t total = a.rows * (int64_t)H;
            for (int64_t u = tid; u < units; u += T) {
                const int h = (int)(u / nw);
                const int i0 = (int)(u - (int64_t)h * nw) * E;
                const int cnt = half - i0 < E ? half - i0 : E;
                const int ja = h * d + i0, jb = ja + half;
                const int64_t ea = r.s + ja, eb = r.s + jb;
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
                    o1[e] = rot(ya, c, -yb, sn);
                    o2[e] = rot(yb, c, ya, sn);
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

// ---------------------------------------------------------------------------
// Split kernels for rows beyond the register budget, out of place: row r is
// cut into chunks of kSplitChunk vectors of its vector grid, one 256-thread
// workgroup per chunk, so a launch of few long rows still fills the GPU (the
// two-pass kernel gives each row one workgroup: 64 rows of 2^20 elements
// kept 64 of 256 CUs busy).  Three launches, no scratch memory and no wait
// between workgroups:
//  1. rmsnorm_split_partial_kernel: each chunk's sum of squares (a fixed
//     tree) goes to the row's staging area, binary32 words from the row's
//     first whole output vector on (one vector per four chunks, inside
//     chunk 0 of the output).
//  2. rmsnorm_split_apply_kernel<..., false>: every chunk adds the row's
//     partials in a fixed order (every workgroup of the row gets the same
//     bits), normalises its chunk and stores it; chunk 0 leaves the staging
//     vectors alone.
//  3. rmsnorm_split_apply_kernel<..., true>: one workgroup per row does the
//     same for the staging vectors, after all of its wavefronts have read
//     the partials they then overwrite.  (Chunk 0 whole in this launch, one
//     workgroup per row, took 8.3 of 75 us at 64 rows of 2^20.)
// x is read twice, as in the two-pass kernel.  In place (out == x) the
// staging area would overwrite x, so those calls take the two-pass kernel.
// ---------------------------------------------------------------------------

// The row's staging area: binary32 words from its first whole output vector.
template <int E>
__device__ __forceinline__ float* split_stage(void* out, const RowSpan<E>& r) {
    return reinterpret_cast<float*>(static_cast<u32x4*>(out) + r.g0 + (r.first != 0 ? 1 : 0));
}

template <typename IO>
__global__ void __launch_bounds__(kSplitThreads)
rmsnorm_split_partial_kernel(const KArgs a, int chunks) {
    constexpr int E = IO::kEpv;
    __shared__ float wsum[kSplitThreads / kWave];
    const int64_t b = blockIdx.x;
    const int64_t row = b / chunks;
    const int c = (int)(b - row * chunks);
    const int64_t whole = a.rows * (int64_t)a.hidden / E;
    const RowSpan<E> r(row, a.hidden);
    u32x4 v[kSplitVpt];
    load_span<IO, kSplitVpt>(a, r, whole, c * kSplitChunk, kSplitThreads, (int)threadIdx.x, v);
    const float s = wave_sum(sum_squares<IO, kSplitVpt>(v));
    if ((threadIdx.x & (kWave - 1)) == 0) wsum[threadIdx.x / kWave] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.0f;
#pragma unroll
        for (int i = 0; i < kSplitThreads / kWave; ++i) t += wsum[i];
        split_stage<E>(a.out, r)[c] = t;
    }
}

template <typename IO, GOp OP, bool STAGE>
__global__ void __launch_bounds__(kSplitThreads)
rmsnorm_split_apply_kernel(const KArgs a, int chunks) {
    constexpr int E = IO::kEpv;
    constexpr int U = kLongUnroll<IO>;
    const int64_t b = blockIdx.x;
    int64_t row;
    int c;
    if constexpr (STAGE) {
        row = b;
        c = 0;
    } else {
        // Row-major over the row's chunk slots (split_slots: padded to a
        // multiple of the 8 XCDs where that keeps each chunk on one XCD at
        // little cost); padding slots exit.  Ordering the grid chunk-major
        // instead made concurrent workgroups read rows a power of two apart,
        // and ran slower (64 rows of 2^20: 79.3 -> 81.9 us).
        const int slots = split_slots(chunks);
        row = b / slots;
        c = (int)(b - row * slots);
        if (c >= chunks) return;
    }
    const int64_t whole = a.rows * (int64_t)a.hidden / E;
    const RowSpan<E> r(row, a.hidden);
    // The row's sum of squares: lane l adds partials l, l + 64, ... in that
    // order (all of them loaded first), then the wavefront tree.  Every
    // wavefront of every workgroup of the row computes the same bits.
    const float* stage = split_stage<E>(a.out, r);
    const int lane = threadIdx.x & (kWave - 1);
    float p[kSplitMaxChunks / kWave];
#pragma unroll
    for (int j = 0; j < kSplitMaxChunks / kWave; ++j) {
        const int i = j * kWave + lane;
        p[j] = i < chunks ? stage[i] : 0.0f;
    }
    float t = 0.0f;
#pragma unroll
    for (int j = 0; j < kSplitMaxChunks / kWave; ++j) t += p[j];
    const float rstd = rstd_of(wave_sum(t), a.hidden_f, a.eps);
    // the staging vectors, row-relative
    const int s0 = r.first != 0 ? 1 : 0;
    const int s1 = s0 + (chunks + 3) / 4;
    if constexpr (STAGE) {
        __syncthreads();  // every wavefront has read the partials
        RowSpan<E> rs = r;
        rs.nch = s1 < r.nch ? s1 : r.nch;
        for (int q0 = s0; q0 < s1; q0 += kSplitThreads * U)
            apply_span<IO, OP, U>(a, rs, row, whole, q0, kSplitThreads, (int)threadIdx.x, rstd);
    } else {
        const int skip_lo = c == 0 ? s0 : 0;
        const int skip_hi = c == 0 ? s1 : 0;
#pragma unroll
        for (int u0 = 0; u0 < kSplitVpt; u0 += U)
            apply_span<IO, OP, U>(a, r, row, whole, c * kSplitChunk + u0 * kSplitThreads, kSplitThreads,
                                  (int)threadIdx.x, rstd, skip_lo, skip_hi);
    }
}

}  // namespace
}  // namespace ltxnorm_detail
