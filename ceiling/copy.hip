// copy.hip -- bandwidth ceiling kernels for the benchmark (not part of the
// library and not declared in include/): streams of 16-byte vectors that
// move the same bytes as a normalisation launch and do no arithmetic, so the
// benchmark can state how close a kernel comes to what this part's HBM
// delivers to plain loads and stores.
//
//   mode 0  plain copy: cached 16-byte loads and stores (bf16x8 when the
//           buffers hold bf16)
//   mode 1  non-temporal copy: the access hints the normalisation kernels
//           use for the activation read and the output write
//   mode 2  non-temporal read only (each thread folds what it read into one
//           word and stores it only if it equals a value the inputs never
//           produce, so the loads cannot be removed)
//   mode 3  non-temporal write only (a constant)
//
// Layout: a workgroup of 256 threads covers `per` * 256 consecutive vectors;
// thread t takes vectors k * 256 + t (k < per), so one instruction of a
// wavefront covers 1 KiB contiguous, and every thread issues all its loads
// before its first store, as the normalisation kernels do.  The grid is one
// workgroup per 256 * per vectors: the dispatcher streams workgroups to the
// CUs until the buffer is done.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

template <int MODE, int PER>
__global__ void __launch_bounds__(kThreads) copy_kernel(u32x4* __restrict__ dst,
                                                        const u32x4* __restrict__ src,
                                                        int64_t nvec, uint32_t* sink) {
    const int64_t base = (int64_t)blockIdx.x * (kThreads * PER) + threadIdx.x;
    u32x4 v[PER];
    if constexpr (MODE != 3) {
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int64_t i = base + (int64_t)k * kThreads;
            if (i < nvec) v[k] = MODE == 0 ? src[i] : __builtin_nontemporal_load(src + i);
            else v[k] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    if constexpr (MODE == 2) {
        uint32_t acc = 0;
#pragma unroll
        for (int k = 0; k < PER; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
        if (acc == 0x7FC17FC1u && sink != nullptr) sink[threadIdx.x] = acc;
    } else {
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int64_t i = base + (int64_t)k * kThreads;
            if (i < nvec) {
                const u32x4 w = MODE == 3 ? u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u} : v[k];
                if constexpr (MODE == 0) dst[i] = w;
                else __builtin_nontemporal_store(w, dst + i);
            }
        }
    }
}

template <int MODE>
const void* pick(int per) {
    switch (per) {
        case 1: return (const void*)&copy_kernel<MODE, 1>;
        case 2: return (const void*)&copy_kernel<MODE, 2>;
        case 4: return (const void*)&copy_kernel<MODE, 4>;
        case 8: return (const void*)&copy_kernel<MODE, 8>;
    }
    return nullptr;
}

}  // namespace

// Enqueue one pass over `nvec` 16-byte vectors on `stream`.  dst and src are
// device pointers, 16-byte aligned (src unused in mode 3, dst in mode 2; sink
// is a device word array of 256 entries for mode 2 or NULL).  Returns 0, or
// -1 for an unknown mode or per, a negative nvec or more than 2^31
// workgroups, or the hipError_t of the launch.
extern "C" __attribute__((visibility("default"))) int ceiling_copy(void* dst, const void* src,
                                                                   int64_t nvec, int mode, int per,
                                                                   void* sink, hipStream_t stream) {
    const void* fn = nullptr;
    switch (mode) {
        case 0: fn = pick<0>(per); break;
        case 1: fn = pick<1>(per); break;
        case 2: fn = pick<2>(per); break;
        case 3: fn = pick<3>(per); break;
    }
    if (fn == nullptr || nvec < 0) return -1;
    if (nvec == 0) return 0;
    const int64_t blocks = (nvec + (int64_t)kThreads * per - 1) / ((int64_t)kThreads * per);
    if (blocks > ((int64_t)1 << 31) - 1) return -1;
    u32x4* d = static_cast<u32x4*>(dst);
    const u32x4* s = static_cast<const u32x4*>(src);
    uint32_t* k = static_cast<uint32_t*>(sink);
    void* params[] = {&d, &s, &nvec, &k};
    const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kThreads), params, 0, stream);
    return e == hipSuccess ? 0 : (int)e;
}
