// The C ABI's host layer (argument validation, ltxnorm_describe_launch,
// status strings) built with AddressSanitizer and exercised without a GPU:
// every call here is rejected by validation or only describes a launch, so
// the dtype launchers are never reached (stubs below abort if they are).
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "ltxnorm.h"
#include "ltxnorm_launch.h"

namespace ltxnorm_detail {
ltxnorm_status launch_bf16(Op, const Request&, hipStream_t) { std::abort(); }
ltxnorm_status launch_f16(Op, const Request&, hipStream_t) { std::abort(); }
ltxnorm_status launch_f32(Op, const Request&, hipStream_t) { std::abort(); }
}  // namespace ltxnorm_detail

int main() {
    // describe: random operations, dtypes (valid and not), shapes and output
    // buffer lengths, including empty and NULL buffers; the text must end
    // inside the buffer and never write past it
    std::mt19937_64 rng(20261203);
    long described = 0, rejected = 0;
    for (int it = 0; it < 200000; ++it) {
        const int op = (int)(rng() % 5);
        const int dt = (int)(rng() % 4);
        int64_t rows = (int64_t)(rng() % 3 == 0 ? rng() % 5000 : rng() % 100000000);
        if (rng() % 50 == 0) rows = -rows - 1;
        int64_t hidden = (int64_t)(rng() % 4 == 0 ? rng() % 70000 : rng() % (1u << 25));
        const int32_t head_dim = (int32_t)(2 * (rng() % 700));
        const int32_t heads = head_dim ? (int32_t)(hidden / head_dim) : 0;
        if (rng() % 3 == 0) hidden = (int64_t)heads * head_dim;
        const size_t len = (size_t)(rng() % 6 == 0 ? rng() % 4 : rng() % 300);
        std::vector<char> buf(len + 1, 'Z');
        char* p = (len == 0 && rng() % 2) ? nullptr : buf.data();
        const ltxnorm_status s =
            ltxnorm_describe_launch((ltxnorm_op)op, rows, hidden, heads, head_dim, (ltxnorm_dtype)dt, p, len);
        if (s == LTXNORM_OK) {
            ++described;
            if (p && len && strnlen(p, len) >= len) { std::printf("unterminated\n"); return 1; }
            if (buf[len] != 'Z') { std::printf("overrun\n"); return 1; }
        } else {
            ++rejected;
        }
    }
    for (int c = -5; c < 20; ++c)
        if (ltxnorm_status_str((ltxnorm_status)c) == nullptr) { std::printf("null status string\n"); return 1; }
    // rejected calls (fake, never dereferenced addresses): NULL, alignment,
    // aliasing, eps, NULL tables, rows_per_sample, dtype; rows == 0 is OK
    char* A = reinterpret_cast<char*>(0x10000);
    char* M = A + 4;
    char* X = A + (1 << 20);
    const ltxnorm_status r[8] = {
        ltxnorm_rmsnorm_fwd(nullptr, X, nullptr, 16, 3072, 1e-6f, nullptr),
        ltxnorm_rmsnorm_fwd(M, X, nullptr, 16, 3072, 1e-6f, nullptr),
        ltxnorm_rmsnorm_fwd(A + 16, A, nullptr, 16, 3072, 1e-6f, nullptr),
        ltxnorm_rmsnorm_fwd(A, X, nullptr, 16, 3072, -1.0f, nullptr),
        ltxnorm_rmsnorm_rope_fwd(A, X, nullptr, nullptr, nullptr, 16, 2048, 32, 64, 16, 1e-6f, nullptr),
        ltxnorm_rmsnorm_adaln_fwd(A, X, nullptr, M, nullptr, 16, 2048, 0, 1e-6f, nullptr),
        ltxnorm_rmsnorm_fwd_dt(A, X, nullptr, 16, 3072, 1e-6f, (ltxnorm_dtype)9, nullptr),
        ltxnorm_rmsnorm_fwd(A, A, nullptr, 0, 3072, 1e-6f, nullptr)};
    std::printf("statuses");
    for (ltxnorm_status s : r) std::printf(" %d", (int)s);
    std::printf("\ndescribed %ld rejected %ld\n", described, rejected);
    return 0;
}
