// The library used through its C ABI alone: HIP runtime calls and
// include/ltxnorm.h, no Python and no PyTorch.  Buffers come from hipMalloc,
// work goes on a stream this program creates, and every output element is
// compared with the CPU oracle (oracle/oracle.c, linked in; test
// infrastructure) under the parity rule of the Python tests: |gpu - ref| <=
// max(ulp(ref), 2^-16 m) for bf16 outputs, |gpu - ref32| <= 2^-18 (|ref32| +
// m) for binary32 outputs, m the magnitude sum of a rotated or modulated
// output's two terms (0 for RMSNorm).  Status codes of rejected calls are
// checked too.  Prints one line per case and "ok" at the end; exits 0 only
// if everything passed.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "ltxnorm.h"

extern "C" {
int oracle_rmsnorm_dt(double* y, const void* x, const void* w, int64_t rows, int64_t hidden,
                      float eps, int dtype);
int oracle_rmsnorm_rope_dt(double* y, double* mag, const void* x, const void* w,
                           const float* cos_tab, const float* sin_tab, int64_t rows,
                           int64_t hidden, int32_t heads, int32_t head_dim, int64_t seq_len,
                           float eps, int dtype);
int oracle_rmsnorm_rope_interleaved_dt(double* y, double* mag, const void* x, const void* w,
                                       const float* cos_tab, const float* sin_tab, int64_t rows,
                                       int64_t hidden, int32_t heads, int32_t head_dim,
                                       int64_t seq_len, float eps, int dtype);
int oracle_rmsnorm_adaln_dt(double* y, double* mag, const void* x, const void* w,
                            const void* scale, const void* shift, int64_t rows, int64_t hidden,
                            int64_t rows_per_sample, float eps, int dtype);
void oracle_round_dt(const double* y, int64_t n, float* ref32, void* ref_out, int dtype);
}

namespace {

constexpr int kOracleBf16 = 0, kOracleF16 = 1, kOracleF32 = 2;
int g_failures = 0;

#define HIP_OK(call)                                                                  \
    do {                                                                              \
        hipError_t e_ = (call);                                                       \
        if (e_ != hipSuccess) {                                                       \
            std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            std::exit(2);                                                             \
        }                                                                             \
    } while (0)

void expect(bool ok, const char* what) {
    std::printf("%s %s\n", ok ? "pass" : "FAIL", what);
    if (!ok) ++g_failures;
}

// Seeded test inputs: a 64-bit LCG, normal-ish values from the sum of four
// uniforms, rounded to bf16 by nearest-even on the bit pattern.
struct Rng {
    uint64_t s;
    double uniform() {
        s = s * 6364136223846793005ULL + 1442695040888963407ULL;
        return (double)(s >> 11) * (1.0 / 9007199254740992.0);
    }
    double normal() { return (uniform() + uniform() + uniform() + uniform() - 2.0) * 1.7320508; }
};

uint16_t to_bf16(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

double from_bf16(uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

std::vector<uint16_t> bf16_values(Rng& r, size_t n, double scale, double offset) {
    std::vector<uint16_t> v(n);
    for (auto& e : v) e = to_bf16((float)(offset + scale * r.normal()));
    return v;
}

// bf16 spacing at v's binade (2^-133 for zero)
double ulp16(double v) {
    if (v == 0.0) return std::ldexp(1.0, -133);
    int e;
    std::frexp(std::fabs(v), &e);
    return std::ldexp(1.0, e - 8);
}

// Element-wise comparison of bf16 output bits with the oracle's double result.
bool compare_bf16(const std::vector<uint16_t>& got, const std::vector<double>& y,
                  const std::vector<double>* mag, const char* label) {
    const int64_t n = (int64_t)y.size();
    std::vector<uint16_t> ref(n);
    oracle_round_dt(y.data(), n, nullptr, ref.data(), kOracleBf16);
    int64_t bad = 0, exact = 0;
    for (int64_t i = 0; i < n; ++i) {
        const double g = from_bf16(got[i]), r = from_bf16(ref[i]);
        if (got[i] == ref[i]) ++exact;
        double tol = ulp16(r);
        if (mag) tol = std::fmax(tol, std::ldexp((*mag)[i], -16));
        if (!(std::fabs(g - r) <= tol) && !(std::isnan(g) && std::isnan(r))) {
            if (bad < 3) std::printf("  %s: element %lld got %.9g ref %.9g\n", label, (long long)i, g, r);
            ++bad;
        }
    }
    std::printf("  %s: %lld elements, %lld bit-exact, %lld outside the rule\n", label,
                (long long)n, (long long)exact, (long long)bad);
    return bad == 0;
}

struct Dev {
    void* p = nullptr;
    explicit Dev(size_t bytes) { HIP_OK(hipMalloc(&p, bytes)); }
    ~Dev() { (void)hipFree(p); }
};

template <typename T>
void upload(void* d, const std::vector<T>& h) {
    HIP_OK(hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice));
}

template <typename T>
std::vector<T> download(const void* d, size_t n) {
    std::vector<T> h(n);
    HIP_OK(hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost));
    return h;
}

// cos/sin tables [seq_len, d/2] for theta = 10000, in double rounded once
void tables(int64_t seq_len, int d, std::vector<float>& c, std::vector<float>& s) {
    c.resize(seq_len * (d / 2));
    s.resize(c.size());
    for (int64_t p = 0; p < seq_len; ++p)
        for (int i = 0; i < d / 2; ++i) {
            const double a = (double)p * std::pow(10000.0, -2.0 * i / d);
            c[p * (d / 2) + i] = (float)std::cos(a);
            s[p * (d / 2) + i] = (float)std::sin(a);
        }
}

void check_rmsnorm(hipStream_t st, int64_t rows, int64_t hidden, uint64_t seed) {
    Rng r{seed};
    const auto x = bf16_values(r, rows * hidden, 1.0, 0.0);
    const auto w = bf16_values(r, hidden, 0.25, 1.0);
    const size_t nb = rows * hidden * 2;
    Dev dx(nb), dy(nb), dw(hidden * 2);
    upload(dx.p, x);
    upload(dw.p, w);
    char label[96];
    std::snprintf(label, sizeof label, "rmsnorm bf16 %lldx%lld", (long long)rows, (long long)hidden);
    const ltxnorm_status s = ltxnorm_rmsnorm_fwd(dy.p, dx.p, dw.p, rows, hidden, 1e-6f, st);
    HIP_OK(hipStreamSynchronize(st));
    std::vector<double> y(rows * hidden);
    oracle_rmsnorm_dt(y.data(), x.data(), w.data(), rows, hidden, 1e-6f, kOracleBf16);
    expect(s == LTXNORM_OK && compare_bf16(download<uint16_t>(dy.p, rows * hidden), y, nullptr, label),
           label);
    // in place: out == x gives the same bits
    const auto out_of_place = download<uint16_t>(dy.p, rows * hidden);
    const ltxnorm_status s2 = ltxnorm_rmsnorm_fwd(dx.p, dx.p, dw.p, rows, hidden, 1e-6f, st);
    HIP_OK(hipStreamSynchronize(st));
    std::snprintf(label, sizeof label, "rmsnorm in place %lldx%lld", (long long)rows, (long long)hidden);
    expect(s2 == LTXNORM_OK && download<uint16_t>(dx.p, rows * hidden) == out_of_place, label);
}

void check_rope(hipStream_t st, bool interleaved, int64_t rows, int heads, int d, int64_t seq_len) {
    Rng r{(uint64_t)(17 + d + interleaved)};
    const int64_t hidden = (int64_t)heads * d;
    const auto x = bf16_values(r, rows * hidden, 1.0, 0.0);
    const auto w = bf16_values(r, hidden, 0.25, 1.0);
    std::vector<float> c, s;
    tables(seq_len, d, c, s);
    Dev dx(rows * hidden * 2), dy(rows * hidden * 2), dw(hidden * 2), dc(c.size() * 4),
        ds(s.size() * 4);
    upload(dx.p, x);
    upload(dw.p, w);
    upload(dc.p, c);
    upload(ds.p, s);
    const ltxnorm_status status =
        interleaved
            ? ltxnorm_rmsnorm_rope_interleaved_fwd(dy.p, dx.p, dw.p, (const float*)dc.p,
                                                   (const float*)ds.p, rows, hidden, heads, d,
                                                   seq_len, 1e-6f, st)
            : ltxnorm_rmsnorm_rope_fwd(dy.p, dx.p, dw.p, (const float*)dc.p, (const float*)ds.p,
                                       rows, hidden, heads, d, seq_len, 1e-6f, st);
    HIP_OK(hipStreamSynchronize(st));
    std::vector<double> y(rows * hidden), mag(rows * hidden);
    if (interleaved)
        oracle_rmsnorm_rope_interleaved_dt(y.data(), mag.data(), x.data(), w.data(), c.data(),
                                           s.data(), rows, hidden, heads, d, seq_len, 1e-6f,
                                           kOracleBf16);
    else
        oracle_rmsnorm_rope_dt(y.data(), mag.data(), x.data(), w.data(), c.data(), s.data(), rows,
                               hidden, heads, d, seq_len, 1e-6f, kOracleBf16);
    char label[96];
    std::snprintf(label, sizeof label, "rope %s %lldx%dx%d seq %lld",
                  interleaved ? "interleaved" : "rotate-half", (long long)rows, heads, d,
                  (long long)seq_len);
    expect(status == LTXNORM_OK &&
               compare_bf16(download<uint16_t>(dy.p, rows * hidden), y, &mag, label),
           label);
}

void check_adaln(hipStream_t st, int64_t rows, int64_t hidden, int64_t rps) {
    Rng r{99};
    const int64_t samples = (rows + rps - 1) / rps;
    const auto x = bf16_values(r, rows * hidden, 1.0, 0.0);
    const auto w = bf16_values(r, hidden, 0.25, 1.0);
    const auto sc = bf16_values(r, samples * hidden, 0.25, 0.0);
    const auto sh = bf16_values(r, samples * hidden, 0.25, 0.0);
    Dev dx(rows * hidden * 2), dy(rows * hidden * 2), dw(hidden * 2), dsc(sc.size() * 2),
        dsh(sh.size() * 2);
    upload(dx.p, x);
    upload(dw.p, w);
    upload(dsc.p, sc);
    upload(dsh.p, sh);
    const ltxnorm_status s =
        ltxnorm_rmsnorm_adaln_fwd(dy.p, dx.p, dw.p, dsc.p, dsh.p, rows, hidden, rps, 1e-6f, st);
    HIP_OK(hipStreamSynchronize(st));
    std::vector<double> y(rows * hidden), mag(rows * hidden);
    oracle_rmsnorm_adaln_dt(y.data(), mag.data(), x.data(), w.data(), sc.data(), sh.data(), rows,
                            hidden, rps, 1e-6f, kOracleBf16);
    char label[96];
    std::snprintf(label, sizeof label, "adaln %lldx%lld, %lld rows per sample", (long long)rows,
                  (long long)hidden, (long long)rps);
    expect(s == LTXNORM_OK && compare_bf16(download<uint16_t>(dy.p, rows * hidden), y, &mag, label),
           label);
}

void check_f32(hipStream_t st, int64_t rows, int64_t hidden) {
    Rng r{7};
    std::vector<float> x(rows * hidden), w(hidden);
    for (auto& e : x) e = (float)r.normal();
    for (auto& e : w) e = (float)(1.0 + 0.25 * r.normal());
    Dev dx(x.size() * 4), dy(x.size() * 4), dw(w.size() * 4);
    upload(dx.p, x);
    upload(dw.p, w);
    const ltxnorm_status s =
        ltxnorm_rmsnorm_fwd_dt(dy.p, dx.p, dw.p, rows, hidden, 1e-6f, LTXNORM_F32, st);
    HIP_OK(hipStreamSynchronize(st));
    std::vector<double> y(x.size());
    oracle_rmsnorm_dt(y.data(), x.data(), w.data(), rows, hidden, 1e-6f, kOracleF32);
    std::vector<float> ref32(x.size());
    oracle_round_dt(y.data(), (int64_t)y.size(), ref32.data(), nullptr, kOracleF32);
    const auto got = download<float>(dy.p, x.size());
    int64_t bad = 0;
    for (size_t i = 0; i < got.size(); ++i)
        if (!(std::fabs((double)got[i] - ref32[i]) <= std::ldexp(std::fabs((double)ref32[i]), -18)))
            ++bad;
    char label[96];
    std::snprintf(label, sizeof label, "rmsnorm fp32 %lldx%lld (%lld outside the rule)",
                  (long long)rows, (long long)hidden, (long long)bad);
    expect(s == LTXNORM_OK && bad == 0, label);
}

// fp16 through the _dt entry point: within one fp16 ulp of the oracle's
// rounded result (values encoded with the host's IEEE half conversion).
double from_f16(uint16_t b) {
    _Float16 h;
    std::memcpy(&h, &b, 2);
    return (double)h;
}

double ulp_f16(double v) {
    const double a = std::fabs(v);
    if (a < std::ldexp(1.0, -14)) return std::ldexp(1.0, -24);
    int e;
    std::frexp(a, &e);
    return std::ldexp(1.0, e - 11);
}

void check_f16(hipStream_t st, int64_t rows, int64_t hidden) {
    Rng r{77};
    std::vector<uint16_t> x(rows * hidden), w(hidden);
    for (auto& e : x) {
        const _Float16 h = (_Float16)r.normal();
        std::memcpy(&e, &h, 2);
    }
    for (auto& e : w) {
        const _Float16 h = (_Float16)(1.0 + 0.25 * r.normal());
        std::memcpy(&e, &h, 2);
    }
    Dev dx(x.size() * 2), dy(x.size() * 2), dw(w.size() * 2);
    upload(dx.p, x);
    upload(dw.p, w);
    const ltxnorm_status s =
        ltxnorm_rmsnorm_fwd_dt(dy.p, dx.p, dw.p, rows, hidden, 1e-6f, LTXNORM_F16, st);
    HIP_OK(hipStreamSynchronize(st));
    std::vector<double> y(x.size());
    oracle_rmsnorm_dt(y.data(), x.data(), w.data(), rows, hidden, 1e-6f, kOracleF16);
    std::vector<uint16_t> ref(x.size());
    oracle_round_dt(y.data(), (int64_t)y.size(), nullptr, ref.data(), kOracleF16);
    const auto got = download<uint16_t>(dy.p, x.size());
    int64_t bad = 0;
    for (size_t i = 0; i < got.size(); ++i) {
        const double g = from_f16(got[i]), f = from_f16(ref[i]);
        if (!(std::fabs(g - f) <= ulp_f16(f))) ++bad;
    }
    char label[96];
    std::snprintf(label, sizeof label, "rmsnorm fp16 %lldx%lld (%lld beyond one ulp)",
                  (long long)rows, (long long)hidden, (long long)bad);
    expect(s == LTXNORM_OK && bad == 0, label);
}

void check_statuses(hipStream_t st) {
    Dev a(1 << 20);
    char* base = static_cast<char*>(a.p);
    expect(ltxnorm_version() == LTXNORM_ABI_VERSION, "version matches the header");
    expect(std::strlen(ltxnorm_status_str(LTXNORM_ERR_ALIAS)) > 0, "status strings");
    expect(ltxnorm_rmsnorm_fwd(base + 2, base + 65536, nullptr, 4, 64, 1e-6f, st) == LTXNORM_ERR_ALIGN,
           "misaligned out is ERR_ALIGN");
    expect(ltxnorm_rmsnorm_fwd(base, nullptr, nullptr, 4, 64, 1e-6f, st) == LTXNORM_ERR_NULL,
           "NULL x is ERR_NULL");
    expect(ltxnorm_rmsnorm_fwd(base + 16, base, nullptr, 4, 64, 1e-6f, st) == LTXNORM_ERR_ALIAS,
           "partial overlap of out and x is ERR_ALIAS");
    expect(ltxnorm_rmsnorm_fwd(nullptr, nullptr, nullptr, 0, 64, 1e-6f, st) == LTXNORM_OK,
           "no rows: OK, nothing launched");
    expect(ltxnorm_rmsnorm_fwd_dt(base, base + 65536, nullptr, 4, 64, 1e-6f, (ltxnorm_dtype)7, st) ==
               LTXNORM_ERR_UNSUPPORTED,
           "unknown dtype is ERR_UNSUPPORTED");
    expect(ltxnorm_rmsnorm_rope_fwd(base, base + 65536, nullptr, (const float*)(base + 131072),
                                    (const float*)(base + 196608), 4, 64, 2, 30, 8, 1e-6f, st) ==
               LTXNORM_ERR_SHAPE,
           "heads * head_dim != hidden is ERR_SHAPE");
    HIP_OK(hipStreamSynchronize(st));
}

}  // namespace

int main() {
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
        std::printf("no GPU\n");
        return 2;
    }
    hipStream_t st;
    HIP_OK(hipStreamCreate(&st));
    check_statuses(st);
    check_rmsnorm(st, 37, 3072, 1);     // three wavefronts per row
    check_rmsnorm(st, 129, 2048, 2);    // one wavefront per row
    check_rmsnorm(st, 50, 3076, 3);     // rows that start inside a vector
    check_rmsnorm(st, 3000, 96, 4);     // short rows, several per wavefront
    check_rmsnorm(st, 1001, 320, 6);    // 16-lane segments, 3 vectors per lane
    check_rope(st, false, 64, 32, 64, 16);
    check_rope(st, true, 64, 32, 64, 16);
    check_rope(st, false, 20, 16, 72, 7);
    check_rope(st, false, 333, 1, 128, 9);   // one head per row: the partner in the lane's other slot
    check_adaln(st, 10, 1024, 5);
    check_adaln(st, 301, 1152, 100);    // 32-lane segments, 5 vectors per lane
    // rows past the register budget: 17 chunks of 2048 vectors, out of place
    // in chunks over many workgroups, in place two passes (the same bits)
    check_rmsnorm(st, 5, 262147, 7);
    check_adaln(st, 3, 262144, 2);
    check_rope(st, true, 3, 1024, 256, 5);
    check_f32(st, 9, 1000);
    check_f16(st, 37, 3072);            // three wavefronts per row
    check_f16(st, 1001, 320);           // 16-lane segments
    HIP_OK(hipStreamDestroy(st));
    std::printf(g_failures == 0 ? "ok\n" : "%d failures\n", g_failures);
    return g_failures == 0 ? 0 : 1;
}
