// Parity of the block-attention C ABI called from C++ alone: device buffers
// from hipMalloc, no Python and no torch.  Seeded N(0,1) inputs rounded to
// bf16, blockattn_fwd and blockattn_bwd on a HIP stream, and the fp64 oracle
// (oracle/blockattn_oracle.c, test infrastructure) on the same bf16 values.
// Tolerances: out, dq, dk, dv max abs <= 2e-2 and mean abs <= 2e-3; lse max
// abs <= 1e-3.  Also checks the status codes of calls the library must
// reject before launching anything.  Exit status 0 when every check passes.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "blockattn.h"

extern "C" {
int oracle_fwd(const double *q, const double *k, const double *v, const int32_t *offsets,
               int batch, int64_t T, int H, int D, int B, int W, double scale, double *out,
               double *lse);
int oracle_bwd(const double *q, const double *k, const double *v, const double *dout,
               const int32_t *offsets, int batch, int64_t T, int H, int D, int B, int W,
               double scale, double *dq, double *dk, double *dv);
}

namespace {

int failures = 0;

#define HIP_OK(x)                                                                      \
    do {                                                                               \
        hipError_t e_ = (x);                                                           \
        if (e_ != hipSuccess) {                                                        \
            std::printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, \
                        __LINE__);                                                     \
            std::exit(2);                                                              \
        }                                                                              \
    } while (0)

// splitmix64, then Box-Muller: a seeded standard normal stream.
struct Normal {
    uint64_t s;
    explicit Normal(uint64_t seed) : s(seed) {}
    uint64_t next() {
        uint64_t z = (s += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
    double uniform() { return ((next() >> 11) + 0.5) * (1.0 / 9007199254740992.0); }
    float operator()() {
        const double u1 = uniform(), u2 = uniform();
        return (float)(std::sqrt(-2.0 * std::log(u1)) * std::cos(6.283185307179586 * u2));
    }
};

// float -> bf16 bits, round to nearest even (finite inputs).
uint16_t to_bf16(float x) {
    uint32_t u;
    std::memcpy(&u, &x, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
double from_bf16(uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return (double)f;
}

struct Errors {
    double max_abs = 0, sum_abs = 0;
    size_t n = 0;
};
Errors compare(const std::vector<uint16_t> &got, const std::vector<double> &ref) {
    Errors e;
    for (size_t i = 0; i < ref.size(); ++i) {
        const double d = std::fabs(from_bf16(got[i]) - ref[i]);
        e.max_abs = std::fmax(e.max_abs, d);
        e.sum_abs += d;
    }
    e.n = ref.size();
    return e;
}
void check(const char *what, const char *name, const Errors &e, double max_tol, double mean_tol) {
    const double mean = e.n ? e.sum_abs / (double)e.n : 0.0;
    const bool ok = e.max_abs <= max_tol && mean <= mean_tol;
    std::printf("  %-4s max abs %.3e  mean abs %.3e  %s\n", name, e.max_abs, mean,
                ok ? "ok" : "FAIL");
    if (!ok) {
        std::printf("FAIL %s %s\n", what, name);
        ++failures;
    }
}

template <typename T>
T *to_device(const std::vector<T> &h) {
    T *d = nullptr;
    HIP_OK(hipMalloc(&d, h.size() * sizeof(T) + 16));
    if (!h.empty()) HIP_OK(hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice));
    return d;
}
template <typename T>
std::vector<T> to_host(const T *d, size_t n) {
    std::vector<T> h(n);
    if (n) HIP_OK(hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost));
    return h;
}

void run_case(const std::vector<int> &lengths, int H, int D, int B, int W, uint64_t seed,
              hipStream_t stream) {
    char what[160];
    std::snprintf(what, sizeof what, "users=%zu H=%d D=%d B=%d W=%d seed=%llu",
                  lengths.size(), H, D, B, W, (unsigned long long)seed);
    std::printf("case %s\n", what);
    std::fflush(stdout);
    const int batch = (int)lengths.size();
    std::vector<int32_t> off(batch + 1, 0);
    for (int u = 0; u < batch; ++u) off[u + 1] = off[u] + lengths[u];
    const int64_t T = off[batch];
    const size_t n = (size_t)T * H * D;
    Normal rng(seed);
    std::vector<uint16_t> hq(n), hk(n), hv(n), hdo(n);
    for (auto *t : {&hq, &hk, &hv, &hdo})
        for (auto &x : *t) x = to_bf16(rng());
    const double scale = 1.0 / std::sqrt((double)D);

    // library, through the C ABI
    uint16_t *q = to_device(hq), *k = to_device(hk), *v = to_device(hv), *dout = to_device(hdo);
    int32_t *doff = to_device(off);
    uint16_t *out, *dq, *dk, *dv;
    float *lse;
    HIP_OK(hipMalloc(&out, n * 2 + 16));
    HIP_OK(hipMalloc(&dq, n * 2 + 16));
    HIP_OK(hipMalloc(&dk, n * 2 + 16));
    HIP_OK(hipMalloc(&dv, n * 2 + 16));
    HIP_OK(hipMalloc(&lse, (size_t)H * T * 4 + 16));
    const size_t ws_bytes = blockattn_bwd_workspace_size(T, batch, H, BLOCKATTN_BF16);
    void *ws = nullptr;
    HIP_OK(hipMalloc(&ws, ws_bytes + 256));
    blockattn_status st = blockattn_fwd(q, k, v, doff, batch, T, H, D, B, W, (float)scale,
                                        BLOCKATTN_BF16, out, lse, stream);
    if (st != BLOCKATTN_OK) {
        std::printf("FAIL %s blockattn_fwd: %s\n", what, blockattn_status_string(st));
        ++failures;
    }
    st = blockattn_bwd(q, k, v, out, dout, lse, doff, batch, T, H, D, B, W, (float)scale,
                       BLOCKATTN_BF16, dq, dk, dv, ws, ws_bytes, stream);
    if (st != BLOCKATTN_OK) {
        std::printf("FAIL %s blockattn_bwd: %s\n", what, blockattn_status_string(st));
        ++failures;
    }
    HIP_OK(hipStreamSynchronize(stream));
    const auto gout = to_host(out, n), gdq = to_host(dq, n), gdk = to_host(dk, n),
               gdv = to_host(dv, n);
    const auto glse = to_host(lse, (size_t)H * T);

    // oracle, on the same bf16 values
    std::vector<double> dqv(n), dkv(n), dvv(n), ddo(n), ro(n), rl((size_t)H * T), rdq(n),
        rdk(n), rdv(n);
    for (size_t i = 0; i < n; ++i) {
        dqv[i] = from_bf16(hq[i]);
        dkv[i] = from_bf16(hk[i]);
        dvv[i] = from_bf16(hv[i]);
        ddo[i] = from_bf16(hdo[i]);
    }
    if (oracle_fwd(dqv.data(), dkv.data(), dvv.data(), off.data(), batch, T, H, D, B, W, scale,
                   ro.data(), rl.data()) != 0 ||
        oracle_bwd(dqv.data(), dkv.data(), dvv.data(), ddo.data(), off.data(), batch, T, H, D,
                   B, W, scale, rdq.data(), rdk.data(), rdv.data()) != 0) {
        std::printf("FAIL %s: oracle rejected the case\n", what);
        ++failures;
        return;
    }
    check(what, "out", compare(gout, ro), 2e-2, 2e-3);
    Errors el;
    for (size_t i = 0; i < rl.size(); ++i) {
        const double d = std::fabs((double)glse[i] - rl[i]);
        el.max_abs = std::fmax(el.max_abs, d);
        el.sum_abs += d;
    }
    el.n = rl.size();
    check(what, "lse", el, 1e-3, 1e-3);
    check(what, "dq", compare(gdq, rdq), 2e-2, 2e-3);
    check(what, "dk", compare(gdk, rdk), 2e-2, 2e-3);
    check(what, "dv", compare(gdv, rdv), 2e-2, 2e-3);
    for (void *p : {(void *)q, (void *)k, (void *)v, (void *)dout, (void *)doff, (void *)out,
                    (void *)dq, (void *)dk, (void *)dv, (void *)lse, ws})
        HIP_OK(hipFree(p));
}

// Calls the library must refuse before any launch (pointers are never
// dereferenced on these paths).
void check_rejections(hipStream_t stream) {
    std::printf("status codes\n");
    void *p = nullptr;
    HIP_OK(hipMalloc(&p, 1 << 20));
    const int32_t *off = (const int32_t *)p;
    struct Want {
        const char *what;
        blockattn_status got, want;
    } cases[] = {
        {"head_dim 48", blockattn_fwd(p, p, p, off, 1, 16, 1, 48, 16, 1, 0.1f, BLOCKATTN_BF16, p,
                                      (float *)p, stream),
         BLOCKATTN_ERR_UNSUPPORTED},
        {"window 0", blockattn_fwd(p, p, p, off, 1, 16, 1, 64, 16, 0, 0.1f, BLOCKATTN_BF16, p,
                                   (float *)p, stream),
         BLOCKATTN_ERR_INVALID_ARGUMENT},
        {"non-finite scale", blockattn_fwd(p, p, p, off, 1, 16, 1, 64, 16, 1, NAN,
                                           BLOCKATTN_BF16, p, (float *)p, stream),
         BLOCKATTN_ERR_INVALID_ARGUMENT},
        {"null out", blockattn_fwd(p, p, p, off, 1, 16, 1, 64, 16, 1, 0.1f, BLOCKATTN_BF16,
                                   nullptr, (float *)p, stream),
         BLOCKATTN_ERR_INVALID_ARGUMENT},
        {"workspace too small",
         blockattn_bwd(p, p, p, p, p, (const float *)p, off, 1, 16, 1, 64, 16, 1, 0.1f,
                       BLOCKATTN_BF16, p, p, p, p, 8, stream),
         BLOCKATTN_ERR_WORKSPACE},
        {"empty batch", blockattn_fwd(nullptr, nullptr, nullptr, nullptr, 0, 0, 1, 64, 16, 1,
                                      0.1f, BLOCKATTN_BF16, nullptr, nullptr, stream),
         BLOCKATTN_OK},
        {"mx_fwd head_dim 32", blockattn_mx_fwd(p, p, p, p, p, off, 1, 16, 1, 32, 16, 1, 0.1f, p,
                                                (float *)p, stream),
         BLOCKATTN_ERR_UNSUPPORTED},
        {"mxpv_fwd head_dim 32", blockattn_mxpv_fwd(p, p, p, p, p, p, off, 1, 16, 1, 32, 16, 1,
                                                    0.1f, p, (float *)p, stream),
         BLOCKATTN_ERR_UNSUPPORTED},
        {"mx_bwd head_dim 32",
         blockattn_mx_bwd(p, p, p, p, p, p, p, p, p, p, p, p, p, p, p, (const float *)p, off, 1,
                          16, 1, 32, 16, 1, 0.1f, p, p, p, p, 1 << 20, stream),
         BLOCKATTN_ERR_UNSUPPORTED},
        {"mx_bwd misaligned scale",
         blockattn_mx_bwd(p, p, p, p, p, p, p, p, p, (char *)p + 2, p, p, p, p, p,
                          (const float *)p, off, 1, 16, 1, 64, 16, 1, 0.1f, p, p, p, p, 1 << 20,
                          stream),
         BLOCKATTN_ERR_INVALID_ARGUMENT},
        {"mx_bwd null dout_t",
         blockattn_mx_bwd(p, p, p, p, p, p, p, p, p, p, p, p, nullptr, p, p, (const float *)p,
                          off, 1, 16, 1, 64, 16, 1, 0.1f, p, p, p, p, 1 << 20, stream),
         BLOCKATTN_ERR_INVALID_ARGUMENT},
        {"mx_bwd workspace small",
         blockattn_mx_bwd(p, p, p, p, p, p, p, p, p, p, p, p, p, p, p, (const float *)p, off, 1,
                          16, 1, 64, 16, 1, 0.1f, p, p, p, p, 8, stream),
         BLOCKATTN_ERR_WORKSPACE},
    };
    for (const Want &w : cases) {
        const bool ok = w.got == w.want;
        std::printf("  %-22s %s (%s)\n", w.what, blockattn_status_string(w.got),
                    ok ? "ok" : "FAIL");
        if (!ok) ++failures;
    }
    HIP_OK(hipFree(p));
}

}  // namespace

int main() {
    std::printf("blockattn ABI version %d\n", blockattn_abi_version());
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    check_rejections(stream);
    run_case({300, 17, 0, 129, 1000}, 2, 64, 64, 2, 11, stream);
    run_case({700, 256, 40}, 2, 128, 256, 3, 12, stream);
    run_case({513, 5, 260}, 3, 32, 48, 2, 13, stream);
    HIP_OK(hipStreamDestroy(stream));
    std::printf("%s (%d failure%s)\n", failures ? "FAILED" : "PASSED", failures,
                failures == 1 ? "" : "s");
    return failures ? 1 : 0;
}
