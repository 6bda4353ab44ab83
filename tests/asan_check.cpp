// Host AddressSanitizer run of the C ABI's argument checks and of the fp64
// oracle.  Built with the host side of the library instrumented (hipcc
// -Xarch_host -fsanitize=address; device code is not), and run without a
// GPU: every call below is one the library must reject, or treat as empty,
// before any HIP call, so the checks and their error paths execute under the
// sanitizer.  The oracle runs on small seeded inputs, including empty users,
// one-token users and block or window sizes far beyond the users.
// Exit status 0 when every check passes (the sanitizer aborts on a fault).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "blockattn.h"

extern "C" {
int oracle_fwd(const double *q, const double *k, const double *v, const int32_t *offsets,
               int batch, int64_t T, int H, int D, int B, int W, double scale, double *out,
               double *lse);
int oracle_bwd(const double *q, const double *k, const double *v, const double *dout,
               const int32_t *offsets, int batch, int64_t T, int H, int D, int B, int W,
               double scale, double *dq, double *dk, double *dv);
int oracle_gdpa_fwd(const double *q, const double *k, const double *v, const int32_t *offsets,
                    int batch, int64_t T, int H, int D, int B, int W, double scale, int act,
                    double *out);
int oracle_gdpa_bwd(const double *q, const double *k, const double *v, const double *dout,
                    const int32_t *offsets, int batch, int64_t T, int H, int D, int B, int W,
                    double scale, int act, double *dq, double *dk, double *dv);
int64_t oracle_pair_count(const int32_t *offsets, int batch, int B, int W);
int oracle_mxpv_fwd(const double *q, const double *k, const double *v, const int32_t *offsets,
                    int batch, int64_t T, int H, int D, int B, int W, double scale, double *out,
                    double *lse);
int oracle_mxpv_slack(const double *q, const double *k, const double *v,
                      const int32_t *offsets, int batch, int64_t T, int H, int D, int B, int W,
                      double scale, const double *eps2, double *slack);
int oracle_mx_bwd(const double *q, const double *k, const double *v, const double *dout,
                  const double *out, const double *lse, const double *qt, const double *kt,
                  const double *dot_t, const int32_t *offsets, int batch, int64_t T, int H,
                  int D, int B, int W, double scale, int quant, double *dq, double *dk,
                  double *dv);
int oracle_mx_bwd_bounds(const double *q, const double *k, const double *v,
                         const double *dout, const double *out, const double *lse,
                         const double *qt, const double *kt, const double *dot_t,
                         const int32_t *offsets, int batch, int64_t T, int H, int D, int B,
                         int W, double scale, double rho, double *dq, double *dk, double *dv,
                         double *sl_dq, double *sl_dk, double *sl_dv, double *ab_dq,
                         double *ab_dk, double *ab_dv);
void oracle_mx_quantize_block(double *x, int64_t n);
}

namespace {

int failures = 0;

void expect(bool ok, const char *what) {
    if (!ok) {
        std::printf("FAIL: %s\n", what);
        ++failures;
    }
}

// An aligned, non-null address that is never dereferenced on these paths.
void *const kFake = reinterpret_cast<void *>(uintptr_t(0x1000));

blockattn_status fwd(int32_t batch, int64_t T, int32_t H, int32_t D, int32_t B, int32_t W,
                     float scale, int dtype, void *q, void *out, void *lse,
                     const int32_t *offsets) {
    return blockattn_fwd(q, kFake, kFake, offsets, batch, T, H, D, B, W, scale,
                         (blockattn_dtype)dtype, out, (float *)lse, nullptr);
}

void abi_checks() {
    const int32_t *off = (const int32_t *)kFake;
    const float nan = std::nanf("");
    expect(fwd(-1, 100, 2, 64, 64, 2, 0.125f, 0, kFake, kFake, kFake, off) ==
               BLOCKATTN_ERR_INVALID_ARGUMENT, "negative batch");
    expect(fwd(2, -5, 2, 64, 64, 2, 0.125f, 0, kFake, kFake, kFake, off) ==
               BLOCKATTN_ERR_INVALID_ARGUMENT, "negative T");
    expect(fwd(2, 100, 0, 64, 64, 2, 0.125f, 0, kFake, kFake, kFake, off) ==
               BLOCKATTN_ERR_INVALID_ARGUMENT, "H = 0");
    expect(fwd(2, 100, 2, 64, 0, 2, 0.125f, 0, kFake, kFake, kFake, off) ==
               BLOCKATTN_ERR_INVALID_ARGUMENT, "B = 0");
    expect(fwd(2, 100, 2, 64, 64, 0, 0.125f, 0, kFake, kFake, kFake, off) ==
               BLOCKATTN_ERR_INVALID_ARGUMENT, "W = 0");
    expect(fwd(2, 100, 2, 64, 64, 2, nan, 0, kFake, kFake, kFake, off) ==
               BLOCKATTN_ERR_INVALID_ARGUMENT, "NaN scale");
    expect(fwd(2, 100, 2, 64, 64, 2, 0.125f, 7, kFake, kFake, kFake, off) ==
               BLOCKATTN_ERR_INVALID_ARGUMENT, "unknown dtype");
    expect(fwd(2, 100, 2, 48, 64, 2, 0.125f, 0, kFake, kFake, kFake, off) ==
               BLOCKATTN_ERR_UNSUPPORTED, "D = 48");
    expect(fwd(1, (int64_t)1 << 31, 2, 64, 64, 2, 0.125f, 0, kFake, kFake, kFake, off) ==
               BLOCKATTN_ERR_UNSUPPORTED, "T = 2^31");
    expect(fwd(2, 100, 200000, 128, 64, 2, 0.125f, 0, kFake, kFake, kFake, off) ==
               BLOCKATTN_ERR_UNSUPPORTED, "128 H D 4 >= 2^32");
    expect(fwd(2, 100, INT32_MAX, 32, INT32_MAX, INT32_MAX, 0.125f, 0, kFake, kFake, kFake,
               off) == BLOCKATTN_ERR_UNSUPPORTED, "H = 2^31-1");
    expect(fwd(2, 100, 2, 64, 64, 2, 0.125f, 0, nullptr, kFake, kFake, off) ==
               BLOCKATTN_ERR_INVALID_ARGUMENT, "null q");
    expect(fwd(2, 100, 2, 64, 64, 2, 0.125f, 0, kFake, (char *)kFake + 8, kFake, off) ==
               BLOCKATTN_ERR_INVALID_ARGUMENT, "misaligned out");
    expect(fwd(2, 100, 2, 64, 64, 2, 0.125f, 0, kFake, kFake, kFake, nullptr) ==
               BLOCKATTN_ERR_INVALID_ARGUMENT, "null offsets");
    expect(fwd(2, 0, 2, 64, INT32_MAX, INT32_MAX, 0.125f, 0, nullptr, nullptr, nullptr,
               nullptr) == BLOCKATTN_OK, "empty call with huge B, W");
    expect(blockattn_bwd(kFake, kFake, kFake, kFake, nullptr, (float *)kFake, off, 2, 100, 2, 64,
                         64, 2, 0.125f, BLOCKATTN_BF16, kFake, kFake, kFake, kFake, 1 << 20,
                         nullptr) == BLOCKATTN_ERR_INVALID_ARGUMENT, "bwd null dout");
    expect(blockattn_bwd(kFake, kFake, kFake, kFake, kFake, (float *)kFake, off, 2, 100, 2, 64,
                         64, 2, 0.125f, BLOCKATTN_BF16, kFake, kFake, kFake, nullptr, 0,
                         nullptr) == BLOCKATTN_ERR_WORKSPACE, "bwd without workspace");
    expect(blockattn_bwd(kFake, kFake, kFake, kFake, kFake, (float *)kFake, off, 2, 100, 2, 64,
                         64, 2, 0.125f, BLOCKATTN_BF16, kFake, kFake, kFake, (char *)kFake + 64,
                         1 << 20, nullptr) == BLOCKATTN_ERR_WORKSPACE, "misaligned workspace");
    expect(blockattn_bwd_noalloc(kFake, kFake, kFake, kFake, kFake, (float *)kFake, off, 2,
                                 (int64_t)4 << 20, 8, 64, 64, 2, 0.125f, BLOCKATTN_BF16, kFake,
                                 kFake, kFake, nullptr) == BLOCKATTN_ERR_WORKSPACE,
           "noalloc beyond its array");
    expect(blockattn_mx_fwd(kFake, kFake, kFake, kFake, kFake, off, 2, 100, 2, 32, 64, 2, 0.125f,
                            kFake, (float *)kFake, nullptr) == BLOCKATTN_ERR_UNSUPPORTED,
           "mx D = 32");
    expect(blockattn_mxpv_fwd(kFake, kFake, kFake, kFake, kFake, kFake, off, 2, 100, 2, 32, 64,
                              2, 0.125f, kFake, (float *)kFake, nullptr) ==
               BLOCKATTN_ERR_UNSUPPORTED, "mxpv D = 32");
    expect(blockattn_mxpv_fwd(kFake, kFake, kFake, kFake, nullptr, kFake, off, 2, 100, 2, 64, 64,
                              2, 0.125f, kFake, (float *)kFake, nullptr) ==
               BLOCKATTN_ERR_INVALID_ARGUMENT, "mxpv null v_t");
    expect(blockattn_mx_bwd(kFake, kFake, kFake, kFake, kFake, kFake, kFake, kFake, kFake, kFake,
                            kFake, kFake, kFake, kFake, kFake, (const float *)kFake, off, 2, 100,
                            2, 32, 64, 2, 0.125f, kFake, kFake, kFake, kFake, 1 << 20,
                            nullptr) == BLOCKATTN_ERR_UNSUPPORTED, "mx_bwd D = 32");
    expect(blockattn_mx_bwd(kFake, kFake, kFake, kFake, kFake, kFake, kFake, kFake, kFake,
                            (char *)kFake + 2, kFake, kFake, kFake, kFake, kFake,
                            (const float *)kFake, off, 2, 100, 2, 64, 64, 2, 0.125f, kFake,
                            kFake, kFake, kFake, 1 << 20, nullptr) ==
               BLOCKATTN_ERR_INVALID_ARGUMENT, "mx_bwd misaligned scale");
    expect(blockattn_mx_bwd(kFake, kFake, kFake, kFake, kFake, kFake, kFake, kFake, kFake, kFake,
                            kFake, kFake, kFake, kFake, kFake, (const float *)kFake, off, 2, 100,
                            2, 64, 64, 2, 0.125f, kFake, kFake, kFake, kFake, 16,
                            nullptr) == BLOCKATTN_ERR_WORKSPACE, "mx_bwd workspace small");
    expect(blockattn_mx_bwd(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                            nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                            nullptr, off, 2, 0, 2, 64, INT32_MAX, INT32_MAX, 0.125f, nullptr,
                            nullptr, nullptr, nullptr, 0, nullptr) == BLOCKATTN_OK,
           "mx_bwd empty");
    expect(blockattn_rope(kFake, kFake, off, 2, 100, 2, 64, 0.f, BLOCKATTN_BF16, kFake, kFake,
                          nullptr) == BLOCKATTN_ERR_INVALID_ARGUMENT, "rope base 0");
    expect(blockattn_gdpa_fwd(kFake, kFake, kFake, off, 2, 100, 2, 64, 64, 2, 0.125f, 3,
                              BLOCKATTN_BF16, kFake, nullptr) == BLOCKATTN_ERR_INVALID_ARGUMENT,
           "gdpa activation 3");
    expect(blockattn_bwd_workspace_size(-1, 1, 8, BLOCKATTN_BF16) == SIZE_MAX, "ws T < 0");
    expect(blockattn_bwd_workspace_size(100, 2, 8, BLOCKATTN_FP32) == 0, "ws fp32");
    for (int s = -1; s <= 5; ++s) expect(blockattn_status_string((blockattn_status)s) != nullptr,
                                         "status string");
}

// Small seeded values (splitmix64 -> [-1, 1)).
std::vector<double> values(size_t n, uint64_t seed) {
    std::vector<double> x(n);
    for (size_t i = 0; i < n; ++i) {
        uint64_t z = (seed += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        x[i] = (double)((z ^ (z >> 31)) >> 11) * (2.0 / 9007199254740992.0) - 1.0;
    }
    return x;
}

void oracle_checks() {
    struct Case { std::vector<int32_t> len; int H, D, B, W; };
    const Case cases[] = {{{0, 1, 37, 0, 70}, 2, 8, 4, 2},
                          {{5, 64}, 1, 4, 1, 3},
                          {{129, 3}, 3, 16, 64, 1},
                          {{40, 13}, 2, 4, INT32_MAX, INT32_MAX},
                          {{}, 1, 4, 8, 2}};
    for (const Case &c : cases) {
        std::vector<int32_t> off(c.len.size() + 1, 0);
        for (size_t u = 0; u < c.len.size(); ++u) off[u + 1] = off[u] + c.len[u];
        const int batch = (int)c.len.size();
        const int64_t T = off[batch];
        const size_t n = (size_t)T * c.H * c.D;
        auto q = values(n, 1), k = values(n, 2), v = values(n, 3), d = values(n, 4);
        std::vector<double> o(n), lse((size_t)c.H * T), dq(n), dk(n), dv(n);
        expect(oracle_fwd(q.data(), k.data(), v.data(), off.data(), batch, T, c.H, c.D, c.B, c.W,
                          0.5, o.data(), lse.data()) == 0, "oracle_fwd");
        expect(oracle_bwd(q.data(), k.data(), v.data(), d.data(), off.data(), batch, T, c.H, c.D,
                          c.B, c.W, 0.5, dq.data(), dk.data(), dv.data()) == 0, "oracle_bwd");
        for (int act = 1; act <= 2; ++act) {
            expect(oracle_gdpa_fwd(q.data(), k.data(), v.data(), off.data(), batch, T, c.H, c.D,
                                   c.B, c.W, 0.5, act, o.data()) == 0, "oracle_gdpa_fwd");
            expect(oracle_gdpa_bwd(q.data(), k.data(), v.data(), d.data(), off.data(), batch, T,
                                   c.H, c.D, c.B, c.W, 0.5, act, dq.data(), dk.data(),
                                   dv.data()) == 0, "oracle_gdpa_bwd");
        }
        for (double x : o) expect(std::isfinite(x), "finite output");
        expect(oracle_pair_count(off.data(), batch, c.B, c.W) >= 0, "pair count");
        // the MXFP8 definitions on the same shapes (the values need not be
        // codes: the oracle's quantization applies to whatever it is given)
        expect(oracle_mxpv_fwd(q.data(), k.data(), v.data(), off.data(), batch, T, c.H, c.D, c.B,
                               c.W, 0.5, o.data(), lse.data()) == 0, "oracle_mxpv_fwd");
        std::vector<double> eps2((size_t)c.H * T, 1e-3), sl(n);
        expect(oracle_mxpv_slack(q.data(), k.data(), v.data(), off.data(), batch, T, c.H, c.D,
                                 c.B, c.W, 0.5, eps2.data(), sl.data()) == 0, "oracle_mxpv_slack");
        expect(oracle_fwd(q.data(), k.data(), v.data(), off.data(), batch, T, c.H, c.D, c.B, c.W,
                          0.5, o.data(), lse.data()) == 0, "oracle_fwd for the mx backward");
        for (int quant = 0; quant <= 1; ++quant)
            expect(oracle_mx_bwd(q.data(), k.data(), v.data(), d.data(), o.data(), lse.data(),
                                 q.data(), k.data(), d.data(), off.data(), batch, T, c.H, c.D,
                                 c.B, c.W, 0.5, quant, dq.data(), dk.data(), dv.data()) == 0,
                   "oracle_mx_bwd");
        std::vector<double> s1(n), s2(n), s3(n), a1(n), a2(n), a3(n);
        expect(oracle_mx_bwd_bounds(q.data(), k.data(), v.data(), d.data(), o.data(), lse.data(),
                                    q.data(), k.data(), d.data(), off.data(), batch, T, c.H, c.D,
                                    c.B, c.W, 0.5, 1.0 / 2048, dq.data(), dk.data(), dv.data(),
                                    s1.data(), s2.data(), s3.data(), a1.data(), a2.data(),
                                    a3.data()) == 0, "oracle_mx_bwd_bounds");
        for (double x : dq) expect(std::isfinite(x), "finite mx dq");
    }
    // the block rule on odd lengths, zeros and a lone value
    for (int64_t len : {0, 1, 31, 33, 95}) {
        std::vector<double> b = values((size_t)len, 7);
        if (len > 2) b[1] = 0.0;
        oracle_mx_quantize_block(b.data(), len);
        for (double x : b) expect(std::isfinite(x), "finite block codes");
    }
    oracle_mx_quantize_block(nullptr, 5);
    // malformed offsets are rejected, not read past
    const int32_t bad[3] = {0, 9, 4};
    std::vector<double> x(64, 0.0), y(64, 0.0), l(16, 0.0);
    expect(oracle_fwd(x.data(), x.data(), x.data(), bad, 2, 4, 1, 4, 4, 1, 1.0, y.data(),
                      l.data()) == -1, "decreasing offsets rejected");
}

}  // namespace

int main() {
    abi_checks();
    oracle_checks();
    std::printf("%s (%d failures)\n", failures ? "FAILED" : "PASSED", failures);
    return failures ? 1 : 0;
}
