/*
 * Block-attention oracle: plain, slow, fp64 CPU implementation of the
 * definition.  TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load this library; the
 * product path never calls it and shares no code with it.
 *
 * What it computes.  "GEM (Meta)" (aiwiki.ai), section "Custom kernels",
 * says BlockAttention splits long user-history self-attention into
 * independent 64-token block computations; the ai.info news item, section
 * "Kunlun changes how GEM scales", and the sysdesai.com summary, section
 * "Kunlun Architecture Details", say block attention is sparse attention
 * arranged in blocks whose cost is linear in sequence length for a fixed
 * window.  "GEM (Meta)", section "Training infrastructure", says the
 * sequences are jagged (per-user lengths, no padding).  The pages give no
 * formula; the readings taken here are:
 *
 *   - each user u owns tokens [offsets[u], offsets[u+1]) of a packed
 *     [T, H, D] tensor; indices below are local to the user;
 *   - blocks of B tokens start at the user's first token (the last one may
 *     be partial) and never straddle users;
 *   - query i sees key j iff  j <= i  and  floor(i/B) - floor(j/B) <= W-1,
 *     i.e. its own block up to itself plus the W-1 previous blocks;
 *   - scores s_ij = scale * <q_i, k_j>, softmax over the visible set,
 *     O_i = sum_j P_ij v_j, lse_i = ln sum_j exp(s_ij)  (natural log,
 *     scale included);
 *   - backward: dP_ij = <dO_i, v_j>, delta_i = sum_j P_ij dP_ij,
 *     dS_ij = P_ij (dP_ij - delta_i), dQ_i = scale sum_j dS_ij k_j,
 *     dK_j = scale sum_i dS_ij q_i, dV_j = sum_i P_ij dO_i.
 *
 * The softmax is two-pass (max, then sum of exponentials) over the visible
 * range of each query, in fp64; delta comes from P and dP, not from <dO,O>.
 * Work is split over (user, head) pairs with OpenMP; every output element is
 * written by exactly one thread in a fixed order, so results do not depend
 * on the thread count.
 *
 * Layouts: q, k, v, out, dout, dq, dk, dv are fp64 [T, H, D] row-major;
 * lse is fp64 [H, T]; offsets is int32 [batch+1].
 * Return value: 0 on success, -1 on invalid arguments or malformed offsets,
 * -2 if scratch memory could not be allocated.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* First local key index visible to local query i (window start). */
static int64_t first_visible(int64_t i, int64_t B, int64_t W)
{
    int64_t blk = i / B - (W - 1);
    return (blk < 0 ? 0 : blk) * B;
}

static int check_args(const int32_t *offsets, int batch, int64_t T, int H, int D,
                      int B, int W)
{
    if (batch < 0 || T < 0 || H < 1 || D < 1 || B < 1 || W < 1 || !offsets)
        return -1;
    if (offsets[0] != 0 || (int64_t)offsets[batch] != T)
        return -1;
    for (int u = 0; u < batch; ++u)
        if (offsets[u + 1] < offsets[u])
            return -1;
    return 0;
}

/* Scratch length for one query's visible scores: at most W * B keys, and
 * never more than the longest user (so huge B or W cost nothing). */
static size_t visible_max(const int32_t *offsets, int batch, int B, int W)
{
    int64_t lmax = 1;
    for (int u = 0; u < batch; ++u) {
        const int64_t L = (int64_t)offsets[u + 1] - offsets[u];
        if (L > lmax)
            lmax = L;
    }
    const int64_t wb = (int64_t)W * (int64_t)B;
    return (size_t)(wb < lmax ? wb : lmax);
}

static double dot(const double *a, const double *b, int D)
{
    double s = 0.0;
    for (int d = 0; d < D; ++d)
        s += a[d] * b[d];
    return s;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the OpenMP thread count of later calls (n >= 1); results do not
 * depend on it.  Used to time the oracle on one thread. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Sum over all users of the number of visible keys per query (one head). */
int64_t oracle_pair_count(const int32_t *offsets, int batch, int B, int W)
{
    if (batch < 0 || B < 1 || W < 1 || !offsets)
        return -1;
    int64_t total = 0;
    for (int u = 0; u < batch; ++u) {
        int64_t L = (int64_t)offsets[u + 1] - offsets[u];
        for (int64_t i = 0; i < L; ++i)
            total += i - first_visible(i, B, W) + 1;
    }
    return total;
}

/* Forward pass: out [T,H,D] and lse [H,T]. */
int oracle_fwd(const double *q, const double *k, const double *v,
               const int32_t *offsets, int batch, int64_t T, int H, int D,
               int B, int W, double scale, double *out, double *lse)
{
    if (check_args(offsets, batch, T, H, D, B, W))
        return -1;
    int status = 0;
    const int64_t npairs = (int64_t)batch * H;
    const int64_t rs = (int64_t)H * D; /* token stride */
    const size_t nvis = visible_max(offsets, batch, B, W);
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * nvis);
        if (!s) {
#pragma omp atomic write
            status = -2;
        }
#pragma omp for schedule(static)
        for (int64_t p = 0; p < npairs; ++p) {
            if (!s)
                continue;
            const int u = (int)(p / H), h = (int)(p % H);
            const int64_t t0 = offsets[u];
            const int64_t L = (int64_t)offsets[u + 1] - t0;
            for (int64_t i = 0; i < L; ++i) {
                const double *qi = q + (t0 + i) * rs + (int64_t)h * D;
                const int64_t j0 = first_visible(i, B, W);
                const int64_t n = i - j0 + 1;
                /* pass 1: scores and their maximum */
                double m = -INFINITY;
                for (int64_t t = 0; t < n; ++t) {
                    const double *kj = k + (t0 + j0 + t) * rs + (int64_t)h * D;
                    s[t] = scale * dot(qi, kj, D);
                    if (s[t] > m)
                        m = s[t];
                }
                /* pass 2: normaliser */
                double l = 0.0;
                for (int64_t t = 0; t < n; ++t)
                    l += exp(s[t] - m);
                double *oi = out + (t0 + i) * rs + (int64_t)h * D;
                for (int d = 0; d < D; ++d)
                    oi[d] = 0.0;
                for (int64_t t = 0; t < n; ++t) {
                    const double pij = exp(s[t] - m) / l;
                    const double *vj = v + (t0 + j0 + t) * rs + (int64_t)h * D;
                    for (int d = 0; d < D; ++d)
                        oi[d] += pij * vj[d];
                }
                lse[(int64_t)h * T + t0 + i] = m + log(l);
            }
        }
        free(s);
    }
    return status;
}

/* Backward pass: dq, dk, dv [T,H,D] from the upstream gradient dout. */
int oracle_bwd(const double *q, const double *k, const double *v,
               const double *dout, const int32_t *offsets, int batch, int64_t T,
               int H, int D, int B, int W, double scale, double *dq, double *dk,
               double *dv)
{
    if (check_args(offsets, batch, T, H, D, B, W))
        return -1;
    int status = 0;
    const int64_t npairs = (int64_t)batch * H;
    const int64_t rs = (int64_t)H * D;
    const size_t nvis = visible_max(offsets, batch, B, W);
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * nvis);
        double *dp = (double *)malloc(sizeof(double) * nvis);
        if (!s || !dp) {
#pragma omp atomic write
            status = -2;
        }
#pragma omp for schedule(static)
        for (int64_t p = 0; p < npairs; ++p) {
            if (!s || !dp)
                continue;
            const int u = (int)(p / H), h = (int)(p % H);
            const int64_t t0 = offsets[u];
            const int64_t L = (int64_t)offsets[u + 1] - t0;
            /* this thread owns rows [t0, t0+L) of head h in dk and dv */
            for (int64_t i = 0; i < L; ++i) {
                double *dki = dk + (t0 + i) * rs + (int64_t)h * D;
                double *dvi = dv + (t0 + i) * rs + (int64_t)h * D;
                for (int d = 0; d < D; ++d)
                    dki[d] = dvi[d] = 0.0;
            }
            for (int64_t i = 0; i < L; ++i) {
                const double *qi = q + (t0 + i) * rs + (int64_t)h * D;
                const double *doi = dout + (t0 + i) * rs + (int64_t)h * D;
                const int64_t j0 = first_visible(i, B, W);
                const int64_t n = i - j0 + 1;
                double m = -INFINITY;
                for (int64_t t = 0; t < n; ++t) {
                    const double *kj = k + (t0 + j0 + t) * rs + (int64_t)h * D;
                    s[t] = scale * dot(qi, kj, D);
                    if (s[t] > m)
                        m = s[t];
                }
                double l = 0.0;
                for (int64_t t = 0; t < n; ++t)
                    l += exp(s[t] - m);
                /* s[] now holds P_ij, dp[] holds dP_ij */
                double delta = 0.0;
                for (int64_t t = 0; t < n; ++t) {
                    const double *vj = v + (t0 + j0 + t) * rs + (int64_t)h * D;
                    s[t] = exp(s[t] - m) / l;
                    dp[t] = dot(doi, vj, D);
                    delta += s[t] * dp[t];
                }
                double *dqi = dq + (t0 + i) * rs + (int64_t)h * D;
                for (int d = 0; d < D; ++d)
                    dqi[d] = 0.0;
                for (int64_t t = 0; t < n; ++t) {
                    const int64_t j = t0 + j0 + t;
                    const double *kj = k + j * rs + (int64_t)h * D;
                    double *dkj = dk + j * rs + (int64_t)h * D;
                    double *dvj = dv + j * rs + (int64_t)h * D;
                    const double ds = s[t] * (dp[t] - delta);
                    for (int d = 0; d < D; ++d) {
                        dqi[d] += scale * ds * kj[d];
                        dkj[d] += scale * ds * qi[d];
                        dvj[d] += s[t] * doi[d];
                    }
                }
            }
        }
        free(s);
        free(dp);
    }
    return status;
}

/*
 * Dense probability matrix of one (user, head): P [L, L] row-major, zero
 * where a key is not visible.  Meant for tiny inputs (row-sum and mask
 * checks); L = offsets[u+1] - offsets[u].
 */
int oracle_probs(const double *q, const double *k, const int32_t *offsets,
                 int batch, int64_t T, int H, int D, int B, int W, double scale,
                 int u, int h, double *P)
{
    if (check_args(offsets, batch, T, H, D, B, W) || u < 0 || u >= batch ||
        h < 0 || h >= H)
        return -1;
    const int64_t rs = (int64_t)H * D;
    const int64_t t0 = offsets[u];
    const int64_t L = (int64_t)offsets[u + 1] - t0;
    memset(P, 0, sizeof(double) * (size_t)(L * L));
    for (int64_t i = 0; i < L; ++i) {
        const double *qi = q + (t0 + i) * rs + (int64_t)h * D;
        const int64_t j0 = first_visible(i, B, W);
        double m = -INFINITY;
        for (int64_t j = j0; j <= i; ++j) {
            const double sij =
                scale * dot(qi, k + (t0 + j) * rs + (int64_t)h * D, D);
            P[i * L + j] = sij;
            if (sij > m)
                m = sij;
        }
        double l = 0.0;
        for (int64_t j = j0; j <= i; ++j)
            l += exp(P[i * L + j] - m);
        for (int64_t j = j0; j <= i; ++j)
            P[i * L + j] = exp(P[i * L + j] - m) / l;
    }
    return 0;
}

/*
 * Generalized dot-product attention on the block pattern.  "GEM (Meta)",
 * section "Custom kernels", describes GDPA as dot-product attention whose
 * softmax is replaced by an activation such as GELU or SiLU.  The pages give
 * no normalisation; the reading taken is none: for each visible pair
 *     x_ij = scale * <q_i, k_j>,   P_ij = act(x_ij),   O_i = sum_j P_ij v_j,
 * with act = SiLU (act == 1: x / (1 + exp(-x))) or GELU (act == 2, the erf
 * form: x * Phi(x), Phi the standard normal CDF).  Backward of sum(dO * O):
 *     dP_ij = <dO_i, v_j>,  dS_ij = act'(x_ij) dP_ij,
 *     dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,
 *     dV_j = sum_i P_ij dO_i.
 * Same layouts, visibility rule, threading and return codes as above;
 * act outside {1, 2} is an invalid argument.
 */
static double act_value(int act, double x)
{
    if (act == 1)
        return x / (1.0 + exp(-x));
    return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
}

static double act_slope(int act, double x)
{
    if (act == 1) {
        const double sg = 1.0 / (1.0 + exp(-x));
        return sg * (1.0 + x * (1.0 - sg));
    }
    const double cdf = 0.5 * (1.0 + erf(x / sqrt(2.0)));
    const double pdf = exp(-0.5 * x * x) / sqrt(2.0 * 3.14159265358979323846);
    return cdf + x * pdf;
}

/* The forward sum, or (absolute != 0) the same sum of absolute terms,
 * sum_j |P_ij| |v_j|: the magnitude a rounding error of each term is
 * relative to, which the GPU parity tests scale their bound by. */
static int gdpa_fwd_sum(const double *q, const double *k, const double *v,
                        const int32_t *offsets, int batch, int64_t T, int H, int D,
                        int B, int W, double scale, int act, int absolute, double *out)
{
    if (check_args(offsets, batch, T, H, D, B, W) || (act != 1 && act != 2))
        return -1;
    const int64_t npairs = (int64_t)batch * H;
    const int64_t rs = (int64_t)H * D;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npairs; ++p) {
        const int u = (int)(p / H), h = (int)(p % H);
        const int64_t t0 = offsets[u];
        const int64_t L = (int64_t)offsets[u + 1] - t0;
        for (int64_t i = 0; i < L; ++i) {
            const double *qi = q + (t0 + i) * rs + (int64_t)h * D;
            double *oi = out + (t0 + i) * rs + (int64_t)h * D;
            for (int d = 0; d < D; ++d)
                oi[d] = 0.0;
            for (int64_t j = first_visible(i, B, W); j <= i; ++j) {
                const double *kj = k + (t0 + j) * rs + (int64_t)h * D;
                const double *vj = v + (t0 + j) * rs + (int64_t)h * D;
                const double pij = act_value(act, scale * dot(qi, kj, D));
                for (int d = 0; d < D; ++d)
                    oi[d] += absolute ? fabs(pij) * fabs(vj[d]) : pij * vj[d];
            }
        }
    }
    return 0;
}

int oracle_gdpa_fwd(const double *q, const double *k, const double *v,
                    const int32_t *offsets, int batch, int64_t T, int H, int D,
                    int B, int W, double scale, int act, double *out)
{
    return gdpa_fwd_sum(q, k, v, offsets, batch, T, H, D, B, W, scale, act, 0, out);
}

int oracle_gdpa_fwd_abs(const double *q, const double *k, const double *v,
                        const int32_t *offsets, int batch, int64_t T, int H, int D,
                        int B, int W, double scale, int act, double *out)
{
    return gdpa_fwd_sum(q, k, v, offsets, batch, T, H, D, B, W, scale, act, 1, out);
}

/* The backward sums, or (absolute != 0) the same sums of absolute terms:
 * |scale| sum_j |dS_ij| |k_j|, |scale| sum_i |dS_ij| |q_i| and
 * sum_i |P_ij| |dO_i|. */
static int gdpa_bwd_sum(const double *q, const double *k, const double *v,
                        const double *dout, const int32_t *offsets, int batch,
                        int64_t T, int H, int D, int B, int W, double scale, int act,
                        int absolute, double *dq, double *dk, double *dv)
{
    if (check_args(offsets, batch, T, H, D, B, W) || (act != 1 && act != 2))
        return -1;
    const int64_t npairs = (int64_t)batch * H;
    const int64_t rs = (int64_t)H * D;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npairs; ++p) {
        const int u = (int)(p / H), h = (int)(p % H);
        const int64_t t0 = offsets[u];
        const int64_t L = (int64_t)offsets[u + 1] - t0;
        for (int64_t i = 0; i < L; ++i)
            for (int d = 0; d < D; ++d) {
                const int64_t o = (t0 + i) * rs + (int64_t)h * D + d;
                dq[o] = dk[o] = dv[o] = 0.0;
            }
        for (int64_t i = 0; i < L; ++i) {
            const double *qi = q + (t0 + i) * rs + (int64_t)h * D;
            const double *doi = dout + (t0 + i) * rs + (int64_t)h * D;
            double *dqi = dq + (t0 + i) * rs + (int64_t)h * D;
            for (int64_t j = first_visible(i, B, W); j <= i; ++j) {
                const int64_t oj = (t0 + j) * rs + (int64_t)h * D;
                const double x = scale * dot(qi, k + oj, D);
                const double pij = act_value(act, x);
                const double ds = act_slope(act, x) * dot(doi, v + oj, D);
                for (int d = 0; d < D; ++d) {
                    if (absolute) {
                        dqi[d] += fabs(scale * ds) * fabs(k[oj + d]);
                        dk[oj + d] += fabs(scale * ds) * fabs(qi[d]);
                        dv[oj + d] += fabs(pij) * fabs(doi[d]);
                    } else {
                        dqi[d] += scale * ds * k[oj + d];
                        dk[oj + d] += scale * ds * qi[d];
                        dv[oj + d] += pij * doi[d];
                    }
                }
            }
        }
    }
    return 0;
}

int oracle_gdpa_bwd(const double *q, const double *k, const double *v,
                    const double *dout, const int32_t *offsets, int batch,
                    int64_t T, int H, int D, int B, int W, double scale, int act,
                    double *dq, double *dk, double *dv)
{
    return gdpa_bwd_sum(q, k, v, dout, offsets, batch, T, H, D, B, W, scale, act, 0, dq,
                        dk, dv);
}

int oracle_gdpa_bwd_abs(const double *q, const double *k, const double *v,
                        const double *dout, const int32_t *offsets, int batch,
                        int64_t T, int H, int D, int B, int W, double scale, int act,
                        double *dq, double *dk, double *dv)
{
    return gdpa_bwd_sum(q, k, v, dout, offsets, batch, T, H, D, B, W, scale, act, 1, dq,
                        dk, dv);
}

/* ------------------------------------------------------------------------
 * MXFP8 attention with the weights quantized too.  "GEM (Meta)" (aiwiki.ai),
 * section "Custom kernels", says production attention runs in MXFP8, and
 * section "Ultra-low-precision training" that the matmuls are block-scaled
 * MXFP8 end to end.  For P.V that means the softmax weights are themselves
 * quantized to E4M3 with one shared power-of-two scale per 32 elements
 * along the product's contraction axis (the keys).  The pages say no more;
 * the readings taken here:
 *
 *   - q, k, v arrive decoded (exact fp64 values of their MXFP8 codes);
 *     scores s_ij, visibility and lse are those of oracle_fwd;
 *   - with t_ij = s_ij log2(e), a weight is 2^t_ij up to a factor common to
 *     the row, which cancels;
 *   - the keys of a query fall into blocks of 32 consecutive positions
 *     counted from its user's first token (block index = local key / 32),
 *     so a user's result does not depend on the other users of the batch;
 *     a block may hold keys the query does not see, which weigh 0;
 *   - in block b, with F_b = floor(max of t_ij over its visible keys), each
 *     visible weight is stored as 2^(F_b - 7) * R(2^(t_ij - F_b + 7)), R the
 *     nearest E4M3 value, ties to the even code.  The argument stays below
 *     2^8 (the E4M3 maximum is 448), so nothing saturates;
 *   - O_i = sum_j Pq_ij v_j / sum_j 2^t_ij: the normaliser and lse come
 *     from the unquantized weights.
 * Shifting every t_ij of a row by an integer shifts every F_b by the same
 * integer and leaves the codes, hence O_i, unchanged.
 */

static const double kLog2e = 1.4426950408889634; /* log2(e) */

/* Nearest E4M3 value to x >= 0 (x < 2^8 + 2^4), ties to the even code:
 * subnormals are multiples of 2^-9 below 2^-6, normals have 3 fraction
 * bits. */
double oracle_e4m3_round(double x)
{
    if (!(x > 0.0))
        return 0.0;
    int e;
    (void)frexp(x, &e); /* x = f 2^e, f in [0.5, 1): floor(log2 x) = e - 1 */
    const int q = e - 1 < -6 ? -9 : e - 1 - 3; /* exponent of the quantum */
    return ldexp(rint(ldexp(x, -q)), q);      /* rint: nearest, ties even */
}

/* The block maxima F_b of row i: t[0..n) are the row's t_ij for local keys
 * j0 .. j0 + n - 1; fb[] gets F of each key's block. */
static void block_floor(const double *t, int64_t n, int64_t g0, double *fb)
{
    int64_t a = 0;
    while (a < n) {
        const int64_t blk = (g0 + a) / 32;
        int64_t e = a;
        double mx = -INFINITY;
        while (e < n && (g0 + e) / 32 == blk) {
            if (t[e] > mx)
                mx = t[e];
            ++e;
        }
        const double f = floor(mx);
        for (int64_t x = a; x < e; ++x)
            fb[x] = f;
        a = e;
    }
}

/* Forward with quantized weights: out [T,H,D], lse [H,T]. */
int oracle_mxpv_fwd(const double *q, const double *k, const double *v,
                    const int32_t *offsets, int batch, int64_t T, int H, int D,
                    int B, int W, double scale, double *out, double *lse)
{
    if (check_args(offsets, batch, T, H, D, B, W))
        return -1;
    int status = 0;
    const int64_t npairs = (int64_t)batch * H;
    const int64_t rs = (int64_t)H * D;
    const size_t nvis = visible_max(offsets, batch, B, W);
#pragma omp parallel
    {
        double *t = (double *)malloc(sizeof(double) * nvis * 2);
        if (!t) {
#pragma omp atomic write
            status = -2;
        }
#pragma omp for schedule(static)
        for (int64_t p = 0; p < npairs; ++p) {
            if (!t)
                continue;
            double *fb = t + nvis;
            const int u = (int)(p / H), h = (int)(p % H);
            const int64_t t0 = offsets[u];
            const int64_t L = (int64_t)offsets[u + 1] - t0;
            for (int64_t i = 0; i < L; ++i) {
                const double *qi = q + (t0 + i) * rs + (int64_t)h * D;
                const int64_t j0 = first_visible(i, B, W);
                const int64_t n = i - j0 + 1;
                double m = -INFINITY;
                for (int64_t x = 0; x < n; ++x) {
                    const double *kj = k + (t0 + j0 + x) * rs + (int64_t)h * D;
                    t[x] = scale * dot(qi, kj, D) * kLog2e;
                    if (t[x] > m)
                        m = t[x];
                }
                /* weights relative to 2^M, M = floor of the row maximum
                 * (an integer shift, which changes no code) */
                const double M = floor(m);
                block_floor(t, n, j0, fb);
                double l = 0.0;
                for (int64_t x = 0; x < n; ++x)
                    l += exp2(t[x] - M);
                double *oi = out + (t0 + i) * rs + (int64_t)h * D;
                for (int d = 0; d < D; ++d)
                    oi[d] = 0.0;
                for (int64_t x = 0; x < n; ++x) {
                    const double pq =
                        ldexp(oracle_e4m3_round(exp2(t[x] - fb[x] + 7.0)), (int)(fb[x] - 7.0 - M));
                    const double *vj = v + (t0 + j0 + x) * rs + (int64_t)h * D;
                    for (int d = 0; d < D; ++d)
                        oi[d] += pq * vj[d];
                }
                for (int d = 0; d < D; ++d)
                    oi[d] /= l;
                lse[(int64_t)h * T + t0 + i] = (M + log2(l)) / kLog2e;
            }
        }
        free(t);
    }
    return status;
}

/* Parity allowance for oracle_mxpv_fwd (test support, not part of the
 * definition).  A computation whose t_ij are off by at most eps2[h*T + i]
 * (log2 units) may round a weight to the neighbouring E4M3 value when its
 * scaled argument lies that close to a midpoint, and may pick F_b one
 * apart when the block maximum lies that close to an integer (which moves
 * only the weights below 2^(F_b - 13), the E4M3 subnormal range).  For each
 * output element, slack = sum_j a_ij |v_jd| / l_i, with a_ij the largest
 * change of Pq_ij those flips allow (0 for a weight no flip can reach). */
int oracle_mxpv_slack(const double *q, const double *k, const double *v,
                      const int32_t *offsets, int batch, int64_t T, int H, int D,
                      int B, int W, double scale, const double *eps2, double *slack)
{
    if (check_args(offsets, batch, T, H, D, B, W))
        return -1;
    int status = 0;
    const int64_t npairs = (int64_t)batch * H;
    const int64_t rs = (int64_t)H * D;
    const size_t nvis = visible_max(offsets, batch, B, W);
#pragma omp parallel
    {
        double *t = (double *)malloc(sizeof(double) * nvis * 2);
        if (!t) {
#pragma omp atomic write
            status = -2;
        }
#pragma omp for schedule(static)
        for (int64_t p = 0; p < npairs; ++p) {
            if (!t)
                continue;
            double *fb = t + nvis;
            const int u = (int)(p / H), h = (int)(p % H);
            const int64_t t0 = offsets[u];
            const int64_t L = (int64_t)offsets[u + 1] - t0;
            for (int64_t i = 0; i < L; ++i) {
                const double *qi = q + (t0 + i) * rs + (int64_t)h * D;
                const int64_t j0 = first_visible(i, B, W);
                const int64_t n = i - j0 + 1;
                const double e = eps2[(int64_t)h * T + t0 + i];
                double m = -INFINITY;
                for (int64_t x = 0; x < n; ++x) {
                    const double *kj = k + (t0 + j0 + x) * rs + (int64_t)h * D;
                    t[x] = scale * dot(qi, kj, D) * kLog2e;
                    if (t[x] > m)
                        m = t[x];
                }
                const double M = floor(m);
                block_floor(t, n, j0, fb);
                /* the unquantized normaliser, at its smallest */
                double l = 0.0;
                for (int64_t x = 0; x < n; ++x)
                    l += exp2(t[x] - M - e);
                double *si = slack + (t0 + i) * rs + (int64_t)h * D;
                for (int d = 0; d < D; ++d)
                    si[d] = 0.0;
                for (int64_t x = 0; x < n; ++x) {
                    /* is the block's maximum within e of an integer? */
                    int64_t a = x;
                    const int64_t g = j0; /* local index of key x = 0 */
                    while (a > 0 && (g + a - 1) / 32 == (g + x) / 32)
                        --a;
                    double bm = -INFINITY;
                    for (int64_t y = a; y < n && (g + y) / 32 == (g + x) / 32; ++y)
                        if (t[y] > bm)
                            bm = t[y];
                    const double fr = bm - floor(bm);
                    const int f_flip = fr <= e || 1.0 - fr <= e;
                    /* the scaled argument and its reach */
                    const double xs = exp2(t[x] - fb[x] + 7.0);
                    const double lo = xs * exp2(-e), hi = xs * exp2(e);
                    const int code_flip = oracle_e4m3_round(lo) != oracle_e4m3_round(hi);
                    double a_ij = 0.0;
                    if (code_flip) /* one E4M3 step at the larger end */
                        a_ij = oracle_e4m3_round(hi) - oracle_e4m3_round(lo);
                    if (f_flip) /* the subnormal quantum of the grid one F below */
                        a_ij += 2.0 * ldexp(1.0, -9);
                    a_ij = ldexp(a_ij, (int)(fb[x] - 7.0 - M));
                    if (a_ij == 0.0)
                        continue;
                    const double *vj = v + (t0 + j0 + x) * rs + (int64_t)h * D;
                    for (int d = 0; d < D; ++d)
                        si[d] += a_ij * fabs(vj[d]) / l;
                }
            }
        }
        free(t);
    }
    return status;
}

/*
 * MXFP8 backward.  "GEM (Meta)", section "Ultra-low-precision training":
 * the attention kernel runs its matrix products as block-scaled MXFP8 in the
 * backward pass as well as in the forward.  Nothing more is given; the
 * readings taken here:
 *   - every product takes MXFP8 operands whose scale blocks run along that
 *     product's contraction: S = scale Q K^T and dP = dO V^T along head
 *     dims (q, k, v, dout: head-dim blocks, as in the forward); dV = P^T dO
 *     and dK = scale dS^T Q along queries, dQ = scale dS K along keys.  Q, K
 *     and dO therefore enter the last three products through a second
 *     quantization along tokens (qt, kt, dot: blocks of 32 tokens counted
 *     from the user's first token), which the caller supplies.  All arrays
 *     here hold decoded values;
 *   - P_ij = exp(s_ij - lse_i) with the forward's lse, and
 *     delta_i = <dO_i, O_i> with the forward's O (both given), the row
 *     statistic of the FlashAttention backward; dS_ij = P_ij (dP_ij - delta_i);
 *   - the operands formed inside the backward are quantized along their
 *     product's contraction: P over each key's queries (for dV), dS over
 *     each key's queries (for dK) and over each query's keys (for dQ), in
 *     blocks of 32 positions counted from the user's first token, where a
 *     position that is not visible holds 0.  In a block whose largest
 *     magnitude is a > 0, each x is stored as 2^E R(x 2^-E) with
 *     E = max(floor(log2 a) - 7, -127) (the E8M0 range) and R the nearest
 *     E4M3 value, ties to the even code, sign kept.  |x 2^-E| < 2^8, so
 *     nothing saturates: the rule of the forward's weights (oracle_mxpv_fwd);
 *   - dQ_i = scale sum_j dSq_ij kt_j, dK_j = scale sum_i dSq_ij qt_i (the
 *     query-blocked dSq), dV_j = sum_i Pq_ij dot_i.
 * With quant = 0 the quantization is skipped: with the exact O and lse and
 * qt = q, kt = k, dot = dout this is oracle_bwd.
 * Layouts: every tensor fp64 [T, H, D]; lse fp64 [H, T].
 */

/* Quantizes n values x[0], x[st], ... as one block, in place. */
static void mx_block(double *x, int64_t n, int64_t st)
{
    double a = 0.0;
    for (int64_t i = 0; i < n; ++i)
        if (fabs(x[i * st]) > a)
            a = fabs(x[i * st]);
    if (!(a > 0.0))
        return; /* all zero */
    int e;
    (void)frexp(a, &e);
    const int E = e - 8 < -127 ? -127 : e - 8; /* floor(log2 a) - 7 */
    for (int64_t i = 0; i < n; ++i) {
        const double y = x[i * st];
        x[i * st] = copysign(ldexp(oracle_e4m3_round(ldexp(fabs(y), -E)), E), y);
    }
}

/* The block rule with a given exponent E, |y| clipped below 2^(E + 8). */
static double mx_at(double y, int E)
{
    const double lim = ldexp(1.0, E + 8) * (1.0 - 0x1p-40);
    const double m = fabs(y) < lim ? fabs(y) : lim;
    return copysign(ldexp(oracle_e4m3_round(ldexp(m, -E)), E), y);
}

static int mx_exp(double a)
{
    int e;
    (void)frexp(a, &e);
    return e - 8 < -127 ? -127 : e - 8;
}

/* Parity allowance of one block (test support): x[] the exact values, err[]
 * bounds on how far a computation's values may be from them (0 for exact
 * zeros), q[] the quantized x.  A computation may take its block exponent
 * from any maximum within the errors and round any value within its error:
 * a[] gets the largest change of each quantized value those allow. */
static void mx_block_reach(const double *x, const double *err, const double *q,
                           int64_t n, int64_t st, double *a)
{
    double lo = 0.0, hi = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        const double m = fabs(x[i * st]);
        if (m - err[i * st] > lo)
            lo = m - err[i * st];
        if (m + err[i * st] > hi)
            hi = m + err[i * st];
    }
    for (int64_t i = 0; i < n; ++i) {
        const double y = x[i * st], e = err[i * st];
        double r = 0.0;
        if (!(hi > 0.0)) {
            r = 0.0;
        } else if (!(lo > 0.0)) { /* the maximum may be near 0: any code */
            r = fabs(q[i * st]) + 2.0 * (fabs(y) + e);
        } else {
            for (int E = mx_exp(lo); E <= mx_exp(hi); ++E) {
                const double d0 = fabs(mx_at(y - e, E) - q[i * st]);
                const double d1 = fabs(mx_at(y + e, E) - q[i * st]);
                r = fmax(r, fmax(d0, d1));
            }
        }
        a[i * st] = r;
    }
}

static int mx_bwd_core(const double *q, const double *k, const double *v,
                       const double *dout, const double *out, const double *lse,
                       const double *qt, const double *kt, const double *dot_t,
                       const int32_t *offsets, int batch, int64_t T, int H,
                       int D, int B, int W, double scale, int quant, double rho,
                       double *dq, double *dk, double *dv, double *sl_dq,
                       double *sl_dk, double *sl_dv, double *ab_dq, double *ab_dk,
                       double *ab_dv)
{
    if (check_args(offsets, batch, T, H, D, B, W))
        return -1;
    const int bounds = sl_dq != NULL;
    int status = 0;
    const int64_t npairs = (int64_t)batch * H;
    const int64_t rs = (int64_t)H * D;
    /* keys seen by one block of 32 queries */
    const int64_t nk = (int64_t)visible_max(offsets, batch, B, W) + 32;
    const double sa = fabs(scale);
#pragma omp parallel
    {
        /* per 32-query block: P, dS (exact), their quantized copies along
         * queries and along keys, error bounds and flip allowances */
        const int nbuf = bounds ? 10 : 5;
        double *buf = (double *)calloc((size_t)(32 * nk * nbuf), sizeof(double));
        if (!buf) {
#pragma omp atomic write
            status = -2;
        }
#pragma omp for schedule(dynamic)
        for (int64_t p = 0; p < npairs; ++p) {
            if (!buf)
                continue;
            double *P = buf, *S = P + 32 * nk;               /* P, dS [32][nk] */
            double *PqT = S + 32 * nk, *SqT = PqT + 32 * nk; /* along queries */
            double *Sq = SqT + 32 * nk;                      /* along keys */
            /* (bounds only) error bounds of P and dS, and the allowances of
             * PqT, SqT and Sq */
            double *eP = Sq + 32 * nk, *eS = eP + 32 * nk;
            double *aP = eS + 32 * nk, *aST = aP + 32 * nk, *aS = aST + 32 * nk;
            const int u = (int)(p / H), h = (int)(p % H);
            const int64_t t0 = offsets[u];
            const int64_t L = (int64_t)offsets[u + 1] - t0;
            const int64_t ho = (int64_t)h * D;
            for (int64_t i = 0; i < L; ++i)
                for (int d = 0; d < D; ++d) {
                    const int64_t o = (t0 + i) * rs + ho + d;
                    dk[o] = dv[o] = dq[o] = 0.0;
                    if (bounds)
                        sl_dq[o] = sl_dk[o] = sl_dv[o] = ab_dq[o] = ab_dk[o] = ab_dv[o] = 0.0;
                }
            for (int64_t i0 = 0; i0 < L; i0 += 32) {
                const int64_t ni = L - i0 < 32 ? L - i0 : 32;
                const int64_t k0 = first_visible(i0, B, W); /* keys k0 .. */
                const int64_t kn = i0 + ni - k0;            /* .. k0 + kn - 1 */
                for (int64_t x = 0; x < 32 * nk; ++x)
                    P[x] = S[x] = 0.0;
                if (bounds)
                    for (int64_t x = 0; x < 32 * nk; ++x)
                        eP[x] = eS[x] = 0.0;
                /* P and dS of the block's queries (row r, column c = key k0 + c) */
                for (int64_t r = 0; r < ni; ++r) {
                    const int64_t i = i0 + r;
                    const double *qi = q + (t0 + i) * rs + ho;
                    const double *doi = dout + (t0 + i) * rs + ho;
                    const double *oi = out + (t0 + i) * rs + ho;
                    const double li = lse[(int64_t)h * T + t0 + i];
                    const double delta = dot(doi, oi, D);
                    double dabs = 0.0;
                    if (bounds)
                        for (int d = 0; d < D; ++d)
                            dabs += fabs(doi[d] * oi[d]);
                    for (int64_t j = first_visible(i, B, W); j <= i; ++j) {
                        const double *kj = k + (t0 + j) * rs + ho;
                        const double *vj = v + (t0 + j) * rs + ho;
                        const double s = scale * dot(qi, kj, D);
                        const double pij = exp(s - li);
                        const double dp = dot(doi, vj, D);
                        const int64_t x = r * nk + (j - k0);
                        P[x] = pij;
                        S[x] = pij * (dp - delta);
                        if (bounds) {
                            /* score and dP products within rho of their
                             * magnitude sums; fp32 exponent arguments and
                             * delta's fp32 sum */
                            double qk = 0.0, dv_ = 0.0;
                            for (int d = 0; d < D; ++d) {
                                qk += fabs(qi[d] * kj[d]);
                                dv_ += fabs(doi[d] * vj[d]);
                            }
                            const double et = rho * sa * qk * kLog2e +
                                              0x1p-20 * (4.0 + fabs(s * kLog2e) + fabs(li * kLog2e));
                            eP[x] = pij * (exp2(et) - 1.0);
                            const double edp = rho * (dv_ + fabs(delta)) + 0x1p-16 * dabs;
                            eS[x] = eP[x] * fabs(dp - delta) + (pij + eP[x]) * edp +
                                    0x1p-22 * fabs(S[x]);
                        }
                    }
                }
                /* along queries: one block per key (the 32 queries are one
                 * block: i0 is a multiple of 32) */
                memcpy(PqT, P, sizeof(double) * 32 * nk);
                memcpy(SqT, S, sizeof(double) * 32 * nk);
                if (quant)
                    for (int64_t c = 0; c < kn; ++c) {
                        mx_block(PqT + c, ni, nk);
                        mx_block(SqT + c, ni, nk);
                    }
                /* along keys: blocks of 32 local keys in each query's row */
                memcpy(Sq, S, sizeof(double) * 32 * nk);
                if (quant)
                    for (int64_t r = 0; r < ni; ++r)
                        for (int64_t c = 0; c < kn;) {
                            const int64_t j = k0 + c;
                            const int64_t e = (j / 32 + 1) * 32 - k0; /* block end */
                            const int64_t n = (e < kn ? e : kn) - c;
                            mx_block(Sq + r * nk + c, n, 1);
                            c += n;
                        }
                if (bounds) {
                    if (quant) {
                        for (int64_t c = 0; c < kn; ++c) {
                            mx_block_reach(P + c, eP + c, PqT + c, ni, nk, aP + c);
                            mx_block_reach(S + c, eS + c, SqT + c, ni, nk, aST + c);
                        }
                        for (int64_t r = 0; r < ni; ++r)
                            for (int64_t c = 0; c < kn;) {
                                const int64_t j = k0 + c;
                                const int64_t e = (j / 32 + 1) * 32 - k0;
                                const int64_t n = (e < kn ? e : kn) - c;
                                mx_block_reach(S + r * nk + c, eS + r * nk + c, Sq + r * nk + c,
                                               n, 1, aS + r * nk + c);
                                c += n;
                            }
                    } else {
                        for (int64_t x = 0; x < 32 * nk; ++x) {
                            aP[x] = eP[x];
                            aST[x] = aS[x] = eS[x];
                        }
                    }
                }
                /* the three products */
                for (int64_t r = 0; r < ni; ++r) {
                    const int64_t i = i0 + r;
                    double *dqi = dq + (t0 + i) * rs + ho;
                    for (int64_t c = 0; c < kn; ++c) {
                        const int64_t x = r * nk + c;
                        const double *ktj = kt + (t0 + k0 + c) * rs + ho;
                        if (Sq[x] != 0.0)
                            for (int d = 0; d < D; ++d)
                                dqi[d] += scale * Sq[x] * ktj[d];
                        if (bounds && (Sq[x] != 0.0 || aS[x] != 0.0))
                            for (int d = 0; d < D; ++d) {
                                const int64_t o = (t0 + i) * rs + ho + d;
                                sl_dq[o] += sa * aS[x] * fabs(ktj[d]);
                                ab_dq[o] += sa * fabs(Sq[x] * ktj[d]);
                            }
                    }
                }
                for (int64_t c = 0; c < kn; ++c) {
                    const int64_t j = k0 + c;
                    double *dkj = dk + (t0 + j) * rs + ho;
                    double *dvj = dv + (t0 + j) * rs + ho;
                    for (int64_t r = 0; r < ni; ++r) {
                        const int64_t x = r * nk + c;
                        const double *qti = qt + (t0 + i0 + r) * rs + ho;
                        const double *dti = dot_t + (t0 + i0 + r) * rs + ho;
                        for (int d = 0; d < D; ++d) {
                            dkj[d] += scale * SqT[x] * qti[d];
                            dvj[d] += PqT[x] * dti[d];
                        }
                        if (bounds)
                            for (int d = 0; d < D; ++d) {
                                const int64_t o = (t0 + j) * rs + ho + d;
                                sl_dk[o] += sa * aST[x] * fabs(qti[d]);
                                ab_dk[o] += sa * fabs(SqT[x] * qti[d]);
                                sl_dv[o] += aP[x] * fabs(dti[d]);
                                ab_dv[o] += fabs(PqT[x] * dti[d]);
                            }
                    }
                }
            }
        }
        free(buf);
    }
    return status;
}

/* MXFP8 backward (definition above): dq, dk, dv [T,H,D]. */
int oracle_mx_bwd(const double *q, const double *k, const double *v,
                  const double *dout, const double *out, const double *lse,
                  const double *qt, const double *kt, const double *dot_t,
                  const int32_t *offsets, int batch, int64_t T, int H, int D,
                  int B, int W, double scale, int quant, double *dq, double *dk,
                  double *dv)
{
    return mx_bwd_core(q, k, v, dout, out, lse, qt, kt, dot_t, offsets, batch, T, H, D,
                       B, W, scale, quant, 0.0, dq, dk, dv, NULL, NULL, NULL, NULL,
                       NULL, NULL);
}

/* Parity allowance for oracle_mx_bwd (test support, not part of the
 * definition), with the same dq, dk, dv.  A computation whose score and dP
 * products are within rho of sum_d |scale q_d k_d| and
 * sum_d |dO_d v_d| + |delta|, whose exponent arguments, delta and dS carry
 * fp32 rounding, and which follows the quantization rule on its own values,
 * may take another block exponent where a block's maximum lies that close
 * to a power of two and round to a neighbouring code where a value lies
 * that close to a midpoint.  sl_* = sum over the contraction of the largest
 * change those flips allow to each quantized operand times |the other
 * operand|; ab_* = the same sum of |quantized operand| |other operand|
 * (what the products' own rounding is relative to). */
int oracle_mx_bwd_bounds(const double *q, const double *k, const double *v,
                         const double *dout, const double *out, const double *lse,
                         const double *qt, const double *kt, const double *dot_t,
                         const int32_t *offsets, int batch, int64_t T, int H, int D,
                         int B, int W, double scale, double rho, double *dq,
                         double *dk, double *dv, double *sl_dq, double *sl_dk,
                         double *sl_dv, double *ab_dq, double *ab_dk, double *ab_dv)
{
    return mx_bwd_core(q, k, v, dout, out, lse, qt, kt, dot_t, offsets, batch, T, H, D,
                       B, W, scale, 1, rho, dq, dk, dv, sl_dq, sl_dk, sl_dv, ab_dq, ab_dk,
                       ab_dv);
}

/* The block rule of oracle_mx_bwd applied to x[0..n) in place (exported so
 * that the rule itself can be pinned). */
void oracle_mx_quantize_block(double *x, int64_t n)
{
    if (x && n > 0)
        mx_block(x, n, 1);
}
