// Backward block attention on bf16 MFMA (gfx950), one launch.
//
// The production block-attention kernel fuses its backward pass ("GEM (Meta)"
// on aiwiki.ai, section "Custom kernels").  Here every 128-row tile of a
// (user, head) is worked on by two workgroups of the same launch:
//
//   query role  (rows = queries i):  dQ_i = scale * sum_j dS_ij k_j
//   key role    (rows = keys j):     dK_j = scale * sum_i dS_ij q_i,
//                                    dV_j = sum_i P_ij dO_i
//
// with P_ij = exp(scale <q_i,k_j> - lse_i), dP_ij = <dO_i, v_j>,
// dS_ij = P_ij (dP_ij - delta_i) and delta_i = <dO_i, O_i> recomputed by
// both roles while staging.  Each output element has exactly one owner, so
// there are no atomics and the result is deterministic.  Visibility is the
// block window: local query i sees local key j iff j <= i and
// floor(i/B) - floor(j/B) < W, i.e. key j is seen by queries
// j <= i < (floor(j/B) + W) * B.
//
// Layouts follow the forward kernel: 32x32x16 bf16 MFMAs, one query (query
// role) or one key (key role) per lane column, operand rows loaded through
// the bit-swap permutation sigma so accumulator octets are the operands of
// the next product.  The query role keeps Q^T and dO^T in registers and
// streams K, V (as is) and K^T through LDS; the key role keeps K^T and V^T
// in registers and streams Q, dO (as is), Q^T and dO^T through LDS.
#include "common.h"
#include "kernels.h"

namespace ba {
namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kTileRows = 128;
constexpr int kKC = 64;        // rows per staged chunk
constexpr int kPad = 8;

__device__ __forceinline__ int sigma32(int a) {
    return (a & ~12) | ((a & 4) << 1) | ((a & 8) >> 1);
}
__device__ __forceinline__ int sigma(int x) { return (x & ~31) | sigma32(x & 31); }

__device__ __forceinline__ int window_start(int row, int B, int W) {
    return max(0, row / B - W + 1) * B;
}
// One past the last query that sees key `key` (queries end at L).
__device__ __forceinline__ int window_end(int key, int B, int W, int L) {
    return (int)min((int64_t)(key / B + W) * B, (int64_t)L);
}

template <int D>
struct BwdSmem {
    union {
        struct {
            bf16 k[kKC][D + kPad];   // rows permuted by sigma
            bf16 v[kKC][D + kPad];   // rows permuted by sigma
            bf16 kt[D][kKC + kPad];  // head-dim rows permuted by sigma
        } qr;
        struct {
            bf16 q[kKC][D + kPad];
            bf16 dob[kKC][D + kPad];
            bf16 qt[D][kKC + kPad];
            bf16 dot[D][kKC + kPad];
            float lse2[kKC];  // log2-domain lse of the chunk's queries
            float dlt[kKC];   // delta of the chunk's queries
        } kr;
    };
};

// A chunk of 64 rows x D of one tensor as 4x4 units (4 rows x 4 columns,
// one 8-byte load per row) spread over the workgroup.
template <int D>
struct Units {
    static constexpr int kCount = kKC / 4 * D / 4;
    static constexpr int kPer = (kCount + kThreads - 1) / kThreads;
    uint2 x[kPer][4];
};

template <int D>
__device__ __forceinline__ void load_units(Units<D> &u, const bf16 *__restrict__ src,
                                           int64_t base, int64_t rs, int c0, int end) {
#pragma unroll
    for (int i = 0; i < Units<D>::kPer; ++i) {
        const int id = threadIdx.x + i * kThreads;
        const int r4 = id / (D / 4), d4 = id % (D / 4);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int row = c0 + r4 * 4 + kk;
            uint2 x = make_uint2(0u, 0u);
            if (id < Units<D>::kCount && row < end)
                x = *(const uint2 *)(src + base + (int64_t)row * rs + d4 * 4);
            u.x[i][kk] = x;
        }
    }
}

// Natural layout: chunk row r goes to LDS row sigma(r).
template <int D>
__device__ __forceinline__ void store_rows(const Units<D> &u, bf16 (*dst)[D + kPad]) {
#pragma unroll
    for (int i = 0; i < Units<D>::kPer; ++i) {
        const int id = threadIdx.x + i * kThreads;
        if (id >= Units<D>::kCount) break;
        const int r4 = id / (D / 4), d4 = id % (D / 4);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) *(uint2 *)&dst[sigma(r4 * 4 + kk)][d4 * 4] = u.x[i][kk];
    }
}

// Transposed layout: column d goes to LDS row sigma(d), rows along it.
template <int D>
__device__ __forceinline__ void store_cols(const Units<D> &u, bf16 (*dst)[kKC + kPad]) {
#pragma unroll
    for (int i = 0; i < Units<D>::kPer; ++i) {
        const int id = threadIdx.x + i * kThreads;
        if (id >= Units<D>::kCount) break;
        const int r4 = id / (D / 4), d4 = id % (D / 4);
        const uint2 *x = u.x[i];
        uint2 c0, c1, c2, c3;
        c0.x = (x[0].x & 0xffffu) | (x[1].x << 16);
        c0.y = (x[2].x & 0xffffu) | (x[3].x << 16);
        c1.x = (x[0].x >> 16) | (x[1].x & 0xffff0000u);
        c1.y = (x[2].x >> 16) | (x[3].x & 0xffff0000u);
        c2.x = (x[0].y & 0xffffu) | (x[1].y << 16);
        c2.y = (x[2].y & 0xffffu) | (x[3].y << 16);
        c3.x = (x[0].y >> 16) | (x[1].y & 0xffff0000u);
        c3.y = (x[2].y >> 16) | (x[3].y & 0xffff0000u);
        *(uint2 *)&dst[sigma(d4 * 4 + 0)][r4 * 4] = c0;
        *(uint2 *)&dst[sigma(d4 * 4 + 1)][r4 * 4] = c1;
        *(uint2 *)&dst[sigma(d4 * 4 + 2)][r4 * 4] = c2;
        *(uint2 *)&dst[sigma(d4 * 4 + 3)][r4 * 4] = c3;
    }
}

__device__ __forceinline__ float dot_bf16x2(uint32_t a, uint32_t b, float acc) {
    acc = fmaf(__uint_as_float(a << 16), __uint_as_float(b << 16), acc);
    return fmaf(__uint_as_float(a & 0xffff0000u), __uint_as_float(b & 0xffff0000u), acc);
}

// delta of the chunk's rows from dO and O units: 4 partial dots per unit,
// summed over the D/4 consecutive lanes that share the unit's rows.
template <int D>
__device__ __forceinline__ void store_delta(const Units<D> &dou, const Units<D> &ou, float *dlt) {
#pragma unroll
    for (int i = 0; i < Units<D>::kPer; ++i) {
        const int id = threadIdx.x + i * kThreads;
        float part[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            float a = dot_bf16x2(dou.x[i][kk].x, ou.x[i][kk].x, 0.f);
            part[kk] = dot_bf16x2(dou.x[i][kk].y, ou.x[i][kk].y, a);
        }
#pragma unroll
        for (int o = 1; o < D / 4; o <<= 1)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) part[kk] += __shfl_xor(part[kk], o, 64);
        if (id < Units<D>::kCount && id % (D / 4) == 0) {
            const int r4 = id / (D / 4);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) dlt[r4 * 4 + kk] = part[kk];
        }
    }
}

template <int D>
__device__ __forceinline__ void store_out(bf16 *dst, const f32x16 (&acc)[D / 32], float mul,
                                          int g) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            bf16x8 x;
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = (bf16)(acc[dt][half * 8 + i] * mul);
            *(bf16x8 *)(dst + dt * 32 + half * 16 + g * 8) = x;
        }
}

// Loads one row of a [T,H,D] tensor as MFMA B operands (lane = row).
template <int D>
__device__ __forceinline__ void load_operand(bf16x8 (&op)[D / 16], const bf16 *__restrict__ src,
                                             int64_t off, bool valid, int g) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        bf16x8 x = {};
        if (valid) x = *(const bf16x8 *)(src + off + ks * 16 + g * 8);
        op[ks] = x;
    }
}

// ------------------------------------------------------------ query role

template <int D>
__device__ void query_role(const Shape &s, const Tile &t, BwdSmem<D> &sm,
                           const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                           const bf16 *__restrict__ v, const bf16 *__restrict__ out,
                           const bf16 *__restrict__ dout, const float *__restrict__ lse,
                           bf16 *__restrict__ dq) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int qi = lane & 31, g = lane >> 5;
    const int64_t rs = (int64_t)s.H * D;
    const int64_t base = t.tok0 * rs + (int64_t)t.h * D;
    const int row0 = t.blk * kTileRows;
    const int row_end = min(row0 + kTileRows, t.len);
    const int wr0 = row0 + w * 32;
    const int my_row = wr0 + qi;
    const bool wave_live = wr0 < row_end;
    const bool my_valid = my_row < row_end;
    const int w_last = min(wr0 + 31, row_end - 1);
    const int wave_klo = window_start(wr0, s.B, s.W);
    const int wave_klo_max = window_start(max(wr0, w_last), s.B, s.W);
    const int my_klo = window_start(my_row, s.B, s.W);
    const float c = s.scale * kLog2e;

    bf16x8 qop[D / 16], doop[D / 16];
    load_operand<D>(qop, q, base + (int64_t)my_row * rs, my_valid, g);
    load_operand<D>(doop, dout, base + (int64_t)my_row * rs, my_valid, g);
    float my_lse2 = 0.f, my_dlt = 0.f;
    if (my_valid) {
        my_lse2 = lse[(int64_t)t.h * s.T + t.tok0 + my_row] * kLog2e;
        float a = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            const bf16x8 o = *(const bf16x8 *)(out + base + (int64_t)my_row * rs + ks * 16 + g * 8);
            const uint4 ou = __builtin_bit_cast(uint4, o);
            const uint4 du = __builtin_bit_cast(uint4, doop[ks]);
            a = dot_bf16x2(du.x, ou.x, a);
            a = dot_bf16x2(du.y, ou.y, a);
            a = dot_bf16x2(du.z, ou.z, a);
            a = dot_bf16x2(du.w, ou.w, a);
        }
        my_dlt = a;
    }
    my_dlt += __shfl_xor(my_dlt, 32, 64);

    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};

    const int kbeg = window_start(row0, s.B, s.W);
    Units<D> ku, vu;
    load_units<D>(ku, k, base, rs, kbeg, row_end);
    load_units<D>(vu, v, base, rs, kbeg, row_end);
    for (int c0 = kbeg; c0 < row_end; c0 += kKC) {
        __syncthreads();
        store_rows<D>(ku, sm.qr.k);
        store_cols<D>(ku, sm.qr.kt);
        store_rows<D>(vu, sm.qr.v);
        __syncthreads();
        if (c0 + kKC < row_end) {
            load_units<D>(ku, k, base, rs, c0 + kKC, row_end);
            load_units<D>(vu, v, base, rs, c0 + kKC, row_end);
        }
        if (!wave_live) continue;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const int a0 = c0 + st * 32;
            if (!(a0 <= w_last && a0 + 31 >= wave_klo)) continue;
            const bool msk = a0 + 31 > wr0 || a0 < wave_klo_max;
            f32x16 sc = {}, dp = {};
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const bf16x8 ka = *(const bf16x8 *)&sm.qr.k[st * 32 + qi][ks * 16 + g * 8];
                sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qop[ks], sc, 0, 0, 0);
                const bf16x8 va = *(const bf16x8 *)&sm.qr.v[st * 32 + qi][ks * 16 + g * 8];
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, doop[ks], dp, 0, 0, 0);
            }
            bf16x8 dsb[2];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = __builtin_amdgcn_exp2f(fmaf(sc[r], c, -my_lse2));
                if (msk) {
                    const int key = a0 + (r >> 3) * 16 + g * 8 + (r & 7);
                    p = (key > my_row || key < my_klo) ? 0.f : p;
                }
                dsb[r >> 3][r & 7] = (bf16)(p * (dp[r] - my_dlt));
            }
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const bf16x8 a =
                        *(const bf16x8 *)&sm.qr.kt[dt * 32 + qi][st * 32 + kk * 16 + g * 8];
                    acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsb[kk], acc[dt], 0, 0,
                                                                      0);
                }
        }
    }
    if (my_valid) store_out<D>(dq + base + (int64_t)my_row * rs, acc, s.scale, g);
}

// -------------------------------------------------------------- key role

template <int D>
__device__ void key_role(const Shape &s, const Tile &t, BwdSmem<D> &sm,
                         const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                         const bf16 *__restrict__ v, const bf16 *__restrict__ out,
                         const bf16 *__restrict__ dout, const float *__restrict__ lse,
                         bf16 *__restrict__ dk, bf16 *__restrict__ dv) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int qi = lane & 31, g = lane >> 5;
    const int64_t rs = (int64_t)s.H * D;
    const int64_t base = t.tok0 * rs + (int64_t)t.h * D;
    const int row0 = t.blk * kTileRows;
    const int row_end = min(row0 + kTileRows, t.len);   // keys of this tile end here
    const int wk0 = row0 + w * 32;
    const int my_key = wk0 + qi;
    const bool wave_live = wk0 < row_end;
    const bool my_valid = my_key < row_end;
    const int wk_last = min(wk0 + 31, row_end - 1);
    const int qend = window_end(row_end - 1, s.B, s.W, t.len);  // queries of the tile end here
    const int wave_qend_min = window_end(wk0, s.B, s.W, t.len);
    const int wave_qend_max = window_end(max(wk0, wk_last), s.B, s.W, t.len);
    const int my_qend = window_end(my_key, s.B, s.W, t.len);
    const float c = s.scale * kLog2e;

    bf16x8 kop[D / 16], vop[D / 16];
    load_operand<D>(kop, k, base + (int64_t)my_key * rs, my_valid, g);
    load_operand<D>(vop, v, base + (int64_t)my_key * rs, my_valid, g);

    f32x16 adk[D / 32], adv[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) adk[dt] = adv[dt] = f32x16{};

    Units<D> qu, du, ou;
    float lse_next = 0.f;
    const float *lse_h = lse + (int64_t)t.h * s.T + t.tok0;
    load_units<D>(qu, q, base, rs, row0, qend);
    load_units<D>(du, dout, base, rs, row0, qend);
    load_units<D>(ou, out, base, rs, row0, qend);
    if (tid < kKC && row0 + tid < qend) lse_next = lse_h[row0 + tid] * kLog2e;
    for (int c0 = row0; c0 < qend; c0 += kKC) {
        __syncthreads();
        store_rows<D>(qu, sm.kr.q);
        store_cols<D>(qu, sm.kr.qt);
        store_rows<D>(du, sm.kr.dob);
        store_cols<D>(du, sm.kr.dot);
        store_delta<D>(du, ou, sm.kr.dlt);
        if (tid < kKC) sm.kr.lse2[tid] = lse_next;
        __syncthreads();
        if (c0 + kKC < qend) {
            load_units<D>(qu, q, base, rs, c0 + kKC, qend);
            load_units<D>(du, dout, base, rs, c0 + kKC, qend);
            load_units<D>(ou, out, base, rs, c0 + kKC, qend);
            lse_next = (tid < kKC && c0 + kKC + tid < qend) ? lse_h[c0 + kKC + tid] * kLog2e
                                                            : 0.f;
        }
        if (!wave_live) continue;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const int a0 = c0 + st * 32;  // first query of the sub-tile
            if (!(a0 + 31 >= wk0 && a0 < wave_qend_max)) continue;
            const bool msk = a0 < wk_last || a0 + 31 >= wave_qend_min;
            f32x16 sc = {}, dp = {};
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const bf16x8 qa = *(const bf16x8 *)&sm.kr.q[st * 32 + qi][ks * 16 + g * 8];
                sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kop[ks], sc, 0, 0, 0);
                const bf16x8 da = *(const bf16x8 *)&sm.kr.dob[st * 32 + qi][ks * 16 + g * 8];
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vop[ks], dp, 0, 0, 0);
            }
            // register r of lane g holds query a0 + 16(r/8) + 8g + r%8
            float pf[16];
            bf16x8 pb[2], dsb[2];
            float pmax = 0.f;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int qrow = st * 32 + hh * 16 + g * 8;
                const float4 l0 = *(const float4 *)&sm.kr.lse2[qrow];
                const float4 l1 = *(const float4 *)&sm.kr.lse2[qrow + 4];
                const float4 d0 = *(const float4 *)&sm.kr.dlt[qrow];
                const float4 d1 = *(const float4 *)&sm.kr.dlt[qrow + 4];
                const float ls[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
                const float ds[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int r = hh * 8 + i;
                    float p = __builtin_amdgcn_exp2f(fmaf(sc[r], c, -ls[i]));
                    if (msk) {
                        const int qq = a0 + hh * 16 + g * 8 + i;
                        p = (qq < my_key || qq >= my_qend) ? 0.f : p;
                    }
                    pf[r] = p;
                    pmax = fmaxf(pmax, p);
                    pb[hh][i] = (bf16)p;
                    dsb[hh][i] = (bf16)(p * (dp[r] - ds[i]));
                }
            }
            // Rows that see few keys have weights near 1, where bf16 rounding
            // of P (2^-9 relative) would dominate dV.  There P is split into
            // bf16 hi + lo and dV takes a second product; elsewhere P < 1/16
            // bounds the rounding error per term by 2^-13.
            const bool split = __any(pmax > 0.0625f);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int col = st * 32 + kk * 16 + g * 8;
                    const bf16x8 da = *(const bf16x8 *)&sm.kr.dot[dt * 32 + qi][col];
                    adv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, pb[kk], adv[dt], 0, 0, 0);
                    if (split) {
                        bf16x8 lo;
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            lo[i] = (bf16)(pf[kk * 8 + i] - (float)pb[kk][i]);
                        adv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, lo, adv[dt], 0, 0, 0);
                    }
                    const bf16x8 qa = *(const bf16x8 *)&sm.kr.qt[dt * 32 + qi][col];
                    adk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, dsb[kk], adk[dt], 0, 0, 0);
                }
        }
    }
    if (my_valid) {
        store_out<D>(dk + base + (int64_t)my_key * rs, adk, s.scale, g);
        store_out<D>(dv + base + (int64_t)my_key * rs, adv, 1.f, g);
    }
}

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_mfma(
    Shape s, const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ out, const bf16 *__restrict__ dout, const float *__restrict__ lse,
    bf16 *__restrict__ dq, bf16 *__restrict__ dk, bf16 *__restrict__ dv) {
    __shared__ int sh[8];
    __shared__ __align__(16) BwdSmem<D> sm;
    Tile t;
    if (!decode_tile<kThreads>(s, kTileRows, 2, t, sh)) return;
    if (t.sub == 0)
        query_role<D>(s, t, sm, q, k, v, out, dout, lse, dq);
    else
        key_role<D>(s, t, sm, q, k, v, out, dout, lse, dk, dv);
}

template <int D>
hipError_t launch_t(const Shape &s, const void *q, const void *k, const void *v, const void *out,
                    const void *dout, const float *lse, void *dq, void *dk, void *dv,
                    hipStream_t st) {
    const int64_t grid = grid_upper_bound(s.T, s.batch, kTileRows, 2, s.H);
    hipLaunchKernelGGL((bwd_mfma<D>), dim3((unsigned)grid), dim3(kThreads), 0, st, s,
                       (const bf16 *)q, (const bf16 *)k, (const bf16 *)v, (const bf16 *)out,
                       (const bf16 *)dout, lse, (bf16 *)dq, (bf16 *)dk, (bf16 *)dv);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_bwd(const Shape &s, const void *q, const void *k, const void *v,
                           const void *out, const void *dout, const float *lse, void *dq,
                           void *dk, void *dv, hipStream_t st) {
    switch (s.D) {
    case 32: return launch_t<32>(s, q, k, v, out, dout, lse, dq, dk, dv, st);
    case 64: return launch_t<64>(s, q, k, v, out, dout, lse, dq, dk, dv, st);
    case 128: return launch_t<128>(s, q, k, v, out, dout, lse, dq, dk, dv, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace ba
