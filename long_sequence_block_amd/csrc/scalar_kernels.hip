// Scalar (vector-ALU FMA) block-attention kernels: the fp32 path.
//
// One wave per tile of 64 rows, one lane per row, fp32 arithmetic with an
// online softmax in the base-2 domain.  K/V (forward, dQ) or Q/dO (dK/dV)
// rows are staged through LDS in chunks of 64 tokens and read as broadcasts.
// The attention pattern is the block window of "GEM (Meta)" (aiwiki.ai),
// section "Custom kernels": local query i sees local key j iff j <= i and
// floor(i/B) - floor(j/B) < W.
#include "common.h"
#include "kernels.h"

namespace ba {
namespace {

constexpr int kRows = 64;   // rows per tile = lanes per workgroup
constexpr int kChunk = 64;  // tokens staged in LDS per step

template <typename TI, int D>
__device__ __forceinline__ void load_row(const TI *p, float *r) {
#pragma unroll
    for (int d = 0; d < D; ++d) r[d] = to_f32(p[d]);
}

template <int D>
__device__ __forceinline__ void zero_row(float *r) {
#pragma unroll
    for (int d = 0; d < D; ++d) r[d] = 0.f;
}

// Turns a gradient row back by the rotary angles of position pos (the
// backward of the rotary embedding applied to q or k; the angles are those
// of rope_sincos).  Nothing to do when s.rope_base is 0.
template <typename TI, int D>
__device__ __forceinline__ void rope_back(const Shape &s, int pos, float *r) {
    if (!(s.rope_base > 0.f)) return;
    const double lb = log2((double)s.rope_base);
#pragma unroll
    for (int d = 0; d < D / 2; ++d) {
        float sn, cs;
        rope_sincos<TI>((double)pos * exp2(-2.0 * d / D * lb) * kInv2Pi, sn, cs);
        const float a = r[d], b = r[d + D / 2];
        r[d] = a * cs + b * sn;
        r[d + D / 2] = b * cs - a * sn;
    }
}

// Forward.  Tile = rows [row0, row0+64) of one query block.  ACT != kSoftmax:
// P = act(scale s) with no normalisation (generalized dot-product attention).
template <typename TI, int D, int ACT>
__global__ __launch_bounds__(kRows) void fwd_scalar(Shape s, const TI *__restrict__ q,
                                                    const TI *__restrict__ k,
                                                    const TI *__restrict__ v,
                                                    TI *__restrict__ out,
                                                    float *__restrict__ lse, int tpb) {
    __shared__ int sh[8];
    __shared__ float ks[kChunk][D + 1];
    __shared__ float vs[kChunk][D + 1];
    Tile t;
    if (!decode_tile<kRows>(s, s.B, tpb, t, sh)) return;
    const int lane = threadIdx.x;
    const int64_t rs = (int64_t)s.H * D;
    const int row0 = t.blk * s.B + t.sub * kRows;
    const int row_end = min(row0 + kRows, (int)min((int64_t)t.blk * s.B + s.B, (int64_t)t.len));
    const int i = row0 + lane;  // local query row of this lane
    const bool valid = i < row_end;
    const int kstart = max(0, t.blk - s.W + 1) * s.B;
    const float c = s.scale * kLog2e;

    float qr[D], acc[D];
    zero_row<D>(acc);
    if (valid) load_row<TI, D>(q + (t.tok0 + i) * rs + (int64_t)t.h * D, qr);
    else zero_row<D>(qr);
    float m = -INFINITY, l = 0.f;

    for (int c0 = kstart; c0 < row_end; c0 += kChunk) {
        const int n = min(kChunk, row_end - c0);
        __syncthreads();
        for (int e = lane; e < n * D; e += kRows) {
            const int r = e / D, d = e % D;
            const int64_t g = (t.tok0 + c0 + r) * rs + (int64_t)t.h * D + d;
            ks[r][d] = to_f32(k[g]);
            vs[r][d] = to_f32(v[g]);
        }
        __syncthreads();
        if (!valid) continue;
        const int jend = min(n, i - c0 + 1);
        for (int r = 0; r < jend; ++r) {
            float dot = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) dot = fmaf(qr[d], ks[r][d], dot);
            if constexpr (ACT != kSoftmax) {
                const float p = act_value<ACT>(dot * s.scale);
#pragma unroll
                for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vs[r][d], acc[d]);
                continue;
            }
            const float x = dot * c;
            if (x > m) {
                const float a = exp2f(m - x);
                l *= a;
#pragma unroll
                for (int d = 0; d < D; ++d) acc[d] *= a;
                m = x;
            }
            const float p = exp2f(x - m);
            l += p;
#pragma unroll
            for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vs[r][d], acc[d]);
        }
    }
    if (!valid) return;
    const float inv = ACT == kSoftmax ? 1.f / l : 1.f;
    TI *o = out + (t.tok0 + i) * rs + (int64_t)t.h * D;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = from_f32<TI>(acc[d] * inv);
    if (ACT == kSoftmax) lse[(int64_t)t.h * s.T + t.tok0 + i] = (m + log2f(l)) * kLn2;
}

// Backward, query role: dQ_i = scale * sum_j P_ij (dP_ij - delta_i) k_j with
// delta_i = <dO_i, O_i>; for ACT != kSoftmax, dQ_i = scale * sum_j
// act'(scale s_ij) dP_ij k_j (out and lse are not read).
template <typename TI, int D, int ACT>
__device__ void bwd_dq_tile(const Shape &s, const Tile &t, int row0, const TI *__restrict__ q,
                            const TI *__restrict__ k, const TI *__restrict__ v,
                            const TI *__restrict__ out, const TI *__restrict__ dout,
                            const float *__restrict__ lse, TI *__restrict__ dq,
                            float (*ks)[D + 1], float (*vs)[D + 1]) {
    const int lane = threadIdx.x;
    const int64_t rs = (int64_t)s.H * D;
    const int row_end = min(row0 + kRows, (int)min((int64_t)t.blk * s.B + s.B, (int64_t)t.len));
    const int i = row0 + lane;
    const bool valid = i < row_end;
    const int kstart = max(0, t.blk - s.W + 1) * s.B;
    const float c = s.scale * kLog2e;

    float qr[D], dor[D], acc[D];
    float dlt = 0.f, lse2 = 0.f;
    zero_row<D>(acc);
    if (valid) {
        const int64_t g = (t.tok0 + i) * rs + (int64_t)t.h * D;
        load_row<TI, D>(q + g, qr);
        load_row<TI, D>(dout + g, dor);
        if constexpr (ACT == kSoftmax) {
#pragma unroll
            for (int d = 0; d < D; ++d) dlt = fmaf(dor[d], to_f32(out[g + d]), dlt);
            lse2 = lse[(int64_t)t.h * s.T + t.tok0 + i] * kLog2e;
        }
    } else {
        zero_row<D>(qr);
        zero_row<D>(dor);
    }
    for (int c0 = kstart; c0 < row_end; c0 += kChunk) {
        const int n = min(kChunk, row_end - c0);
        __syncthreads();
        for (int e = lane; e < n * D; e += kRows) {
            const int r = e / D, d = e % D;
            const int64_t g = (t.tok0 + c0 + r) * rs + (int64_t)t.h * D + d;
            ks[r][d] = to_f32(k[g]);
            vs[r][d] = to_f32(v[g]);
        }
        __syncthreads();
        if (!valid) continue;
        const int jend = min(n, i - c0 + 1);
        for (int r = 0; r < jend; ++r) {
            float sdot = 0.f, pdot = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                sdot = fmaf(qr[d], ks[r][d], sdot);
                pdot = fmaf(dor[d], vs[r][d], pdot);
            }
            const float ds = ACT == kSoftmax ? exp2f(sdot * c - lse2) * (pdot - dlt)
                                             : act_slope<ACT>(sdot * s.scale) * pdot;
#pragma unroll
            for (int d = 0; d < D; ++d) acc[d] = fmaf(ds, ks[r][d], acc[d]);
        }
    }
    if (!valid) return;
    TI *o = dq + (t.tok0 + i) * rs + (int64_t)t.h * D;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= s.scale;
    rope_back<TI, D>(s, i, acc);
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = from_f32<TI>(acc[d]);
}

// Backward, key role: dK_j = scale * sum_i dS_ij q_i and dV_j = sum_i P_ij dO_i
// over the queries that see key j: i in [j, min(L, (kb+W)*B)).  delta_i is
// recomputed from O and dO for each staged query chunk.
template <typename TI, int D, int ACT>
__device__ void bwd_dkdv_tile(const Shape &s, const Tile &t, int row0,
                              const TI *__restrict__ q, const TI *__restrict__ k,
                              const TI *__restrict__ v, const TI *__restrict__ out,
                              const TI *__restrict__ dout, const float *__restrict__ lse,
                              TI *__restrict__ dk, TI *__restrict__ dv, float (*qs)[D + 1],
                              float (*dos)[D + 1], float *ls, float *dls) {
    const int lane = threadIdx.x;
    const int64_t rs = (int64_t)s.H * D;
    const int row_end = min(row0 + kRows, (int)min((int64_t)t.blk * s.B + s.B, (int64_t)t.len));
    const int j = row0 + lane;  // local key row of this lane
    const bool valid = j < row_end;
    const int qend = (int)min(((int64_t)t.blk + s.W) * s.B, (int64_t)t.len);
    const float c = s.scale * kLog2e;

    float kr[D], vr[D], ak[D], av[D];
    zero_row<D>(ak);
    zero_row<D>(av);
    if (valid) {
        const int64_t g = (t.tok0 + j) * rs + (int64_t)t.h * D;
        load_row<TI, D>(k + g, kr);
        load_row<TI, D>(v + g, vr);
    } else {
        zero_row<D>(kr);
        zero_row<D>(vr);
    }
    for (int c0 = row0; c0 < qend; c0 += kChunk) {
        const int n = min(kChunk, qend - c0);
        __syncthreads();
        for (int e = lane; e < n * D; e += kRows) {
            const int r = e / D, d = e % D;
            const int64_t g = (t.tok0 + c0 + r) * rs + (int64_t)t.h * D + d;
            qs[r][d] = to_f32(q[g]);
            dos[r][d] = to_f32(dout[g]);
        }
        if (ACT == kSoftmax && lane < n) {
            const int64_t g = (t.tok0 + c0 + lane) * rs + (int64_t)t.h * D;
            float dlt = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) dlt = fmaf(to_f32(dout[g + d]), to_f32(out[g + d]), dlt);
            ls[lane] = lse[(int64_t)t.h * s.T + t.tok0 + c0 + lane] * kLog2e;
            dls[lane] = dlt;
        }
        __syncthreads();
        if (!valid) continue;
        const int rbeg = max(0, j - c0);
        for (int r = rbeg; r < n; ++r) {
            float sdot = 0.f, pdot = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                sdot = fmaf(qs[r][d], kr[d], sdot);
                pdot = fmaf(dos[r][d], vr[d], pdot);
            }
            float p, ds;
            if constexpr (ACT == kSoftmax) {
                p = exp2f(sdot * c - ls[r]);
                ds = p * (pdot - dls[r]);
            } else {
                float gr;
                act_value_slope<ACT>(sdot * s.scale, p, gr);
                ds = gr * pdot;
            }
#pragma unroll
            for (int d = 0; d < D; ++d) {
                ak[d] = fmaf(ds, qs[r][d], ak[d]);
                av[d] = fmaf(p, dos[r][d], av[d]);
            }
        }
    }
    if (!valid) return;
    const int64_t g = (t.tok0 + j) * rs + (int64_t)t.h * D;
#pragma unroll
    for (int d = 0; d < D; ++d) ak[d] *= s.scale;
    rope_back<TI, D>(s, j, ak);
#pragma unroll
    for (int d = 0; d < D; ++d) {
        dk[g + d] = from_f32<TI>(ak[d]);
        dv[g + d] = from_f32<TI>(av[d]);
    }
}

// Backward: one launch.  Every block has 2*tpb sub-tiles: the first tpb
// compute dQ rows, the next tpb compute dK/dV rows of the same block.
template <typename TI, int D, int ACT>
__global__ __launch_bounds__(kRows) void bwd_scalar(
    Shape s, const TI *__restrict__ q, const TI *__restrict__ k, const TI *__restrict__ v,
    const TI *__restrict__ out, const TI *__restrict__ dout, const float *__restrict__ lse,
    TI *__restrict__ dq, TI *__restrict__ dk, TI *__restrict__ dv, int tpb) {
    __shared__ int sh[8];
    __shared__ float as[kChunk][D + 1];
    __shared__ float bs[kChunk][D + 1];
    __shared__ float ls[kChunk], dls[kChunk];
    Tile t;
    if (!decode_tile<kRows>(s, s.B, 2 * tpb, t, sh)) return;
    const int row0 = t.blk * s.B + (t.sub % tpb) * kRows;
    if (t.sub < tpb)
        bwd_dq_tile<TI, D, ACT>(s, t, row0, q, k, v, out, dout, lse, dq, as, bs);
    else
        bwd_dkdv_tile<TI, D, ACT>(s, t, row0, q, k, v, out, dout, lse, dk, dv, as, bs, ls, dls);
}

template <typename TI, int D, int ACT>
hipError_t launch_fwd_act(const Shape &s, const void *q, const void *k, const void *v, void *out,
                          float *lse, hipStream_t st) {
    const int tpb = (int)(((int64_t)s.B + kRows - 1) / kRows);
    const int64_t grid = grid_upper_bound(s.T, s.batch, s.B, tpb, s.H);
    hipLaunchKernelGGL((fwd_scalar<TI, D, ACT>), dim3((unsigned)grid), dim3(kRows), 0, st, s,
                       (const TI *)q, (const TI *)k, (const TI *)v, (TI *)out, lse, tpb);
    return hipGetLastError();
}

template <typename TI, int D, int ACT>
hipError_t launch_bwd_act(const Shape &s, const void *q, const void *k, const void *v,
                          const void *out, const void *dout, const float *lse, void *dq,
                          void *dk, void *dv, hipStream_t st) {
    const int tpb = (int)(((int64_t)s.B + kRows - 1) / kRows);
    const int64_t grid = grid_upper_bound(s.T, s.batch, s.B, 2 * tpb, s.H);
    hipLaunchKernelGGL((bwd_scalar<TI, D, ACT>), dim3((unsigned)grid), dim3(kRows), 0, st, s,
                       (const TI *)q, (const TI *)k, (const TI *)v, (const TI *)out,
                       (const TI *)dout, lse, (TI *)dq, (TI *)dk, (TI *)dv, tpb);
    return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_d(const Shape &s, const void *q, const void *k, const void *v, void *out,
                        float *lse, hipStream_t st) {
    switch (s.act) {
    case kSoftmax: return launch_fwd_act<float, D, kSoftmax>(s, q, k, v, out, lse, st);
    case kSilu: return launch_fwd_act<float, D, kSilu>(s, q, k, v, out, lse, st);
    case kGelu: return launch_fwd_act<float, D, kGelu>(s, q, k, v, out, lse, st);
    }
    return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_bwd_d(const Shape &s, const void *q, const void *k, const void *v,
                        const void *out, const void *dout, const float *lse, void *dq, void *dk,
                        void *dv, hipStream_t st) {
    switch (s.act) {
    case kSoftmax:
        return launch_bwd_act<float, D, kSoftmax>(s, q, k, v, out, dout, lse, dq, dk, dv, st);
    case kSilu:
        return launch_bwd_act<float, D, kSilu>(s, q, k, v, out, dout, lse, dq, dk, dv, st);
    case kGelu:
        return launch_bwd_act<float, D, kGelu>(s, q, k, v, out, dout, lse, dq, dk, dv, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_scalar_fwd(const Shape &s, bool bf16_io, const void *q, const void *k,
                             const void *v, void *out, float *lse, hipStream_t st) {
    if (bf16_io) return hipErrorInvalidValue;  // bf16 storage runs on the MFMA kernels
    switch (s.D) {
    case 32: return launch_fwd_d<32>(s, q, k, v, out, lse, st);
    case 64: return launch_fwd_d<64>(s, q, k, v, out, lse, st);
    case 128: return launch_fwd_d<128>(s, q, k, v, out, lse, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_scalar_bwd(const Shape &s, bool bf16_io, const void *q, const void *k,
                             const void *v, const void *out, const void *dout,
                             const float *lse, void *dq, void *dk, void *dv,
                             hipStream_t st) {
    if (bf16_io) return hipErrorInvalidValue;
    switch (s.D) {
    case 32: return launch_bwd_d<32>(s, q, k, v, out, dout, lse, dq, dk, dv, st);
    case 64: return launch_bwd_d<64>(s, q, k, v, out, dout, lse, dq, dk, dv, st);
    case 128: return launch_bwd_d<128>(s, q, k, v, out, dout, lse, dq, dk, dv, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace ba
