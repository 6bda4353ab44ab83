// Rotary position embedding of Q and K, rotate-half form, with positions
// local to each user ("GEM (Meta)" on aiwiki.ai, section "Custom kernels":
// the production block-attention kernel carries a rotary embedding and
// fuses its backward; the form, base and positions are readings, stated in
// include/blockattn.h).
//
// The kernel reads and writes each element once, so it is bound by HBM.  A
// workgroup finds the positions of its tokens once (a 64-way search of the
// offsets, then a short scan), keeps them and each pair's turns per position
// in LDS, and rotates Q and K rows with the angle reduced to a fraction of a
// turn in fp64, so large positions lose no accuracy.
#include "common.h"
#include "kernels.h"
#include "mfma_util.h"

namespace ba {
namespace {

constexpr int kRopeThreads = 256;

// Eight consecutive elements of a row as fp32, and back (RNE for bf16).
__device__ __forceinline__ void load8(const bf16 *p, float (&x)[8]) {
    const bf16x8 v = *(const bf16x8 *)p;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
}
__device__ __forceinline__ void load8(const float *p, float (&x)[8]) {
    const float4 a = *(const float4 *)p, b = *(const float4 *)(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void store8(bf16 *p, const float (&x)[8]) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const bf16x2 h = pack_bf16(x[e], x[e + 1]);
        v[e] = h[0];
        v[e + 1] = h[1];
    }
    *(bf16x8 *)p = v;
}
__device__ __forceinline__ void store8(float *p, const float (&x)[8]) {
    *(float4 *)p = make_float4(x[0], x[1], x[2], x[3]);
    *(float4 *)(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}

// The user that owns token t: the largest u < batch with offsets[u] <= t,
// found by the 64 lanes of one wave probing 64 splitters at a time, so a
// batch of n users takes about log64(n) rounds.  Every read stays inside
// offsets[1 .. batch-1] and the range shrinks every round, also for
// malformed offsets.
__device__ int user_of(const int32_t *off, int batch, int T, int64_t t, int lane) {
    int lo = 0, hi = batch;  // the answer is in [lo, hi)
    while (hi - lo > 1) {
        const int span = hi - lo - 1;  // candidates lo+1 .. hi-1
        const int p = lo + 1 + (int)(((int64_t)span * lane) >> 6);
        const bool le = clamp_off(off[p], T) <= t;
        const int cnt = __popcll(__ballot(le));
        const int nlo = cnt > 0 ? __shfl(p, cnt - 1, 64) : lo;
        const int nhi = cnt < 64 ? __shfl(p, cnt, 64) : hi;
        lo = nlo;
        hi = nhi;
    }
    return lo;
}

constexpr int kRopeTok = 32;   // tokens per workgroup
constexpr int kRopeBatch = 4;  // items per thread whose loads are all issued first

// A workgroup rotates the rows of kRopeTok consecutive tokens.  An item is
// (token, head, group of 8 pairs); thread i takes items i, i + 256, ... in
// batches of kRopeBatch, loading every row of a batch before it stores any
// (outputs may alias inputs, so the compiler could not reorder them itself).
template <typename TI, int D>
__global__ __launch_bounds__(kRopeThreads) void rope_kernel(
    const TI *q, const TI *k, const int32_t *__restrict__ offsets, int batch, int T, int H,
    double turns_log2, TI *q_rot, TI *k_rot) {
    constexpr int G = D / 16;  // groups of 8 pairs per row
    __shared__ double rrev[D / 2];  // turns per position of each pair
    __shared__ int pos_sh[kRopeTok];
    __shared__ int u0;
    const int tid = threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.x * kRopeTok;
    const int ntok = (int)min((int64_t)kRopeTok, (int64_t)T - t0);
    if (tid < 64) {
        const int u = user_of(offsets, batch, T, t0, tid);
        if (tid == 0) u0 = u;
    }
    // pair d turns by base^(-2d/D) radians per position
    if (tid < D / 2) rrev[tid] = exp2(-2.0 * tid / D * turns_log2) * kInv2Pi;
    __syncthreads();
    if (tid < ntok) {
        const int64_t t = t0 + tid;
        int u = u0;
        while (u + 1 < batch && clamp_off(offsets[u + 1], T) <= t) ++u;
        pos_sh[tid] = (int)(t - clamp_off(offsets[u], T));
    }
    __syncthreads();

    const int items = ntok * H * G;
    const int64_t rs = (int64_t)H * D;
    for (int i0 = tid; i0 < items; i0 += kRopeThreads * kRopeBatch) {
        float lo[kRopeBatch][2][8], hi[kRopeBatch][2][8];
        int64_t base[kRopeBatch];
        int pos[kRopeBatch], grp[kRopeBatch];
        bool live[kRopeBatch];
#pragma unroll
        for (int b = 0; b < kRopeBatch; ++b) {
            const int it = i0 + b * kRopeThreads;
            live[b] = it < items;
            const int tl = live[b] ? it / (H * G) : 0, rem = live[b] ? it % (H * G) : 0;
            const int h = rem / G;
            grp[b] = rem % G;
            pos[b] = pos_sh[tl];
            base[b] = (t0 + tl) * rs + (int64_t)h * D + 8 * grp[b];
            if (live[b]) {
                load8(q + base[b], lo[b][0]);
                load8(q + base[b] + D / 2, hi[b][0]);
                load8(k + base[b], lo[b][1]);
                load8(k + base[b] + D / 2, hi[b][1]);
            }
        }
#pragma unroll
        for (int b = 0; b < kRopeBatch; ++b) {
            if (!live[b]) continue;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float sn, cs;
                rope_sincos<TI>((double)pos[b] * rrev[8 * grp[b] + e], sn, cs);
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    const float x = lo[b][w][e], y = hi[b][w][e];
                    lo[b][w][e] = x * cs - y * sn;
                    hi[b][w][e] = y * cs + x * sn;
                }
            }
            store8(q_rot + base[b], lo[b][0]);
            store8(q_rot + base[b] + D / 2, hi[b][0]);
            store8(k_rot + base[b], lo[b][1]);
            store8(k_rot + base[b] + D / 2, hi[b][1]);
        }
    }
}

template <typename TI, int D>
hipError_t launch_t(const Shape &s, const void *q, const void *k, void *q_rot, void *k_rot,
                    hipStream_t st) {
    const int64_t grid = (s.T + kRopeTok - 1) / kRopeTok;
    hipLaunchKernelGGL((rope_kernel<TI, D>), dim3((unsigned)grid), dim3(kRopeThreads), 0, st,
                       (const TI *)q, (const TI *)k, s.offsets, s.batch, (int)s.T, s.H,
                       log2((double)s.rope_base), (TI *)q_rot, (TI *)k_rot);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rope(const Shape &s, bool bf16_io, const void *q, const void *k, void *q_rot,
                       void *k_rot, hipStream_t st) {
    switch (s.D) {
    case 32:
        return bf16_io ? launch_t<bf16, 32>(s, q, k, q_rot, k_rot, st)
                       : launch_t<float, 32>(s, q, k, q_rot, k_rot, st);
    case 64:
        return bf16_io ? launch_t<bf16, 64>(s, q, k, q_rot, k_rot, st)
                       : launch_t<float, 64>(s, q, k, q_rot, k_rot, st);
    case 128:
        return bf16_io ? launch_t<bf16, 128>(s, q, k, q_rot, k_rot, st)
                       : launch_t<float, 128>(s, q, k, q_rot, k_rot, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace ba
