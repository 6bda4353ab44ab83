// Shared device-side definitions of the block-attention kernels (gfx950).
//
// The jagged tile scheduler lives here: the pages stress that user histories
// are jagged and that padding them would waste compute ("GEM (Meta)",
// sections "Training infrastructure" and "Custom kernels"), so every kernel
// enumerates exactly the blocks that exist, on the device, from the int32
// offsets, without any host read of them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ba {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Sizes of one call.  Tensors are [T, H, D]; row statistics are [H, T].
struct Shape {
    const int32_t *offsets;
    int batch;
    int64_t T;
    int H;
    int D;
    int B;  // block size (tokens)
    int W;  // window in blocks, own block included
    float scale;
    float rope_base;  // > 0: the backward returns gradients through a rotary
                      // embedding with this base (see rope_sincos); 0: none
    int act;          // score function: kSoftmax, or a GDPA activation
};

// Score functions.  kSoftmax is block attention proper.  The others are
// generalized dot-product attention ("GEM (Meta)" on aiwiki.ai, section
// "Custom kernels": the softmax replaced by an activation such as GELU or
// SiLU), read as P_ij = act(scale <q_i, k_j>) with no normalisation.
enum { kSoftmax = 0, kSilu = 1, kGelu = 2 };

// act(x) and act'(x) in fp32.  SiLU: x s(x) with the logistic s(x) =
// 1 / (1 + 2^(-x log2 e)), slope s(x) (1 + x (1 - s(x))); it tends to 0 (and
// slope 0) for large negative x, where 2^(...) overflows to +inf.  GELU, the
// erf form: x Phi(x), slope Phi(x) + x phi(x), with Phi the standard normal
// CDF and phi its density.
template <int ACT>
__device__ __forceinline__ void act_value_slope(float x, float &a, float &g) {
    if constexpr (ACT == kSilu) {
        const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
        a = x * sg;
        g = sg * (1.f + x * (1.f - sg));
    } else {
        const float cdf = 0.5f * (1.f + erff(x * 0.70710678118654752f));
        const float pdf =
            0.39894228040143268f * __builtin_amdgcn_exp2f(-0.5f * 1.4426950408889634f * x * x);
        a = x * cdf;
        g = cdf + x * pdf;
    }
}
template <int ACT>
__device__ __forceinline__ float act_value(float x) {
    float a, g;
    act_value_slope<ACT>(x, a, g);
    return a;
}
template <int ACT>
__device__ __forceinline__ float act_slope(float x) {
    float a, g;
    act_value_slope<ACT>(x, a, g);
    return g;
}

// One tile of work: sub-tile `sub` of row unit `blk` (local to the user), head
// h, of user `user` whose tokens start at packed index tok0 and who has len
// tokens.  Callers turn `sub` into rows (and, for the backward, a role).
struct Tile {
    int user;
    int blk;
    int sub;
    int h;
    int64_t tok0;
    int len;
};

__device__ __forceinline__ int clamp_off(int32_t o, int T) { return o < 0 ? 0 : (o > T ? T : o); }

// Inclusive prefix sum over the NT threads of a workgroup (NT a multiple of
// 64): wave-level shuffles, then one LDS pass over the wave totals.  Also
// returns the workgroup total.  `sh` holds NT/64 ints.
template <int NT, typename I = int>
__device__ __forceinline__ I wg_inclusive_scan(I v, I *sh, I &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const I y = __shfl_up(v, o, 64);
        if (lane >= o) v += y;
    }
    if (NT == 64) {
        total = __shfl(v, 63, 64);
        return v;
    }
    if (lane == 63) sh[wave] = v;
    __syncthreads();
    I add = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const I x = sh[w];
        add += w < wave ? x : 0;
        tot += x;
    }
    __syncthreads();
    total = tot;
    return v + add;
}

// Workgroups are dealt round-robin over the 8 XCDs in id order.  The logical
// tile of a workgroup is chosen so that each XCD works through runs of kRun
// consecutive logical tiles: neighbouring tiles, which read the same K/V
// rows, then share one XCD's L2.  The map is a bijection on [0, grid) when
// grid is a multiple of 8 * kRun.
constexpr int kRun = 16;
__device__ __forceinline__ int logical_tile() {
    const int b = blockIdx.x, xcd = b & 7, j = b >> 3;
    return ((j / kRun) * 8 + xcd) * kRun + (j % kRun);
}

// Maps this workgroup to its tile.  A user's rows are cut into units of R
// rows; the logical order is user, then head, then unit, then sub-tile (tpb
// per unit), so consecutive tiles are consecutive row units of one (user,
// head).  Tiles exist only for rows that exist: a jagged batch costs no
// padding.  Returns false for a workgroup beyond the last tile (the grid is
// an upper bound, since the host never reads the offsets).  Each pass of the
// scan covers NT * UPT users.  `sh` must hold NT/64 + 4 ints in LDS.  All
// results are wave-uniform.
template <int NT, int UPT = 1>
__device__ bool decode_tile(const Shape &s, int R, int tpb, Tile &t, int *sh) {
    const int tid = threadIdx.x;
    const int lt = logical_tile();
    const int T = (int)s.T;
    int base = 0;
    for (int c0 = 0; c0 < s.batch; c0 += NT * UPT) {
        // UPT consecutive users per thread: UPT + 1 offsets, read once
        const int u0 = c0 + tid * UPT;
        int n[UPT], a[UPT], L[UPT];
        int sum = 0;
        if constexpr (UPT == 1) {
            n[0] = a[0] = L[0] = 0;
            if (u0 < s.batch) {  // both offsets in one branch
                a[0] = clamp_off(s.offsets[u0], T);
                const int e = clamp_off(s.offsets[u0 + 1], T);
                L[0] = e > a[0] ? e - a[0] : 0;
                n[0] = (int)(((int64_t)L[0] + R - 1) / R * tpb * s.H);
            }
            sum = n[0];
        } else {
            int prev = u0 < s.batch ? clamp_off(s.offsets[u0], T) : 0;
#pragma unroll
            for (int i = 0; i < UPT; ++i) {
                n[i] = a[i] = L[i] = 0;
                if (u0 + i < s.batch) {
                    const int e = clamp_off(s.offsets[u0 + i + 1], T);
                    a[i] = prev;
                    L[i] = e > prev ? e - prev : 0;
                    n[i] = (int)(((int64_t)L[i] + R - 1) / R * tpb * s.H);
                    prev = e;
                }
                sum += n[i];
            }
        }
        int chunk;
        const int incl = wg_inclusive_scan<NT>(sum, sh, chunk);
        // the thread of the owning user passes on its rows (no second read
        // of the offsets)
        int first = base + incl - sum;
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            if (n[i] > 0 && lt >= first && lt < first + n[i]) {
                sh[NT / 64] = u0 + i;
                sh[NT / 64 + 1] = lt - first;
                sh[NT / 64 + 2] = a[i];
                sh[NT / 64 + 3] = L[i];
            }
            first += n[i];
        }
        base += chunk;
        if (lt < base) break;  // uniform: base and lt are the same in every thread
    }
    if (lt >= base) return false;
    __syncthreads();
    const int u = __builtin_amdgcn_readfirstlane(sh[NT / 64]);
    const int local = __builtin_amdgcn_readfirstlane(sh[NT / 64 + 1]);
    const int a = __builtin_amdgcn_readfirstlane(sh[NT / 64 + 2]);
    const int L = __builtin_amdgcn_readfirstlane(sh[NT / 64 + 3]);
    const int per_head = (int)(((int64_t)L + R - 1) / R * tpb);
    t.user = u;
    t.h = local / per_head;
    const int rem = local - t.h * per_head;
    t.blk = rem / tpb;
    t.sub = rem - t.blk * tpb;
    t.tok0 = a;
    t.len = L;
    return true;
}

// Grid size for a tile space: an upper bound on the real tile count
// (sum_u ceil(L_u/R) <= T/R + batch), rounded up to a multiple of 8 * kRun.
inline int64_t grid_upper_bound(int64_t T, int batch, int R, int tpb, int H) {
    const int64_t blocks = (T + R - 1) / R + batch;
    const int64_t g = blocks * tpb * H;
    return (g + 8 * kRun - 1) / (8 * kRun) * (8 * kRun);
}

// Rotary embedding angles.  Pair d (features d and d + D/2) of a token at
// position p turns by p * base^(-2d/D) radians; the kernels carry it as
// `turns` = that angle / (2 pi), computed in fp64, and reduce it to
// [-1/2, 1/2] turn before taking the sine and cosine, so large positions
// keep full accuracy.  bf16 paths use the hardware's turn-based sine and
// cosine (fp32); the fp32 path takes them in fp64.
constexpr double kInv2Pi = 0.15915494309189533577;
template <typename TI>
__device__ __forceinline__ void rope_sincos(double turns, float &s, float &c);
template <>
__device__ __forceinline__ void rope_sincos<bf16>(double turns, float &s, float &c) {
    const float f = (float)(turns - rint(turns));
    s = __builtin_amdgcn_sinf(f);
    c = __builtin_amdgcn_cosf(f);
}
template <>
__device__ __forceinline__ void rope_sincos<float>(double turns, float &s, float &c) {
    double sd, cd;
    sincos((turns - rint(turns)) * 6.283185307179586477, &sd, &cd);
    s = (float)sd;
    c = (float)cd;
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename TO> __device__ __forceinline__ TO from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

}  // namespace ba
