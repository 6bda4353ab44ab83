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
};

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

__device__ __forceinline__ int64_t clamp_off(int32_t o, int64_t T) {
    int64_t x = o;
    return x < 0 ? 0 : (x > T ? T : x);
}

// Tiles of user u: ceil(L/R) row units of R rows, each with tpb sub-tiles,
// times H heads.
__device__ __forceinline__ int64_t user_tiles(const Shape &s, int u, int R, int tpb) {
    const int64_t a = clamp_off(s.offsets[u], s.T);
    const int64_t b = clamp_off(s.offsets[u + 1], s.T);
    const int64_t L = b > a ? b - a : 0;
    return ((L + R - 1) / R) * (int64_t)tpb * s.H;
}

// Inclusive prefix sum over the NT threads of a workgroup (NT a multiple of
// 64): wave-level shuffles, then one LDS pass over the wave totals.
template <int NT>
__device__ __forceinline__ int64_t wg_inclusive_scan(int64_t v, int64_t *sh) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int64_t y = __shfl_up(v, o, 64);
        if (lane >= o) v += y;
    }
    if (NT > 64) {
        if (lane == 63) sh[wave] = v;
        __syncthreads();
        int64_t add = 0;
        for (int w = 0; w < wave; ++w) add += sh[w];
        v += add;
        __syncthreads();
    }
    return v;
}

// Maps this workgroup to its tile.  A user's rows are cut into units of R
// rows (t.blk is the unit index); the logical tile order is user-major, then
// unit, then sub-tile (tpb per unit), then head, so the tiles that share K/V
// rows (same user and head, neighbouring units) are close.
// Consecutive workgroup ids are dealt round-robin over the 8 XCDs of the
// chip; the remap below gives each XCD one contiguous run of logical tiles
// (so neighbouring blocks share that XCD's L2) and balances the real tile
// count over the XCDs.  Needs gridDim.x to be a multiple of 8 and at least
// the real tile count rounded up to one.  Returns false for an idle
// workgroup.  `sh` must hold NT/64 + 4 int64 values in LDS.
template <int NT>
__device__ bool decode_tile(const Shape &s, int R, int tpb, Tile &t, int64_t *sh) {
    const int tid = threadIdx.x;
    // pass 1: total number of tiles
    int64_t total = 0;
    for (int c0 = 0; c0 < s.batch; c0 += NT) {
        const int u = c0 + tid;
        const int64_t n = u < s.batch ? user_tiles(s, u, R, tpb) : 0;
        const int64_t inc = wg_inclusive_scan<NT>(n, sh);
        if (tid == NT - 1) sh[NT / 64] = inc;
        __syncthreads();
        total += sh[NT / 64];
        __syncthreads();
    }
    // XCD-aware remap of the workgroup id onto a logical tile
    const int xcd = blockIdx.x & 7;
    const int64_t j = blockIdx.x >> 3;
    const int64_t per = total >> 3, rem = total & 7;
    if (j >= per + (xcd < rem ? 1 : 0)) return false;
    const int64_t lt = xcd * per + (xcd < rem ? xcd : rem) + j;
    // pass 2: find the user whose tile range holds lt
    int64_t base = 0;
    for (int c0 = 0; c0 < s.batch; c0 += NT) {
        const int u = c0 + tid;
        const int64_t n = u < s.batch ? user_tiles(s, u, R, tpb) : 0;
        const int64_t inc = wg_inclusive_scan<NT>(n, sh);
        if (u < s.batch && n > 0 && lt >= base + inc - n && lt < base + inc) {
            sh[NT / 64 + 1] = u;
            sh[NT / 64 + 2] = lt - (base + inc - n);
        }
        if (tid == NT - 1) sh[NT / 64] = inc;
        __syncthreads();
        const int64_t chunk = sh[NT / 64];
        const bool done = lt < base + chunk;
        base += chunk;
        if (done) break;
        __syncthreads();
    }
    const int u = (int)sh[NT / 64 + 1];
    const int64_t local = sh[NT / 64 + 2];
    const int64_t h = local % s.H;
    const int64_t rest = local / s.H;
    t.user = u;
    t.h = (int)h;
    t.blk = (int)(rest / tpb);
    t.sub = (int)(rest % tpb);
    t.tok0 = clamp_off(s.offsets[u], s.T);
    const int64_t e = clamp_off(s.offsets[u + 1], s.T);
    t.len = (int)(e > t.tok0 ? e - t.tok0 : 0);
    return true;
}

// Grid size for a tile space: an upper bound on the real tile count
// (sum_u ceil(L_u/R) <= T/R + batch), rounded up to a multiple of 8.
inline int64_t grid_upper_bound(int64_t T, int batch, int R, int tpb, int H) {
    const int64_t blocks = (T + R - 1) / R + batch;
    const int64_t g = blocks * tpb * H;
    return (g + 7) / 8 * 8;
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename TO> __device__ __forceinline__ TO from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

}  // namespace ba
