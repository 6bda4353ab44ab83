// Device helpers shared by the bf16 MFMA kernels (gfx950).
#pragma once

#include "common.h"

namespace ba {

// sigma swaps bits 2 and 3 of a row index inside each group of 32 rows.
// Operand rows stored at LDS row sigma(m) make register r of an MFMA
// 32x32x16 accumulator (lane group g = lane/32) hold logical row
// 16(r/8) + 8g + r%8, i.e. 8 consecutive rows per register octet, which is
// the B-operand layout of the next 16-deep product.
__device__ __forceinline__ int sigma32(int a) {
    return (a & ~12) | ((a & 4) << 1) | ((a & 8) >> 1);
}
__device__ __forceinline__ int sigma(int x) { return (x & ~31) | sigma32(x & 31); }

// rho: operand row m holds logical row (m & 3) | ((m >> 3) & 3) << 2 |
// ((m >> 2) & 1) << 4 inside each group of 32 rows, which makes register r
// of lane group g of a 32x32 accumulator hold logical row 16g + r: 16
// consecutive rows per lane, the operand layout of the 64-deep block-scaled
// fp8 product (lane (n, g) holds elements 16g .. 16g + 15 of each 32-element
// block).
__device__ __forceinline__ int rho32(int m) {
    return (m & 3) | (((m >> 3) & 3) << 2) | (((m >> 2) & 1) << 4);
}
__device__ __forceinline__ int rho(int x) { return (x & ~31) | rho32(x & 31); }

// First local key visible to local query `row`: its own block plus the W-1
// previous blocks, clipped at the user's first token.
__device__ __forceinline__ int window_start(int row, int B, int W) {
    return max(0, row / B - W + 1) * B;
}
// One past the last local query that sees local key `key` (queries end at L).
__device__ __forceinline__ int window_end(int key, int B, int W, int L) {
    return (int)min(((int64_t)(key / B) + W) * B, (int64_t)L);
}

// Buffer resource over `rows` rows of stride `rs` elements starting at
// `base`, ending after D bf16 columns of the last row: reads past it return
// zero without touching memory.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const bf16 *base, int rows,
                                                           int64_t rs) {
    const uint32_t bytes = rows > 0 ? (uint32_t)((int64_t)(rows - 1) * rs * 2 + D * 2) : 0u;
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, bytes, 0x00020000);
}

// The same range as a raw 4-dword buffer descriptor (for instructions issued
// from inline assembly): base address, 16-bit high part and stride 0, byte
// count, and the dword-format word of gfx9 raw buffers.
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x2 __attribute__((ext_vector_type(2)));  // packed fp8 conversions
template <int D>
__device__ __forceinline__ i32x4 row_desc(const bf16 *base, int rows, int64_t rs) {
    const uint32_t bytes = rows > 0 ? (uint32_t)((int64_t)(rows - 1) * rs * 2 + D * 2) : 0u;
    const uint64_t a = (uint64_t)base;
    return i32x4{(int)(uint32_t)a, (int)((a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store16(uint4 x, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, off, 0, 0);
}
__device__ __forceinline__ void buf_store4(float x, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off, 0, 0);
}
// Raw buffer resource over `bytes` bytes at `base`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bytes_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

// Value of lane^32 combined with this lane's (one VALU op on gfx950).
__device__ __forceinline__ float swap_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Transpose of a 4x4 bf16 block held as 4 rows of uint2 (columns 0,1 in .x,
// 2,3 in .y): c[j] receives column j as (row0, row1) in .x, (row2, row3) in .y.
__device__ __forceinline__ void transpose4x4(const uint2 (&x)[4], uint2 (&c)[4]) {
    c[0] = make_uint2(__builtin_amdgcn_perm(x[1].x, x[0].x, 0x05040100u),
                      __builtin_amdgcn_perm(x[3].x, x[2].x, 0x05040100u));
    c[1] = make_uint2(__builtin_amdgcn_perm(x[1].x, x[0].x, 0x07060302u),
                      __builtin_amdgcn_perm(x[3].x, x[2].x, 0x07060302u));
    c[2] = make_uint2(__builtin_amdgcn_perm(x[1].y, x[0].y, 0x05040100u),
                      __builtin_amdgcn_perm(x[3].y, x[2].y, 0x05040100u));
    c[3] = make_uint2(__builtin_amdgcn_perm(x[1].y, x[0].y, 0x07060302u),
                      __builtin_amdgcn_perm(x[3].y, x[2].y, 0x07060302u));
}

// Two floats rounded to bf16 (nearest even) in one packed register.
__device__ __forceinline__ bf16x2 pack_bf16(float a, float b) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    return __builtin_convertvector((f32x2){a, b}, bf16x2);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace ba
