// Forward block attention on bf16 MFMA (gfx950).
//
// The pattern is the block window of "GEM (Meta)" (aiwiki.ai), section
// "Custom kernels" (self-attention as independent fixed-size token blocks)
// and the ai.info news item, section "Kunlun changes how GEM scales" (sparse
// attention in blocks, linear cost at a fixed window): local query i sees
// local key j iff j <= i and floor(i/B) - floor(j/B) < W.
//
// Work split.  A workgroup of 4 waves owns 128 consecutive rows of one user
// and one head; wave w owns rows [row0 + 32w, row0 + 32w + 32).  The tile
// does not depend on B: every row carries its own window start, so any B
// that is a multiple of 16 works, and B = 64/128/256 need no window masks.
// Keys are streamed in chunks of 64 from the window start of the tile's
// first row: K into LDS as is, V transposed into LDS, with the next chunk's
// global loads in flight while the current chunk is computed.
//
// Per chunk and wave, with 32x32x16 bf16 MFMAs and fp32 accumulation:
//   S^T = K Q^T   (K from LDS, Q^T held in registers for the whole tile)
//   mask (causal, window) only on the sub-tiles that straddle a boundary
//   online softmax in the base-2 domain; each lane owns one query, so the
//   row max needs one exchange with lane^32 and the row sum none until the
//   end; a row's running max is only moved when it grows by more than 2^8
//   O^T += V^T P^T (V^T from LDS, P^T straight from the S^T accumulators)
//
// Lane layouts of v_mfma_f32_32x32x16_bf16 (g = lane/32, i = 0..7):
//   A[m][k]: lane holds A[lane%32][8g + i];  B[k][n]: lane holds B[8g + i][lane%32]
//   C[m][n]: lane, register r holds C[8(r/4) + 4g + r%4][lane%32].
// Loading A row m from key sigma(m), where sigma swaps bits 2 and 3, makes
// C register r of lane (g) hold key 16(r/8) + 8g + r%8: registers 0..7 and
// 8..15 are then exactly the B operands of the two 16-key PV products.  The
// same permutation on the rows of V^T gives each lane 8 consecutive output
// columns per register octet.
#include "common.h"
#include "kernels.h"

namespace ba {
namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kTileRows = 128;
constexpr int kKC = 64;        // keys per staged chunk
constexpr int kPad = 8;        // bf16 padding per LDS row (16 bytes)

__device__ __forceinline__ int sigma32(int a) {
    return (a & ~12) | ((a & 4) << 1) | ((a & 8) >> 1);
}
__device__ __forceinline__ int sigma(int x) { return (x & ~31) | sigma32(x & 31); }

__device__ __forceinline__ int window_start(int row, int B, int W) {
    return max(0, row / B - W + 1) * B;
}

template <int D>
struct FwdSmem {
    bf16 k[kKC][D + kPad];   // row r holds key sigma(r) of the chunk
    bf16 vt[D][kKC + kPad];  // row r holds head-dim column sigma(r), keys along the row
};

template <int D>
struct ChunkRegs {
    static constexpr int KP = kKC * D / 8 / kThreads;               // 16-byte K pieces
    static constexpr int VU = (kKC / 4 * D / 4 + kThreads - 1) / kThreads;  // 4x4 V units
    bf16x8 k[KP];
    uint2 v[VU][4];
};

// Global -> registers for keys [c0, c0 + 64) of one (user, head); keys at or
// beyond kend read as zero.
template <int D>
__device__ __forceinline__ void load_chunk(ChunkRegs<D> &r, const bf16 *__restrict__ k,
                                           const bf16 *__restrict__ v, int64_t base,
                                           int64_t rs, int c0, int kend) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < ChunkRegs<D>::KP; ++i) {
        const int p = tid + i * kThreads;
        const int key = c0 + p / (D / 8);
        const int c8 = p % (D / 8);
        bf16x8 x = {};
        if (key < kend) x = *(const bf16x8 *)(k + base + (int64_t)key * rs + c8 * 8);
        r.k[i] = x;
    }
#pragma unroll
    for (int i = 0; i < ChunkRegs<D>::VU; ++i) {
        const int u = tid + i * kThreads;
        const int k4 = u / (D / 4), d4 = u % (D / 4);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int key = c0 + k4 * 4 + kk;
            uint2 x = make_uint2(0u, 0u);
            if (u < kKC / 4 * D / 4 && key < kend)
                x = *(const uint2 *)(v + base + (int64_t)key * rs + d4 * 4);
            r.v[i][kk] = x;
        }
    }
}

// Registers -> LDS: K rows permuted by sigma, V transposed (4x4 per thread).
template <int D>
__device__ __forceinline__ void store_chunk(const ChunkRegs<D> &r, FwdSmem<D> &sm) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < ChunkRegs<D>::KP; ++i) {
        const int p = tid + i * kThreads;
        const int row = p / (D / 8), c8 = p % (D / 8);
        *(bf16x8 *)&sm.k[sigma(row)][c8 * 8] = r.k[i];
    }
#pragma unroll
    for (int i = 0; i < ChunkRegs<D>::VU; ++i) {
        const int u = tid + i * kThreads;
        if (u >= kKC / 4 * D / 4) break;
        const int k4 = u / (D / 4), d4 = u % (D / 4);
        const uint2 *x = r.v[i];
        // column dd of the 4x4 block: (key0, key1) in .x, (key2, key3) in .y
        uint2 c0, c1, c2, c3;
        c0.x = (x[0].x & 0xffffu) | (x[1].x << 16);
        c0.y = (x[2].x & 0xffffu) | (x[3].x << 16);
        c1.x = (x[0].x >> 16) | (x[1].x & 0xffff0000u);
        c1.y = (x[2].x >> 16) | (x[3].x & 0xffff0000u);
        c2.x = (x[0].y & 0xffffu) | (x[1].y << 16);
        c2.y = (x[2].y & 0xffffu) | (x[3].y << 16);
        c3.x = (x[0].y >> 16) | (x[1].y & 0xffff0000u);
        c3.y = (x[2].y >> 16) | (x[3].y & 0xffff0000u);
        *(uint2 *)&sm.vt[sigma(d4 * 4 + 0)][k4 * 4] = c0;
        *(uint2 *)&sm.vt[sigma(d4 * 4 + 1)][k4 * 4] = c1;
        *(uint2 *)&sm.vt[sigma(d4 * 4 + 2)][k4 * 4] = c2;
        *(uint2 *)&sm.vt[sigma(d4 * 4 + 3)][k4 * 4] = c3;
    }
}

template <int D>
__global__ __launch_bounds__(kThreads) void fwd_mfma(Shape s, const bf16 *__restrict__ q,
                                                     const bf16 *__restrict__ k,
                                                     const bf16 *__restrict__ v,
                                                     bf16 *__restrict__ out,
                                                     float *__restrict__ lse) {
    __shared__ int64_t sh[8];
    __shared__ __align__(16) FwdSmem<D> sm;
    Tile t;
    if (!decode_tile<kThreads>(s, kTileRows, 1, t, sh)) return;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int qi = lane & 31, g = lane >> 5;
    const int64_t rs = (int64_t)s.H * D;
    const int64_t base = t.tok0 * rs + (int64_t)t.h * D;
    const int row0 = t.blk * kTileRows;
    const int row_end = min(row0 + kTileRows, t.len);  // rows and keys end here
    const int wr0 = row0 + w * 32;
    const int my_row = wr0 + qi;
    const bool wave_live = wr0 < row_end;
    const int w_last = min(wr0 + 31, row_end - 1);
    const int wave_klo = window_start(wr0, s.B, s.W);
    const int wave_klo_max = window_start(max(wr0, w_last), s.B, s.W);
    const int my_klo = window_start(my_row, s.B, s.W);
    // Fold the sign of scale into Q so that c >= 0 and max commutes with it.
    const float c = fabsf(s.scale) * kLog2e;
    const uint32_t qsign = s.scale < 0.f ? 0x80008000u : 0u;

    bf16x8 qreg[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        bf16x8 x = {};
        if (my_row < row_end) {
            x = *(const bf16x8 *)(q + base + (int64_t)my_row * rs + ks * 16 + g * 8);
            uint4 u = __builtin_bit_cast(uint4, x);
            u.x ^= qsign;
            u.y ^= qsign;
            u.z ^= qsign;
            u.w ^= qsign;
            x = __builtin_bit_cast(bf16x8, u);
        }
        qreg[ks] = x;
    }

    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
    float m = -INFINITY, l = 0.f;

    const int kbeg = window_start(row0, s.B, s.W);
    ChunkRegs<D> regs;
    load_chunk<D>(regs, k, v, base, rs, kbeg, row_end);
    for (int c0 = kbeg; c0 < row_end; c0 += kKC) {
        __syncthreads();
        store_chunk<D>(regs, sm);
        __syncthreads();
        if (c0 + kKC < row_end) load_chunk<D>(regs, k, v, base, rs, c0 + kKC, row_end);
        if (!wave_live) continue;

        bool act[2], msk[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const int a = c0 + st * 32;
            act[st] = a <= w_last && a + 31 >= wave_klo;
            msk[st] = a + 31 > wr0 || a < wave_klo_max;
        }
        if (!act[0] && !act[1]) continue;

        f32x16 sc[2];
        float mx = -INFINITY;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            sc[st] = f32x16{};
            if (!act[st]) continue;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const bf16x8 a = *(const bf16x8 *)&sm.k[st * 32 + qi][ks * 16 + g * 8];
                sc[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], sc[st], 0, 0, 0);
            }
            if (msk[st]) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = c0 + st * 32 + (r >> 3) * 16 + g * 8 + (r & 7);
                    if (key > my_row || key < my_klo) sc[st][r] = -INFINITY;
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[st][r]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // Lazy rescale: a row keeps a stale max unless its scores grew past it
        // by 2^8.  The decision is per row (alpha is exactly 1 for rows that
        // keep theirs), so a row's rounding never depends on other rows.
        const bool grow = (m == -INFINITY) || (mx - m) * c > 8.f;
        if (__any(grow)) {
            const float mn = grow ? fmaxf(m, mx) : m;
            const float alpha = (m == -INFINITY) ? 0.f : exp2f((m - mn) * c);
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
            m = mn;
        }
        const float mc = (m == -INFINITY) ? 0.f : m * c;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            if (!act[st]) continue;
            bf16x8 pb[2];
            if (msk[st]) {
                // masked scores are -inf; c may be 0, so zero their weight here
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p = __builtin_amdgcn_exp2f(fmaf(sc[st][r], c, -mc));
                    p = sc[st][r] == -INFINITY ? 0.f : p;
                    l += p;
                    pb[r >> 3][r & 7] = (bf16)p;
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(sc[st][r], c, -mc));
                    l += p;
                    pb[r >> 3][r & 7] = (bf16)p;
                }
            }
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const bf16x8 a =
                        *(const bf16x8 *)&sm.vt[dt * 32 + qi][st * 32 + kk * 16 + g * 8];
                    acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kk], acc[dt], 0,
                                                                      0, 0);
                }
            }
        }
    }

    const float lt = l + __shfl_xor(l, 32, 64);
    if (!wave_live || my_row >= row_end) return;
    const float inv = 1.f / lt;
    bf16 *o = out + base + (int64_t)my_row * rs;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            bf16x8 x;
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = (bf16)(acc[dt][half * 8 + i] * inv);
            *(bf16x8 *)(o + dt * 32 + half * 16 + g * 8) = x;
        }
    }
    if (g == 0) lse[(int64_t)t.h * s.T + t.tok0 + my_row] = (m * c + log2f(lt)) * kLn2;
}

template <int D>
hipError_t launch_t(const Shape &s, const void *q, const void *k, const void *v, void *out,
                    float *lse, hipStream_t st) {
    const int64_t grid = grid_upper_bound(s.T, s.batch, kTileRows, 1, s.H);
    hipLaunchKernelGGL((fwd_mfma<D>), dim3((unsigned)grid), dim3(kThreads), 0, st, s,
                       (const bf16 *)q, (const bf16 *)k, (const bf16 *)v, (bf16 *)out, lse);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_fwd(const Shape &s, const void *q, const void *k, const void *v,
                           void *out, float *lse, hipStream_t st) {
    switch (s.D) {
    case 32: return launch_t<32>(s, q, k, v, out, lse, st);
    case 64: return launch_t<64>(s, q, k, v, out, lse, st);
    case 128: return launch_t<128>(s, q, k, v, out, lse, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace ba
