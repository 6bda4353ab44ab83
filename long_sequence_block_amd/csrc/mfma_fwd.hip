// Forward block attention on bf16 MFMA (gfx950).
//
// The pattern is the block window of "GEM (Meta)" (aiwiki.ai), section
// "Custom kernels" (self-attention as independent fixed-size token blocks)
// and the ai.info news item, section "Kunlun changes how GEM scales" (sparse
// attention in blocks, linear cost at a fixed window): local query i sees
// local key j iff j <= i and floor(i/B) - floor(j/B) < W.
//
// Work split.  A workgroup of 4 waves owns 128 consecutive rows of one user
// and one head; each wave owns 32 of them (which 32 rotates with the tile so
// that the causal imbalance between waves does not always land on the same
// SIMD).  Every row carries its own window start, so any B that is a
// multiple of 16 works.  Keys are streamed in chunks of 64 from the window
// start of the tile's first row, through two LDS buffers: while the waves
// compute on one, the next chunk's global loads are in flight and are
// written into the other, with one barrier per chunk.  Global loads go
// through buffer resources sized to the chunk's valid rows, so keys past the
// tile's last row read as zero without a branch.
//
// Per chunk and wave, with 32x32x16 bf16 MFMAs and fp32 accumulation:
//   S^T = K Q^T   (K from LDS, Q^T held in registers for the whole tile)
//   mask (causal, window) only on the sub-tiles that straddle a boundary
//   online softmax in the base-2 domain; each lane owns one query, so the
//   row max needs one lane^32 exchange and the row sum none until the end;
//   a row's running max is only moved when it grows by more than 2^8
//   O^T += V^T P^T (V^T from LDS, P^T straight from the S^T accumulators)
//
// Lane layouts of v_mfma_f32_32x32x16_bf16 (g = lane/32, i = 0..7):
//   A[m][k]: lane holds A[lane%32][8g + i];  B[k][n]: lane holds B[8g + i][lane%32]
//   C[m][n]: lane, register r holds C[8(r/4) + 4g + r%4][lane%32].
// Storing key row m at LDS row sigma(m), where sigma swaps bits 2 and 3,
// makes C register r of lane (g) hold key 16(r/8) + 8g + r%8: registers
// 0..7 and 8..15 are then exactly the B operands of the two 16-key PV
// products.  The same permutation on the rows of V^T gives each lane 8
// consecutive output columns per register octet.
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
struct FwdBuf {
    bf16 k[kKC][D + kPad];   // row r holds key sigma(r) of the chunk
    bf16 vt[D][kKC + kPad];  // row r holds head-dim column sigma(r), keys along the row
};

// One chunk of K and V in registers on its way from HBM to LDS: K as 16-byte
// row pieces, V as 4 keys x 4 columns units (transposed on the way to LDS).
template <int D>
struct Stage {
    static constexpr int KP = kKC * D / 8 / kThreads;
    static constexpr int VUnits = kKC / 4 * D / 4;
    static constexpr int VU = (VUnits + kThreads - 1) / kThreads;
    uint4 k[KP];
    uint2 v[VU][4];
};

// Buffer resource over `rows` rows (of stride `rs` elements) starting at
// `base`, covering D columns of the last row: reads past it return zero.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const bf16 *base, int rows,
                                                           int64_t rs) {
    const uint32_t bytes = rows > 0 ? (uint32_t)((int64_t)(rows - 1) * rs * 2 + D * 2) : 0u;
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, bytes, 0x00020000);
}

template <int D>
__device__ __forceinline__ void load_chunk(Stage<D> &r, __amdgpu_buffer_rsrc_t kr,
                                           __amdgpu_buffer_rsrc_t vr, uint32_t rsb) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < Stage<D>::KP; ++i) {
        const int p = tid + i * kThreads;
        const int row = p / (D / 8), c8 = p % (D / 8);
        r.k[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                               kr, row * rsb + c8 * 16, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < Stage<D>::VU; ++i) {
        const int u = tid + i * kThreads;
        const int k4 = u % (kKC / 4), d4 = u / (kKC / 4);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            uint2 x = make_uint2(0u, 0u);
            if (u < Stage<D>::VUnits)
                x = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                                  vr, (k4 * 4 + kk) * rsb + d4 * 8, 0, 0));
            r.v[i][kk] = x;
        }
    }
}

// Registers -> LDS: K rows permuted by sigma, V transposed (4x4 per thread).
// The 16 consecutive lanes that share a column group write one 128-byte run
// of a V^T row, so the stores are free of bank conflicts.
template <int D>
__device__ __forceinline__ void store_chunk(const Stage<D> &r, FwdBuf<D> &sm) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < Stage<D>::KP; ++i) {
        const int p = tid + i * kThreads;
        const int row = p / (D / 8), c8 = p % (D / 8);
        *(uint4 *)&sm.k[sigma(row)][c8 * 8] = r.k[i];
    }
#pragma unroll
    for (int i = 0; i < Stage<D>::VU; ++i) {
        const int u = tid + i * kThreads;
        if (u >= Stage<D>::VUnits) break;
        const int k4 = u % (kKC / 4), d4 = u / (kKC / 4);
        const uint2 *x = r.v[i];
        // column dd of the 4x4 unit: (key0, key1) in .x, (key2, key3) in .y
        uint2 c[4];
        c[0] = make_uint2(__builtin_amdgcn_perm(x[1].x, x[0].x, 0x05040100u),
                          __builtin_amdgcn_perm(x[3].x, x[2].x, 0x05040100u));
        c[1] = make_uint2(__builtin_amdgcn_perm(x[1].x, x[0].x, 0x07060302u),
                          __builtin_amdgcn_perm(x[3].x, x[2].x, 0x07060302u));
        c[2] = make_uint2(__builtin_amdgcn_perm(x[1].y, x[0].y, 0x05040100u),
                          __builtin_amdgcn_perm(x[3].y, x[2].y, 0x05040100u));
        c[3] = make_uint2(__builtin_amdgcn_perm(x[1].y, x[0].y, 0x07060302u),
                          __builtin_amdgcn_perm(x[3].y, x[2].y, 0x07060302u));
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) *(uint2 *)&sm.vt[sigma(d4 * 4 + dd)][k4 * 4] = c[dd];
    }
}

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

// Waves per SIMD the register budget is sized for (2 workgroups of 4 waves
// per CU at D = 128, 3 below).
template <int D>
constexpr int kWavesPerSimd = D == 128 ? 2 : 3;

template <int D>
__global__ __launch_bounds__(kThreads, kWavesPerSimd<D>) void fwd_mfma(Shape s, const bf16 *__restrict__ q,
                                                     const bf16 *__restrict__ k,
                                                     const bf16 *__restrict__ v,
                                                     bf16 *__restrict__ out,
                                                     float *__restrict__ lse) {
    __shared__ int sh[8];
    __shared__ __align__(16) FwdBuf<D> sm[2];
    Tile t;
    if (!decode_tile<kThreads>(s, kTileRows, 1, t, sh)) return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = ((tid >> 6) + t.blk) & 3;  // row group of this wave
    const int qi = lane & 31, g = lane >> 5;
    const int64_t rs = (int64_t)s.H * D;
    const uint32_t rsb = (uint32_t)(rs * 2);
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
    // Fold the sign of scale into Q so that c > 0 and max commutes with it;
    // c is kept away from 0 so that masked scores (-inf) stay -inf.
    const float c = fmaxf(fabsf(s.scale) * kLog2e, 1e-30f);
    const float grow_thr = 8.f / c;
    const uint32_t qsign = s.scale < 0.f ? 0x80008000u : 0u;

    bf16x8 qreg[D / 16];
    {
        const bf16 *qrow = q + base + (int64_t)my_row * rs;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            uint4 u = make_uint4(0u, 0u, 0u, 0u);
            if (my_row < row_end) u = *(const uint4 *)(qrow + ks * 16 + g * 8);
            u.x ^= qsign;
            u.y ^= qsign;
            u.z ^= qsign;
            u.w ^= qsign;
            qreg[ks] = __builtin_bit_cast(bf16x8, u);
        }
    }

    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
    float m = -INFINITY, l = 0.f;

    const int kbeg = window_start(row0, s.B, s.W);
    const int nchunks = (row_end - kbeg + kKC - 1) / kKC;
    const bf16 *kb = k + base + (int64_t)kbeg * rs;
    const bf16 *vb = v + base + (int64_t)kbeg * rs;
    Stage<D> st;
    {
        const int rows = min(kKC, row_end - kbeg);
        load_chunk<D>(st, row_rsrc<D>(kb, rows, rs), row_rsrc<D>(vb, rows, rs), rsb);
        store_chunk<D>(st, sm[0]);
        if (nchunks > 1) {
            const int rows1 = min(kKC, row_end - kbeg - kKC);
            load_chunk<D>(st, row_rsrc<D>(kb + kKC * rs, rows1, rs),
                          row_rsrc<D>(vb + kKC * rs, rows1, rs), rsb);
        }
        __syncthreads();
    }

    for (int ci = 0; ci < nchunks; ++ci) {
        const FwdBuf<D> &bf = sm[ci & 1];
        const int c0 = kbeg + ci * kKC;
        if (wave_live) {
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
                const int a = c0 + sub * 32;
                if (!(a <= w_last && a + 31 >= wave_klo)) continue;
                f32x16 sc = {};
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks) {
                    const bf16x8 ka = *(const bf16x8 *)&bf.k[sub * 32 + qi][ks * 16 + g * 8];
                    sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[ks], sc, 0, 0, 0);
                }
                if (a + 31 > wr0 || a < wave_klo_max) {
                    // key of register r: a + 8g + 16(r/8) + r%8; visible iff
                    // my_klo <= key <= my_row
                    const int x = a + 8 * g - my_klo;
                    const uint32_t span = (uint32_t)(my_row - my_klo);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if ((uint32_t)(x + 16 * (r >> 3) + (r & 7)) > span) sc[r] = -INFINITY;
                }
                float mx = sc[0];
#pragma unroll
                for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
                mx = swap_max(mx);
                // Lazy rescale: a row keeps a stale max unless its scores grew
                // past it by 2^8 (in the exp2 domain).  The decision is per row,
                // so a row's rounding never depends on other rows.
                const bool grow = mx > m + grow_thr;
                if (__builtin_amdgcn_ballot_w64(grow)) {
                    const float alpha = grow ? __builtin_amdgcn_exp2f((m - mx) * c) : 1.f;
                    m = grow ? mx : m;
                    l *= alpha;
#pragma unroll
                    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
                }
                const float mc = m == -INFINITY ? 0.f : m * c;
                bf16x8 pb[2];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(sc[r], c, -mc));
                    l += p;
                    pb[r >> 3][r & 7] = (bf16)p;
                }
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        const bf16x8 va =
                            *(const bf16x8 *)&bf.vt[dt * 32 + qi][sub * 32 + kk * 16 + g * 8];
                        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kk], acc[dt],
                                                                          0, 0, 0);
                    }
            }
        }
        if (ci + 1 < nchunks) {
            store_chunk<D>(st, sm[(ci + 1) & 1]);
            if (ci + 2 < nchunks) {
                const int off = (ci + 2) * kKC;
                const int rows = min(kKC, row_end - kbeg - off);
                load_chunk<D>(st, row_rsrc<D>(kb + off * rs, rows, rs),
                              row_rsrc<D>(vb + off * rs, rows, rs), rsb);
            }
        }
        __syncthreads();
    }

    const float lt = swap_sum(l);
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
