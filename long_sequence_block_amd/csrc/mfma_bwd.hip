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
// dS_ij = P_ij (dP_ij - delta_i) and delta_i = <dO_i, O_i>, recomputed by
// both roles from O and dO.  Each output element has exactly one owner, so
// there are no atomics and no workspace, and the result is deterministic.
// Visibility is the block window: local query i sees local key j iff j <= i
// and floor(i/B) - floor(j/B) < W, so key j is seen by queries
// j <= i < (floor(j/B) + W) * B.
//
// Layouts follow the forward kernel: 32x32x16 bf16 MFMAs, one query (query
// role) or one key (key role) per lane column; streamed rows sit in LDS
// tiles (lds_tile.h) at row sigma(m), so accumulator octets are the operands
// of the next product, and the products that contract along the streamed
// rows read them with transposed LDS reads.  The query role keeps its Q and
// dO rows in registers and streams K and V; the key role keeps K and V rows
// and streams Q, dO, O and lse.  Chunks of 64 rows go from HBM straight into
// three rotating LDS tiles; the key role computes delta (and lse * log2 e)
// of chunk c+1 from the LDS copies while chunk c is consumed, so it needs no
// extra barrier.
#include "kernels.h"
#include "lds_tile.h"

namespace ba {
namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kTileRows = 128;
constexpr int kKC = 64;        // rows per streamed chunk
constexpr int NB = 3;          // LDS chunk buffers in rotation

// Waves per SIMD the register budget is sized for.
template <int D>
constexpr int kWavesPerSimd = D == 128 ? 1 : 2;

// One chunk buffer: the query role uses tiles 0 (K) and 1 (V), the key role
// tiles 0 (Q), 1 (dO), 2 (O) and the raw lse of the chunk's queries.
template <int D>
struct BwdChunk {
    bf16 t[3][kKC * D];
    float lse[kKC];
};
template <int D>
struct BwdSmem {
    BwdChunk<D> c[NB];
    float lse2[NB][kKC];  // lse * log2(e), per key-role chunk
    float dlt[NB][kKC];   // delta, per key-role chunk
};

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

// Loads one row of a [T,H,D] tensor as MFMA B operands (lane column = row).
template <int D>
__device__ __forceinline__ void load_operand(bf16x8 (&op)[D / 16], const bf16 *row, bool valid,
                                             int g) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        uint4 x = make_uint4(0u, 0u, 0u, 0u);
        if (valid) x = *(const uint4 *)(row + ks * 16 + g * 8);
        op[ks] = __builtin_bit_cast(bf16x8, x);
    }
}

__device__ __forceinline__ float dot8(bf16x8 a, bf16x8 b, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 0, 1),
                                          __builtin_shufflevector(b, b, 0, 1), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 2, 3),
                                          __builtin_shufflevector(b, b, 2, 3), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 4, 5),
                                          __builtin_shufflevector(b, b, 4, 5), acc, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 6, 7),
                                           __builtin_shufflevector(b, b, 6, 7), acc, false);
}

// Waits for the chunk about to be consumed and joins the barrier; `ahead`
// says whether the next chunk's loads (kDma instructions) may stay in flight.
template <int kDma>
__device__ __forceinline__ void chunk_barrier(bool ahead) {
    if (ahead)
        wait_vm_barrier<kDma>();
    else
        wait_vm_barrier<0>();
}

// Per-lane LDS offsets shared by both roles.
template <int D>
struct ReadOffsets {
    int rd[D / 16];       // row reads, per 16-column step
    int trd[2][D / 32];   // transposed reads, per half and 32-column block
    __device__ ReadOffsets(int lane) {
        const int qi = lane & 31, g = lane >> 5;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) rd[ks] = row_read_offset<D>(qi, g) ^ (ks << 5);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) trd[h][dt] = tr_read_offset<D>(lane, h, dt);
    }
};

// ------------------------------------------------------------ query role

template <int D>
__device__ void query_role(const Shape &s, const Tile &t, BwdSmem<D> &sm, int wave,
                           const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                           const bf16 *__restrict__ v, const bf16 *__restrict__ out,
                           const bf16 *__restrict__ dout, const float *__restrict__ lse,
                           bf16 *__restrict__ dq) {
    using G = TileGeom<D>;
    constexpr int kDma = 2 * G::kDmaPerWave;
    const int lane = threadIdx.x & 63;
    const int w = (wave + t.blk) & 3;
    const int qi = lane & 31, g = lane >> 5;
    const int64_t rs = (int64_t)s.H * D;
    const uint32_t rsb = (uint32_t)(rs * 2);
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

    const int kbeg = window_start(row0, s.B, s.W);
    const int nch = (row_end - kbeg + kKC - 1) / kKC;
    const bf16 *kb = k + base + (int64_t)kbeg * rs;
    const bf16 *vb = v + base + (int64_t)kbeg * rs;
    lds_t *lds = (lds_t *)&sm;
    uint32_t voff[G::kDmaPerWave];
    dma_offsets<D>(voff, wave, lane, rsb);
    auto issue = [&](int ci, int buf) {
        const int off = ci * kKC, rows = min(kKC, row_end - kbeg - off);
        lds_t *b = lds + buf * (int)sizeof(BwdChunk<D>);
        dma_tile<D>(row_desc<D>(kb + off * rs, rows, rs), b, voff, wave);
        dma_tile<D>(row_desc<D>(vb + off * rs, rows, rs), b + G::kBytes, voff, wave);
    };

    if (nch > 0) issue(0, 0);
    bf16x8 qop[D / 16], doop[D / 16];
    load_operand<D>(qop, q + base + (int64_t)my_row * rs, my_valid, g);
    load_operand<D>(doop, dout + base + (int64_t)my_row * rs, my_valid, g);
    float my_lse2 = 0.f, my_dlt = 0.f;
    if (my_valid) {
        my_lse2 = lse[(int64_t)t.h * s.T + t.tok0 + my_row] * kLog2e;
        const bf16 *orow = out + base + (int64_t)my_row * rs;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            my_dlt = dot8(doop[ks], *(const bf16x8 *)(orow + ks * 16 + g * 8), my_dlt);
    }
    my_dlt = swap_sum(my_dlt);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): only tile loads in flight from here
    if (nch > 1) issue(1, 1);
    const ReadOffsets<D> ro(lane);

    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};

    auto step = [&](int ci, auto buf_c) {
        constexpr int buf = decltype(buf_c)::value;
        chunk_barrier<kDma>(ci + 1 < nch);
        if (ci + 2 < nch) issue(ci + 2, (buf + 2) % NB);
        if (!wave_live) return;
        const lds_t *kt = lds + buf * (int)sizeof(BwdChunk<D>);
        const lds_t *vt = kt + G::kBytes;
        const int c0 = kbeg + ci * kKC;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int a = c0 + sub * 32;
            if (!(a <= w_last && a + 31 >= wave_klo)) continue;
            f32x16 sc = {}, dp = {};
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                sc = mfma32(lds_read16(kt + sub * 32 * G::kRowBytes + ro.rd[ks]), qop[ks], sc);
                dp = mfma32(lds_read16(vt + sub * 32 * G::kRowBytes + ro.rd[ks]), doop[ks], dp);
            }
            const bool masked = a + 31 > wr0 || a < wave_klo_max;
            // key of register r: a + 8g + 16(r/8) + r%8; visible iff
            // my_klo <= key <= my_row
            const int x = a + 8 * g - my_klo;
            const uint32_t span = (uint32_t)(my_row - my_klo);
            bf16x8 dsb[2];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = __builtin_amdgcn_exp2f(fmaf(sc[r], c, -my_lse2));
                if (masked && (uint32_t)(x + 16 * (r >> 3) + (r & 7)) > span) p = 0.f;
                dsb[r >> 3][r & 7] = (bf16)(p * (dp[r] - my_dlt));
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const lds_t *kr = kt + (sub * 32 + kk * 16) * G::kRowBytes;
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
                    acc[dt] = mfma32(lds_read_tr(kr + ro.trd[0][dt], kr + ro.trd[1][dt]),
                                     dsb[kk], acc[dt]);
            }
        }
    };
    for (int ci = 0; ci < nch; ci += NB) {
        step(ci, std::integral_constant<int, 0>{});
        if (ci + 1 < nch) step(ci + 1, std::integral_constant<int, 1>{});
        if (ci + 2 < nch) step(ci + 2, std::integral_constant<int, 2>{});
    }
    if (my_valid) store_out<D>(dq + base + (int64_t)my_row * rs, acc, s.scale, g);
}

// -------------------------------------------------------------- key role

template <int D>
__device__ void key_role(const Shape &s, const Tile &t, BwdSmem<D> &sm, int wave,
                         const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                         const bf16 *__restrict__ v, const bf16 *__restrict__ out,
                         const bf16 *__restrict__ dout, const float *__restrict__ lse,
                         bf16 *__restrict__ dk, bf16 *__restrict__ dv) {
    using G = TileGeom<D>;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = (wave + t.blk) & 3;
    const int qi = lane & 31, g = lane >> 5;
    const int64_t rs = (int64_t)s.H * D;
    const uint32_t rsb = (uint32_t)(rs * 2);
    const int64_t base = t.tok0 * rs + (int64_t)t.h * D;
    const int row0 = t.blk * kTileRows;
    const int row_end = min(row0 + kTileRows, t.len);  // keys of this tile end here
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

    const int nch = (qend - row0 + kKC - 1) / kKC;
    const bf16 *qb = q + base + (int64_t)row0 * rs;
    const bf16 *db = dout + base + (int64_t)row0 * rs;
    const bf16 *ob = out + base + (int64_t)row0 * rs;
    const float *lsb = lse + (int64_t)t.h * s.T + t.tok0 + row0;
    lds_t *lds = (lds_t *)&sm;
    uint32_t voff[G::kDmaPerWave];
    dma_offsets<D>(voff, wave, lane, rsb);
    auto issue = [&](int ci, int buf) {
        const int off = ci * kKC, rows = min(kKC, qend - row0 - off);
        lds_t *b = lds + buf * (int)sizeof(BwdChunk<D>);
        dma_tile<D>(row_desc<D>(qb + off * rs, rows, rs), b, voff, wave);
        dma_tile<D>(row_desc<D>(db + off * rs, rows, rs), b + G::kBytes, voff, wave);
        dma_tile<D>(row_desc<D>(ob + off * rs, rows, rs), b + 2 * G::kBytes, voff, wave);
        if (wave == 0) {
            // 64 lse values, 4 bytes per lane
            const uint64_t a = (uint64_t)(lsb + off);
            const i32x4 desc{(int)(uint32_t)a, (int)((a >> 32) & 0xffffu), rows * 4, 0x00020000};
            const uint32_t dst = (uint32_t)(uintptr_t)(b + 3 * G::kBytes);
            asm volatile(
                "s_mov_b32 m0, %0\n\t"
                "s_nop 0\n\t"
                "buffer_load_dword %1, %2, 0 offen lds"
                :
                : "s"(dst), "v"((uint32_t)lane * 4u), "s"(desc)
                : "memory", "m0");
        }
    };
    // delta and lse * log2(e) of chunk buffer `buf` (its loads complete and
    // visible): 4 threads per row, each over D/4 columns.
    auto prep = [&](int buf) {
        const lds_t *b = lds + buf * (int)sizeof(BwdChunk<D>);
        const int r = tid >> 2, part = tid & 3;
        const int p = sigma(r);
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) {
            const int off = G::at(p, part * (D / 32) + i);
            d = dot8(lds_read16(b + G::kBytes + off), lds_read16(b + 2 * G::kBytes + off), d);
        }
        d += __shfl_xor(d, 1, 64);
        d += __shfl_xor(d, 2, 64);
        if (part == 0) {
            sm.dlt[buf][r] = d;
            sm.lse2[buf][r] = sm.c[buf].lse[r] * kLog2e;
        }
    };

    if (nch > 0) issue(0, 0);
    bf16x8 kop[D / 16], vop[D / 16];
    load_operand<D>(kop, k + base + (int64_t)my_key * rs, my_valid, g);
    load_operand<D>(vop, v + base + (int64_t)my_key * rs, my_valid, g);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): chunk 0 and the K, V rows are in
    if (nch > 1) issue(1, 1);
    asm volatile("s_barrier" ::: "memory");
    if (nch > 0) prep(0);
    const ReadOffsets<D> ro(lane);

    f32x16 adk[D / 32], adv[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) adk[dt] = adv[dt] = f32x16{};

    auto step = [&](int ci, auto buf_c) {
        constexpr int buf = decltype(buf_c)::value;
        wait_vm_barrier<0>();
        if (ci + 2 < nch) issue(ci + 2, (buf + 2) % NB);
        if (ci + 1 < nch) prep((buf + 1) % NB);
        if (!wave_live) return;
        const lds_t *qt = lds + buf * (int)sizeof(BwdChunk<D>);
        const lds_t *dt_ = qt + G::kBytes;
        const int c0 = row0 + ci * kKC;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int a = c0 + sub * 32;  // first query of the sub-tile
            if (!(a + 31 >= wk0 && a < wave_qend_max)) continue;
            f32x16 sc = {}, dp = {};
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                sc = mfma32(lds_read16(qt + sub * 32 * G::kRowBytes + ro.rd[ks]), kop[ks], sc);
                dp = mfma32(lds_read16(dt_ + sub * 32 * G::kRowBytes + ro.rd[ks]), vop[ks], dp);
            }
            const bool masked = a < wk_last || a + 31 >= wave_qend_min;
            // query of register r: a + 8g + 16(r/8) + r%8; it sees this
            // lane's key iff my_key <= query < my_qend
            const int x = a + 8 * g - my_key;
            const uint32_t span = (uint32_t)max(my_qend - my_key, 0);
            float pf[16];
            bf16x8 pb[2], dsb[2];
            float pmax = 0.f;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int qrow = sub * 32 + hh * 16 + g * 8;
                const float4 l0 = *(const float4 *)&sm.lse2[buf][qrow];
                const float4 l1 = *(const float4 *)&sm.lse2[buf][qrow + 4];
                const float4 d0 = *(const float4 *)&sm.dlt[buf][qrow];
                const float4 d1 = *(const float4 *)&sm.dlt[buf][qrow + 4];
                const float ls[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
                const float ds[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int r = hh * 8 + i;
                    float p = __builtin_amdgcn_exp2f(fmaf(sc[r], c, -ls[i]));
                    if (masked && (uint32_t)(x + 16 * hh + i) >= span) p = 0.f;
                    pf[r] = p;
                    pmax = fmaxf(pmax, p);
                    pb[hh][i] = (bf16)p;
                    dsb[hh][i] = (bf16)(p * (dp[r] - ds[i]));
                }
            }
            // Rows that see few keys have weights near 1, where bf16
            // rounding of P (2^-9 relative) would dominate dV.  There P is
            // split into bf16 hi + lo and dV takes a second product;
            // elsewhere P < 1/16 bounds the rounding error per term by 2^-13.
            const bool split = __builtin_amdgcn_ballot_w64(pmax > 0.0625f) != 0;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const lds_t *qr = qt + (sub * 32 + kk * 16) * G::kRowBytes;
                const lds_t *dr = dt_ + (sub * 32 + kk * 16) * G::kRowBytes;
                bf16x8 lo;
                if (split) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) lo[i] = (bf16)(pf[kk * 8 + i] - (float)pb[kk][i]);
                }
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) {
                    const bf16x8 da = lds_read_tr(dr + ro.trd[0][dt], dr + ro.trd[1][dt]);
                    adv[dt] = mfma32(da, pb[kk], adv[dt]);
                    if (split) adv[dt] = mfma32(da, lo, adv[dt]);
                    adk[dt] = mfma32(lds_read_tr(qr + ro.trd[0][dt], qr + ro.trd[1][dt]),
                                     dsb[kk], adk[dt]);
                }
            }
        }
    };
    for (int ci = 0; ci < nch; ci += NB) {
        step(ci, std::integral_constant<int, 0>{});
        if (ci + 1 < nch) step(ci + 1, std::integral_constant<int, 1>{});
        if (ci + 2 < nch) step(ci + 2, std::integral_constant<int, 2>{});
    }
    if (my_valid) {
        store_out<D>(dk + base + (int64_t)my_key * rs, adk, s.scale, g);
        store_out<D>(dv + base + (int64_t)my_key * rs, adv, 1.f, g);
    }
}

template <int D>
__global__ __launch_bounds__(kThreads, kWavesPerSimd<D>) void bwd_mfma(
    Shape s, const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ out, const bf16 *__restrict__ dout, const float *__restrict__ lse,
    bf16 *__restrict__ dq, bf16 *__restrict__ dk, bf16 *__restrict__ dv) {
    __shared__ int sh[8];
    __shared__ __align__(1024) BwdSmem<D> sm;
    Tile t;
    if (!decode_tile<kThreads>(s, kTileRows, 2, t, sh)) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t.sub == 0)
        query_role<D>(s, t, sm, wave, q, k, v, out, dout, lse, dq);
    else
        key_role<D>(s, t, sm, wave, q, k, v, out, dout, lse, dk, dv);
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
