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
// dS_ij = P_ij (dP_ij - delta_i) and delta_i = <dO_i, O_i>.  A first,
// memory-bound launch writes delta and lse * log2(e) of every row to the
// workspace; the main launch then never reads O.  Each output element of the
// main launch has exactly one owner, so there are no atomics and the result
// is deterministic.  Visibility is the block window: local query i sees
// local key j iff j <= i and floor(i/B) - floor(j/B) < W, so key j is seen by
// queries j <= i < (floor(j/B) + W) * B.
//
// Layouts follow the forward kernel: 32x32x16 bf16 MFMAs, one query (query
// role) or one key (key role) per lane column; streamed rows sit in LDS
// tiles (lds_tile.h) at row sigma(m), so accumulator octets are the operands
// of the next product, and the products that contract along the streamed
// rows read them with transposed LDS reads.  The query role keeps its Q and
// dO rows in registers and streams K and V; the key role keeps K and V rows
// and streams Q, dO and the two row statistics.  Chunks of 64 rows go from
// HBM straight into two LDS buffers in turn, one barrier per chunk.
#include "kernels.h"
#include "lds_tile.h"

namespace ba {
namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kTileRows = 128;
constexpr int kKC = 64;        // rows per streamed chunk
constexpr int NB = 2;          // LDS chunk buffers in rotation

// Waves per SIMD the register budget is sized for.
template <int D>
constexpr int kWavesPerSimd = D == 128 ? 1 : 2;

// One chunk buffer: the query role uses tiles 0 (K) and 1 (V), the key role
// tiles 0 (Q) and 1 (dO) and the row statistics of the chunk's queries.
template <int D>
struct BwdChunk {
    bf16 t[2][kKC * D];
    float lse2[kKC];  // lse * log2(e)
    float dlt[kKC];   // delta
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
__device__ void query_role(const Shape &s, const Tile &t, BwdChunk<D> *sm, int wave,
                           const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                           const bf16 *__restrict__ v, const bf16 *__restrict__ dout,
                           const float *__restrict__ ws_lse2, const float *__restrict__ ws_dlt,
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
    lds_t *lds = (lds_t *)sm;
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
        const int64_t i = (int64_t)t.h * s.T + t.tok0 + my_row;
        my_lse2 = ws_lse2[i];
        my_dlt = ws_dlt[i];
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): only tile loads in flight from here
    const ReadOffsets<D> ro(lane);

    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};

    auto step = [&](int ci, auto buf_c) {
        constexpr int buf = decltype(buf_c)::value;
        wait_vm_barrier<0>();
        if (ci + 1 < nch) issue(ci + 1, buf ^ 1);
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
            float pr[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], c, -my_lse2));
            if (masked) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if ((uint32_t)(x + 16 * (r >> 3) + (r & 7)) > span) pr[r] = 0.f;
            }
            bf16x8 dsb[2];
#pragma unroll
            for (int r = 0; r < 16; ++r) dsb[r >> 3][r & 7] = (bf16)(pr[r] * (dp[r] - my_dlt));
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
    }
    if (my_valid) store_out<D>(dq + base + (int64_t)my_row * rs, acc, s.scale, g);
}

// -------------------------------------------------------------- key role

template <int D>
__device__ void key_role(const Shape &s, const Tile &t, BwdChunk<D> *sm, int wave,
                         const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                         const bf16 *__restrict__ v, const bf16 *__restrict__ dout,
                         const float *__restrict__ ws_lse2, const float *__restrict__ ws_dlt,
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
    const int64_t srow = (int64_t)t.h * s.T + t.tok0 + row0;
    lds_t *lds = (lds_t *)sm;
    uint32_t voff[G::kDmaPerWave];
    dma_offsets<D>(voff, wave, lane, rsb);
    // A chunk: Q and dO tiles by every wave, the 64 lse2 and delta values
    // (4 bytes per lane) by waves 0 and 1.
    auto issue = [&](int ci, int buf) {
        const int off = ci * kKC, rows = min(kKC, qend - row0 - off);
        lds_t *b = lds + buf * (int)sizeof(BwdChunk<D>);
        dma_tile<D>(row_desc<D>(qb + off * rs, rows, rs), b, voff, wave);
        dma_tile<D>(row_desc<D>(db + off * rs, rows, rs), b + G::kBytes, voff, wave);
        if (wave < 2) {
            const float *src = (wave == 0 ? ws_lse2 : ws_dlt) + srow + off;
            const uint64_t a = (uint64_t)src;
            const i32x4 desc{(int)(uint32_t)a, (int)((a >> 32) & 0xffffu), rows * 4, 0x00020000};
            const uint32_t dst = (uint32_t)(uintptr_t)(b + 2 * G::kBytes + wave * kKC * 4);
            asm volatile(
                "s_mov_b32 m0, %0\n\t"
                "s_nop 0\n\t"
                "buffer_load_dword %1, %2, 0 offen lds"
                :
                : "s"(dst), "v"((uint32_t)lane * 4u), "s"(desc)
                : "memory", "m0");
        }
    };

    if (nch > 0) issue(0, 0);
    bf16x8 kop[D / 16], vop[D / 16];
    load_operand<D>(kop, k + base + (int64_t)my_key * rs, my_valid, g);
    load_operand<D>(vop, v + base + (int64_t)my_key * rs, my_valid, g);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): only tile loads in flight from here
    const ReadOffsets<D> ro(lane);

    f32x16 adk[D / 32], adv[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) adk[dt] = adv[dt] = f32x16{};

    auto step = [&](int ci, auto buf_c) {
        constexpr int buf = decltype(buf_c)::value;
        wait_vm_barrier<0>();
        if (ci + 1 < nch) issue(ci + 1, buf ^ 1);
        if (!wave_live) return;
        const BwdChunk<D> &cb = sm[buf];
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
                const float4 l0 = *(const float4 *)&cb.lse2[qrow];
                const float4 l1 = *(const float4 *)&cb.lse2[qrow + 4];
                const float4 d0 = *(const float4 *)&cb.dlt[qrow];
                const float4 d1 = *(const float4 *)&cb.dlt[qrow + 4];
                const float ls[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
                const float ds[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int r = hh * 8 + i;
                    pf[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], c, -ls[i]));
                    dp[r] -= ds[i];
                }
            }
            if (masked) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if ((uint32_t)(x + 16 * (r >> 3) + (r & 7)) >= span) pf[r] = 0.f;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                pmax = fmaxf(pmax, pf[r]);
                pb[r >> 3][r & 7] = (bf16)pf[r];
                dsb[r >> 3][r & 7] = (bf16)(pf[r] * dp[r]);
            }
            // Where a weight exceeds 1/4 (queries that see few keys), bf16
            // rounding of P (up to 2^-8 relative) is split off into a bf16 lo
            // part and dV takes a second product; elsewhere each term's
            // rounding error stays below 2^-10 |dO|, well under the bf16
            // rounding of dV itself.  About 2% of sub-tiles split on N(0,1)
            // inputs.
            const bool split = __builtin_amdgcn_ballot_w64(pmax > 0.25f) != 0;
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
    }
    if (my_valid) {
        store_out<D>(dk + base + (int64_t)my_key * rs, adk, s.scale, g);
        store_out<D>(dv + base + (int64_t)my_key * rs, adv, 1.f, g);
    }
}

// Row statistics of the backward pass: delta = <dO, O> (fp32 from bf16
// products) and lse * log2(e), for every (head, token), into [H, T] arrays.
// One thread per row; consecutive lanes take consecutive tokens of one head.
template <int D>
__global__ __launch_bounds__(256) void bwd_rowstats(Shape s, const bf16 *__restrict__ out,
                                                    const bf16 *__restrict__ dout,
                                                    const float *__restrict__ lse,
                                                    float *__restrict__ ws_lse2,
                                                    float *__restrict__ ws_dlt) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int h = blockIdx.y;
    if (t >= s.T) return;
    const int64_t row = (t * s.H + h) * D;
    float d = 0.f;
#pragma unroll
    for (int i = 0; i < D / 8; ++i)
        d = dot8(*(const bf16x8 *)(dout + row + i * 8), *(const bf16x8 *)(out + row + i * 8), d);
    const int64_t o = (int64_t)h * s.T + t;
    ws_dlt[o] = d;
    ws_lse2[o] = lse[o] * kLog2e;
}

template <int D>
__global__ __launch_bounds__(kThreads, kWavesPerSimd<D>) void bwd_mfma(
    Shape s, const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ dout, const float *__restrict__ ws_lse2,
    const float *__restrict__ ws_dlt, bf16 *__restrict__ dq, bf16 *__restrict__ dk,
    bf16 *__restrict__ dv) {
    __shared__ int sh[8];
    __shared__ __align__(1024) BwdChunk<D> sm[NB];
    Tile t;
    if (!decode_tile<kThreads>(s, kTileRows, 2, t, sh)) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t.sub == 0)
        query_role<D>(s, t, sm, wave, q, k, v, dout, ws_lse2, ws_dlt, dq);
    else
        key_role<D>(s, t, sm, wave, q, k, v, dout, ws_lse2, ws_dlt, dk, dv);
}

template <int D>
hipError_t launch_t(const Shape &s, const void *q, const void *k, const void *v, const void *out,
                    const void *dout, const float *lse, void *dq, void *dk, void *dv,
                    float *ws, hipStream_t st) {
    float *ws_lse2 = ws, *ws_dlt = ws + s.H * s.T;
    hipLaunchKernelGGL((bwd_rowstats<D>), dim3((unsigned)((s.T + 255) / 256), (unsigned)s.H),
                       dim3(256), 0, st, s, (const bf16 *)out, (const bf16 *)dout, lse, ws_lse2,
                       ws_dlt);
    const int64_t grid = grid_upper_bound(s.T, s.batch, kTileRows, 2, s.H);
    hipLaunchKernelGGL((bwd_mfma<D>), dim3((unsigned)grid), dim3(kThreads), 0, st, s,
                       (const bf16 *)q, (const bf16 *)k, (const bf16 *)v, (const bf16 *)dout,
                       (const float *)ws_lse2, (const float *)ws_dlt, (bf16 *)dq, (bf16 *)dk,
                       (bf16 *)dv);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_bwd(const Shape &s, const void *q, const void *k, const void *v,
                           const void *out, const void *dout, const float *lse, void *dq,
                           void *dk, void *dv, float *ws, hipStream_t st) {
    switch (s.D) {
    case 32: return launch_t<32>(s, q, k, v, out, dout, lse, dq, dk, dv, ws, st);
    case 64: return launch_t<64>(s, q, k, v, out, dout, lse, dq, dk, dv, ws, st);
    case 128: return launch_t<128>(s, q, k, v, out, dout, lse, dq, dk, dv, ws, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace ba
