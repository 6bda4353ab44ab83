// Backward block attention on bf16 MFMA (gfx950).
//
// The production block-attention kernel fuses its backward pass ("GEM (Meta)"
// on aiwiki.ai, section "Custom kernels").  Every 128-row tile of a
// (user, head) is worked on twice, in two roles:
//
//   query role  (rows = queries i):  dQ_i = scale * sum_j dS_ij k_j
//   key role    (rows = keys j):     dK_j = scale * sum_i dS_ij q_i,
//                                    dV_j = sum_i P_ij dO_i
//
// with P_ij = exp(scale <q_i,k_j> - lse_i), dP_ij = <dO_i, v_j>,
// dS_ij = P_ij (dP_ij - delta_i) and delta_i = sum_j P_ij dP_ij.  Each output
// element has exactly one owner, so there are no atomics on outputs and the
// result is deterministic.  Visibility is the block window: local query i
// sees local key j iff j <= i and floor(i/B) - floor(j/B) < W, so key j is
// seen by queries j <= i < (floor(j/B) + W) * B.
//
// delta.  <dO_i, O_i> equals delta_i only for the exact O; the forward's O
// is rounded to bf16, and with near-one-hot weights that rounding moves dS
// enough to show in dQ and dK.  So the query role starts from delta'_i =
// <dO_i, O_i> of the bf16 O and, from the same fp32 values that form dS,
// sums eps_i = sum_j P_ij (dP_ij - delta'_i) = delta_i - delta'_i (the P_ij
// of a row sum to 1) together with C_i = sum_j P_ij k_j (one more product,
// on the transposed K it already reads).  Then
//     dQ_i = scale sum_j P_ij (dP_ij - delta'_i) k_j - scale eps_i C_i,
// and it writes delta_i and lse_i * log2(e) for the key role, which
// therefore runs after it.
//
// Launches (softmax):
//   1. bwd_tile_index (one workgroup): per-user tile counts from the jagged
//      offsets, their prefix sums, the total, and zeroed queue counters.
//   2. bwd_table: the tile table (one 16-byte entry per (user, head, unit,
//      role)).
//   3. bwd_mfma, query pass, then 4. bwd_mfma, key pass: as many workgroups
//      as fit on the GPU at once; each takes tiles of its pass from a queue
//      counter until it runs dry.  While it works on one tile it already
//      holds the next tile's table entry, has issued the next tile's first
//      chunk and operand rows, and has requested the index of the tile after
//      that, so per-tile set-up latency is hidden.
// The activation variants (no delta) run both roles in one bwd_mfma launch.
//
// Layouts follow the forward kernel: 32x32x16 bf16 MFMAs, one query (query
// role) or one key (key role) per lane column; streamed rows sit in LDS
// tiles (lds_tile.h) at row sigma(m), so accumulator octets are the operands
// of the next product, and the products that contract along the streamed
// rows read them with transposed LDS reads.  The query role keeps its Q and
// dO rows in registers and streams K and V; the key role keeps K and V rows
// and streams Q, dO and the two row statistics of each query.  Chunks of 64 rows go from
// HBM straight into two LDS buffers in turn, one barrier per chunk.
#include <algorithm>
#include <atomic>

#include "kernels.h"
#include "lds_tile.h"

namespace ba {
namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kTileRows = kBwdTileRows;
constexpr int kKC = 64;        // rows per streamed chunk

// Tile queues.  Workgroups are dealt to the 8 XCDs round-robin, so group
// blockIdx % 8 runs on one XCD.  Each group takes the tiles of its own runs
// of kRunTiles consecutive tiles (8 units of one (user, head): neighbours
// that read the same rows) from its own counter, so those rows are shared
// in that XCD's L2.  Any placement of workgroups gives the same result.
constexpr int kQueues = 8;
constexpr int kRunTiles = 16;
// The key pass's queue counters start here in the counter block (the query
// pass, or a launch running both roles, uses ctr[0 .. kQueues); ctr[kQueues]
// holds the tile count).
constexpr int kPass1Ctr = 16;

// Waves per SIMD the register budget is sized for.
template <int D>
constexpr int kWavesPerSimd = D == 128 ? 1 : 2;

// One chunk buffer: the query role uses tiles 0 (K) and 1 (V), the key role
// tiles 0 (Q) and 1 (dO) and the row statistics of the chunk's queries.
template <int D>
struct BwdChunk {
    bf16 t[2][kKC * D];
    float lse2[kKC];  // lse * log2(e)
    float ndlt[kKC];  // -delta
};

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

// A decoded tile; every field is wave-uniform.
struct BwdTile {
    int role;           // 0: query role, 1: key role
    int h, blk, len, tok0;
    int row0, row_end;  // the tile's own rows (local indices)
    int sbeg, send;     // the streamed rows
    int nch;            // chunks of streamed rows
};

// Table entry: {tok0, len, unit, 2 * head + role}.
__device__ __forceinline__ BwdTile make_tile(const Shape &s, int4 e) {
    BwdTile t;
    t.tok0 = __builtin_amdgcn_readfirstlane(e.x);
    t.len = __builtin_amdgcn_readfirstlane(e.y);
    t.blk = __builtin_amdgcn_readfirstlane(e.z);
    const int hr = __builtin_amdgcn_readfirstlane(e.w);
    t.h = hr >> 1;
    t.role = hr & 1;
    t.row0 = t.blk * kTileRows;
    t.row_end = min(t.row0 + kTileRows, t.len);
    if (t.role == 0) {  // keys of the window of the tile's queries
        t.sbeg = window_start(t.row0, s.B, s.W);
        t.send = t.row_end;
    } else {            // queries that see the tile's keys
        t.sbeg = t.row0;
        t.send = window_end(t.row_end - 1, s.B, s.W, t.len);
    }
    t.nch = (t.send - t.sbeg + kKC - 1) / kKC;
    return t;
}

// The rows a wave owns in a tile: 32 rows, rotated with the unit index so
// that the SIMDs share the lighter and heavier row groups evenly.
__device__ __forceinline__ int wave_rows(const BwdTile &t, int wave) {
    return t.row0 + ((wave + t.blk) & 3) * 32;
}

// The registers a wave keeps for one tile: the MFMA B operands of its own
// row (Q and dO for the query role, K and V for the key role) and, for the
// query role, the row's lse * log2(e) and -delta.
template <int D>
struct Ops {
    bf16x8 a[D / 16], b[D / 16];
    float lse2, ndlt;
};

// LDS staging of a tile's own rows (two 64-row TileGeom tiles per tensor)
// and, for the query role, their row statistics.  The next tile's rows land
// here while the current tile's last chunk is worked on.
template <int D>
struct OpsLds {
    bf16 a[2][kKC * D];
    bf16 b[2][kKC * D];
    float lse2[kTileRows];
    float ndlt[kTileRows];
};

// Output store instructions per wave and tile.  The counts are fixed
// (buffer instructions clip rows past the tile instead of branching around
// them), so the next tile's first wait can allow for exactly these.
// The softmax query role also stores its rows' exact -delta and
// lse * log2(e) for the key pass (two more).
template <int D, int ACT>
constexpr int kStores(int role) { return role == 0 ? D / 16 + (ACT == kSoftmax ? 2 : 0) : D / 8; }

// Writes a wave's 32 rows of one output (scaled by mul) as bf16; rows past
// the tile are clipped by the buffer range.  With a rotary table (rrev, in
// LDS: turns per position of each pair), the rows are first turned back by
// their position's angles, which is the backward of the rotary embedding
// applied to q and k before attention: the gradient with respect to the
// unrotated input is R(p)^T times the gradient with respect to the rotated
// one.  The lane holds column 32 dt + 16 half + 8 g + e in register
// 8 half + e of acc[dt], so both columns of a pair (c, c + D/2) are in the
// same lane: acc[dt + D/64] for D >= 64, the other half for D = 32.
template <int D>
__device__ __forceinline__ void store_rows(bf16 *dst_tile, int rows, int64_t rs, uint32_t lrow,
                                           const f32x16 (&acc)[D / 32], float mul, int g,
                                           const __attribute__((address_space(3))) double *rrev,
                                           int pos) {
    const auto r = row_rsrc<D>(dst_tile, rows, rs);
    const uint32_t off = lrow * (uint32_t)(rs * 2) + (uint32_t)g * 16u;
    f32x16 x[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) x[dt][e] = acc[dt][e] * mul;
    if (rrev) {
        constexpr int kLoTiles = D == 32 ? 1 : D / 64;
        constexpr int kHalves = D == 32 ? 1 : 2;
#pragma unroll
        for (int dt = 0; dt < kLoTiles; ++dt)
#pragma unroll
            for (int half = 0; half < kHalves; ++half)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int c = 32 * dt + 16 * half + 8 * g + e;
                    const int dh = D == 32 ? 0 : dt + D / 64;
                    const int rl = 8 * half + e, rh = D == 32 ? 8 + e : rl;
                    float sn, cs;
                    rope_sincos<bf16>((double)pos * rrev[c], sn, cs);
                    const float a = x[dt][rl], b = x[dh][rh];
                    x[dt][rl] = a * cs + b * sn;
                    x[dh][rh] = b * cs - a * sn;
                }
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            bf16x8 y;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x2 p = pack_bf16(x[dt][half * 8 + 2 * j], x[dt][half * 8 + 2 * j + 1]);
                y[2 * j] = p[0];
                y[2 * j + 1] = p[1];
            }
            buf_store16(__builtin_bit_cast(uint4, y), r, off + (uint32_t)(dt * 64 + half * 32));
        }
}

// ------------------------------------------------------------ query role

// Per-tile window bounds of a wave's 32 rows (wave-uniform) and of each
// lane's row, computed once per tile.  Query role: keys [klo, last] are
// visited, sub-tiles with a key below klo_max or above first row wr0 are
// masked, and key j is visible to the lane iff (x0 + j) <= span (unsigned).
struct QWin {
    int klo, last, klo_max, wr0;
    int x0;
    uint32_t span;
};
__device__ __forceinline__ QWin query_win(const Shape &s, const BwdTile &t, int wave, int lane) {
    QWin w;
    w.wr0 = wave_rows(t, wave);
    w.last = min(w.wr0 + 31, t.row_end - 1);
    w.klo = window_start(w.wr0, s.B, s.W);
    w.klo_max = window_start(max(w.wr0, w.last), s.B, s.W);
    const int my_row = w.wr0 + (lane & 31);
    const int my_klo = window_start(my_row, s.B, s.W);
    w.x0 = 8 * (lane >> 5) - my_klo;
    w.span = (uint32_t)(my_row - my_klo);
    return w;
}

// One 64-key chunk of the query role: S^T and dP^T for each 32-key
// sub-tile, then dQ^T += K^T dS^T.  c0 = first key of the chunk.
//
// Softmax: dP starts from -delta' (delta' = <dO, O> of the forward's bf16 O),
// and the chunk also accumulates, for the exact delta, the lane's share of
// eps = sum_j P_ij (dP_ij - delta'_i) (fp32, from the same values as dS) and
// acc_c = C^T = K^T P^T, i.e. C_i = sum_j P_ij k_j, with the transposed K
// operand the dQ product already reads.
template <int D, int ACT>
__device__ __forceinline__ void query_chunk(const Shape &s, const QWin &w, int lane,
                                            const lds_t *kt, int c0, const Ops<D> &op,
                                            const f32x16 &ndlt, const ReadOffsets<D> &ro,
                                            f32x16 (&acc)[D / 32], f32x16 (&acc_c)[D / 32],
                                            float &eps) {
    using G = TileGeom<D>;
    const float c = s.scale * kLog2e;
    const lds_t *vt = kt + G::kBytes;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
        const int a = c0 + sub * 32;
        if (!(a <= w.last && a + 31 >= w.klo)) continue;
        // Every LDS read of the sub-tile is issued before its first use, so
        // their latencies overlap each other and the products.
        const lds_t *ks_ = kt + sub * 32 * G::kRowBytes;
        const lds_t *vs_ = vt + sub * 32 * G::kRowBytes;
        bf16x8 ka[D / 16], va[D / 16];
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            ka[ks] = lds_read16(ks_ + ro.rd[ks]);
            va[ks] = lds_read16(vs_ + ro.rd[ks]);
        }
        f32x16 sc = mfma32(ka[0], op.a[0], f32x16{});
#pragma unroll
        for (int ks = 1; ks < D / 16; ++ks) sc = mfma32(ka[ks], op.a[ks], sc);
        // dP^T starts from -delta of the lane's query: the products leave
        // dP - delta (the activation variants have no delta).
        f32x16 dp = mfma32(va[0], op.b[0], ACT == kSoftmax ? ndlt : f32x16{});
#pragma unroll
        for (int ks = 1; ks < D / 16; ++ks) dp = mfma32(va[ks], op.b[ks], dp);
        bf16x8 ktr[2][D / 32];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                const lds_t *kr = ks_ + kk * 16 * G::kRowBytes;
                ktr[kk][dt] = lds_read_tr(kr + ro.trd[0][dt], kr + ro.trd[1][dt]);
            }
        // dS = pr * dp: pr = P for the softmax, act'(scale s) for GDPA
        float pr[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
            pr[r] = ACT == kSoftmax ? __builtin_amdgcn_exp2f(fmaf(sc[r], c, -op.lse2))
                                    : act_slope<ACT>(sc[r] * s.scale);
        // Issue order: all operand reads, the S products, the transposed
        // reads, then each dP product followed by a share of the
        // exponentials (which need only S), so one wave keeps both its
        // matrix and vector pipes busy.
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * (D / 16), 0);
        __builtin_amdgcn_sched_group_barrier(0x008, D / 16, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * (D / 32), 0);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 32 / (D / 16), 0);
        }
        const bool masked = a + 31 > w.wr0 || a < w.klo_max;
        // key of register r: a + 8g + 16(r/8) + r%8; visible iff
        // my_klo <= key <= my_row
        const int x = a + w.x0;
        if (masked) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if ((uint32_t)(x + 16 * (r >> 3) + (r & 7)) > w.span) pr[r] = 0.f;
        }
        bf16x8 dsb[2];
        float es[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = kk * 8 + 2 * j;
                const float d0 = pr[r] * dp[r], d1 = pr[r + 1] * dp[r + 1];
                if (ACT == kSoftmax) es[j] += d0 + d1;
                const bf16x2 v2 = pack_bf16(d0, d1);
                dsb[kk][2 * j] = v2[0];
                dsb[kk][2 * j + 1] = v2[1];
            }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) acc[dt] = mfma32(ktr[kk][dt], dsb[kk], acc[dt]);
        if constexpr (ACT == kSoftmax) {
            eps += (es[0] + es[1]) + (es[2] + es[3]);
            bf16x8 pb[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = kk * 8 + 2 * j;
                    const bf16x2 p2 = pack_bf16(pr[r], pr[r + 1]);
                    pb[kk][2 * j] = p2[0];
                    pb[kk][2 * j + 1] = p2[1];
                }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
                    acc_c[dt] = mfma32(ktr[kk][dt], pb[kk], acc_c[dt]);
        }
    }
}

// -------------------------------------------------------------- key role

// Key role: queries [wk0, qend_max) are visited, sub-tiles with a query
// below wk_last or at or past qend_min are masked, and query i sees the
// lane's key iff (x0 + i) < span (unsigned).
struct KWin {
    int wk0, qend_max, wk_last, qend_min;
    int x0;
    uint32_t span;
};
__device__ __forceinline__ KWin key_win(const Shape &s, const BwdTile &t, int wave, int lane) {
    KWin w;
    w.wk0 = wave_rows(t, wave);
    w.wk_last = min(w.wk0 + 31, t.row_end - 1);
    w.qend_min = window_end(w.wk0, s.B, s.W, t.len);
    w.qend_max = window_end(max(w.wk0, w.wk_last), s.B, s.W, t.len);
    const int my_key = w.wk0 + (lane & 31);
    const int my_qend = window_end(my_key, s.B, s.W, t.len);
    w.x0 = 8 * (lane >> 5) - my_key;
    w.span = (uint32_t)max(my_qend - my_key, 0);
    return w;
}

// One 64-query chunk of the key role: S and dP for each 32-query sub-tile,
// then dV^T += dO^T P and dK^T += Q^T dS.  c0 = first query of the chunk;
// cb holds the chunk's row statistics.
template <int D, int ACT>
__device__ __forceinline__ void key_chunk(const Shape &s, const KWin &w, int lane,
                                          const lds_t *qt, const BwdChunk<D> &cb, int c0,
                                          const Ops<D> &op, const ReadOffsets<D> &ro,
                                          f32x16 (&adk)[D / 32], f32x16 (&adv)[D / 32]) {
    using G = TileGeom<D>;
    const int g = lane >> 5;
    const float c = s.scale * kLog2e;
    const lds_t *dt_ = qt + G::kBytes;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
        const int a = c0 + sub * 32;  // first query of the sub-tile
        if (!(a + 31 >= w.wk0 && a < w.qend_max)) continue;
        const lds_t *qs_ = qt + sub * 32 * G::kRowBytes;
        const lds_t *ds_ = dt_ + sub * 32 * G::kRowBytes;
        bf16x8 qa[D / 16], da[D / 16];
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            qa[ks] = lds_read16(qs_ + ro.rd[ks]);
            da[ks] = lds_read16(ds_ + ro.rd[ks]);
        }
        // lse2 and -delta of the sub-tile's queries, in register order:
        // register r holds query a + 8g + 16(r/8) + r%8.
        f32x16 ls, nd;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int qrow = sub * 32 + hh * 16 + g * 8;
            const float4 l0 = *(const float4 *)&cb.lse2[qrow];
            const float4 l1 = *(const float4 *)&cb.lse2[qrow + 4];
            const float4 d0 = *(const float4 *)&cb.ndlt[qrow];
            const float4 d1 = *(const float4 *)&cb.ndlt[qrow + 4];
            ls[hh * 8 + 0] = l0.x; ls[hh * 8 + 1] = l0.y; ls[hh * 8 + 2] = l0.z;
            ls[hh * 8 + 3] = l0.w; ls[hh * 8 + 4] = l1.x; ls[hh * 8 + 5] = l1.y;
            ls[hh * 8 + 6] = l1.z; ls[hh * 8 + 7] = l1.w;
            nd[hh * 8 + 0] = d0.x; nd[hh * 8 + 1] = d0.y; nd[hh * 8 + 2] = d0.z;
            nd[hh * 8 + 3] = d0.w; nd[hh * 8 + 4] = d1.x; nd[hh * 8 + 5] = d1.y;
            nd[hh * 8 + 6] = d1.z; nd[hh * 8 + 7] = d1.w;
        }
        f32x16 sc = mfma32(qa[0], op.a[0], f32x16{});
#pragma unroll
        for (int ks = 1; ks < D / 16; ++ks) sc = mfma32(qa[ks], op.a[ks], sc);
        // dP starts from -delta of each query: the products leave dP - delta
        // (the activation variants have no delta).
        f32x16 dp = mfma32(da[0], op.b[0], ACT == kSoftmax ? nd : f32x16{});
#pragma unroll
        for (int ks = 1; ks < D / 16; ++ks) dp = mfma32(da[ks], op.b[ks], dp);
        bf16x8 qtr[2][D / 32], dtr[2][D / 32];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                const lds_t *qr = qs_ + kk * 16 * G::kRowBytes;
                const lds_t *dr = ds_ + kk * 16 * G::kRowBytes;
                dtr[kk][dt] = lds_read_tr(dr + ro.trd[0][dt], dr + ro.trd[1][dt]);
                qtr[kk][dt] = lds_read_tr(qr + ro.trd[0][dt], qr + ro.trd[1][dt]);
            }
        // P, and the factor of dS = gf * dp (P itself for the softmax,
        // act'(scale s) for GDPA)
        float pf[16], gf[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if constexpr (ACT == kSoftmax)
                pf[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], c, -ls[r]));
            else
                act_value_slope<ACT>(sc[r] * s.scale, pf[r], gf[r]);
        }
        // Issue order as in the query role.
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * (D / 16) + 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, D / 16, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 8 * (D / 32), 0);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 32 / (D / 16), 0);
        }
        const bool masked = a < w.wk_last || a + 31 >= w.qend_min;
        // query of register r (a + 8g + 16(r/8) + r%8) sees this lane's key
        // iff my_key <= query < my_qend
        const int x = a + w.x0;
        if (masked) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if ((uint32_t)(x + 16 * (r >> 3) + (r & 7)) >= w.span) pf[r] = gf[r] = 0.f;
        }
        if constexpr (ACT == kSoftmax) {
#pragma unroll
            for (int r = 0; r < 16; ++r) gf[r] = pf[r];
        }
        // P in bf16 (and, for the softmax, its largest value, compared as
        // bits since the weights are >= 0), then the dV products, which need
        // only P; dS needs dP.
        uint32_t pmax = 0u;
        bf16x8 pb[2], dsb[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = kk * 8 + 2 * j;
                pmax = max(pmax, max(__float_as_uint(pf[r]), __float_as_uint(pf[r + 1])));
                const bf16x2 p2 = pack_bf16(pf[r], pf[r + 1]);
                pb[kk][2 * j] = p2[0];
                pb[kk][2 * j + 1] = p2[1];
            }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) adv[dt] = mfma32(dtr[kk][dt], pb[kk], adv[dt]);
        // Where a weight exceeds 1/4 (queries that see few keys), bf16
        // rounding of P (up to 2^-8 relative) is split off into a bf16 lo
        // part and dV takes a second product; elsewhere each term's rounding
        // error stays below 2^-10 |dO|, well under the bf16 rounding of dV
        // itself.  About 2% of sub-tiles split on N(0,1) inputs.
        // (Softmax only: activation weights are O(1) throughout, and their
        // sums are bounded relative to their own magnitude.)
        if (ACT == kSoftmax && __builtin_amdgcn_ballot_w64(pmax > __float_as_uint(0.25f)) != 0) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 lo;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = kk * 8 + 2 * j;
                    const bf16x2 l2 = pack_bf16(pf[r] - (float)pb[kk][2 * j],
                                                pf[r + 1] - (float)pb[kk][2 * j + 1]);
                    lo[2 * j] = l2[0];
                    lo[2 * j + 1] = l2[1];
                }
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) adv[dt] = mfma32(dtr[kk][dt], lo, adv[dt]);
            }
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = kk * 8 + 2 * j;
                const bf16x2 s2 = pack_bf16(gf[r] * dp[r], gf[r + 1] * dp[r + 1]);
                dsb[kk][2 * j] = s2[0];
                dsb[kk][2 * j + 1] = s2[1];
            }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) adk[dt] = mfma32(qtr[kk][dt], dsb[kk], adk[dt]);
    }
}

// ------------------------------------------------------------ pre-passes

// Tile counts per user (ceil(L / 128) units x 2 roles x H heads), their
// exclusive prefix sums into ubase[0..batch], the total into ctr[kQueues],
// and the queue counters of both passes ctr[0 .. kQueues) and
// ctr[kPass1Ctr .. kPass1Ctr + kQueues) = 0.  One workgroup.  Sums are
// capped at `cap` (the table's capacity, which well-formed offsets never
// reach), so malformed offsets cannot make the table writes overrun.
__global__ __launch_bounds__(1024) void bwd_tile_index(Shape s, int cap, int *__restrict__ ctr,
                                                       int *__restrict__ ubase) {
    __shared__ long long sh[16];
    const int T = (int)s.T;
    long long run = 0;
    for (int c0 = 0; c0 < s.batch; c0 += 1024) {
        const int u = c0 + (int)threadIdx.x;
        long long n = 0;
        if (u < s.batch) {
            const int a = clamp_off(s.offsets[u], T), b = clamp_off(s.offsets[u + 1], T);
            const int L = b > a ? b - a : 0;
            n = (long long)((L + kTileRows - 1) / kTileRows) * 2 * s.H;
        }
        long long total;
        const long long incl = wg_inclusive_scan<1024, long long>(n, sh, total);
        if (u < s.batch) ubase[u] = (int)min(run + incl - n, (long long)cap);
        run += total;
    }
    if (threadIdx.x == 0) {
        const int n = (int)min(run, (long long)cap);
        ubase[s.batch] = n;
        for (int i = 0; i < kQueues; ++i) ctr[i] = ctr[kPass1Ctr + i] = 0;
        ctr[kQueues] = n;
    }
}

// Workgroup u writes the table entries of user u in the order head, unit,
// role.
__global__ __launch_bounds__(256) void bwd_table(Shape s, const int *__restrict__ ubase,
                                                 int4 *__restrict__ table) {
    const int u = (int)blockIdx.x;
    const int j0 = ubase[u], j1 = ubase[u + 1];
    if (j1 <= j0) return;
    const int T = (int)s.T;
    const int a = clamp_off(s.offsets[u], T), e = clamp_off(s.offsets[u + 1], T);
    const int L = e - a;
    const int per_head = (L + kTileRows - 1) / kTileRows * 2;
    for (int j = j0 + (int)threadIdx.x; j < j1; j += 256) {
        const int loc = j - j0, h = loc / per_head, rem = loc - h * per_head;
        table[j] = make_int4(a, L, rem >> 1, (h << 1) | (rem & 1));
    }
}

// ------------------------------------------------------------ main kernel

// Kernel arguments and per-wave constants of the main kernel.
template <int D>
struct BwdArgs {
    Shape s;
    const bf16 *q, *k, *v, *dout;
    const bf16 *out;     // the forward's O (softmax query role: delta' = <dO, O>)
    const float *lse;    // the forward's lse [H, T]
    const float *ws_lse2, *ws_ndlt;
    int *ctr;         // this group's queue counter
    const int4 *table;
    int tstride, toff;  // tile n of this launch is table[n * tstride + toff]
    float *ndlt_out;    // where the query role writes its rows' exact -delta
    float *lse2_out;    // and their lse * log2(e)
    bf16 *dq, *dk, *dv;
    int ntiles;
    int group, ngroups;
    int wave, lane;
    lds_t *lds;       // chunk buffers
    BwdChunk<D> *sm;
    OpsLds<D> *ol;    // the tile's own rows
    int *ring;        // the next tile's index, by tile parity
    int *entry;       // the next tile's table entry (dwords 0..3)
    // rotary table (turns per position of each pair) or null
    const __attribute__((address_space(3))) double *rrev;
    uint32_t voff[TileGeom<D>::kDmaPerWave];
};

// Where a workgroup is in its stream of tiles.
struct BwdSched {
    int kt;         // tiles done
    int buf;        // LDS buffer of the next chunk
    int prev_role;  // role of the previous tile (-1: none)
};

// LDS byte address of a pointer into LDS (generic pointers to LDS carry the
// offset in their low 32 bits).
__device__ __forceinline__ uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)p; }
__device__ __forceinline__ uint32_t lds_addr(const lds_t *p) { return (uint32_t)(uintptr_t)p; }

// Tile index of the n-th request of a group.  The table is cut into rounds
// of ngroups runs of kRunTiles tiles; a group takes one run of each round,
// in snake order (run `group` of even rounds, run ngroups-1-group of odd
// ones), so a group that drew a costly run in one round draws a cheap end of
// the next where run costs trend along the table.
// (Saturated at INT32_MAX, which no tile index reaches.)
__device__ __forceinline__ int queue_tile(int n, int group, int ngroups) {
    const int r = n / kRunTiles;
    const int gq = (r & 1) ? ngroups - 1 - group : group;
    const int64_t j = ((int64_t)r * ngroups + gq) * kRunTiles + n % kRunTiles;
    return (int)min(j, (int64_t)INT32_MAX);
}

// One dword per lane from `src` (`bytes` valid, the rest zero) into LDS at
// byte address `dst`: 64 lanes x 4 bytes.
__device__ __forceinline__ void dma_dwords(const void *src, uint32_t bytes, uint32_t dst,
                                           int lane) {
    const uint64_t a = (uint64_t)src;
    const i32x4 desc{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                     __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffffu)),
                     __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
    const uint32_t d = __builtin_amdgcn_readfirstlane(dst);
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %1, %2, 0 offen lds"
        :
        : "s"(d), "v"((uint32_t)lane * 4u), "s"(desc)
        : "memory", "m0");
}

// Issues this wave's share of chunk ci of tile t into buffer `buf`.
template <int D>
__device__ __forceinline__ void issue_chunk(const BwdArgs<D> &A, const BwdTile &t, int ci,
                                            int buf) {
    using G = TileGeom<D>;
    const int64_t rs = (int64_t)A.s.H * D;
    const int off = t.sbeg + ci * kKC, rows = min(kKC, t.send - off);
    const int64_t base = ((int64_t)t.tok0 + off) * rs + (int64_t)t.h * D;
    lds_t *b = A.lds + buf * (int)sizeof(BwdChunk<D>);
    // (uniform branches rather than pointer selects, which the compiler
    // would turn into an indexed copy of the arguments in scratch memory)
    if (t.role == 0) {
        dma_tile<D>(row_desc<D>(A.k + base, rows, rs), b, A.voff, A.wave);
        dma_tile<D>(row_desc<D>(A.v + base, rows, rs), b + G::kBytes, A.voff, A.wave);
    } else {
        dma_tile<D>(row_desc<D>(A.q + base, rows, rs), b, A.voff, A.wave);
        dma_tile<D>(row_desc<D>(A.dout + base, rows, rs), b + G::kBytes, A.voff, A.wave);
        // the chunk's 64 lse2 and -delta values
        const int64_t so = (int64_t)t.h * A.s.T + t.tok0 + off;
        if (A.wave == 0)
            dma_dwords(A.ws_lse2 + so, (uint32_t)rows * 4u, lds_addr(b + 2 * G::kBytes), A.lane);
        else if (A.wave == 1)
            dma_dwords(A.ws_ndlt + so, (uint32_t)rows * 4u, lds_addr(b + 2 * G::kBytes + kKC * 4),
                       A.lane);
    }
}

// Issues this wave's share of tile t's own rows (and, for the query role,
// their row statistics) into the operand staging area.
template <int D, int ACT>
__device__ __forceinline__ void issue_ops(const BwdArgs<D> &A, const BwdTile &t) {
    const int64_t rs = (int64_t)A.s.H * D;
    const int64_t base = ((int64_t)t.tok0 + t.row0) * rs + (int64_t)t.h * D;
    const int rows = t.row_end - t.row0;
    auto rows_of = [&](const bf16 *src, bf16 (&dst)[2][kKC * D]) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int r = max(0, min(kKC, rows - half * kKC));
            dma_tile<D>(row_desc<D>(src + base + (int64_t)half * kKC * rs, r, rs),
                        (lds_t *)dst[half], A.voff, A.wave);
        }
    };
    if (t.role == 0) {
        rows_of(A.q, A.ol->a);
        rows_of(A.dout, A.ol->b);
        // waves 0 and 2: the forward's lse of rows 64 (w >> 1) ..
        const int half = A.wave >> 1;
        const int r = max(0, min(kKC, rows - half * kKC));
        const int64_t so = (int64_t)t.h * A.s.T + t.tok0 + t.row0 + half * kKC;
        if (ACT == kSoftmax && !(A.wave & 1))
            dma_dwords(A.lse + so, (uint32_t)r * 4u, lds_addr(A.ol->lse2 + half * kKC), A.lane);
    } else {
        rows_of(A.k, A.ol->a);
        rows_of(A.v, A.ol->b);
    }
}

// Reads this wave's operand registers from the staging area: lane
// (qi, g) takes row wave_rows + qi, 16-byte granules 2ks + g.
template <int D>
__device__ __forceinline__ void read_ops(const BwdArgs<D> &A, const BwdTile &t, Ops<D> &op) {
    using G = TileGeom<D>;
    const int qi = A.lane & 31, g = A.lane >> 5;
    const int lr = wave_rows(t, A.wave) - t.row0 + qi;  // 0 .. 127
    const int half = lr >> 6, p = sigma(lr & 63);      // physical row of logical row lr
    const lds_t *ta = (const lds_t *)A.ol->a[half];
    const lds_t *tb = (const lds_t *)A.ol->b[half];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        const int o = G::at(p, 2 * ks + g);
        op.a[ks] = lds_read16(ta + o);
        op.b[ks] = lds_read16(tb + o);
    }
    // (query role: the forward's lse; -delta' is set by the caller)
    op.lse2 = t.role == 0 ? A.ol->lse2[lr] * kLog2e : 0.f;
    op.ndlt = 0.f;
}

// The lane's 16-byte granules 2ks + g (ks < D/16) of its own row of the
// forward's O for query-role tile t, by plain buffer loads (rows past the
// tile read as zero): the granules of dO that read_ops gives the lane, so
// the lane's dot product covers half of the row and its lane^32 partner the
// other half.  Issued before a tile's output stores, so the next tile's
// first wait covers them.
template <int D>
__device__ __forceinline__ void load_orows(const BwdArgs<D> &A, const BwdTile &t,
                                           bf16x8 (&o)[D / 16]) {
    const int64_t rs = (int64_t)A.s.H * D;
    const auto r = row_rsrc<D>(A.out + ((int64_t)t.tok0 + t.row0) * rs + (int64_t)t.h * D,
                               t.row_end - t.row0, rs);
    const uint32_t lr = (uint32_t)(wave_rows(t, A.wave) - t.row0 + (A.lane & 31));
    const uint32_t off = lr * (uint32_t)(rs * 2) + (uint32_t)(A.lane >> 5) * 16u;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
        o[ks] = __builtin_bit_cast(bf16x8, buf_load16(r, off + (uint32_t)ks * 32u));
}

// Works through tile t (of role ROLE, whose own rows and first chunk are in
// flight or landed) and sets up the next one: returns false when the queue
// has run dry, else the next tile in tn with its rows and first chunk issued.
//
// orow: the softmax query role's O granules of tile t's rows on entry (see
// load_orows), and of the next tile's rows on return.
template <int D, int ROLE, int ACT>
__device__ __forceinline__ bool run_tile(const BwdArgs<D> &A, const ReadOffsets<D> &ro,
                                         BwdSched &sc, const BwdTile &t, BwdTile &tn,
                                         bf16x8 (&orow)[D / 16]) {
    // accumulator sets: dQ (and C, softmax) or dK and dV
    constexpr int NA = ROLE == 0 && ACT != kSoftmax ? 1 : 2;
    const int tid = threadIdx.x, g = A.lane >> 5;
    // The tile's rows and first chunk have landed; only the previous tile's
    // output stores may still be in flight.
    if (sc.prev_role < 0)
        wait_vm_barrier<0>();
    else if (sc.prev_role == 0)
        wait_vm_barrier<kStores<D, ACT>(0)>();
    else
        wait_vm_barrier<kStores<D, ACT>(1)>();
    Ops<D> op;
    read_ops<D>(A, t, op);
    if (ROLE == 0 && ACT == kSoftmax) {
        // delta' = <dO, O> of the lane's row (fp32 sums of bf16 products)
        float d = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) d = dot8(op.b[ks], orow[ks], d);
        op.ndlt = -swap_sum(d);
    }
    // Index of the next tile (published at the end of the previous one).
    const int jn = __builtin_amdgcn_readfirstlane(A.ring[(sc.kt + 1) & 1]);
    // The next tile's 16-byte entry goes straight into LDS (lanes 0..3 one
    // dword each, the rest past the range); the chunk waits cover it.
    if (jn < A.ntiles && A.wave == 0)
        dma_dwords(A.table + ((int64_t)jn * A.tstride + A.toff), 16u, lds_addr(A.entry), A.lane);
    // A one-chunk tile needs the entry in this same step, and must not
    // overwrite the staging area before every wave has read its rows.
    if (t.nch == 1) wait_vm_barrier<0>();
    // Request the index of the tile after next.  Only its raw count is kept
    // across the chunk loop; waiting for it happens at the end of the tile,
    // where what else is in flight (the next tile's first DMAs) is needed by
    // the next wait anyway.
    int pend = 0;
    if (tid == 0) pend = atomicAdd(A.ctr, 1);

    f32x16 acc[NA][D / 32];
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) acc[i][dt] = f32x16{};
    f32x16 ndlt;
    if (ROLE == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) ndlt[r] = op.ndlt;
    }
    const bool live = wave_rows(t, A.wave) < t.row_end;
    QWin qw;
    KWin kw;
    if (ROLE == 0)
        qw = query_win(A.s, t, A.wave, A.lane);
    else
        kw = key_win(A.s, t, A.wave, A.lane);
    float eps = 0.f;  // softmax query role: this lane's share of delta - delta'
    bool has_next = false;
    for (int ci = 0; ci < t.nch; ++ci) {
        if (ci > 0) wait_vm_barrier<0>();  // chunk ci has landed
        if (ci + 1 < t.nch) {
            issue_chunk<D>(A, t, ci + 1, sc.buf ^ 1);
        } else if (jn < A.ntiles) {
            const int *e = A.entry;
            tn = make_tile(A.s, make_int4(e[0], e[1], e[2], e[3]));
            issue_chunk<D>(A, tn, 0, sc.buf ^ 1);
            issue_ops<D, ACT>(A, tn);
            has_next = true;
        }
        const lds_t *b = A.lds + sc.buf * (int)sizeof(BwdChunk<D>);
        const int c0 = t.sbeg + ci * kKC;
        if (live) {
            if (ROLE == 0)
                query_chunk<D, ACT>(A.s, qw, A.lane, b, c0, op, ndlt, ro, acc[0], acc[NA - 1],
                                    eps);
            else
                key_chunk<D, ACT>(A.s, kw, A.lane, b, A.sm[sc.buf], c0, op, ro, acc[0],
                                  acc[NA - 1]);
        }
        sc.buf ^= 1;
    }
    // (read in every lane by a convergent readfirstlane, which the compiler
    // cannot move into the lane-0 branch, so the wait for the atomic is on
    // every path and no register stays pending into the next tile)
    const int jnn = queue_tile(__builtin_amdgcn_readfirstlane(pend), A.group, A.ngroups);
    if (tid == 0) A.ring[sc.kt & 1] = jnn;
    // Outputs: a fixed number of stores per wave (rows past the tile are
    // clipped), which the next tile's first wait allows for.
    const int64_t rs = (int64_t)A.s.H * D;
    const int64_t obase = ((int64_t)t.tok0 + t.row0) * rs + (int64_t)t.h * D;
    const int rows = t.row_end - t.row0;
    const uint32_t lrow = (uint32_t)(wave_rows(t, A.wave) - t.row0 + (A.lane & 31));
    const int pos = t.row0 + (int)lrow;  // local index of the lane's row
    if (ROLE == 0 && ACT == kSoftmax && has_next) load_orows<D>(A, tn, orow);
    if (ROLE == 0 && ACT == kSoftmax) {
        // The exact delta_i = delta'_i + eps_i (sum_j P_ij = 1), and
        // dQ_i = scale sum_j P_ij (dP_ij - delta_i) k_j
        //      = (the dS-with-delta' sum) - scale eps_i C_i.
        // (query i's keys are split between lanes i and i + 32)
        const float e = swap_sum(eps);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[0][dt][r] = fmaf(-e, acc[NA - 1][dt][r], acc[0][dt][r]);
        // -delta and lse * log2(e) of the lane's row for the key pass (lanes
        // g = 1 and rows past the tile fall outside the buffer range: two
        // stores per wave)
        const int64_t so = (int64_t)t.h * A.s.T + t.tok0 + t.row0;
        const uint32_t sb = g == 0 ? lrow * 4u : 0x80000000u;
        buf_store4(op.ndlt - e, bytes_rsrc(A.ndlt_out + so, (uint32_t)rows * 4u), sb);
        buf_store4(op.lse2, bytes_rsrc(A.lse2_out + so, (uint32_t)rows * 4u), sb);
    }
    if (ROLE == 0) {
        store_rows<D>(A.dq + obase, rows, rs, lrow, acc[0], A.s.scale, g, A.rrev, pos);
    } else {
        store_rows<D>(A.dk + obase, rows, rs, lrow, acc[0], A.s.scale, g, A.rrev, pos);
        store_rows<D>(A.dv + obase, rows, rs, lrow, acc[NA - 1], 1.f, g, nullptr, pos);
    }
    sc.prev_role = ROLE;
    ++sc.kt;
    return has_next;
}

// PASS 0 runs the query-role tiles, PASS 1 the key-role tiles, PASS 2 both.
// The softmax backward runs PASS 0 and then PASS 1 as two launches: the
// query role computes each row's exact delta, which the key role needs.
// The activation variants have no delta and run PASS 2.
template <int D, int ACT, int PASS>
__global__ __launch_bounds__(kThreads, kWavesPerSimd<D>) void bwd_mfma(
    Shape s, const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ dout, const bf16 *__restrict__ out, const float *__restrict__ lse,
    float *__restrict__ ws_lse2, float *__restrict__ ws_ndlt, int *__restrict__ ctr,
    const int4 *__restrict__ table, bf16 *__restrict__ dq, bf16 *__restrict__ dk,
    bf16 *__restrict__ dv) {
    static_assert(!(ACT == kSoftmax && PASS == 2),
                  "the softmax key role must run after every query role has written delta");
    __shared__ __align__(1024) BwdChunk<D> sm[2];
    __shared__ __align__(1024) OpsLds<D> ol;
    __shared__ int ring[2];  // the next tile's index, by tile parity
    __shared__ int entry[64];  // 64 lanes x 4 bytes; dwords 0..3 hold the entry
    __shared__ double rrev[D / 2];  // rotary turns per position of each pair
    const int tid = threadIdx.x;
    BwdArgs<D> A;
    A.s = s;
    A.q = q;
    A.k = k;
    A.v = v;
    A.dout = dout;
    A.out = out;
    A.lse = lse;
    A.ws_lse2 = ws_lse2;
    A.ws_ndlt = ws_ndlt;
    A.lse2_out = ws_lse2;
    A.ngroups = min((int)gridDim.x, kQueues);
    A.group = (int)blockIdx.x % A.ngroups;
    A.ctr = ctr + (PASS == 1 ? kPass1Ctr : 0) + A.group;
    A.table = table;
    A.tstride = PASS == 2 ? 1 : 2;
    A.toff = PASS == 2 ? 0 : PASS;
    A.ndlt_out = ws_ndlt;
    A.dq = dq;
    A.dk = dk;
    A.dv = dv;
    A.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    A.lane = tid & 63;
    A.lds = (lds_t *)sm;
    A.sm = sm;
    A.ol = &ol;
    A.ring = ring;
    A.entry = entry;
    A.rrev = nullptr;
    if (s.rope_base > 0.f) {
        if (tid < D / 2) rrev[tid] = exp2(-2.0 * tid / D * log2((double)s.rope_base)) * kInv2Pi;
        A.rrev = (const __attribute__((address_space(3))) double *)rrev;
    }
    dma_offsets<D>(A.voff, A.wave, A.lane, (uint32_t)((int64_t)s.H * D * 2));
    const ReadOffsets<D> ro(A.lane);

    if (tid == 0) {
        ring[0] = queue_tile(atomicAdd(A.ctr, 1), A.group, A.ngroups);
        ring[1] = queue_tile(atomicAdd(A.ctr, 1), A.group, A.ngroups);
    }
    __syncthreads();
    // (every unit has one tile of each role, so a single-role pass has half
    // the table's tiles)
    const int ntab = __builtin_amdgcn_readfirstlane(ctr[kQueues]);
    A.ntiles = PASS == 2 ? ntab : ntab / 2;
    const int j0 = __builtin_amdgcn_readfirstlane(ring[0]);
    if (j0 >= A.ntiles) return;
    BwdTile t = make_tile(s, table[(int64_t)j0 * A.tstride + A.toff]);
    issue_chunk<D>(A, t, 0, 0);
    issue_ops<D, ACT>(A, t);
    bf16x8 orow[D / 16];
    if (PASS == 0 && ACT == kSoftmax) load_orows<D>(A, t, orow);

    BwdSched sc{0, 0, -1};
    for (;;) {
        BwdTile tn;
        bool more;
        if constexpr (PASS == 0)
            more = run_tile<D, 0, ACT>(A, ro, sc, t, tn, orow);
        else if constexpr (PASS == 1)
            more = run_tile<D, 1, ACT>(A, ro, sc, t, tn, orow);
        else
            more = t.role == 0 ? run_tile<D, 0, ACT>(A, ro, sc, t, tn, orow)
                               : run_tile<D, 1, ACT>(A, ro, sc, t, tn, orow);
        if (!more) break;
        t = tn;
    }
}

// Workgroups of bwd_mfma<D, ACT, PASS> that fit on the current device at once.
template <int D, int ACT, int PASS>
int resident_workgroups() {
    // one per instantiation and device; concurrent first calls may both
    // compute it, and store the same value
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    if (dev >= 0 && dev < 64) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, bwd_mfma<D, ACT, PASS>, kThreads, 0) !=
            hipSuccess ||
        per < 1)
        per = 1;
    const int n = cus * per;
    if (dev >= 0 && dev < 64) cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

template <int D, int ACT>
hipError_t launch_act(const Shape &s, const void *q, const void *k, const void *v,
                      const void *out, const void *dout, const float *lse, void *dq, void *dk,
                      void *dv, void *ws, hipStream_t st) {
    const BwdWorkspace w = bwd_workspace_layout(ws, s.T, s.batch, s.H);
    const int64_t max_tiles = bwd_max_tiles(s.T, s.batch, s.H);
    hipLaunchKernelGGL(bwd_tile_index, dim3(1), dim3(1024), 0, st, s, (int)max_tiles, w.ctr,
                       w.ubase);
    hipLaunchKernelGGL(bwd_table, dim3((unsigned)s.batch), dim3(256), 0, st, s,
                       (const int *)w.ubase, w.table);
    auto main_pass = [&](auto pass_c) {
        constexpr int PASS = decltype(pass_c)::value;
        const int64_t grid = std::min<int64_t>(PASS == 2 ? max_tiles : max_tiles / 2,
                                               (int64_t)resident_workgroups<D, ACT, PASS>());
        hipLaunchKernelGGL((bwd_mfma<D, ACT, PASS>), dim3((unsigned)std::max<int64_t>(grid, 1)),
                           dim3(kThreads), 0, st, s, (const bf16 *)q, (const bf16 *)k,
                           (const bf16 *)v, (const bf16 *)dout, (const bf16 *)out, lse, w.lse2,
                           w.ndlt, w.ctr, (const int4 *)w.table, (bf16 *)dq, (bf16 *)dk,
                           (bf16 *)dv);
    };
    if constexpr (ACT == kSoftmax) {
        main_pass(std::integral_constant<int, 0>{});
        main_pass(std::integral_constant<int, 1>{});
    } else {
        main_pass(std::integral_constant<int, 2>{});
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_t(const Shape &s, const void *q, const void *k, const void *v, const void *out,
                    const void *dout, const float *lse, void *dq, void *dk, void *dv,
                    void *ws, hipStream_t st) {
    switch (s.act) {
    case kSoftmax: return launch_act<D, kSoftmax>(s, q, k, v, out, dout, lse, dq, dk, dv, ws, st);
    case kSilu: return launch_act<D, kSilu>(s, q, k, v, out, dout, lse, dq, dk, dv, ws, st);
    case kGelu: return launch_act<D, kGelu>(s, q, k, v, out, dout, lse, dq, dk, dv, ws, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_mfma_bwd(const Shape &s, const void *q, const void *k, const void *v,
                           const void *out, const void *dout, const float *lse, void *dq,
                           void *dk, void *dv, void *ws, hipStream_t st) {
    switch (s.D) {
    case 32: return launch_t<32>(s, q, k, v, out, dout, lse, dq, dk, dv, ws, st);
    case 64: return launch_t<64>(s, q, k, v, out, dout, lse, dq, dk, dv, ws, st);
    case 128: return launch_t<128>(s, q, k, v, out, dout, lse, dq, dk, dv, ws, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace ba
