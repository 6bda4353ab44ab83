// Backward block attention in MXFP8 on the block-scaled fp8 matrix cores
// (gfx950).
//
// "GEM (Meta)", section "Ultra-low-precision training": the attention kernel
// runs its matrix products as block-scaled MXFP8 in the backward pass as well
// as the forward.  All five products here are
// v_mfma_scale_f32_32x32x64_f8f6f4, each with its operands' scale blocks
// along its own contraction:
//   query pass (one wave per 32 queries i):
//     S^T = K Q^T and dP^T - delta = V dO^T - delta   (head dims: q, k, v,
//       dO head-dim-blocked),
//     dS = P (dP - delta), quantized along the query's keys,
//     dQ^T += K_t^T dS^T                               (keys: k token-blocked);
//   key pass (one wave per 32 keys j):
//     S = Q K^T and dP - delta = dO V^T - delta        (head dims),
//     P and dS quantized along the key's queries,
//     dV^T += dO_t^T P and dK^T += Q_t^T dS            (queries: q, dO
//       token-blocked).
// P_ij = exp(scale s_ij - lse_i) with the forward's lse, and delta_i =
// <dO_i, O_i> with the forward's O.  The query pass computes delta and
// lse * log2(e) of its rows and writes them for the key pass, which runs
// after it.
//
// Quantization of a block of 32 values (one query's keys, or one key's
// queries, 32 positions counted from the user's first token; positions
// outside the window are 0): with a the block's largest magnitude,
// E = max(floor(log2 a) - 7, -127), the codes are the nearest E4M3 values
// of x 2^-E (below 2^8, so none saturates) and the scale byte is E + 127.
// A lane pair (n, n + 32) holds one block: 16 values each.
//
// Layouts, as in the MXFP8 forward: head-dim-blocked E4M3 [T, H, D] with
// E8M0 scales [H, T, D/32]; token-blocked E4M3 transposed [H, D, 32 NB] with
// scales [H, NB, D], NB = ceil(T/32) + batch, user u's local token j at
// column 32 ub + j with ub = ceil(off[u]/32) + u.  Streamed head-dim-blocked
// rows sit at LDS row rho(m) (mfma_util.h), so register r of lane group g of
// a 32-row half's scores is position 16g + r: in register order, the lane's
// bytes of the next product's operand.  Token-blocked chunks are D rows of
// 64 bytes, read as plain rows (physical row m holds head-dim row sigma(m),
// which puts accumulator register 8 half + e at column 16 half + 8 g + e).
// Chunks of 64 positions start on multiples of 32 of the user's tokens and
// go from HBM straight into two LDS buffers in turn, one barrier per chunk.
// One workgroup per 128-row tile, found by the forward's tile decode.
#include "kernels.h"
#include "lds_tile.h"

namespace ba {
namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kTileRows = 128;
constexpr int kKC = 64;        // positions per streamed chunk

typedef float f32x4v __attribute__((ext_vector_type(4)));

// Waves per SIMD the register budget is sized for: ROLE 0 is the query
// pass (one accumulator set), ROLE 1 the key pass (two).
template <int D, int ROLE>
constexpr int kWaves = ROLE == 0 ? (D == 128 ? 2 : 3) : (D == 128 ? 1 : 2);

// One chunk buffer: tiles of 64 x D bytes, each followed by a 1 KiB area
// for its scales.  Query pass: K, V (head-dim-blocked), K_t (token-blocked).
// Key pass: Q, dO, Q_t, dO_t, then lse * log2(e) and -delta of the chunk's
// 64 queries.
template <int D>
struct MxBuf {
    static constexpr int kTile = 64 * D + 1024;
    static constexpr int kStats = 4 * kTile;
    static constexpr int kBytes[2] = {3 * kTile, 4 * kTile + 1024};
};

struct MxBwdArgs {
    const uint8_t *q, *qsc, *k, *ksc, *v, *vsc, *dout, *dosc;  // head-dim-blocked
    const uint8_t *qt, *qtsc, *kt, *ktsc, *dot, *dotsc;        // token-blocked
    const bf16 *out;    // the forward's O
    const float *lse;   // the forward's lse [H, T]
    float *lse2, *ndlt; // [H, T]: lse * log2(e) and -delta, query pass -> key pass
    bf16 *dq, *dk, *dv;
};

// The lane's operand bytes of its own head-dim-blocked row (rows that do not
// exist read as zero codes with scale 2^0): lane (n, g) takes bytes
// 64i + 16g .. + 15 and 64i + 32 + 16g .. + 15 of the row, and the scale of
// block 2i + g.
template <int D>
__device__ __forceinline__ void own_row(const uint8_t *x, const uint8_t *xsc, const Shape &s,
                                        int64_t tok, int h, bool ok, int g, i32x8 (&f)[D / 64],
                                        int (&sc)[D / 64]) {
    const uint8_t *p = x + tok * ((int64_t)s.H * D) + (int64_t)h * D;
    const uint8_t *ps = xsc + ((int64_t)h * s.T + tok) * (D / 32);
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
        uint4 lo = make_uint4(0u, 0u, 0u, 0u), hi = lo;
        int b = 127;
        if (ok) {
            lo = *(const uint4 *)(p + 64 * i + 16 * g);
            hi = *(const uint4 *)(p + 64 * i + 32 + 16 * g);
            b = ps[2 * i + g];
        }
        f[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        sc[i] = b;
    }
}

// Head-dim-blocked rows [tok, tok + rows) of head h into a tile at physical
// rows rho(m) (rows past `rows` arrive as zeros).
template <int D>
__device__ __forceinline__ void dma_rows8(const uint8_t *x, const Shape &s, int64_t tok, int rows,
                                          int h, lds_t *dst,
                                          const uint32_t (&voff)[TileGeom<D / 2>::kDmaPerWave],
                                          int wave) {
    const int64_t rs = (int64_t)s.H * D / 2;  // row stride in bf16 units
    const bf16 *base = (const bf16 *)x + tok * rs + (int64_t)h * (D / 2);
    dma_tile<D / 2>(row_desc<D / 2>(base, rows, rs), dst, voff, wave);
}

// How many bytes before the scales of row tok, head h ([H, T, D/32]) the
// dword-aligned window that dma_scales loads starts.
template <int D>
__device__ __forceinline__ int scale_mis(const Shape &s, int h, int64_t tok) {
    return (int)((((int64_t)h * s.T + tok) * (D / 32)) & 3);
}

// The scales of rows [tok, tok + rows) into LDS at dst, from mis bytes
// before them (one wave).  The dword window ends at most 3 bytes past the
// last scale; only at the tensor's end can that pass it, and then the
// window is read byte by byte.
template <int D>
__device__ __forceinline__ void dma_scales(const uint8_t *xsc, const Shape &s, int h, int64_t tok,
                                           int rows, lds_t *dst, int lane) {
    const int64_t first = ((int64_t)h * s.T + tok) * (D / 32);
    const int mis = (int)(first & 3);
    const uint32_t nb = (uint32_t)(max(rows, 0) * (D / 32) + mis);
    const uint32_t nbr = (nb + 3) & ~3u;
    const int64_t wbeg = first - mis, total = (int64_t)s.H * s.T * (D / 32);
    if (wbeg + nbr <= total)
        dma_dwords_lds(xsc + wbeg, nbr, lds_addr_of(dst), lane);
    else
        bytes_to_lds(xsc + wbeg, (uint32_t)(total - wbeg), lds_addr_of(dst), lane);
}

// 64 positions of token-blocked rows of head h, from column 32 ub + c: D/64
// tiles of 64 head-dim rows x 64 bytes, and (wave sw) the two blocks' 2 x D
// scales at dst + 64 D.
template <int D>
__device__ __forceinline__ void dma_trows(const uint8_t *x, const uint8_t *xsc, const Shape &s,
                                          int h, int64_t ub, int c, lds_t *dst,
                                          const uint32_t (&voffv)[1], int wave, int lane,
                                          int sw) {
    const int64_t nblk = (s.T + 31) / 32 + s.batch, Tp = 32 * nblk;
    const int64_t tot = (int64_t)s.H * D * Tp;
#pragma unroll
    for (int j = 0; j < D / 64; ++j) {
        const int64_t o = ((int64_t)h * D + 64 * j) * Tp + 32 * ub + c;
        const uint64_t a = (uint64_t)(x + o);
        const uint32_t range = (uint32_t)min(63 * Tp + 64, tot - o);
        dma_tile<32>(i32x4{(int)(uint32_t)a, (int)((a >> 32) & 0xffffu), (int)range, 0x00020000},
                     dst + j * 4096, voffv, wave);
    }
    if (wave == sw) {
        const int64_t so = ((int64_t)h * nblk + ub + c / 32) * D;
        const uint32_t nb = (uint32_t)min((int64_t)2 * D, (int64_t)s.H * nblk * D - so);
        dma_dwords_lds(xsc + so, nb, lds_addr_of(dst + 64 * D), lane);
    }
}

// Block-scaled E4M3 codes of the 16 values x[] of this lane; the lane pair
// (n, n + 32) holds one block of 32.  Returns the scale byte E + 127.  The
// scaled conversion divides by 2 to the power of its scale operand's
// exponent field, so the fp32 bit pattern (E + 127) << 23 gives x 2^-E for
// every E in [-127, 127] (checked on gfx950 against the plain conversion of
// x 2^-E, including E = -127, whose pattern is +0.0).
__device__ __forceinline__ int quant_block(const float (&x)[16], int *w) {
    float a = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) a = fmaxf(a, fabsf(x[r]));
    a = swap_max(a);
    // frexp exponent e (a = f 2^e, f in [0.5, 1)): floor(log2 a) = e - 1
    const int E = a > 0.f ? max(__builtin_amdgcn_frexp_expf(a) - 8, -127) : -127;
    const float sc = __uint_as_float((uint32_t)(E + 127) << 23);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        i16x2 c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(i16x2{0, 0}, x[4 * j], x[4 * j + 1],
                                                          sc, false);
        c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(c, x[4 * j + 2], x[4 * j + 3], sc, true);
        w[j] = __builtin_bit_cast(int, c);
    }
    return E + 127;
}

// Reads a 32-row half (rows 32 h ..) of a head-dim-blocked tile: the lane's
// operand bytes (row read offsets rd) and scales (sbase: the tile's scale
// window, already at the lane's row and g).
template <int D>
__device__ __forceinline__ void read_half8(const lds_t *tile, const lds_t *sbase, int h,
                                           const int (&rd)[D / 32], i32x8 (&f)[D / 64],
                                           int (&sc)[D / 64]) {
    using G8 = TileGeom<D / 2, 1>;
    const lds_t *t8 = tile + h * 32 * G8::kRowBytes;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
        const uint4 lo = __builtin_bit_cast(uint4, lds_read16(t8 + rd[2 * i]));
        const uint4 hi = __builtin_bit_cast(uint4, lds_read16(t8 + rd[2 * i + 1]));
        f[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        sc[i] = *(const __attribute__((address_space(3))) uint8_t *)(sbase + h * 32 * (D / 32) +
                                                                     2 * i);
    }
}

// One head-dim contraction: sum_i of the block-scaled products of a[i] (A
// rows) and b[i] (B columns) onto acc.
template <int D>
__device__ __forceinline__ f32x16 hd_product(const i32x8 (&a)[D / 64], const int (&as)[D / 64],
                                             const i32x8 (&b)[D / 64], const int (&bs)[D / 64],
                                             f32x16 acc) {
#pragma unroll
    for (int i = 0; i < D / 64; ++i)
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[i], acc, 0, 0, 0, as[i], 0,
                                                             bs[i]);
    return acc;
}

// acc[dt] += T^T X for a token-blocked tile T (D rows of 64 bytes; the
// lane's row read rdv and scale byte offset tsrd) and the quantized operand
// x (scale byte xs of the lane's block g).
template <int D>
__device__ __forceinline__ void tok_product(const lds_t *tt, int rdv, int tsrd, const i32x8 &x,
                                            int xs, f32x16 (&acc)[D / 32]) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
        const int tb = (dt >> 1) * 4096 + (dt & 1) * 2048;
        const uint4 lo = __builtin_bit_cast(uint4, lds_read16(tt + tb + rdv));
        const uint4 hi = __builtin_bit_cast(uint4, lds_read16(tt + tb + (rdv ^ 32)));
        const i32x8 a = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                              (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        const int as = *(const __attribute__((address_space(3))) uint8_t *)(tt + 64 * D + tsrd +
                                                                          32 * dt);
        acc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, x, acc[dt], 0, 0, 0, as, 0,
                                                                 xs);
    }
}

// Writes a wave's 32 rows of one output (acc * mul) as bf16 (row `row` of
// the lane; rows at or past row_end are skipped).
template <int D>
__device__ __forceinline__ void store_out(bf16 *dst, const Shape &s, const Tile &t, int row,
                                          int row_end, int g, const f32x16 (&acc)[D / 32],
                                          float mul) {
    if (row >= row_end) return;
    bf16 *o = dst + (t.tok0 + row) * ((int64_t)s.H * D) + (int64_t)t.h * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            bf16x8 x;
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = (bf16)(acc[dt][half * 8 + i] * mul);
            *(bf16x8 *)(o + dt * 32 + half * 16 + g * 8) = x;
        }
}

template <int D, int ROLE, int UPT>
__global__ __launch_bounds__(kThreads, (kWaves<D, ROLE>)) void bwd_mx(Shape s, MxBwdArgs A) {
    using G8 = TileGeom<D / 2, 1>;  // a head-dim-blocked row of D bytes
    constexpr int kBuf = MxBuf<D>::kBytes[ROLE];
    constexpr int kT = MxBuf<D>::kTile;
    __shared__ int sh[8];
    __shared__ __align__(1024) unsigned char sm[2 * kBuf];
    Tile t;
    if (!decode_tile<kThreads, UPT>(s, kTileRows, 1, t, sh)) return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int w = (wave + t.blk) & 3;  // row group of this wave
    const int qi = lane & 31, g = lane >> 5;
    const int row0 = t.blk * kTileRows;
    const int row_end = min(row0 + kTileRows, t.len);
    const int wr0 = row0 + w * 32;  // the wave's first row (query or key)
    const int my = wr0 + qi;
    const bool wave_live = wr0 < row_end;
    const int w_last = min(wr0 + 31, row_end - 1);
    const float c = s.scale * kLog2e;
    const int64_t ub = (t.tok0 + 31) / 32 + t.user;  // the user's first token block
    lds_t *lds = (lds_t *)sm;

    // streamed positions [sbeg, send): keys of the tile's queries (query
    // pass, back to a multiple of 32) or queries that see its keys (key pass)
    const int sbeg = ROLE == 0 ? window_start(row0, s.B, s.W) & ~31 : row0;
    const int send = ROLE == 0 ? row_end : window_end(row_end - 1, s.B, s.W, t.len);
    const int nch = (send - sbeg + kKC - 1) / kKC;

    uint32_t voff8[G8::kDmaPerWave];
    dma_offsets<D / 2, true, 1>(voff8, wave, lane, (uint32_t)(s.H * D));
    uint32_t voffv[1];
    dma_offsets<32, false, 1>(voffv, wave, lane,
                              (uint32_t)(32 * ((s.T + 31) / 32 + s.batch)));
    auto issue = [&](int ci, int buf) {
        const int off = sbeg + ci * kKC, rows = min(kKC, t.len - off);
        const int64_t tok = t.tok0 + off;
        lds_t *b = lds + buf * kBuf;
        if constexpr (ROLE == 0) {
            dma_rows8<D>(A.k, s, tok, rows, t.h, b, voff8, wave);
            dma_rows8<D>(A.v, s, tok, rows, t.h, b + kT, voff8, wave);
            dma_trows<D>(A.kt, A.ktsc, s, t.h, ub, off, b + 2 * kT, voffv, wave, lane, 1);
            if (wave == 0) dma_scales<D>(A.ksc, s, t.h, tok, rows, b + 64 * D, lane);
            if (wave == 2) dma_scales<D>(A.vsc, s, t.h, tok, rows, b + kT + 64 * D, lane);
        } else {
            dma_rows8<D>(A.q, s, tok, rows, t.h, b, voff8, wave);
            dma_rows8<D>(A.dout, s, tok, rows, t.h, b + kT, voff8, wave);
            dma_trows<D>(A.qt, A.qtsc, s, t.h, ub, off, b + 2 * kT, voffv, wave, lane, 1);
            dma_trows<D>(A.dot, A.dotsc, s, t.h, ub, off, b + 3 * kT, voffv, wave, lane, 3);
            if (wave == 0) dma_scales<D>(A.qsc, s, t.h, tok, rows, b + 64 * D, lane);
            if (wave == 2) dma_scales<D>(A.dosc, s, t.h, tok, rows, b + kT + 64 * D, lane);
            // the chunk's lse * log2(e) and -delta (rows past the user read 0)
            const int64_t so = (int64_t)t.h * s.T + tok;
            const uint32_t nb = (uint32_t)max(rows, 0) * 4u;
            if (wave == 1) dma_dwords_lds(A.lse2 + so, nb, lds_addr_of(b + MxBuf<D>::kStats), lane);
            if (wave == 3)
                dma_dwords_lds(A.ndlt + so, nb, lds_addr_of(b + MxBuf<D>::kStats + 256), lane);
        }
    };
    if (nch > 0) issue(0, 0);

    // The wave's own rows: Q and dO (query pass) or K and V (key pass).
    const bool ok = my < row_end;
    i32x8 fa[D / 64], fb[D / 64];
    int sa[D / 64], sb[D / 64];
    own_row<D>(ROLE == 0 ? A.q : A.k, ROLE == 0 ? A.qsc : A.ksc, s, t.tok0 + my, t.h, ok, g, fa,
               sa);
    own_row<D>(ROLE == 0 ? A.dout : A.v, ROLE == 0 ? A.dosc : A.vsc, s, t.tok0 + my, t.h, ok, g,
               fb, sb);
    float lse2 = 0.f, ndlt = 0.f;
    if constexpr (ROLE == 0) {
        // delta = <dO, O> of the lane's row: the lane's dO bytes (both
        // blocks of each 64-element group: scales 2i and 2i + 1) against the
        // same columns of the forward's O, fp32; the lane pair holds the row.
        float d = 0.f, l = 0.f;
        if (ok) {
            const int64_t tok = t.tok0 + my;
            const bf16 *orow = A.out + tok * ((int64_t)s.H * D) + (int64_t)t.h * D;
            const uint8_t *ps = A.dosc + ((int64_t)t.h * s.T + tok) * (D / 32);
#pragma unroll
            for (int i = 0; i < D / 64; ++i)
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const float f = ldexpf(1.f, (int)ps[2 * i + half] - 127);
                    const uint4 o0 = *(const uint4 *)(orow + 64 * i + 32 * half + 16 * g);
                    const uint4 o1 = *(const uint4 *)(orow + 64 * i + 32 * half + 16 * g + 8);
                    const uint32_t ow[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
                    float part = 0.f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int code = fb[i][4 * half + j];
                        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(code, false);
                        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(code, true);
                        part = fmaf(lo[0], __uint_as_float(ow[2 * j] << 16), part);
                        part = fmaf(lo[1], __uint_as_float(ow[2 * j] & 0xffff0000u), part);
                        part = fmaf(hi[0], __uint_as_float(ow[2 * j + 1] << 16), part);
                        part = fmaf(hi[1], __uint_as_float(ow[2 * j + 1] & 0xffff0000u), part);
                    }
                    d = fmaf(part, f, d);
                }
            l = A.lse[(int64_t)t.h * s.T + tok] * kLog2e;
        }
        ndlt = -swap_sum(d);
        lse2 = l;
        if (ok && g == 0) {
            const int64_t so = (int64_t)t.h * s.T + t.tok0 + my;
            A.ndlt[so] = ndlt;
            A.lse2[so] = lse2;
        }
    }
    // Own rows (and chunk 0) complete here, so inside the chunk loop the
    // only vector memory operations in flight are the tile loads that the
    // loop waits for itself.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    // Per-lane LDS read offsets: row reads of head-dim-blocked tiles (lane
    // (qi, g): physical row qi, granules 2ks + g), the lane's row in their
    // scale windows (physical row qi holds position rho(qi)), and the
    // token-blocked tile's row read and scale (head-dim row sigma(qi) of
    // block g).
    int rd[D / 32];
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) rd[ks] = row_read_offset<D / 2, 1>(qi, g) ^ (ks << 5);
    const int srd = rho32(qi) * (D / 32) + g;
    const int rdv = row_read_offset<32, 1>(qi, g);
    const int tsrd = g * D + sigma32(qi);

    // Window bounds.  Query pass: the lane's query `my` sees keys
    // [klo, my]; key pass: the lane's key `my` is seen by queries
    // [my, qend).  Wave-uniform: the first/last positions any lane needs and
    // the ranges where every lane sees everything.
    const int my_lo = ROLE == 0 ? window_start(my, s.B, s.W) : my;
    const uint32_t span = ROLE == 0 ? (uint32_t)(my - my_lo)
                                    : (uint32_t)max(window_end(my, s.B, s.W, t.len) - my, 0);
    const int lo_min = ROLE == 0 ? window_start(wr0, s.B, s.W) : wr0;          // first needed
    const int hi_max = ROLE == 0 ? w_last + 1 : window_end(w_last, s.B, s.W, t.len);  // end
    const int full_lo = ROLE == 0 ? window_start(w_last, s.B, s.W) : w_last;
    const int full_hi = ROLE == 0 ? wr0 + 1 : window_end(wr0, s.B, s.W, t.len);

    f32x16 acc[ROLE == 0 ? 1 : 2][D / 32];
#pragma unroll
    for (int i = 0; i < (ROLE == 0 ? 1 : 2); ++i)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) acc[i][dt] = f32x16{};

    auto step = [&](int ci, auto buf_c) {
        constexpr int buf = decltype(buf_c)::value;
        wait_vm_barrier<0>();
        if (ci + 1 < nch) issue(ci + 1, buf ^ 1);
        if (!wave_live) return;
        const lds_t *b = lds + buf * kBuf;
        const int c0 = sbeg + ci * kKC;
        const bool live0 = c0 < hi_max && c0 + 31 >= lo_min;
        const bool live1 = c0 + 32 < hi_max && c0 + 63 >= lo_min;
        if (!live0 && !live1) return;
        int q1[8], q2[8];  // codes: dS (query pass); P and dS (key pass)
        int e1[2], e2[2];  // their scale bytes per half
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int a = c0 + 32 * h;
            // (a half that no lane of the wave sees always counts as masked
            // below, and every position of it fails the visibility test, so
            // it comes out as zeros without a path of its own)
            const bool masked = ROLE == 0 ? (a + 31 > wr0 || a < full_lo)
                                          : (a < w_last || a + 31 >= full_hi);
            const int x0 = a + 16 * g - my_lo;
            // The weights first (scores, P and, in the key pass, P's codes),
            // then dP and dS, so that only one operand half and one product
            // result are live at a time.  Register r is position a + 16g + r;
            // lse * log2(e) and -delta per register belong to the lane's
            // query (query pass) or to the half's queries 16g + r (key pass).
            const lds_t *st = b + MxBuf<D>::kStats + 4 * (a - c0 + 16 * g);
            float p[16];
            {
                i32x8 f1[D / 64];
                int s1[D / 64];
                read_half8<D>(b, b + 64 * D + scale_mis<D>(s, t.h, t.tok0 + c0) + srd, h, rd, f1,
                              s1);
                float l2[16];
                if constexpr (ROLE == 0) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) l2[r] = lse2;
                } else {
#pragma unroll
                    for (int r = 0; r < 16; r += 4) {
                        const f32x4v l4 = *(const __attribute__((address_space(3))) f32x4v *)(
                            st + 4 * r);
#pragma unroll
                        for (int e = 0; e < 4; ++e) l2[r + e] = l4[e];
                    }
                }
                const f32x16 sc = hd_product<D>(f1, s1, fa, sa, f32x16{});
                // (two loops on the wave-uniform flag: the unmasked halves,
                // most of them, carry no visibility test)
                if (masked) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const bool vis = ROLE == 0 ? (uint32_t)(x0 + r) <= span
                                                   : (uint32_t)(x0 + r) < span;
                        p[r] = vis ? __builtin_amdgcn_exp2f(fmaf(sc[r], c, -l2[r])) : 0.f;
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        p[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], c, -l2[r]));
                }
            }
            if constexpr (ROLE == 1) e1[h] = quant_block(p, q1 + 4 * h);
            float ds[16];
            {
                i32x8 f2[D / 64];
                int s2[D / 64];
                read_half8<D>(b + kT, b + kT + 64 * D + scale_mis<D>(s, t.h, t.tok0 + c0) + srd,
                              h, rd, f2, s2);
                f32x16 nd;
                if constexpr (ROLE == 0) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) nd[r] = ndlt;
                } else {
#pragma unroll
                    for (int r = 0; r < 16; r += 4) {
                        const f32x4v d4 = *(const __attribute__((address_space(3))) f32x4v *)(
                            st + 256 + 4 * r);
#pragma unroll
                        for (int e = 0; e < 4; ++e) nd[r + e] = d4[e];
                    }
                }
                const f32x16 dp = hd_product<D>(f2, s2, fb, sb, nd);
#pragma unroll
                for (int r = 0; r < 16; ++r) ds[r] = p[r] * dp[r];
            }
            if constexpr (ROLE == 0)
                e1[h] = quant_block(ds, q1 + 4 * h);
            else
                e2[h] = quant_block(ds, q2 + 4 * h);
        }
        const i32x8 x1 = i32x8{q1[0], q1[1], q1[2], q1[3], q1[4], q1[5], q1[6], q1[7]};
        if constexpr (ROLE == 0) {
            tok_product<D>(b + 2 * kT, rdv, tsrd, x1, g ? e1[1] : e1[0], acc[0]);
        } else {
            const i32x8 x2 = i32x8{q2[0], q2[1], q2[2], q2[3], q2[4], q2[5], q2[6], q2[7]};
            tok_product<D>(b + 3 * kT, rdv, tsrd, x1, g ? e1[1] : e1[0], acc[1]);  // dV += dO_t^T P
            tok_product<D>(b + 2 * kT, rdv, tsrd, x2, g ? e2[1] : e2[0], acc[0]);  // dK += Q_t^T dS
        }
    };
    for (int ci = 0; ci < nch; ci += 2) {
        step(ci, std::integral_constant<int, 0>{});
        if (ci + 1 < nch) step(ci + 1, std::integral_constant<int, 1>{});
    }

    if (!wave_live) return;
    if constexpr (ROLE == 0) {
        store_out<D>(A.dq, s, t, my, row_end, g, acc[0], s.scale);
    } else {
        store_out<D>(A.dk, s, t, my, row_end, g, acc[0], s.scale);
        store_out<D>(A.dv, s, t, my, row_end, g, acc[1], 1.f);
    }
}

template <int D>
hipError_t launch_d(const Shape &s, const MxBwdArgs &a, hipStream_t st) {
    const int64_t grid = grid_upper_bound(s.T, s.batch, kTileRows, 1, s.H);
    auto pass = [&](auto role_c) {
        constexpr int ROLE = decltype(role_c)::value;
        if (s.batch > 4 * kThreads)
            hipLaunchKernelGGL((bwd_mx<D, ROLE, 4>), dim3((unsigned)grid), dim3(kThreads), 0, st,
                               s, a);
        else
            hipLaunchKernelGGL((bwd_mx<D, ROLE, 1>), dim3((unsigned)grid), dim3(kThreads), 0, st,
                               s, a);
    };
    pass(std::integral_constant<int, 0>{});
    pass(std::integral_constant<int, 1>{});
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_bwd_mx(const Shape &s, const MxBwdPtrs &p, void *ws, hipStream_t st) {
    const BwdWorkspace w = bwd_workspace_layout(ws, s.T, s.batch, s.H);
    MxBwdArgs a;
    a.q = (const uint8_t *)p.q;
    a.qsc = (const uint8_t *)p.q_scale;
    a.k = (const uint8_t *)p.k;
    a.ksc = (const uint8_t *)p.k_scale;
    a.v = (const uint8_t *)p.v;
    a.vsc = (const uint8_t *)p.v_scale;
    a.dout = (const uint8_t *)p.dout;
    a.dosc = (const uint8_t *)p.dout_scale;
    a.qt = (const uint8_t *)p.q_t;
    a.qtsc = (const uint8_t *)p.q_t_scale;
    a.kt = (const uint8_t *)p.k_t;
    a.ktsc = (const uint8_t *)p.k_t_scale;
    a.dot = (const uint8_t *)p.dout_t;
    a.dotsc = (const uint8_t *)p.dout_t_scale;
    a.out = (const bf16 *)p.out;
    a.lse = p.lse;
    a.lse2 = w.lse2;
    a.ndlt = w.ndlt;
    a.dq = (bf16 *)p.dq;
    a.dk = (bf16 *)p.dk;
    a.dv = (bf16 *)p.dv;
    switch (s.D) {
    case 64: return launch_d<64>(s, a, st);
    case 128: return launch_d<128>(s, a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace ba
