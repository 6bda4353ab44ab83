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
// SIMD).  Every row carries its own window start, so any B >= 1 works.
// Keys are streamed in chunks of 64 from the window
// start of the tile's first row.  Each chunk's K and V rows go from HBM
// straight into LDS tiles (lds_tile.h) through buffer loads sized to the
// chunk's valid rows (keys past the tile's last row arrive as zeros); NB
// tiles rotate so that the loads of the next NB-1 chunks are in flight while
// one is computed, with one barrier per chunk.
//
// Per chunk and wave, with 32x32x16 bf16 MFMAs and fp32 accumulation:
//   S^T = K Q^T   (K rows from LDS, Q^T held in registers for the whole tile)
//   mask (causal, window) only on the sub-tiles that straddle a boundary
//   online softmax in the base-2 domain; each lane owns one query, so the
//   row max needs one lane^32 exchange and the row sum none until the end;
//   a row's running max is only moved when it grows by more than 2^8
//   O^T += V^T P^T (V^T by transposed LDS reads, P^T straight from the S^T
//   accumulators)
//
// Lane layouts of v_mfma_f32_32x32x16_bf16 (g = lane/32, i = 0..7):
//   A[m][k]: lane holds A[lane%32][8g + i];  B[k][n]: lane holds B[8g + i][lane%32]
//   C[m][n]: lane, register r holds C[8(r/4) + 4g + r%4][lane%32].
// K rows sit at LDS row sigma(m) (sigma swaps bits 2 and 3), which makes C
// register r of lane (g) hold key 16(r/8) + 8g + r%8: registers 0..7 and
// 8..15 are then exactly the B operands of the two 16-key PV products.  The
// transposed V reads take head-dim column sigma(m) for operand row m, so each
// lane ends with 8 consecutive output columns per register octet.
#include "kernels.h"
#include "lds_tile.h"

namespace ba {
namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kTileRows = 128;
constexpr int kKC = 64;        // keys per staged chunk

// LDS tiles in rotation (two: a small footprint lets more workgroups share a
// CU, which hides more latency than a deeper prefetch), and waves per SIMD the
// register budget is sized for (at D = 128 the quantized-weights variant
// fits three: it keeps one half-chunk's scores live at a time and its chunk
// buffers are half the bf16 size).
template <int D>
constexpr int kBufs = 2;
template <int D, int MX = 0>
constexpr int kWavesPerSimd = D == 128 ? (MX == 2 ? 3 : 2) : 4;

template <int D>
struct FwdChunk {
    bf16 k[kKC * D];
    bf16 v[kKC * D];
};

// MX: q and k are MXFP8 (E4M3 bytes [T, H, D], E8M0 block scales [H, T,
// D/32], one per 32 head-dim elements) and the scores come from the
// block-scaled fp8 products (v_mfma_scale_f32_32x32x64_f8f6f4: 64 head-dim
// elements, i.e. two scale blocks, per product).  Its operand layout, from
// an in-bounds probe on gfx950: lane (m, g) holds 16 bytes of each of the
// two blocks, and the scale of (row m, block j) comes from lane m + 32j.
// Those 16-byte reads are exactly the granule reads of a bf16 tile of D/2
// columns, so the fp8 K tile uses that geometry, with the swizzle of tiles
// read only by row reads (lds_tile.h, SW = 1).
//
// MX = 2 takes v in MXFP8 too and quantizes the softmax weights for a
// block-scaled P.V product ("GEM (Meta)", sections "Custom kernels" and
// "Ultra-low-precision training": MXFP8 block-scaled matmuls end to end).
// v arrives transposed and blocked by user: E4M3 [H, D, 32 NB] with
// NB = ceil(T/32) + batch, user u's local token j at column 32 ub + j with
// ub = ceil(off[u] / 32) + u (so users never share a 32-token block), and
// E8M0 scales [H, NB, D], one per 32 tokens of a user's column: the scales
// run along the P.V contraction.  Chunks then start on a multiple of 32
// local tokens (keys before the window are masked), so each 32-key half of
// a chunk is one scale block of v and of the weights, and one 32x32x64
// product takes a whole chunk.  K
// rows sit at LDS row rho(m) (mfma_util.h), so a lane's 16 score registers
// of a half are keys 16g .. 16g + 15: in register order they are the
// lane's bytes of the weights' operand.  v^T rows are plain 16-byte row
// reads of a tile with 64-byte rows.  The running max m is kept as a whole
// number in the log2 domain, so a rescale is an exact power of two and a
// weight's code depends only on its own block: with F = floor(block max of
// s c), the weight p = 2^(s c - m) is stored as 2^(F - 7 - m) times the
// nearest E4M3 value of p 2^(m - F + 7) = 2^(s c - F + 7) < 2^8.  The row
// sum and lse use the unquantized weights.  The two halves of a chunk are
// worked through in turn (one half's scores live at a time); a rescale
// between them moves the first half's block exponent, not its codes.
//
// UPT: users per thread in each pass of the tile decode (4 for batches above
// 1024 users, chosen by the host, which knows the batch size).
template <int D, int ACT, int MX, int UPT>
__global__ __launch_bounds__(kThreads, (kWavesPerSimd<D, MX>)) void fwd_mfma(
    Shape s, const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    bf16 *__restrict__ out, float *__restrict__ lse, const uint8_t *__restrict__ qsc,
    const uint8_t *__restrict__ ksc, const uint8_t *__restrict__ vsc) {
    using G = TileGeom<D>;
    using G8 = TileGeom<(D >= 64 ? D / 2 : 32), 1>;  // an fp8 row of D bytes
    constexpr int NB = kBufs<D>;
    constexpr int kDma = 2 * G::kDmaPerWave;  // DMA instructions per wave per chunk
    __shared__ int sh[8];
    // chunk buffers: K then V tiles (MX = 2: the fp8 K tile, its scales, the
    // fp8 v^T tile at kVOff, its scales; half the bf16 footprint)
    constexpr int kBuf = MX == 2 ? 128 * D + 2048 : (int)sizeof(FwdChunk<D>);
    constexpr int kVOff = MX == 2 ? 64 * D + 1024 : G::kBytes;
    __shared__ __align__(1024) unsigned char sm[NB * kBuf];
    Tile t;
    if (!decode_tile<kThreads, UPT>(s, kTileRows, 1, t, sh)) return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int w = (wave + t.blk) & 3;  // row group of this wave
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
    // (the activation variants take the signed scale instead)
    const uint32_t qsign = MX ? (s.scale < 0.f ? 0x80808080u : 0u)
                              : (ACT == kSoftmax && s.scale < 0.f ? 0x80008000u : 0u);

    const int kwin = window_start(row0, s.B, s.W);
    // (MX = 2: back to a multiple of 32 local tokens)
    const int kbeg = MX == 2 ? kwin - (kwin & 31) : kwin;
    const int nch = (row_end - kbeg + kKC - 1) / kKC;
    // fp8 rows are addressed in bf16 units (half their byte offsets)
    const int64_t rs8 = rs / 2;
    const bf16 *kb = MX ? k + (t.tok0 + kbeg) * rs8 + (int64_t)t.h * (D / 2)
                        : k + base + (int64_t)kbeg * rs;
    const bf16 *vb = v + base + (int64_t)kbeg * rs;
    // byte offset of the first K scale of the tile, [H, T, D/32] layout
    const int64_t ks0 = ((int64_t)t.h * s.T + t.tok0 + kbeg) * (D / 32);
    lds_t *lds = (lds_t *)sm;
    uint32_t voff[G::kDmaPerWave];
    dma_offsets<D>(voff, wave, lane, rsb);
    uint32_t voff8[G8::kDmaPerWave];
    if constexpr (MX)
        dma_offsets<G8::kRowBytes / 2, MX == 2, 1>(voff8, wave, lane, (uint32_t)(rs8 * 2));
    // MX = 2: v^T rows of this head from the tile's first key (byte
    // offsets; the user's columns start at 32 ub), and their scales
    const int64_t nblk = (s.T + 31) / 32 + s.batch, Tp = 32 * nblk;
    const int64_t ub = (t.tok0 + 31) / 32 + t.user;
    const int64_t vb8 = (int64_t)t.h * D * Tp + 32 * ub + kbeg;
    const int64_t vs0 = ((int64_t)t.h * nblk + ub + kbeg / 32) * D;
    uint32_t voffv[1];
    if constexpr (MX == 2) dma_offsets<32, false, 1>(voffv, wave, lane, (uint32_t)Tp);
    // Scales of chunk ci: a dword-aligned window starts `mis` bytes before
    // them and lands in LDS after the fp8 K tile.
    auto scale_mis = [&](int ci) { return (int)((ks0 + (int64_t)ci * kKC * (D / 32)) & 3); };
    auto issue = [&](int ci, int buf) {
        const int off = ci * kKC, rows = min(kKC, row_end - kbeg - off);
        lds_t *b = lds + buf * kBuf;
        if constexpr (MX) {
            dma_tile<G8::kRowBytes / 2>(row_desc<G8::kRowBytes / 2>(kb + off * rs8, rows, rs8), b,
                                        voff8, wave);
            if (wave == 0) {
                const uint8_t *sp = ksc + ks0 + (int64_t)off * (D / 32);
                const int mis = scale_mis(ci);
                const uint32_t nb = (uint32_t)(rows * (D / 32) + mis);
                // The dword window ends at most 3 bytes past the chunk's last
                // scale; only on the last head can that pass the tensor's
                // end, and then the window is read byte by byte instead.
                const int64_t wbeg = ks0 + (int64_t)off * (D / 32) - mis;
                const int64_t total = (int64_t)s.H * s.T * (D / 32);
                if (wbeg + ((nb + 3) & ~3u) <= total)
                    dma_dwords_lds(sp - mis, (nb + 3) & ~3u, lds_addr_of(b + kKC * D), lane);
                else
                    bytes_to_lds(sp - mis, (uint32_t)(total - wbeg), lds_addr_of(b + kKC * D),
                                 lane);
            }
        } else {
            dma_tile<D>(row_desc<D>(kb + off * rs, rows, rs), b, voff, wave);
        }
        if constexpr (MX == 2) {
            // v^T: D rows of 64 key bytes (64-row tiles of 64-byte rows),
            // ranges ending at the tensor's end; and the chunk's 2 x D
            // scales (wave 1)
            const int64_t vtot = (int64_t)s.H * D * Tp;
#pragma unroll
            for (int j = 0; j < D / 64; ++j) {
                const int64_t o = vb8 + off + (int64_t)j * 64 * Tp;
                const uint64_t a = (uint64_t)((const uint8_t *)v + o);
                const uint32_t range = (uint32_t)min(63 * Tp + 64, vtot - o);
                dma_tile<32>(i32x4{(int)(uint32_t)a, (int)((a >> 32) & 0xffffu), (int)range,
                                   0x00020000},
                             b + kVOff + j * 4096, voffv, wave);
            }
            if (wave == 1) {
                const int64_t so = vs0 + (int64_t)(off / 32) * D;
                const uint32_t nb = (uint32_t)min((int64_t)2 * D, (int64_t)s.H * nblk * D - so);
                dma_dwords_lds(vsc + so, nb, lds_addr_of(b + kVOff + 64 * D), lane);
            }
        } else {
            dma_tile<D>(row_desc<D>(vb + off * rs, rows, rs), b + G::kBytes, voff, wave);
        }
    };

    if (nch > 0) issue(0, 0);
    bf16x8 qreg[MX ? 1 : D / 16];
    i32x8 qf8[D >= 64 ? D / 64 : 1];
    int qs8[D >= 64 ? D / 64 : 1];
    if constexpr (MX) {
        // lane (row, g): bytes 64i + 16g .. and 64i + 32 + 16g .. of its row,
        // and the scale of block 2i + g
        const uint8_t *qrow = (const uint8_t *)q + ((t.tok0 + my_row) * rs8 * 2 + (int64_t)t.h * D);
        const uint8_t *srow = qsc + ((int64_t)t.h * s.T + t.tok0 + my_row) * (D / 32);
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
            uint4 lo = make_uint4(0u, 0u, 0u, 0u), hi = lo;
            int sc8 = 127;
            if (my_row < row_end) {
                lo = *(const uint4 *)(qrow + 64 * i + 16 * g);
                hi = *(const uint4 *)(qrow + 64 * i + 32 + 16 * g);
                sc8 = srow[2 * i + g];
            }
            qf8[i] = i32x8{(int)(lo.x ^ qsign), (int)(lo.y ^ qsign), (int)(lo.z ^ qsign),
                           (int)(lo.w ^ qsign), (int)(hi.x ^ qsign), (int)(hi.y ^ qsign),
                           (int)(hi.z ^ qsign), (int)(hi.w ^ qsign)};
            qs8[i] = sc8;
        }
    } else {
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
    // Q (and chunk 0) complete here, so inside the chunk loop the only vector
    // memory operations in flight are the tile loads that the loop waits for
    // itself.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    if (NB == 3 && nch > 1) issue(1, 1);

    // Per-lane LDS read offsets inside a chunk tile (loop-invariant): the
    // chunk, sub-tile and 16-key offsets are added as immediates.
    int rd[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
        rd[ks] = MX ? row_read_offset<G8::kRowBytes / 2, 1>(qi, g) ^ (ks << 5)
                    : row_read_offset<D>(qi, g) ^ (ks << 5);
    // MX: byte offset of the lane's key row in the chunk's scale window
    // (physical row m of the tile holds key sigma(m), or rho(m) for MX = 2)
    const int srd = (MX == 2 ? rho32(qi) : sigma32(qi)) * (D / 32);
    // MX = 2: the lane's v^T row read (physical row qi, granule g of each
    // 32-key block) and its scale byte (head-dim column sigma(qi) of
    // block g)
    const int rdv = row_read_offset<32, 1>(qi, g);
    const int vsrd = g * D + sigma32(qi);
    int trd[2][D / 32];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) trd[h][dt] = tr_read_offset<D>(lane, h, dt);

    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
    // running max (MX = 2: in the log2 domain, a whole number) and the
    // lane's share of the row sum
    float m = -INFINITY, l = 0.f;

    // One chunk held in tile `buf` (a constant, so LDS offsets fold into
    // instruction immediates).
    auto step = [&](int ci, auto buf_c) {
        constexpr int buf = decltype(buf_c)::value;
        if (NB == 3 && ci + 1 < nch)
            wait_vm_barrier<(NB == 3 ? kDma : 0)>();
        else
            wait_vm_barrier<0>();
        if (ci + NB - 1 < nch) issue(ci + NB - 1, (buf + NB - 1) % NB);
        if (!wave_live) return;
        const lds_t *kt = lds + buf * kBuf;
        const lds_t *vt = kt + kVOff;
        const int c0 = kbeg + ci * kKC;
        if constexpr (MX == 2) {
            // halves h = 0, 1: keys c0 + 32h .. c0 + 32h + 31
            const bool live0 = c0 <= w_last && c0 + 31 >= wave_klo;
            const bool live1 = c0 + 32 <= w_last && c0 + 63 >= wave_klo;
            if (!live0 && !live1) return;
            // Each half in turn: scores (register r of lane group g is key
            // a + 16g + r), masked; the running max; weights, their fp32
            // sum, and the E4M3 codes of p 2^-E with
            // E = floor(block max s c) - 7 - m (at most 1; at least -127,
            // the scale's range: weights below 2^-119 of the row's max).
            // The lazy rescale moves m to ceil(max s c) once a score passes
            // m + 8: a whole power of two, so it is exact, and the first
            // half's codes keep their values through its block exponent.
            i32x8 pf8;
            int e8[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int a = c0 + h * 32;
                f32x16 x;
                float bm = -INFINITY;
                if (h ? live1 : live0) {
                    const lds_t *k8 = kt + h * 32 * G8::kRowBytes;
                    const lds_t *sp = kt + kKC * D + scale_mis(ci) + h * 32 * (D / 32) + srd + g;
                    i32x8 kf[D / 64];
                    int ksc8[D / 64];
#pragma unroll
                    for (int i = 0; i < D / 64; ++i) {
                        const uint4 lo = __builtin_bit_cast(uint4, lds_read16(k8 + rd[2 * i]));
                        const uint4 hi = __builtin_bit_cast(uint4, lds_read16(k8 + rd[2 * i + 1]));
                        kf[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                      (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                        ksc8[i] = *(const __attribute__((address_space(3))) uint8_t *)(sp + 2 * i);
                    }
                    x = f32x16{};
#pragma unroll
                    for (int i = 0; i < D / 64; ++i)
                        x = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf[i], qf8[i], x, 0,
                                                                           0, 0, ksc8[i], 0,
                                                                           qs8[i]);
                    if (a + 31 > wr0 || a < wave_klo_max) {
                        const int x0 = a + 16 * g - my_klo;
                        const uint32_t span = (uint32_t)(my_row - my_klo);
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            if ((uint32_t)(x0 + r) > span) x[r] = -INFINITY;
                    }
                    float mh = x[0];
#pragma unroll
                    for (int r = 1; r < 16; ++r) mh = fmaxf(mh, x[r]);
                    bm = swap_max(mh);
                }
                const bool grow = bm * c > m + 8.f;
                if (__builtin_amdgcn_ballot_w64(grow)) {
                    const float mn = grow ? ceilf(bm * c) : m;
                    const int shift = m == -INFINITY ? -1000 : (int)(m - mn);  // <= 0
                    m = mn;
                    const float alpha = ldexpf(1.f, shift);
                    l *= alpha;
#pragma unroll
                    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
                    if (h == 1) {
                        // the first half's block exponent moves with m (its
                        // weights drop below the scale's range only when
                        // they are below 2^-119 of the row's max)
                        e8[0] += shift;
                        if (e8[0] < 0) {
                            e8[0] = 0;
#pragma unroll
                            for (int j = 0; j < 4; ++j) pf8[j] = 0;
                        }
                    }
                }
                const int E = bm == -INFINITY ? -127 : (int)fmaxf(floorf(bm * c) - 7.f - m, -127.f);
                // the scaled conversion divides by 2 to the power of its scale
                // operand's exponent field: 2^E as a bit pattern
                const float esc = __uint_as_float((uint32_t)(E + 127) << 23);
                e8[h] = E + 127;
                // (this half's weights join l before the next half can
                // rescale it)
                float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    int w = 0;
                    if (bm != -INFINITY) {  // (uniform per lane pair; m is finite here)
                        float p[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            p[i] = __builtin_amdgcn_exp2f(fmaf(x[4 * j + i], c, -m));
                            ls[i] += p[i];
                        }
                        i16x2 cv = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(
                            i16x2{0, 0}, p[0], p[1], esc, false);
                        cv = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(cv, p[2], p[3], esc, true);
                        w = __builtin_bit_cast(int, cv);
                    }
                    pf8[4 * h + j] = w;
                }
                l += (ls[0] + ls[1]) + (ls[2] + ls[3]);
            }
            const int ps8 = g ? e8[1] : e8[0];  // the scale of (query, block g)
            // v^T operands and scales, each read just before its product
            // (fewer registers live across the chunk)
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                const int tb = (dt >> 1) * 4096 + (dt & 1) * 2048;
                const uint4 lo = __builtin_bit_cast(uint4, lds_read16(vt + tb + rdv));
                const uint4 hi = __builtin_bit_cast(uint4, lds_read16(vt + tb + (rdv ^ 32)));
                const i32x8 va = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                const int vs8 = *(const __attribute__((address_space(3))) uint8_t *)(
                    vt + 64 * D + vsrd + 32 * dt);
                acc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pf8, acc[dt], 0, 0,
                                                                         0, vs8, 0, ps8);
            }
            return;
        }
        // Softmax and P.V of the sub-tile `sub` (first key a) whose scores
        // are in sc.  The V reads go first so that their latency hides under
        // the vector work.
        auto finish = [&](f32x16 sc, int sub, int a) {
            bf16x8 vtr[2][D / 32];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const lds_t *vr = vt + (sub * 32 + kk * 16) * G::kRowBytes;
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
                    vtr[kk][dt] = lds_read_tr(vr + trd[0][dt], vr + trd[1][dt]);
            }
            if constexpr (ACT != kSoftmax) {
                // P = act(scale s), zero outside the window; no normalisation
                float pv[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) pv[r] = act_value<ACT>(sc[r] * s.scale);
                if (a + 31 > wr0 || a < wave_klo_max) {
                    const int x = a + 8 * g - my_klo;
                    const uint32_t span = (uint32_t)(my_row - my_klo);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if ((uint32_t)(x + 16 * (r >> 3) + (r & 7)) > span) pv[r] = 0.f;
                }
                bf16x8 pa[2];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int r = 2 * j;
                    const bf16x2 p2 = pack_bf16(pv[r], pv[r + 1]);
                    pa[r >> 3][r & 7] = p2[0];
                    pa[r >> 3][(r & 7) + 1] = p2[1];
                }
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int dt = 0; dt < D / 32; ++dt)
                        acc[dt] = mfma32(vtr[kk][dt], pa[kk], acc[dt]);
                return;
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
            // The row sum stays in fp32 (four partial sums): a sum of the
            // bf16-rounded weights would move lse by up to 2^-9 on rows that
            // see few keys.
            bf16x8 pb[2];
            float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int r = 2 * j;
                const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[r], c, -mc));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[r + 1], c, -mc));
                ls[j & 3] += p0 + p1;
                const bf16x2 p2 = pack_bf16(p0, p1);
                pb[r >> 3][r & 7] = p2[0];
                pb[r >> 3][(r & 7) + 1] = p2[1];
            }
            l += (ls[0] + ls[1]) + (ls[2] + ls[3]);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) acc[dt] = mfma32(vtr[kk][dt], pb[kk], acc[dt]);
        };
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int a = c0 + sub * 32;
            if (!(a <= w_last && a + 31 >= wave_klo)) continue;
            f32x16 sc;
            if constexpr (MX) {
                // fp8 K rows and their scales, then the block-scaled products
                const lds_t *k8 = kt + sub * 32 * G8::kRowBytes;
                const lds_t *sp = kt + kKC * D + scale_mis(ci) + sub * 32 * (D / 32) + srd + g;
                i32x8 kf[D / 64];
                int ksc8[D / 64];
#pragma unroll
                for (int i = 0; i < D / 64; ++i) {
                    const uint4 lo = __builtin_bit_cast(uint4, lds_read16(k8 + rd[2 * i]));
                    const uint4 hi = __builtin_bit_cast(uint4, lds_read16(k8 + rd[2 * i + 1]));
                    kf[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                  (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                    ksc8[i] = *(const __attribute__((address_space(3))) uint8_t *)(sp + 2 * i);
                }
                sc = f32x16{};
#pragma unroll
                for (int i = 0; i < D / 64; ++i)
                    sc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf[i], qf8[i], sc, 0, 0,
                                                                        0, ksc8[i], 0, qs8[i]);
            } else {
                // All K reads of the sub-tile first, then the S products.
                bf16x8 ka[D / 16];
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks)
                    ka[ks] = lds_read16(kt + sub * 32 * G::kRowBytes + rd[ks]);
                sc = mfma32(ka[0], qreg[0], f32x16{});
#pragma unroll
                for (int ks = 1; ks < D / 16; ++ks) sc = mfma32(ka[ks], qreg[ks], sc);
            }
            finish(sc, sub, a);
        }
    };
    for (int ci = 0; ci < nch; ci += NB) {
        step(ci, std::integral_constant<int, 0>{});
        if (ci + 1 < nch) step(ci + 1, std::integral_constant<int, 1>{});
        if (NB == 3 && ci + 2 < nch) step(ci + 2, std::integral_constant<int, (NB == 3 ? 2 : 0)>{});
    }

    const float lt = swap_sum(l);
    if (!wave_live || my_row >= row_end) return;
    const float inv = ACT == kSoftmax ? 1.f / lt : 1.f;
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
    if (ACT == kSoftmax && g == 0)
        lse[(int64_t)t.h * s.T + t.tok0 + my_row] = ((MX == 2 ? m : m * c) + log2f(lt)) * kLn2;
}

template <int D, int ACT, int MX = 0>
hipError_t launch_act(const Shape &s, const void *q, const void *k, const void *v, void *out,
                      float *lse, hipStream_t st, const uint8_t *qsc = nullptr,
                      const uint8_t *ksc = nullptr, const uint8_t *vsc = nullptr) {
    const int64_t grid = grid_upper_bound(s.T, s.batch, kTileRows, 1, s.H);
    // one pass of 256 users per thread-scan is fastest up to 1024 users; four
    // users per thread and pass beyond that
    if (s.batch > 4 * kThreads)
        hipLaunchKernelGGL((fwd_mfma<D, ACT, MX, 4>), dim3((unsigned)grid), dim3(kThreads), 0, st,
                           s, (const bf16 *)q, (const bf16 *)k, (const bf16 *)v, (bf16 *)out, lse,
                           qsc, ksc, vsc);
    else
        hipLaunchKernelGGL((fwd_mfma<D, ACT, MX, 1>), dim3((unsigned)grid), dim3(kThreads), 0, st,
                           s, (const bf16 *)q, (const bf16 *)k, (const bf16 *)v, (bf16 *)out, lse,
                           qsc, ksc, vsc);
    return hipGetLastError();
}

template <int D>
hipError_t launch_t(const Shape &s, const void *q, const void *k, const void *v, void *out,
                    float *lse, hipStream_t st) {
    switch (s.act) {
    case kSoftmax: return launch_act<D, kSoftmax>(s, q, k, v, out, lse, st);
    case kSilu: return launch_act<D, kSilu>(s, q, k, v, out, lse, st);
    case kGelu: return launch_act<D, kGelu>(s, q, k, v, out, lse, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_mfma_fwd_mx(const Shape &s, const void *q, const void *q_scale, const void *k,
                              const void *k_scale, const void *v, void *out, float *lse,
                              hipStream_t st) {
    const uint8_t *qs = (const uint8_t *)q_scale, *ks = (const uint8_t *)k_scale;
    switch (s.D) {
    case 64: return launch_act<64, kSoftmax, 1>(s, q, k, v, out, lse, st, qs, ks);
    case 128: return launch_act<128, kSoftmax, 1>(s, q, k, v, out, lse, st, qs, ks);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_mfma_fwd_mxpv(const Shape &s, const void *q, const void *q_scale,
                                const void *k, const void *k_scale, const void *v_t,
                                const void *v_scale, void *out, float *lse, hipStream_t st) {
    const uint8_t *qs = (const uint8_t *)q_scale, *ks = (const uint8_t *)k_scale;
    const uint8_t *vs = (const uint8_t *)v_scale;
    switch (s.D) {
    case 64: return launch_act<64, kSoftmax, 2>(s, q, k, v_t, out, lse, st, qs, ks, vs);
    case 128: return launch_act<128, kSoftmax, 2>(s, q, k, v_t, out, lse, st, qs, ks, vs);
    }
    return hipErrorInvalidValue;
}

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
