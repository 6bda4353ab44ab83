// LDS tiles of 64 rows x D bf16 for the MFMA kernels (gfx950).
//
// A tile is filled straight from HBM by buffer loads that write LDS (no
// VGPRs, no VALU): each wave instruction moves 64 lanes x 16 bytes into one
// contiguous KiB of LDS, and every lane picks which 16-byte granule of which
// source row lands in its slot.  That choice gives the tile two properties:
//
//  * Row permutation: physical row p holds source row sigma(p) (sigma swaps
//    bits 2 and 3, see mfma_util.h), so MFMA accumulators computed from the
//    tile's rows come out in register octets of consecutive rows.
//  * Swizzle: granule gr of physical row p sits at granule gr ^ swz(p).  swz
//    is chosen so that the two read patterns below touch distinct banks:
//    16-byte row reads (lanes 0..31 read physical rows 0..31, one granule)
//    and ds_read_b64_tr_b16 transposed reads (each 16-lane group reads 4
//    consecutive rows, 2 neighbouring granules); it holds whether the LDS
//    serves 128 or 256 bytes per clock.
//
// Transposed reads.  ds_read_b64_tr_b16 gives lane i of each 16-lane group,
// as its element j, element i%4 of the 4 bf16 that source lane 4j + i/4
// addressed.  If source lane s addresses row r0 + s/4 at columns
// c(s%4) .. c(s%4)+3, lane i therefore receives column c(i/4) + i%4 of rows
// r0 .. r0+3: the operand layout an MFMA needs when the contraction runs
// along the tile's rows, read from a row-major tile.
#pragma once

#include "mfma_util.h"

namespace ba {

typedef __attribute__((address_space(3))) char lds_t;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// SW = 1: the swizzle of tiles read only by 16-byte row reads, such as fp8
// tiles (which have no transposed reads).  For 64-byte rows (D = 32) it
// takes row bits 2 and 3, so the 16 lanes that one LDS clock serves (rows
// r .. r + 15 at 256 bytes per clock) all hit distinct banks; the SW = 0
// swizzle there also serves the transposed reads, and rows r and r + 8 of
// a 16-row group share banks.  Wider rows are the same for both.
template <int D, int SW = 0>
struct TileGeom {
    static constexpr int kRowBytes = D * 2;
    static constexpr int kBytes = 64 * kRowBytes;
    static constexpr int kDmaPerWave = D / 32;  // 16-byte DMA instructions per wave (4 waves)

    // Granule XOR of physical row p (bits 0..3 of p only).
    __device__ static int swz(int p) {
        if (D == 32 && SW) return (p >> 2) & 3;
        if (D == 32) return (((p >> 1) & 1) << 1) | ((p >> 2) & 1);
        int f = ((p >> 2) & 1) | (((p ^ (p >> 3)) & 1) << 1) | (((p >> 1) & 1) << 2);
        if (D == 128) f |= (p & 1) << 3;
        return f;
    }
    // Byte offset of granule gr of physical row p.
    __device__ static int at(int p, int gr) { return p * kRowBytes + ((gr ^ swz(p)) << 4); }
};

// Per-lane source offsets (bytes from the first source row) of this wave's
// DMA instructions for one tile; rsb = source row stride in bytes.  They do
// not depend on the chunk, so they are computed once per workgroup.
// Physical row p holds source row sigma(p), or rho(p) with RHO.
template <int D, bool RHO = false, int SW = 0>
__device__ __forceinline__ void dma_offsets(uint32_t (&voff)[TileGeom<D>::kDmaPerWave],
                                            int wave, int lane, uint32_t rsb) {
#pragma unroll
    for (int j = 0; j < TileGeom<D>::kDmaPerWave; ++j) {
        const int slot = (wave * TileGeom<D>::kDmaPerWave + j) * 64 + lane;
        const int p = slot / (D / 8), pg = slot % (D / 8);
        const int gr = pg ^ TileGeom<D, SW>::swz(p);
        voff[j] = (uint32_t)(RHO ? rho(p) : sigma(p)) * rsb + (uint32_t)gr * 16u;
    }
}

// Issues this wave's DMA instructions filling `tile` from the rows that the
// descriptor covers (rows past it arrive as zeros).  They are issued from
// inline assembly: the compiler then does not treat them as pending writes to
// every LDS address (which would make it wait for all of them before any LDS
// read), and the kernels wait for them explicitly with wait_vm_barrier.  Any
// wait the compiler inserts for its own loads stays correct, only stricter.
template <int D>
__device__ __forceinline__ void dma_tile(i32x4 desc, lds_t *tile,
                                         const uint32_t (&voff)[TileGeom<D>::kDmaPerWave],
                                         int wave) {
    // The LDS address and the descriptor are wave-uniform; readfirstlane
    // states it, so they are given to the instruction in scalar registers.
    const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)tile);
    desc = i32x4{__builtin_amdgcn_readfirstlane(desc[0]), __builtin_amdgcn_readfirstlane(desc[1]),
                 __builtin_amdgcn_readfirstlane(desc[2]), __builtin_amdgcn_readfirstlane(desc[3])};
#pragma unroll
    for (int j = 0; j < TileGeom<D>::kDmaPerWave; ++j) {
        const uint32_t dst = __builtin_amdgcn_readfirstlane(
            base + (uint32_t)(wave * TileGeom<D>::kDmaPerWave + j) * 1024u);
        asm volatile(
            "s_mov_b32 m0, %0\n\t"
            "s_nop 0\n\t"
            "buffer_load_dwordx4 %1, %2, 0 offen lds"
            :
            : "s"(dst), "v"(voff[j]), "s"(desc)
            : "memory", "m0");
    }
}

// Waits until at most n of this wave's vector memory operations are in
// flight (and all its LDS operations are done), then joins the workgroup
// barrier.  No cache or fence work: DMA writes to LDS are complete once
// counted, and LDS is coherent within the workgroup.
template <int n>
__device__ __forceinline__ void wait_vm_barrier() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | ((n >> 4) << 14));
    asm volatile("s_barrier" ::: "memory");
}

// Offset (bytes) of the 16-byte row read of MFMA operand rows: lane (qi, g)
// reads physical row qi, granule 2ks + g.  Returns the ks = 0 offset; the
// offset for ks is (that ^ (ks << 5)), and rows 32*sub.. add sub*32*kRowBytes.
template <int D, int SW = 0>
__device__ __forceinline__ int row_read_offset(int qi, int g) {
    return TileGeom<D, SW>::at(qi, g);
}

// Offset (bytes) of the transposed reads that give this lane (m = lane%32,
// g = lane/32) the contraction-along-rows operand A[m][k] = tile[logical row
// k][column 32dt + sigma(m)] for k = 8g + 4h .. 8g + 4h + 3; the reads h = 0
// and 1 make one 8-deep operand.  Logical row 8g + 4h + j is physical row
// 8h + 4g + j.  Logical rows 32*sub + 16*kk.. add (32 sub + 16 kk) rows.
template <int D>
__device__ __forceinline__ int tr_read_offset(int lane, int h, int dt) {
    const int G = lane >> 4, s = lane & 15;
    const int g = G >> 1, dhalf = G & 1;
    const int q = ((s & 1) << 1) | ((s >> 1) & 1);  // column quad, bits swapped (sigma)
    const int p = 8 * h + 4 * g + (s >> 2);
    const int col = 32 * dt + 16 * dhalf + 4 * q;
    return TileGeom<D>::at(p, col >> 3) + ((col >> 2) & 1) * 8;
}

// LDS byte address of a pointer into LDS.
__device__ __forceinline__ uint32_t lds_addr_of(const lds_t *p) { return (uint32_t)(uintptr_t)p; }

// One dword per lane from `src` (4-byte aligned; `bytes` valid, the rest
// zero) into LDS at byte address `dst`: 64 lanes x 4 bytes.
__device__ __forceinline__ void dma_dwords_lds(const void *src, uint32_t bytes, uint32_t dst,
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

// The same 64 dwords as dma_dwords_lds, for a window whose last dword would
// pass the end of its tensor: `bytes` (< 256) are valid.  Each lane loads its
// 4 bytes one by one through a range-checked buffer (bytes past the range
// read as zero) and writes the dword to LDS.  The loads are visible to the
// compiler, which waits for them (and for everything issued before them)
// before the write, so this path is for the rare window at a tensor's end.
__device__ __forceinline__ void bytes_to_lds(const void *src, uint32_t bytes, uint32_t dst,
                                             int lane) {
    const auto r = __builtin_amdgcn_make_buffer_rsrc((void *)src, (short)0, bytes, 0x00020000);
    uint32_t w = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b)
        w |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (uint32_t)lane * 4u + b, 0, 0)
             << (8 * b);
    *(__attribute__((address_space(3))) uint32_t *)(uintptr_t)(dst + (uint32_t)lane * 4u) = w;
}

__device__ __forceinline__ bf16x8 lds_read16(const lds_t *p) {
    return *(const __attribute__((address_space(3))) bf16x8 *)p;
}
__device__ __forceinline__ bf16x8 lds_read_tr(const lds_t *p0, const lds_t *p1) {
    const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4 *)p0);
    const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4 *)p1);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

}  // namespace ba
