// Internal launchers of the block-attention kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace ba {

// Scalar FMA path (fp32 storage; bf16_io must be false).  s.act selects the
// score function, as for the MFMA kernels.
hipError_t launch_scalar_fwd(const Shape &s, bool bf16_io, const void *q, const void *k,
                             const void *v, void *out, float *lse, hipStream_t st);
hipError_t launch_scalar_bwd(const Shape &s, bool bf16_io, const void *q, const void *k,
                             const void *v, const void *out, const void *dout,
                             const float *lse, void *dq, void *dk, void *dv, hipStream_t st);

// Rotary embedding of q and k (rotate-half, per-user positions, base
// s.rope_base) into q_rot and k_rot; bf16 or fp32 storage.
hipError_t launch_rope(const Shape &s, bool bf16_io, const void *q, const void *k, void *q_rot,
                       void *k_rot, hipStream_t st);

// bf16 MFMA forward.
hipError_t launch_mfma_fwd(const Shape &s, const void *q, const void *k, const void *v,
                           void *out, float *lse, hipStream_t st);

// Forward with q and k in MXFP8: E4M3 bytes [T, H, D] and E8M0 block scales
// [H, T, D/32]; v, out bf16.  D 64 or 128.
hipError_t launch_mfma_fwd_mx(const Shape &s, const void *q, const void *q_scale, const void *k,
                              const void *k_scale, const void *v, void *out, float *lse,
                              hipStream_t st);

// Forward with q, k and v in MXFP8 and the softmax weights quantized for a
// block-scaled P.V product: q, k as above; v^T E4M3 [H, D, 32 NB] with
// NB = ceil(T/32) + batch, user u's local token j at column
// 32 (ceil(off[u]/32) + u) + j; v scales E8M0 [H, NB, D] (one per 32 tokens
// of a user's column).  D 64 or 128; D * 32 NB < 2^32.
hipError_t launch_mfma_fwd_mxpv(const Shape &s, const void *q, const void *q_scale,
                                const void *k, const void *k_scale, const void *v_t,
                                const void *v_scale, void *out, float *lse, hipStream_t st);

// bf16 MFMA backward.  Workspace (caller-owned device memory, 256-byte
// aligned): per-(head, token) row statistics lse * log2(e) and -delta, which
// the query pass writes for the key pass, a
// 256-byte block of counters (the tile queues of the query and key passes,
// the tile count), per-user tile prefix sums, and the tile table.  Each
// region starts on a 256-byte boundary.
constexpr int kBwdTileRows = 128;

inline int64_t bwd_max_tiles(int64_t T, int batch, int H) {
    // sum over users of ceil(L_u / 128) <= ceil(T / 128) + batch, x 2 roles
    return ((T + kBwdTileRows - 1) / kBwdTileRows + batch) * 2 * (int64_t)H;
}

struct BwdWorkspace {
    float *lse2, *ndlt;
    int *ctr, *ubase;
    int4 *table;
};

inline size_t ws_align(size_t x) { return (x + 255) / 256 * 256; }

inline size_t bwd_workspace_bytes(int64_t T, int batch, int H) {
    return 2 * ws_align((size_t)H * (size_t)T * sizeof(float)) + 256 +
           ws_align(((size_t)batch + 1) * sizeof(int)) +
           ws_align((size_t)bwd_max_tiles(T, batch, H) * 16);
}

inline BwdWorkspace bwd_workspace_layout(void *ws, int64_t T, int batch, int H) {
    char *p = (char *)ws;
    BwdWorkspace w;
    const size_t stat = ws_align((size_t)H * (size_t)T * sizeof(float));
    w.lse2 = (float *)p;
    w.ndlt = (float *)(p + stat);
    w.ctr = (int *)(p + 2 * stat);
    w.ubase = (int *)(p + 2 * stat + 256);
    w.table = (int4 *)(p + 2 * stat + 256 + ws_align(((size_t)batch + 1) * sizeof(int)));
    return w;
}

hipError_t launch_mfma_bwd(const Shape &s, const void *q, const void *k, const void *v,
                           const void *out, const void *dout, const float *lse, void *dq,
                           void *dk, void *dv, void *ws, hipStream_t st);

// MXFP8 backward (softmax): q, k, v, dout head-dim-blocked as for
// launch_mfma_fwd_mx; q_t, k_t, dout_t token-blocked and transposed as v_t
// for launch_mfma_fwd_mxpv; out bf16 and lse fp32 from the forward; dq, dk,
// dv bf16 [T, H, D].  Workspace as for launch_mfma_bwd (only its two row
// statistic regions are used).  D 64 or 128.
struct MxBwdPtrs {
    const void *q, *q_scale, *k, *k_scale, *v, *v_scale, *dout, *dout_scale;
    const void *q_t, *q_t_scale, *k_t, *k_t_scale, *dout_t, *dout_t_scale;
    const void *out;
    const float *lse;
    void *dq, *dk, *dv;
};
hipError_t launch_mfma_bwd_mx(const Shape &s, const MxBwdPtrs &p, void *ws, hipStream_t st);

}  // namespace ba
