// C ABI of the block-attention library: argument checks, then dispatch to
// the HIP kernels.  The operation, layouts and error rules are documented in
// include/blockattn.h.
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "blockattn.h"
#include "common.h"
#include "kernels.h"

static_assert(BLOCKATTN_GDPA_SILU == ba::kSilu && BLOCKATTN_GDPA_GELU == ba::kGelu,
              "activation codes of the ABI and the kernels agree");

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Checks shared by the forward and backward entry points.  Returns OK when
// the call is valid and has work to do, OK with *empty set when it is valid
// and empty, or an error code.  B and W are normalised in place: a block of
// B >= T tokens holds any user whole, as one of T tokens does, and a window
// of W >= ceil(T/B) blocks covers any user's whole past, as ceil(T/B) does,
// so clamping both to those values changes no result and keeps every index
// the kernels derive from them (W * B <= 2T) far from overflow.
blockattn_status check_common(const int32_t *offsets, int32_t batch, int64_t T,
                              int32_t H, int32_t D, int32_t *B, int32_t *W, float scale,
                              blockattn_dtype dtype, bool *empty) {
    *empty = false;
    if (batch < 0 || T < 0 || H < 1 || *B < 1 || *W < 1 || !isfinite(scale))
        return BLOCKATTN_ERR_INVALID_ARGUMENT;
    if (dtype != BLOCKATTN_BF16 && dtype != BLOCKATTN_FP32)
        return BLOCKATTN_ERR_INVALID_ARGUMENT;
    if (D != 32 && D != 64 && D != 128) return BLOCKATTN_ERR_UNSUPPORTED;
    if (T > (int64_t)INT32_MAX - 1024) return BLOCKATTN_ERR_UNSUPPORTED;
    // 32-bit byte offsets within a 128-row tile: 128 rows of H * D elements
    // (at most 4 bytes each) must span less than 4 GiB
    if ((int64_t)128 * H * D * 4 >= ((int64_t)1 << 32)) return BLOCKATTN_ERR_UNSUPPORTED;
    if (T > 0) {
        if (*B > T) *B = (int32_t)T;
        const int64_t nb = (T + *B - 1) / *B;
        if (*W > nb) *W = (int32_t)nb;
    }
    // the largest grid is the fp32 backward's: 2 * ceil(B/64) row tiles per
    // block, at most ceil(T/B) + batch blocks, times H
    const int64_t tiles =
        ((T + *B - 1) / *B + batch) * 2 * (((int64_t)*B + 63) / 64) * (int64_t)H;
    if (tiles > (int64_t)INT32_MAX - 1024) return BLOCKATTN_ERR_UNSUPPORTED;
    // and the backward's tile table by (ceil(T/128) + batch) * 2 * H
    if (ba::bwd_max_tiles(T, batch, H) > (int64_t)INT32_MAX - 1024)
        return BLOCKATTN_ERR_UNSUPPORTED;
    if (T == 0 || batch == 0) {
        *empty = true;
        return BLOCKATTN_OK;
    }
    if (!offsets) return BLOCKATTN_ERR_INVALID_ARGUMENT;
    return BLOCKATTN_OK;
}

ba::Shape make_shape(const int32_t *offsets, int32_t batch, int64_t T, int32_t H, int32_t D,
                     int32_t B, int32_t W, float scale) {
    ba::Shape s;
    s.offsets = offsets;
    s.batch = batch;
    s.T = T;
    s.H = H;
    s.D = D;
    s.B = B;
    s.W = W;
    s.scale = scale;
    s.rope_base = 0.f;
    s.act = ba::kSoftmax;
    return s;
}

// The forward entry points: block attention (act kSoftmax, writes lse) or
// its activation variants (no lse).
blockattn_status forward(const void *q, const void *k, const void *v, const int32_t *offsets,
                         int32_t batch, int64_t total_tokens, int32_t num_heads,
                         int32_t head_dim, int32_t block_size, int32_t window_blocks,
                         float scale, int act, blockattn_dtype dtype, void *out, float *lse,
                         hipStream_t stream) {
    bool empty;
    blockattn_status st = check_common(offsets, batch, total_tokens, num_heads, head_dim,
                                       &block_size, &window_blocks, scale, dtype, &empty);
    if (st != BLOCKATTN_OK || empty) return st;
    const bool stats = act == ba::kSoftmax;
    if (!q || !k || !v || !out || (stats && !lse)) return BLOCKATTN_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        (stats && !aligned16(lse)))
        return BLOCKATTN_ERR_INVALID_ARGUMENT;
    ba::Shape s = make_shape(offsets, batch, total_tokens, num_heads, head_dim, block_size,
                             window_blocks, scale);
    s.act = act;
    hipError_t e = dtype == BLOCKATTN_BF16
                       ? ba::launch_mfma_fwd(s, q, k, v, out, lse, stream)
                       : ba::launch_scalar_fwd(s, false, q, k, v, out, lse, stream);
    return e == hipSuccess ? BLOCKATTN_OK : BLOCKATTN_ERR_HIP;
}

// The workspace of blockattn_bwd_noalloc: a static device array, one copy per
// GPU, created by the runtime with this file's code object.  Host code never
// uses its name as an address (on the host it is a stand-in, not device
// memory): scratch_address() looks up the device address once per device.
static __device__ __align__(256) unsigned char scratch[BLOCKATTN_NOALLOC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device (null if it cannot be
// obtained), looked up with that device current on its first use and kept.
void *scratch_address() {
    static std::atomic<void *> addr[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = addr[dev].load(std::memory_order_acquire);
    if (p) return p;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev].store(p, std::memory_order_release);
    return p;
}

// The backward entry points: plain (rope_base 0) or through a rotary
// embedding of q and k (rope_base > 0, q and k already rotated).  noalloc:
// the workspace is the static array above (workspace and workspace_bytes
// are ignored), looked up only once the arguments have passed their checks.
blockattn_status backward(const void *q, const void *k, const void *v, const void *out,
                          const void *dout, const float *lse, const int32_t *offsets,
                          int32_t batch, int64_t total_tokens, int32_t num_heads,
                          int32_t head_dim, int32_t block_size, int32_t window_blocks,
                          float scale, float rope_base, int act, blockattn_dtype dtype,
                          void *dq, void *dk, void *dv, void *workspace,
                          size_t workspace_bytes, hipStream_t stream, bool noalloc = false) {
    bool empty;
    blockattn_status st = check_common(offsets, batch, total_tokens, num_heads, head_dim,
                                       &block_size, &window_blocks, scale, dtype, &empty);
    if (st != BLOCKATTN_OK || empty) return st;
    const bool stats = act == ba::kSoftmax;  // out and lse enter only the softmax
    if (!q || !k || !v || !dout || !dq || !dk || !dv || (stats && (!out || !lse)))
        return BLOCKATTN_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) ||
        !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
        (stats && (!aligned16(out) || !aligned16(lse))))
        return BLOCKATTN_ERR_INVALID_ARGUMENT;
    const size_t need = blockattn_bwd_workspace_size(total_tokens, batch, num_heads, dtype);
    if (noalloc) {
        workspace = nullptr;
        workspace_bytes = 0;
        if (need > 0 && need <= BLOCKATTN_NOALLOC_WORKSPACE_BYTES) {
            workspace = scratch_address();
            if (!workspace) return BLOCKATTN_ERR_HIP;
            workspace_bytes = BLOCKATTN_NOALLOC_WORKSPACE_BYTES;
        }
    }
    if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u)))
        return BLOCKATTN_ERR_WORKSPACE;
    ba::Shape s = make_shape(offsets, batch, total_tokens, num_heads, head_dim, block_size,
                             window_blocks, scale);
    s.rope_base = rope_base;
    s.act = act;
    hipError_t e = dtype == BLOCKATTN_BF16
                       ? ba::launch_mfma_bwd(s, q, k, v, out, dout, lse, dq, dk, dv, workspace,
                                             stream)
                       : ba::launch_scalar_bwd(s, false, q, k, v, out, dout, lse, dq, dk, dv,
                                               stream);
    return e == hipSuccess ? BLOCKATTN_OK : BLOCKATTN_ERR_HIP;
}

}  // namespace

extern "C" {

int blockattn_abi_version(void) { return BLOCKATTN_ABI_VERSION; }

const char *blockattn_status_string(blockattn_status status) {
    switch (status) {
    case BLOCKATTN_OK: return "ok";
    case BLOCKATTN_ERR_INVALID_ARGUMENT: return "invalid argument";
    case BLOCKATTN_ERR_UNSUPPORTED: return "unsupported size";
    case BLOCKATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case BLOCKATTN_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

size_t blockattn_bwd_workspace_size(int64_t total_tokens, int32_t batch, int32_t num_heads,
                                    blockattn_dtype dtype) {
    if (total_tokens < 0 || batch < 0 || num_heads < 1 ||
        (dtype != BLOCKATTN_BF16 && dtype != BLOCKATTN_FP32))
        return SIZE_MAX;
    if (dtype == BLOCKATTN_FP32) return 0;  // the fp32 kernels need no workspace
    if (total_tokens == 0 || batch == 0) return 0;  // nothing to launch
    return ba::bwd_workspace_bytes(total_tokens, batch, num_heads);
}

blockattn_status blockattn_fwd(const void *q, const void *k, const void *v,
                               const int32_t *offsets, int32_t batch, int64_t total_tokens,
                               int32_t num_heads, int32_t head_dim, int32_t block_size,
                               int32_t window_blocks, float scale, blockattn_dtype dtype,
                               void *out, float *lse, hipStream_t stream) {
    return forward(q, k, v, offsets, batch, total_tokens, num_heads, head_dim, block_size,
                   window_blocks, scale, ba::kSoftmax, dtype, out, lse, stream);
}

blockattn_status blockattn_bwd(const void *q, const void *k, const void *v, const void *out,
                               const void *dout, const float *lse, const int32_t *offsets,
                               int32_t batch, int64_t total_tokens, int32_t num_heads,
                               int32_t head_dim, int32_t block_size, int32_t window_blocks,
                               float scale, blockattn_dtype dtype, void *dq, void *dk,
                               void *dv, void *workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    return backward(q, k, v, out, dout, lse, offsets, batch, total_tokens, num_heads, head_dim,
                    block_size, window_blocks, scale, 0.f, ba::kSoftmax, dtype, dq, dk, dv,
                    workspace, workspace_bytes, stream);
}

blockattn_status blockattn_bwd_noalloc(const void *q, const void *k, const void *v,
                                       const void *out, const void *dout, const float *lse,
                                       const int32_t *offsets, int32_t batch,
                                       int64_t total_tokens, int32_t num_heads,
                                       int32_t head_dim, int32_t block_size,
                                       int32_t window_blocks, float scale,
                                       blockattn_dtype dtype, void *dq, void *dk, void *dv,
                                       hipStream_t stream) {
    return backward(q, k, v, out, dout, lse, offsets, batch, total_tokens, num_heads, head_dim,
                    block_size, window_blocks, scale, 0.f, ba::kSoftmax, dtype, dq, dk, dv,
                    nullptr, 0, stream, /*noalloc=*/true);
}

blockattn_status blockattn_rope(const void *q, const void *k, const int32_t *offsets,
                                int32_t batch, int64_t total_tokens, int32_t num_heads,
                                int32_t head_dim, float theta_base, blockattn_dtype dtype,
                                void *q_rot, void *k_rot, hipStream_t stream) {
    bool empty;
    // B and W do not enter the embedding; 1 and 1 pass the shared checks
    int32_t one_b = 1, one_w = 1;
    blockattn_status st = check_common(offsets, batch, total_tokens, num_heads, head_dim, &one_b,
                                       &one_w, 1.f, dtype, &empty);
    if (st != BLOCKATTN_OK) return st;
    if (!isfinite(theta_base) || !(theta_base > 0.f)) return BLOCKATTN_ERR_INVALID_ARGUMENT;
    if (empty) return BLOCKATTN_OK;
    if (!q || !k || !q_rot || !k_rot) return BLOCKATTN_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k) || !aligned16(q_rot) || !aligned16(k_rot))
        return BLOCKATTN_ERR_INVALID_ARGUMENT;
    ba::Shape s = make_shape(offsets, batch, total_tokens, num_heads, head_dim, 1, 1, 1.f);
    s.rope_base = theta_base;
    const hipError_t e = ba::launch_rope(s, dtype == BLOCKATTN_BF16, q, k, q_rot, k_rot, stream);
    return e == hipSuccess ? BLOCKATTN_OK : BLOCKATTN_ERR_HIP;
}

blockattn_status blockattn_rope_bwd(const void *q_rot, const void *k_rot, const void *v,
                                    const void *out, const void *dout, const float *lse,
                                    const int32_t *offsets, int32_t batch, int64_t total_tokens,
                                    int32_t num_heads, int32_t head_dim, int32_t block_size,
                                    int32_t window_blocks, float scale, float theta_base,
                                    blockattn_dtype dtype, void *dq, void *dk, void *dv,
                                    void *workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
    if (!isfinite(theta_base) || !(theta_base > 0.f)) return BLOCKATTN_ERR_INVALID_ARGUMENT;
    return backward(q_rot, k_rot, v, out, dout, lse, offsets, batch, total_tokens, num_heads,
                    head_dim, block_size, window_blocks, scale, theta_base, ba::kSoftmax, dtype,
                    dq, dk, dv, workspace, workspace_bytes, stream);
}

blockattn_status blockattn_gdpa_fwd(const void *q, const void *k, const void *v,
                                    const int32_t *offsets, int32_t batch, int64_t total_tokens,
                                    int32_t num_heads, int32_t head_dim, int32_t block_size,
                                    int32_t window_blocks, float scale, int32_t activation,
                                    blockattn_dtype dtype, void *out, hipStream_t stream) {
    if (activation != BLOCKATTN_GDPA_SILU && activation != BLOCKATTN_GDPA_GELU)
        return BLOCKATTN_ERR_INVALID_ARGUMENT;
    return forward(q, k, v, offsets, batch, total_tokens, num_heads, head_dim, block_size,
                   window_blocks, scale, activation, dtype, out, nullptr, stream);
}

blockattn_status blockattn_gdpa_bwd(const void *q, const void *k, const void *v,
                                    const void *dout, const int32_t *offsets, int32_t batch,
                                    int64_t total_tokens, int32_t num_heads, int32_t head_dim,
                                    int32_t block_size, int32_t window_blocks, float scale,
                                    int32_t activation, blockattn_dtype dtype, void *dq,
                                    void *dk, void *dv, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
    if (activation != BLOCKATTN_GDPA_SILU && activation != BLOCKATTN_GDPA_GELU)
        return BLOCKATTN_ERR_INVALID_ARGUMENT;
    return backward(q, k, v, nullptr, dout, nullptr, offsets, batch, total_tokens, num_heads,
                    head_dim, block_size, window_blocks, scale, 0.f, activation, dtype, dq, dk,
                    dv, workspace, workspace_bytes, stream);
}

blockattn_status blockattn_mx_fwd(const void *q, const void *q_scale, const void *k,
                                  const void *k_scale, const void *v, const int32_t *offsets,
                                  int32_t batch, int64_t total_tokens, int32_t num_heads,
                                  int32_t head_dim, int32_t block_size, int32_t window_blocks,
                                  float scale, void *out, float *lse, hipStream_t stream) {
    bool empty;
    blockattn_status st = check_common(offsets, batch, total_tokens, num_heads, head_dim,
                                       &block_size, &window_blocks, scale, BLOCKATTN_BF16, &empty);
    if (st != BLOCKATTN_OK) return st;
    if (head_dim != 64 && head_dim != 128) return BLOCKATTN_ERR_UNSUPPORTED;
    if (empty) return BLOCKATTN_OK;
    if (!q || !q_scale || !k || !k_scale || !v || !out || !lse)
        return BLOCKATTN_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse) ||
        ((uintptr_t)q_scale & 3u) || ((uintptr_t)k_scale & 3u))
        return BLOCKATTN_ERR_INVALID_ARGUMENT;
    const ba::Shape s = make_shape(offsets, batch, total_tokens, num_heads, head_dim, block_size,
                                   window_blocks, scale);
    const hipError_t e = ba::launch_mfma_fwd_mx(s, q, q_scale, k, k_scale, v, out, lse, stream);
    return e == hipSuccess ? BLOCKATTN_OK : BLOCKATTN_ERR_HIP;
}

blockattn_status blockattn_mxpv_fwd(const void *q, const void *q_scale, const void *k,
                                    const void *k_scale, const void *v_t, const void *v_scale,
                                    const int32_t *offsets, int32_t batch, int64_t total_tokens,
                                    int32_t num_heads, int32_t head_dim, int32_t block_size,
                                    int32_t window_blocks, float scale, void *out, float *lse,
                                    hipStream_t stream) {
    bool empty;
    blockattn_status st = check_common(offsets, batch, total_tokens, num_heads, head_dim,
                                       &block_size, &window_blocks, scale, BLOCKATTN_BF16, &empty);
    if (st != BLOCKATTN_OK) return st;
    if (head_dim != 64 && head_dim != 128) return BLOCKATTN_ERR_UNSUPPORTED;
    // v^T rows are addressed with 32-bit byte offsets
    const int64_t tp = ((total_tokens + 31) / 32 + batch) * 32;
    if ((int64_t)head_dim * tp >= ((int64_t)1 << 32)) return BLOCKATTN_ERR_UNSUPPORTED;
    if (empty) return BLOCKATTN_OK;
    if (!q || !q_scale || !k || !k_scale || !v_t || !v_scale || !out || !lse)
        return BLOCKATTN_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v_t) || !aligned16(out) ||
        !aligned16(lse) || ((uintptr_t)q_scale & 3u) || ((uintptr_t)k_scale & 3u) ||
        ((uintptr_t)v_scale & 3u))
        return BLOCKATTN_ERR_INVALID_ARGUMENT;
    const ba::Shape s = make_shape(offsets, batch, total_tokens, num_heads, head_dim, block_size,
                                   window_blocks, scale);
    const hipError_t e =
        ba::launch_mfma_fwd_mxpv(s, q, q_scale, k, k_scale, v_t, v_scale, out, lse, stream);
    return e == hipSuccess ? BLOCKATTN_OK : BLOCKATTN_ERR_HIP;
}

blockattn_status blockattn_mx_bwd(const void *q, const void *q_scale, const void *k,
                                  const void *k_scale, const void *v, const void *v_scale,
                                  const void *dout, const void *dout_scale, const void *q_t,
                                  const void *q_t_scale, const void *k_t, const void *k_t_scale,
                                  const void *dout_t, const void *dout_t_scale, const void *out,
                                  const float *lse, const int32_t *offsets, int32_t batch,
                                  int64_t total_tokens, int32_t num_heads, int32_t head_dim,
                                  int32_t block_size, int32_t window_blocks, float scale,
                                  void *dq, void *dk, void *dv, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    bool empty;
    blockattn_status st = check_common(offsets, batch, total_tokens, num_heads, head_dim,
                                       &block_size, &window_blocks, scale, BLOCKATTN_BF16, &empty);
    if (st != BLOCKATTN_OK) return st;
    if (head_dim != 64 && head_dim != 128) return BLOCKATTN_ERR_UNSUPPORTED;
    // token-blocked rows are addressed with 32-bit byte offsets
    const int64_t tp = ((total_tokens + 31) / 32 + batch) * 32;
    if ((int64_t)head_dim * tp >= ((int64_t)1 << 32)) return BLOCKATTN_ERR_UNSUPPORTED;
    if (empty) return BLOCKATTN_OK;
    const void *ptrs[] = {q, q_scale, k, k_scale, v, v_scale, dout, dout_scale, q_t,
                          q_t_scale, k_t, k_t_scale, dout_t, dout_t_scale, out, lse, dq, dk, dv};
    for (const void *p : ptrs)
        if (!p) return BLOCKATTN_ERR_INVALID_ARGUMENT;
    const void *rows16[] = {q, k, v, dout, q_t, k_t, dout_t, out, lse, dq, dk, dv};
    for (const void *p : rows16)
        if (!aligned16(p)) return BLOCKATTN_ERR_INVALID_ARGUMENT;
    const void *scales4[] = {q_scale, k_scale, v_scale, dout_scale, q_t_scale, k_t_scale,
                             dout_t_scale};
    for (const void *p : scales4)
        if ((uintptr_t)p & 3u) return BLOCKATTN_ERR_INVALID_ARGUMENT;
    const size_t need = blockattn_bwd_workspace_size(total_tokens, batch, num_heads,
                                                     BLOCKATTN_BF16);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u))
        return BLOCKATTN_ERR_WORKSPACE;
    const ba::Shape s = make_shape(offsets, batch, total_tokens, num_heads, head_dim, block_size,
                                   window_blocks, scale);
    const ba::MxBwdPtrs p{q, q_scale, k, k_scale, v, v_scale, dout, dout_scale,
                          q_t, q_t_scale, k_t, k_t_scale, dout_t, dout_t_scale,
                          out, lse, dq, dk, dv};
    const hipError_t e = ba::launch_mfma_bwd_mx(s, p, workspace, stream);
    return e == hipSuccess ? BLOCKATTN_OK : BLOCKATTN_ERR_HIP;
}

blockattn_status blockattn_swa_fwd(const void *q, const void *k, const void *v,
                                   const int32_t *offsets, int32_t batch, int64_t total_tokens,
                                   int32_t num_heads, int32_t head_dim, int32_t window_tokens,
                                   float scale, blockattn_dtype dtype, void *out, float *lse,
                                   hipStream_t stream) {
    return blockattn_fwd(q, k, v, offsets, batch, total_tokens, num_heads, head_dim, 1,
                         window_tokens, scale, dtype, out, lse, stream);
}

blockattn_status blockattn_swa_bwd(const void *q, const void *k, const void *v,
                                   const void *out, const void *dout, const float *lse,
                                   const int32_t *offsets, int32_t batch, int64_t total_tokens,
                                   int32_t num_heads, int32_t head_dim, int32_t window_tokens,
                                   float scale, blockattn_dtype dtype, void *dq, void *dk,
                                   void *dv, void *workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
    return blockattn_bwd(q, k, v, out, dout, lse, offsets, batch, total_tokens, num_heads,
                         head_dim, 1, window_tokens, scale, dtype, dq, dk, dv, workspace,
                         workspace_bytes, stream);
}

}  // extern "C"
