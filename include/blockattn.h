/*
 * blockattn.h -- C ABI of the MI355X (gfx950) jagged block-attention library.
 *
 * Operation.  Block attention replaces full self-attention over a user's
 * engagement history with sparse attention arranged in fixed-size token
 * blocks, making the cost linear in sequence length for a fixed window (ai.info
 * news item, section "Kunlun changes how GEM scales"; sysdesai.com summary,
 * section "Kunlun Architecture Details"; "GEM (Meta)" on aiwiki.ai, section
 * "Custom kernels", which names 64-token blocks).  Histories are jagged: each
 * user has its own length and nothing is padded ("GEM (Meta)", sections
 * "Training infrastructure" and "Custom kernels").
 *
 * Exact pattern computed (the pages give no formula; these are the readings):
 *   user u owns packed tokens [offsets[u], offsets[u+1]);  with i, j local
 *   indices inside that user, query i attends to key j iff
 *       j <= i   and   floor(i/B) - floor(j/B) <= W - 1
 *   (causal; its own block plus the W-1 previous blocks; blocks start at the
 *   user's first token, never straddle users, and the last may be partial).
 *   s_ij = scale * <q_i, k_j>,  P = softmax_j(s),  O_i = sum_j P_ij v_j,
 *   lse_i = ln sum_j exp(s_ij).
 * The backward pass returns dQ, dK, dV of sum(dO * O) (the production kernel
 * fuses its backward, "GEM (Meta)", section "Custom kernels").
 *
 * Layouts.  q, k, v, out, dout, dq, dk, dv: contiguous [T, H, D] (token-major,
 * then head, then head_dim), element type given by `dtype`.  lse: fp32 [H, T].
 * offsets: int32 [batch + 1] in DEVICE memory, offsets[0] = 0, non-decreasing,
 * offsets[batch] = T; zero-length users are allowed.  All tensor pointers are
 * device pointers and must be 16-byte aligned.
 *
 * Ownership and execution.  The caller owns every buffer.  The library never
 * allocates, frees or synchronises, keeps no per-call state, and never reads
 * `offsets` on the host.  Calls are enqueued on `stream` and are asynchronous;
 * calls on different streams may run concurrently if their outputs do not
 * overlap.  Outputs are fully overwritten, never accumulated into.  Results are
 * bitwise deterministic for identical inputs.  Malformed offsets (not
 * satisfying the rules above) give unspecified values but no out-of-bounds
 * memory access: every user range is clamped to [0, T].  Input values are
 * expected to be finite: a NaN or infinity in q, k, v or dout can make NaN
 * any output of the 128-row tiles that read it, rows that do not see that
 * element included (the matrix products multiply masked weights, which are
 * zero, by every value a tile reads, and 0 x NaN is NaN); it never causes an
 * out-of-bounds access.
 *
 * Errors.  Return codes only; nothing throws across the ABI.  Argument checks
 * happen before any HIP call, so an invalid call enqueues nothing.
 */
#ifndef BLOCKATTN_H
#define BLOCKATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BLOCKATTN_ABI_VERSION 9

typedef enum {
    BLOCKATTN_BF16 = 0, /* bf16 storage, fp32 accumulation, MFMA path      */
    BLOCKATTN_FP32 = 1  /* fp32 storage and arithmetic                      */
} blockattn_dtype;

typedef enum {
    BLOCKATTN_OK = 0,
    BLOCKATTN_ERR_INVALID_ARGUMENT = 1, /* batch<0, T<0, H<1, B<1, W<1, non-finite
                                           scale, null or misaligned pointer,
                                           unknown dtype                        */
    BLOCKATTN_ERR_UNSUPPORTED = 2,      /* D not in {32,64,128}; T above
                                           2^31-1025; 128 * H * D * 4 >= 2^32;
                                           launch too large                     */
    BLOCKATTN_ERR_WORKSPACE = 3,        /* workspace needed but null, too small
                                           or not 256-byte aligned              */
    BLOCKATTN_ERR_HIP = 4               /* a HIP launch reported an error       */
} blockattn_status;

/*
 * Forward pass.  Writes out [T,H,D] (dtype) and lse [H,T] (fp32).
 *   batch          number of users (>= 0); offsets has batch+1 entries
 *   total_tokens   T = offsets[batch]; T = 0 or batch = 0 returns OK at once
 *   num_heads      H >= 1;  head_dim D in {32, 64, 128}
 *   block_size     B >= 1 (B = 1 with W = w is the token sliding window of
 *                  w tokens, see blockattn_swa_fwd); any B >= T gives one
 *                  block per user, as B = T does
 *   window_blocks  W >= 1 (W = 1: independent blocks); any W >= ceil(T/B)
 *                  gives causal attention over each whole user
 *   scale          finite multiplier of <q, k> (typically 1/sqrt(D))
 */
blockattn_status blockattn_fwd(const void *q, const void *k, const void *v,
                               const int32_t *offsets, int32_t batch,
                               int64_t total_tokens, int32_t num_heads,
                               int32_t head_dim, int32_t block_size,
                               int32_t window_blocks, float scale,
                               blockattn_dtype dtype, void *out, float *lse,
                               hipStream_t stream);

/*
 * Bytes of device workspace blockattn_bwd needs for these sizes.  For bf16:
 * two fp32 row statistics per (head, token) (lse in base 2 and -delta, with
 * delta_i = sum_j P_ij <dO_i, v_j>), 256 bytes of counters, batch + 1 int32
 * tile prefix sums
 * and a 16-byte tile-table entry per (user, head, 128-row unit, role), i.e.
 * at most 2 * (ceil(T / 128) + batch) * H entries; each region is rounded up
 * to 256 bytes.  0 for fp32 and for empty calls (T or batch 0).  Returns
 * SIZE_MAX for invalid sizes.
 */
size_t blockattn_bwd_workspace_size(int64_t total_tokens, int32_t batch,
                                    int32_t num_heads, blockattn_dtype dtype);

/*
 * Backward pass.  Given the forward inputs, its out and lse, and the upstream
 * gradient dout, writes dq, dk, dv [T,H,D] (dtype; fp32 accumulation).
 * workspace: device memory of at least blockattn_bwd_workspace_size() bytes,
 * 256-byte aligned, owned by the caller, contents on entry ignored; the call
 * uses it as scratch on `stream` (two calls that share a workspace must not
 * overlap), it may be reused once the stream has passed this call, and may
 * be null when the size is 0.  Other arguments as for blockattn_fwd.
 */
blockattn_status blockattn_bwd(const void *q, const void *k, const void *v,
                               const void *out, const void *dout,
                               const float *lse, const int32_t *offsets,
                               int32_t batch, int64_t total_tokens,
                               int32_t num_heads, int32_t head_dim,
                               int32_t block_size, int32_t window_blocks,
                               float scale, blockattn_dtype dtype, void *dq,
                               void *dk, void *dv, void *workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * Token-level sliding-window attention: query i of a user sees keys
 * i - window_tokens < j <= i of the same user.  This is the pattern the pages
 * name as the predecessor of block attention and the baseline of its speedup
 * ("GEM (Meta)", section "Custom kernels"); it is block attention with blocks
 * of one token and a window of window_tokens blocks, and these two calls are
 * exactly blockattn_fwd / blockattn_bwd with block_size 1 and window_blocks
 * window_tokens (same layouts, workspace and errors; window_tokens < 1 is
 * BLOCKATTN_ERR_INVALID_ARGUMENT).
 */
blockattn_status blockattn_swa_fwd(const void *q, const void *k, const void *v,
                                   const int32_t *offsets, int32_t batch,
                                   int64_t total_tokens, int32_t num_heads,
                                   int32_t head_dim, int32_t window_tokens,
                                   float scale, blockattn_dtype dtype, void *out,
                                   float *lse, hipStream_t stream);
blockattn_status blockattn_swa_bwd(const void *q, const void *k, const void *v,
                                   const void *out, const void *dout,
                                   const float *lse, const int32_t *offsets,
                                   int32_t batch, int64_t total_tokens,
                                   int32_t num_heads, int32_t head_dim,
                                   int32_t window_tokens, float scale,
                                   blockattn_dtype dtype, void *dq, void *dk,
                                   void *dv, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * Rotary position embedding.  The production block-attention kernel carries
 * a rotary embedding and fuses its backward ("GEM (Meta)", section "Custom
 * kernels"); the pages give neither its form nor its base nor the positions.
 * Readings: the rotate-half form, angle p * theta_base^(-2d/D) for the pair
 * of features (d, d + D/2), d < D/2, and p the token's index inside its own
 * user (positions restart at every user, like the blocks).  For each token
 * and head of q and k:
 *     x_rot[d]       = x[d] cos - x[d + D/2] sin
 *     x_rot[d + D/2] = x[d + D/2] cos + x[d] sin
 * Writes q_rot and k_rot [T, H, D] (dtype; fp32 arithmetic, the angle reduced
 * in fp64).  q_rot may be q and k_rot may be k (in place); otherwise outputs
 * must not overlap inputs.  theta_base must be finite and > 0 (typically
 * 10000), else BLOCKATTN_ERR_INVALID_ARGUMENT.  Other arguments, layouts and
 * errors as for blockattn_fwd.  The attention forward then runs on q_rot and
 * k_rot (blockattn_fwd), and blockattn_rope_bwd gives the gradients.
 */
blockattn_status blockattn_rope(const void *q, const void *k, const int32_t *offsets,
                                int32_t batch, int64_t total_tokens,
                                int32_t num_heads, int32_t head_dim,
                                float theta_base, blockattn_dtype dtype,
                                void *q_rot, void *k_rot, hipStream_t stream);

/*
 * Backward of blockattn_fwd(q_rot, k_rot, v) with the rotary embedding's
 * backward fused in: takes the rotated q_rot and k_rot (as blockattn_rope
 * wrote them) with v, out, lse and dout, and writes dq and dk with respect
 * to the UNROTATED q and k (each row turned back by its position's angles,
 * R(p)^T, inside the kernel that computes it) and dv.  theta_base as for
 * blockattn_rope; everything else as for blockattn_bwd.
 */
blockattn_status blockattn_rope_bwd(const void *q_rot, const void *k_rot,
                                    const void *v, const void *out,
                                    const void *dout, const float *lse,
                                    const int32_t *offsets, int32_t batch,
                                    int64_t total_tokens, int32_t num_heads,
                                    int32_t head_dim, int32_t block_size,
                                    int32_t window_blocks, float scale,
                                    float theta_base, blockattn_dtype dtype,
                                    void *dq, void *dk, void *dv,
                                    void *workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/*
 * Generalized dot-product attention (GDPA) on the same block pattern: the
 * softmax replaced by an activation ("GEM (Meta)", section "Custom kernels":
 * GDPA replaces the softmax with activations such as GELU or SiLU).  The
 * pages give no normalisation; the reading is none:
 *     x_ij = scale * <q_i, k_j>,  P_ij = act(x_ij),  out_i = sum_j P_ij v_j
 * over the visible keys j of query i, with act SiLU (x / (1 + e^-x)) or GELU
 * (the erf form, x * Phi(x)).  No lse.  blockattn_gdpa_bwd returns dq, dk,
 * dv of sum(dout * out) (dS_ij = act'(x_ij) <dout_i, v_j>); it needs neither
 * out nor lse, and takes the workspace of blockattn_bwd.  activation not in
 * blockattn_gdpa_act is BLOCKATTN_ERR_INVALID_ARGUMENT; everything else as
 * for blockattn_fwd / blockattn_bwd.
 */
typedef enum {
    BLOCKATTN_GDPA_SILU = 1,
    BLOCKATTN_GDPA_GELU = 2
} blockattn_gdpa_act;

blockattn_status blockattn_gdpa_fwd(const void *q, const void *k, const void *v,
                                    const int32_t *offsets, int32_t batch,
                                    int64_t total_tokens, int32_t num_heads,
                                    int32_t head_dim, int32_t block_size,
                                    int32_t window_blocks, float scale,
                                    int32_t activation, blockattn_dtype dtype,
                                    void *out, hipStream_t stream);
blockattn_status blockattn_gdpa_bwd(const void *q, const void *k, const void *v,
                                    const void *dout, const int32_t *offsets,
                                    int32_t batch, int64_t total_tokens,
                                    int32_t num_heads, int32_t head_dim,
                                    int32_t block_size, int32_t window_blocks,
                                    float scale, int32_t activation,
                                    blockattn_dtype dtype, void *dq, void *dk,
                                    void *dv, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/*
 * Forward with q and k in MXFP8.  The pages say production attention runs in
 * MXFP8, a block-scaled FP8 format ("GEM (Meta)", section "Custom kernels"),
 * and give nothing more; the reading is the OCP Microscaling format: each
 * element an E4M3 byte (bias 7, subnormals, no infinities, S.1111.111 NaN),
 * every 32 consecutive head-dim elements sharing one E8M0 scale byte,
 * 2^(e - 127).  Here the score product q.k runs on the block-scaled fp8
 * matrix cores; v, out and the softmax are as in blockattn_fwd (bf16, fp32).
 *   q, k       E4M3 bytes [T, H, D], 16-byte aligned
 *   q_scale,   E8M0 bytes [H, T, D/32] (head-major, like lse), 4-byte
 *   k_scale    aligned; element (t, h, d) has scale [h][t][d / 32]
 *   v          bf16 [T, H, D];  out bf16 [T, H, D];  lse fp32 [H, T]
 * D must be 64 or 128, else BLOCKATTN_ERR_UNSUPPORTED.  Other arguments and
 * errors as for blockattn_fwd.  The block-scaled fp8 products sum with fewer
 * bits than fp32 (measured: within 2^-12 of sum_d |scale q_d k_d| per score).
 * The MXFP8 backward is blockattn_mx_bwd.
 */
blockattn_status blockattn_mx_fwd(const void *q, const void *q_scale,
                                  const void *k, const void *k_scale,
                                  const void *v, const int32_t *offsets,
                                  int32_t batch, int64_t total_tokens,
                                  int32_t num_heads, int32_t head_dim,
                                  int32_t block_size, int32_t window_blocks,
                                  float scale, void *out, float *lse,
                                  hipStream_t stream);

/*
 * Forward with q, k and v in MXFP8 and the P.V product block-scaled too.
 * The pages put production attention in MXFP8 ("GEM (Meta)", section
 * "Custom kernels") and the matmuls in block-scaled MXFP8 end to end
 * (section "Ultra-low-precision training"), which for P.V means the softmax
 * weights are quantized as well.  Reading: each query's weights fall into
 * blocks of 32 keys counted from its user's first token; with F the floor
 * of the block's largest s * log2(e), a weight 2^(s log2 e) (relative to
 * the row) is stored as 2^(F - 7) times the nearest E4M3 value of
 * 2^(s log2 e - F + 7) (ties to even; below 2^8, so nothing saturates).
 * The row sum and lse use the unquantized weights.  v's scales run along
 * the P.V contraction, each user's tokens, so v comes transposed and
 * blocked by user (NB = ceil(T / 32) + batch; user u's blocks start at
 * ub = ceil(offsets[u] / 32) + u, so users never share a block):
 *   q, k, q_scale, k_scale   as for blockattn_mx_fwd
 *   v_t      E4M3 bytes [H, D, 32 * NB], 16-byte aligned: local token j of
 *            user u, column d of head h, at [h][d][32 ub + j]; the columns
 *            no token uses are padding
 *   v_scale  E8M0 bytes [H, NB, D], 4-byte aligned: that element's scale
 *            is [h][ub + j / 32][d]
 *   out      bf16 [T, H, D];  lse fp32 [H, T]
 * A chunk of 64 keys starts on a multiple of 32 of the user's tokens, so
 * the products also read codes and scales just past a user's last token
 * (its padding, the next user's first block): every code of v_t (padding
 * included) must be finite and no scale may be 255 (NaN), or NaN can reach
 * unrelated rows.  D must be 64 or 128 and D * 32 * NB below 2^32,
 * else BLOCKATTN_ERR_UNSUPPORTED.  Other arguments and errors as for
 * blockattn_fwd.  The block-scaled products sum with fewer bits than fp32
 * (see blockattn_mx_fwd).  The MXFP8 backward is blockattn_mx_bwd.
 */
blockattn_status blockattn_mxpv_fwd(const void *q, const void *q_scale,
                                    const void *k, const void *k_scale,
                                    const void *v_t, const void *v_scale,
                                    const int32_t *offsets, int32_t batch,
                                    int64_t total_tokens, int32_t num_heads,
                                    int32_t head_dim, int32_t block_size,
                                    int32_t window_blocks, float scale,
                                    void *out, float *lse, hipStream_t stream);

/*
 * Backward in MXFP8 ("GEM (Meta)", section "Ultra-low-precision training":
 * the attention kernel's block-scaled MXFP8 products run in the backward as
 * well as the forward).  Every product takes operands whose 32-element scale
 * blocks run along its own contraction.  The score and dP products contract
 * head dims: q, k, v and dout come head-dim-blocked.  dV = P^T dO and
 * dK = scale dS^T Q contract queries and dQ = scale dS K contracts keys:
 * q, k and dout come a second time, quantized along each user's tokens and
 * transposed (the caller's producer emits both).  P_ij = exp(scale q_i.k_j -
 * lse_i) with the forward's lse, delta_i = <dO_i, O_i> with the forward's
 * out, dS_ij = P_ij (dP_ij - delta_i).  P and dS are quantized inside the
 * backward along each key's queries (for dV, dK), and dS along each query's
 * keys (for dQ), in blocks of 32 positions counted from the user's first
 * token: with a the block's largest magnitude, each value becomes 2^E times
 * its nearest E4M3 value (ties to even) of x 2^-E,
 * E = max(floor(log2 a) - 7, -127), so nothing saturates.  Softmax only.
 *   q, k, v, dout             E4M3 bytes [T, H, D], 16-byte aligned
 *   q_scale, k_scale,         E8M0 bytes [H, T, D/32], 4-byte aligned, as
 *   v_scale, dout_scale       for blockattn_mx_fwd
 *   q_t, k_t, dout_t          E4M3 bytes [H, D, 32 * NB], 16-byte aligned,
 *                             laid out like blockattn_mxpv_fwd's v_t (user
 *                             u's local token j, column d of head h, at
 *                             [h][d][32 ub + j], ub = ceil(offsets[u] / 32)
 *                             + u, NB = ceil(T / 32) + batch)
 *   q_t_scale, k_t_scale,     E8M0 bytes [H, NB, D], 4-byte aligned, as
 *   dout_t_scale              v_scale of blockattn_mxpv_fwd
 *   out                       bf16 [T, H, D], the forward's output
 *   lse                       fp32 [H, T], the forward's lse
 *   dq, dk, dv                bf16 [T, H, D], written whole
 *   workspace                 as for blockattn_bwd (same size function)
 * The products read codes and scales of the token-blocked tensors just past
 * a user's last token: every code (padding included) must be finite and no
 * scale 255, as for blockattn_mxpv_fwd.  D must be 64 or 128 and D * 32 * NB
 * below 2^32, else BLOCKATTN_ERR_UNSUPPORTED; a null or misaligned pointer
 * is BLOCKATTN_ERR_INVALID_ARGUMENT; other arguments and errors as for
 * blockattn_bwd.  Results are deterministic (no atomics).
 */
blockattn_status blockattn_mx_bwd(const void *q, const void *q_scale,
                                  const void *k, const void *k_scale,
                                  const void *v, const void *v_scale,
                                  const void *dout, const void *dout_scale,
                                  const void *q_t, const void *q_t_scale,
                                  const void *k_t, const void *k_t_scale,
                                  const void *dout_t, const void *dout_t_scale,
                                  const void *out, const float *lse,
                                  const int32_t *offsets, int32_t batch,
                                  int64_t total_tokens, int32_t num_heads,
                                  int32_t head_dim, int32_t block_size,
                                  int32_t window_blocks, float scale, void *dq,
                                  void *dk, void *dv, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/*
 * blockattn_bwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a static device array
 * of BLOCKATTN_NOALLOC_WORKSPACE_BYTES inside the library, one per GPU,
 * created with the library's code object and held until the process ends;
 * this call allocates nothing.  Calls whose blockattn_bwd_workspace_size
 * exceeds that size return BLOCKATTN_ERR_WORKSPACE (64 MiB covers, e.g.,
 * 524288 tokens x 8 heads: 33.6 MB).  Every call on one GPU shares that
 * GPU's array, so calls that overlap on one GPU (other streams, other host
 * threads) race and must be serialised by the caller; each call sets up
 * everything it reads (no state carries over between calls).  Arguments,
 * results and other errors as for blockattn_bwd; BLOCKATTN_ERR_HIP if the
 * array's address cannot be obtained.
 */
#define BLOCKATTN_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
blockattn_status blockattn_bwd_noalloc(const void *q, const void *k, const void *v,
                                       const void *out, const void *dout,
                                       const float *lse, const int32_t *offsets,
                                       int32_t batch, int64_t total_tokens,
                                       int32_t num_heads, int32_t head_dim,
                                       int32_t block_size, int32_t window_blocks,
                                       float scale, blockattn_dtype dtype, void *dq,
                                       void *dk, void *dv, hipStream_t stream);

/* Static, human-readable name of a status code ("unknown status" otherwise). */
const char *blockattn_status_string(blockattn_status status);

/* BLOCKATTN_ABI_VERSION of the loaded library. */
int blockattn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BLOCKATTN_H */
