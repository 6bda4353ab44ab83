// Internal launchers of the block-attention kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace ba {

// Scalar FMA path (fp32 storage, or bf16 storage with fp32 arithmetic).
hipError_t launch_scalar_fwd(const Shape &s, bool bf16_io, const void *q, const void *k,
                             const void *v, void *out, float *lse, hipStream_t st);
hipError_t launch_scalar_bwd(const Shape &s, bool bf16_io, const void *q, const void *k,
                             const void *v, const void *out, const void *dout,
                             const float *lse, void *dq, void *dk, void *dv, hipStream_t st);

// bf16 MFMA forward.
hipError_t launch_mfma_fwd(const Shape &s, const void *q, const void *k, const void *v,
                           void *out, float *lse, hipStream_t st);

// bf16 MFMA backward: a row-statistics launch (delta, lse * log2 e into the
// workspace `ws`, 2 * H * T floats) and one launch of query-role and
// key-role workgroups.
hipError_t launch_mfma_bwd(const Shape &s, const void *q, const void *k, const void *v,
                           const void *out, const void *dout, const float *lse, void *dq,
                           void *dk, void *dv, float *ws, hipStream_t st);

}  // namespace ba
