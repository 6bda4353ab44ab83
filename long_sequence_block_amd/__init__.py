"""MI355X-native (gfx950) jagged block attention.

The computation runs in the HIP library built from ``csrc/`` and exposed
through the C ABI of ``include/blockattn.h``; ``binding`` is its ctypes
binding.  ``workloads`` draws the seeded synthetic inputs.
"""
from .binding import (BF16, FP32, GDPA_GELU, GDPA_SILU, BlockAttnError,  # noqa: F401
                      blockattn_abi_version, blockattn_gdpa_bwd, blockattn_gdpa_fwd,
                      blockattn_mx_fwd, mx_fwd, blockattn_mxpv_fwd, mxpv_fwd,
                      blockattn_mx_bwd, mx_bwd,
                      blockattn_bwd, blockattn_bwd_noalloc, blockattn_bwd_workspace_size,
                      blockattn_fwd, bwd_noalloc, NOALLOC_WORKSPACE_BYTES,
                      blockattn_rope, blockattn_rope_bwd, blockattn_status_string,
                      blockattn_swa_bwd, blockattn_swa_fwd, bwd, fwd, library_path, load,
                      gdpa_bwd, gdpa_fwd, rope, rope_bwd, swa_bwd, swa_fwd)
