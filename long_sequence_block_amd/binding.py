"""Thin ctypes binding of the block-attention C ABI (include/blockattn.h).

Functions named like the C entry points take raw device pointers and sizes
and return the status code, exactly as the C ABI does.  ``fwd`` and ``bwd``
are conveniences that take torch tensors (torch only provides device memory
and the stream), allocate the outputs, call the C ABI and raise on error.
Every step of the computation runs in the HIP library; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .build import LIB, build_library

BF16, FP32 = 0, 1
OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
GDPA_SILU, GDPA_GELU = 1, 2  # blockattn_gdpa_act

# Every symbol include/blockattn.h declares.
EXPORTS = ("blockattn_fwd", "blockattn_bwd", "blockattn_bwd_workspace_size",
           "blockattn_swa_fwd", "blockattn_swa_bwd", "blockattn_rope", "blockattn_rope_bwd",
           "blockattn_gdpa_fwd", "blockattn_gdpa_bwd", "blockattn_mx_fwd", "blockattn_mxpv_fwd",
           "blockattn_mx_bwd", "blockattn_bwd_noalloc", "blockattn_status_string", "blockattn_abi_version")

NOALLOC_WORKSPACE_BYTES = 64 << 20  # BLOCKATTN_NOALLOC_WORKSPACE_BYTES

_lib = None


class BlockAttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


def library_path() -> str:
    return LIB


def load() -> ctypes.CDLL:
    """Loads the built library (building it first only if none is built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        build_library()
    lib = ctypes.CDLL(LIB)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.blockattn_fwd.argtypes = [vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, f32,
                                  ctypes.c_int, vp, vp, vp]
    lib.blockattn_fwd.restype = ctypes.c_int
    lib.blockattn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                  i32, f32, ctypes.c_int, vp, vp, vp, vp, ctypes.c_size_t,
                                  vp]
    lib.blockattn_bwd.restype = ctypes.c_int
    lib.blockattn_bwd_workspace_size.argtypes = [i64, i32, i32, ctypes.c_int]
    lib.blockattn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.blockattn_swa_fwd.argtypes = [vp, vp, vp, vp, i32, i64, i32, i32, i32, f32,
                                      ctypes.c_int, vp, vp, vp]
    lib.blockattn_swa_fwd.restype = ctypes.c_int
    lib.blockattn_swa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                      f32, ctypes.c_int, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.blockattn_swa_bwd.restype = ctypes.c_int
    lib.blockattn_rope.argtypes = [vp, vp, vp, i32, i64, i32, i32, f32, ctypes.c_int, vp, vp,
                                   vp]
    lib.blockattn_rope.restype = ctypes.c_int
    lib.blockattn_rope_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                       i32, f32, f32, ctypes.c_int, vp, vp, vp, vp,
                                       ctypes.c_size_t, vp]
    lib.blockattn_rope_bwd.restype = ctypes.c_int
    lib.blockattn_gdpa_fwd.argtypes = [vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, f32, i32,
                                       ctypes.c_int, vp, vp]
    lib.blockattn_gdpa_fwd.restype = ctypes.c_int
    lib.blockattn_gdpa_bwd.argtypes = [vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, f32,
                                       i32, ctypes.c_int, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.blockattn_gdpa_bwd.restype = ctypes.c_int
    lib.blockattn_mx_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, f32,
                                     vp, vp, vp]
    lib.blockattn_mx_fwd.restype = ctypes.c_int
    lib.blockattn_mxpv_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32,
                                       f32, vp, vp, vp]
    lib.blockattn_mxpv_fwd.restype = ctypes.c_int
    lib.blockattn_mx_bwd.argtypes = [vp] * 17 + [i32, i64, i32, i32, i32, i32, f32, vp, vp, vp,
                                                 vp, ctypes.c_size_t, vp]
    lib.blockattn_mx_bwd.restype = ctypes.c_int
    lib.blockattn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                          i32, f32, ctypes.c_int, vp, vp, vp, vp]
    lib.blockattn_bwd_noalloc.restype = ctypes.c_int
    lib.blockattn_status_string.argtypes = [ctypes.c_int]
    lib.blockattn_status_string.restype = ctypes.c_char_p
    lib.blockattn_abi_version.argtypes = []
    lib.blockattn_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


# ---------------------------------------------------------------- raw C ABI


def blockattn_fwd(q, k, v, offsets, batch, total_tokens, num_heads, head_dim,
                  block_size, window_blocks, scale, dtype, out, lse, stream) -> int:
    return load().blockattn_fwd(q, k, v, offsets, batch, total_tokens, num_heads,
                                head_dim, block_size, window_blocks, scale, dtype,
                                out, lse, stream)


def blockattn_bwd(q, k, v, out, dout, lse, offsets, batch, total_tokens, num_heads,
                  head_dim, block_size, window_blocks, scale, dtype, dq, dk, dv,
                  workspace, workspace_bytes, stream) -> int:
    return load().blockattn_bwd(q, k, v, out, dout, lse, offsets, batch, total_tokens,
                                num_heads, head_dim, block_size, window_blocks, scale,
                                dtype, dq, dk, dv, workspace, workspace_bytes, stream)


def blockattn_bwd_noalloc(q, k, v, out, dout, lse, offsets, batch, total_tokens, num_heads,
                          head_dim, block_size, window_blocks, scale, dtype, dq, dk, dv,
                          stream) -> int:
    return load().blockattn_bwd_noalloc(q, k, v, out, dout, lse, offsets, batch, total_tokens,
                                        num_heads, head_dim, block_size, window_blocks, scale,
                                        dtype, dq, dk, dv, stream)


def blockattn_swa_fwd(q, k, v, offsets, batch, total_tokens, num_heads, head_dim,
                      window_tokens, scale, dtype, out, lse, stream) -> int:
    return load().blockattn_swa_fwd(q, k, v, offsets, batch, total_tokens, num_heads,
                                    head_dim, window_tokens, scale, dtype, out, lse, stream)


def blockattn_swa_bwd(q, k, v, out, dout, lse, offsets, batch, total_tokens, num_heads,
                      head_dim, window_tokens, scale, dtype, dq, dk, dv, workspace,
                      workspace_bytes, stream) -> int:
    return load().blockattn_swa_bwd(q, k, v, out, dout, lse, offsets, batch, total_tokens,
                                    num_heads, head_dim, window_tokens, scale, dtype, dq, dk,
                                    dv, workspace, workspace_bytes, stream)


def blockattn_rope(q, k, offsets, batch, total_tokens, num_heads, head_dim, theta_base, dtype,
                   q_rot, k_rot, stream) -> int:
    return load().blockattn_rope(q, k, offsets, batch, total_tokens, num_heads, head_dim,
                                 theta_base, dtype, q_rot, k_rot, stream)


def blockattn_rope_bwd(q_rot, k_rot, v, out, dout, lse, offsets, batch, total_tokens,
                       num_heads, head_dim, block_size, window_blocks, scale, theta_base, dtype,
                       dq, dk, dv, workspace, workspace_bytes, stream) -> int:
    return load().blockattn_rope_bwd(q_rot, k_rot, v, out, dout, lse, offsets, batch,
                                     total_tokens, num_heads, head_dim, block_size,
                                     window_blocks, scale, theta_base, dtype, dq, dk, dv,
                                     workspace, workspace_bytes, stream)


def blockattn_gdpa_fwd(q, k, v, offsets, batch, total_tokens, num_heads, head_dim,
                       block_size, window_blocks, scale, activation, dtype, out, stream) -> int:
    return load().blockattn_gdpa_fwd(q, k, v, offsets, batch, total_tokens, num_heads,
                                     head_dim, block_size, window_blocks, scale, activation,
                                     dtype, out, stream)


def blockattn_gdpa_bwd(q, k, v, dout, offsets, batch, total_tokens, num_heads, head_dim,
                       block_size, window_blocks, scale, activation, dtype, dq, dk, dv,
                       workspace, workspace_bytes, stream) -> int:
    return load().blockattn_gdpa_bwd(q, k, v, dout, offsets, batch, total_tokens, num_heads,
                                     head_dim, block_size, window_blocks, scale, activation,
                                     dtype, dq, dk, dv, workspace, workspace_bytes, stream)


def blockattn_mx_fwd(q, q_scale, k, k_scale, v, offsets, batch, total_tokens, num_heads,
                     head_dim, block_size, window_blocks, scale, out, lse, stream) -> int:
    return load().blockattn_mx_fwd(q, q_scale, k, k_scale, v, offsets, batch, total_tokens,
                                   num_heads, head_dim, block_size, window_blocks, scale, out,
                                   lse, stream)


def blockattn_mxpv_fwd(q, q_scale, k, k_scale, v_t, v_scale, offsets, batch, total_tokens,
                       num_heads, head_dim, block_size, window_blocks, scale, out, lse,
                       stream) -> int:
    return load().blockattn_mxpv_fwd(q, q_scale, k, k_scale, v_t, v_scale, offsets, batch,
                                     total_tokens, num_heads, head_dim, block_size,
                                     window_blocks, scale, out, lse, stream)


def blockattn_mx_bwd(q, q_scale, k, k_scale, v, v_scale, dout, dout_scale, q_t, q_t_scale,
                     k_t, k_t_scale, dout_t, dout_t_scale, out, lse, offsets, batch,
                     total_tokens, num_heads, head_dim, block_size, window_blocks, scale, dq,
                     dk, dv, workspace, workspace_bytes, stream) -> int:
    return load().blockattn_mx_bwd(q, q_scale, k, k_scale, v, v_scale, dout, dout_scale, q_t,
                                   q_t_scale, k_t, k_t_scale, dout_t, dout_t_scale, out, lse,
                                   offsets, batch, total_tokens, num_heads, head_dim,
                                   block_size, window_blocks, scale, dq, dk, dv, workspace,
                                   workspace_bytes, stream)


def blockattn_bwd_workspace_size(total_tokens, batch, num_heads, dtype) -> int:
    return int(load().blockattn_bwd_workspace_size(total_tokens, batch, num_heads, dtype))


def blockattn_status_string(status: int) -> str:
    return load().blockattn_status_string(status).decode()


def blockattn_abi_version() -> int:
    return int(load().blockattn_abi_version())


status_string = blockattn_status_string

# ------------------------------------------------------ torch conveniences
#
# Streams.  Each call runs on `stream` (default: the current stream).  The
# outputs and the workspace this module allocates are allocated while that
# stream is current, so the caching allocator hands their memory to other
# work only in that stream's order, after the kernels that use it; the
# workspace tensor stays referenced until the C call has been enqueued.
# Tensors the caller passes in are the caller's to keep alive and to order
# (torch's usual rules across streams, e.g. Tensor.record_stream).


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _check_tensor(t, shape, dtype, dev, what):
    """A caller's tensor: the given shape and dtype, contiguous, on device
    dev (a kernel handed a host pointer or a wrong-sized buffer would fault,
    so these are checked before any call)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch tensor")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous {dtype} tensor of shape {tuple(shape)}")
    if not t.is_cuda or t.device != dev:
        raise ValueError(f"{what} must be on {dev}")


def _check_offsets(offsets, dev):
    if (not isinstance(offsets, torch.Tensor) or offsets.dtype != torch.int32
            or offsets.dim() != 1 or offsets.numel() < 1 or not offsets.is_contiguous()
            or not offsets.is_cuda or offsets.device != dev):
        raise ValueError(f"offsets must be a contiguous 1-D int32 tensor of batch + 1 "
                         f"entries on {dev}")


def _check(q, k, v, offsets):
    if not isinstance(q, torch.Tensor) or q.dim() != 3 or not q.is_cuda:
        raise ValueError("q must be a [T, H, D] device tensor")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_tensor(t, q.shape, q.dtype, q.device, n)
    _check_offsets(offsets, q.device)


def _check_like(q, *ts, what="out and dout"):
    for t in ts:
        _check_tensor(t, q.shape, q.dtype, q.device, what)


def _check_lse(lse, H, T, dev):
    _check_tensor(lse, (H, T), torch.float32, dev, "lse")


def _outputs(q, out, lse, out_dtype=None):
    """The forward's out [T, H, D] and lse fp32 [H, T]: the caller's, checked,
    or new ones (called with the call's stream current)."""
    T, H, D = q.shape
    dt = q.dtype if out_dtype is None else out_dtype
    out = torch.empty((T, H, D), dtype=dt, device=q.device) if out is None else out
    lse = torch.empty((H, T), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensor(out, (T, H, D), dt, q.device, "out")
    _check_tensor(lse, (H, T), torch.float32, q.device, "lse")
    return out, lse


def _torch_stream(stream):
    """The torch stream a call runs on: the given one, else the current."""
    return torch.cuda.current_stream() if stream is None else stream


def _workspace(q, offsets, code, workspace):
    """The backward's workspace tensor: the caller's, or a new device buffer
    of blockattn_bwd_workspace_size bytes (None if none is needed).  Called
    with the call's stream current (see above).  Its size and alignment are
    the C call's to check."""
    T, H, _ = q.shape
    need = blockattn_bwd_workspace_size(T, offsets.numel() - 1, H, code)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None and (not isinstance(workspace, torch.Tensor)
                                  or not workspace.is_cuda or workspace.device != q.device
                                  or not workspace.is_contiguous()):
        raise ValueError(f"workspace must be a contiguous tensor on {q.device}")
    return workspace


def _ws_args(ws):
    return (ws.data_ptr(), ws.numel() * ws.element_size()) if ws is not None else (None, 0)


def _grads(q, grads, dtype=None):
    """dq, dk, dv [T, H, D]: the caller's three tensors, checked, or new ones."""
    dt = q.dtype if dtype is None else dtype
    if grads is None:
        return tuple(torch.empty(q.shape, dtype=dt, device=q.device) for _ in range(3))
    if len(grads) != 3:
        raise ValueError("grads must be three tensors (dq, dk, dv)")
    for t, n in zip(grads, ("dq", "dk", "dv")):
        _check_tensor(t, q.shape, dt, q.device, n)
    return tuple(grads)


def fwd(q, k, v, offsets, block_size: int, window_blocks: int, scale: float,
        out=None, lse=None, stream=None):
    """Forward block attention.  Returns (out [T,H,D], lse fp32 [H,T])."""
    _check(q, k, v, offsets)
    T, H, D = q.shape
    st = _torch_stream(stream)
    with torch.cuda.stream(st):
        out, lse = _outputs(q, out, lse)
        rc = blockattn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), offsets.data_ptr(),
                           offsets.numel() - 1, T, H, D, block_size, window_blocks,
                           float(scale), _dtype_code(q), out.data_ptr(), lse.data_ptr(),
                           st.cuda_stream)
    if rc != OK:
        raise BlockAttnError("blockattn_fwd", rc)
    return out, lse


def bwd(q, k, v, out, dout, lse, offsets, block_size: int, window_blocks: int,
        scale: float, grads=None, workspace=None, stream=None):
    """Backward block attention.  Returns (dq, dk, dv), each [T,H,D]."""
    _check(q, k, v, offsets)
    T, H, D = q.shape
    _check_like(q, out, dout)
    _check_lse(lse, H, T, q.device)
    code = _dtype_code(q)
    st = _torch_stream(stream)
    with torch.cuda.stream(st):
        dq, dk, dv = _grads(q, grads)
        ws = _workspace(q, offsets, code, workspace)
        ws_ptr, ws_len = _ws_args(ws)
        rc = blockattn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                           dout.data_ptr(), lse.data_ptr(), offsets.data_ptr(),
                           offsets.numel() - 1, T, H, D, block_size, window_blocks,
                           float(scale), code, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                           ws_ptr, ws_len, st.cuda_stream)
        del ws
    if rc != OK:
        raise BlockAttnError("blockattn_bwd", rc)
    return dq, dk, dv


def bwd_noalloc(q, k, v, out, dout, lse, offsets, block_size: int, window_blocks: int,
                scale: float, grads=None, stream=None):
    """Backward block attention through blockattn_bwd_noalloc (the library's
    static workspace; nothing is allocated for it).  Returns (dq, dk, dv);
    pass grads to have nothing allocated at all."""
    _check(q, k, v, offsets)
    T, H, D = q.shape
    _check_like(q, out, dout)
    _check_lse(lse, H, T, q.device)
    st = _torch_stream(stream)
    with torch.cuda.stream(st):
        dq, dk, dv = _grads(q, grads)
        rc = blockattn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   dout.data_ptr(), lse.data_ptr(), offsets.data_ptr(),
                                   offsets.numel() - 1, T, H, D, block_size, window_blocks,
                                   float(scale), _dtype_code(q), dq.data_ptr(), dk.data_ptr(),
                                   dv.data_ptr(), st.cuda_stream)
    if rc != OK:
        raise BlockAttnError("blockattn_bwd_noalloc", rc)
    return dq, dk, dv


def swa_fwd(q, k, v, offsets, window_tokens: int, scale: float, out=None, lse=None,
            stream=None):
    """Token sliding-window forward (blockattn_swa_fwd).  Returns (out, lse)."""
    _check(q, k, v, offsets)
    T, H, D = q.shape
    st = _torch_stream(stream)
    with torch.cuda.stream(st):
        out, lse = _outputs(q, out, lse)
        rc = blockattn_swa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), offsets.data_ptr(),
                               offsets.numel() - 1, T, H, D, window_tokens, float(scale),
                               _dtype_code(q), out.data_ptr(), lse.data_ptr(), st.cuda_stream)
    if rc != OK:
        raise BlockAttnError("blockattn_swa_fwd", rc)
    return out, lse


def swa_bwd(q, k, v, out, dout, lse, offsets, window_tokens: int, scale: float,
            grads=None, workspace=None, stream=None):
    """Token sliding-window backward (blockattn_swa_bwd).  Returns (dq, dk, dv)."""
    _check(q, k, v, offsets)
    T, H, D = q.shape
    _check_like(q, out, dout)
    _check_lse(lse, H, T, q.device)
    code = _dtype_code(q)
    st = _torch_stream(stream)
    with torch.cuda.stream(st):
        dq, dk, dv = _grads(q, grads)
        ws = _workspace(q, offsets, code, workspace)
        ws_ptr, ws_len = _ws_args(ws)
        rc = blockattn_swa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                               dout.data_ptr(), lse.data_ptr(), offsets.data_ptr(),
                               offsets.numel() - 1, T, H, D, window_tokens, float(scale), code,
                               dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws_ptr, ws_len,
                               st.cuda_stream)
        del ws
    if rc != OK:
        raise BlockAttnError("blockattn_swa_bwd", rc)
    return dq, dk, dv


def rope(q, k, offsets, theta_base: float = 10000.0, q_rot=None, k_rot=None, stream=None):
    """Rotary embedding of q and k (blockattn_rope).  Returns (q_rot, k_rot);
    pass q_rot=q, k_rot=k to rotate in place."""
    _check(q, k, q, offsets)
    T, H, D = q.shape
    st = _torch_stream(stream)
    with torch.cuda.stream(st):
        q_rot = torch.empty_like(q) if q_rot is None else q_rot
        k_rot = torch.empty_like(k) if k_rot is None else k_rot
        _check_like(q, q_rot, k_rot, what="q_rot and k_rot")
        rc = blockattn_rope(q.data_ptr(), k.data_ptr(), offsets.data_ptr(), offsets.numel() - 1,
                            T, H, D, float(theta_base), _dtype_code(q), q_rot.data_ptr(),
                            k_rot.data_ptr(), st.cuda_stream)
    if rc != OK:
        raise BlockAttnError("blockattn_rope", rc)
    return q_rot, k_rot


def rope_bwd(q_rot, k_rot, v, out, dout, lse, offsets, block_size: int, window_blocks: int,
             scale: float, theta_base: float = 10000.0, grads=None, workspace=None,
             stream=None):
    """Backward through attention and the rotary embedding (blockattn_rope_bwd):
    (dq, dk, dv) with dq, dk taken with respect to the unrotated q, k."""
    _check(q_rot, k_rot, v, offsets)
    T, H, D = q_rot.shape
    _check_like(q_rot, out, dout)
    _check_lse(lse, H, T, q_rot.device)
    code = _dtype_code(q_rot)
    st = _torch_stream(stream)
    with torch.cuda.stream(st):
        dq, dk, dv = _grads(q_rot, grads)
        ws = _workspace(q_rot, offsets, code, workspace)
        ws_ptr, ws_len = _ws_args(ws)
        rc = blockattn_rope_bwd(q_rot.data_ptr(), k_rot.data_ptr(), v.data_ptr(),
                                out.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                                offsets.data_ptr(), offsets.numel() - 1, T, H, D, block_size,
                                window_blocks, float(scale), float(theta_base), code,
                                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws_ptr, ws_len,
                                st.cuda_stream)
        del ws
    if rc != OK:
        raise BlockAttnError("blockattn_rope_bwd", rc)
    return dq, dk, dv


def gdpa_fwd(q, k, v, offsets, block_size: int, window_blocks: int, scale: float,
             activation: int, out=None, stream=None):
    """Generalized dot-product attention forward (blockattn_gdpa_fwd): the
    block pattern with P = act(scale q.k), no normalisation.  Returns out."""
    _check(q, k, v, offsets)
    T, H, D = q.shape
    st = _torch_stream(stream)
    with torch.cuda.stream(st):
        out = torch.empty_like(q) if out is None else out
        _check_like(q, out, what="out")
        rc = blockattn_gdpa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), offsets.data_ptr(),
                                offsets.numel() - 1, T, H, D, block_size, window_blocks,
                                float(scale), int(activation), _dtype_code(q), out.data_ptr(),
                                st.cuda_stream)
    if rc != OK:
        raise BlockAttnError("blockattn_gdpa_fwd", rc)
    return out


def gdpa_bwd(q, k, v, dout, offsets, block_size: int, window_blocks: int, scale: float,
             activation: int, grads=None, workspace=None, stream=None):
    """Generalized dot-product attention backward (blockattn_gdpa_bwd).
    Returns (dq, dk, dv)."""
    _check(q, k, v, offsets)
    T, H, D = q.shape
    _check_like(q, dout, what="dout")
    code = _dtype_code(q)
    st = _torch_stream(stream)
    with torch.cuda.stream(st):
        dq, dk, dv = _grads(q, grads)
        ws = _workspace(q, offsets, code, workspace)
        ws_ptr, ws_len = _ws_args(ws)
        rc = blockattn_gdpa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                                offsets.data_ptr(), offsets.numel() - 1, T, H, D, block_size,
                                window_blocks, float(scale), int(activation), code,
                                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws_ptr, ws_len,
                                st.cuda_stream)
        del ws
    if rc != OK:
        raise BlockAttnError("blockattn_gdpa_bwd", rc)
    return dq, dk, dv


def _check_mx_rows(dev, T, H, D, **ts):
    """E4M3 codes [T, H, D] and their E8M0 scales [H, T, D/32] (uint8)."""
    for n, t in ts.items():
        shape = (T, H, D) if not n.endswith("scale") else (H, T, D // 32)
        _check_tensor(t, shape, torch.uint8, dev, n)


def _check_mx_tok(dev, T, H, D, batch, **ts):
    """Token-blocked E4M3 codes [H, D, 32 nb] and scales [H, nb, D] (uint8),
    nb = ceil(T/32) + batch."""
    nb = -(-T // 32) + batch
    for n, t in ts.items():
        shape = (H, D, 32 * nb) if not n.endswith("scale") else (H, nb, D)
        _check_tensor(t, shape, torch.uint8, dev, n)


def mx_fwd(q, q_scale, k, k_scale, v, offsets, block_size: int, window_blocks: int,
           scale: float, out=None, lse=None, stream=None):
    """Forward with q and k in MXFP8 (blockattn_mx_fwd): q, k uint8 [T, H, D]
    E4M3 codes; q_scale, k_scale uint8 [H, T, D/32] E8M0 scales; v bf16.
    Returns (out bf16 [T, H, D], lse fp32 [H, T])."""
    if not isinstance(q, torch.Tensor) or q.dim() != 3 or not q.is_cuda:
        raise ValueError("q must be a [T, H, D] device tensor")
    T, H, D = q.shape
    dev = q.device
    _check_mx_rows(dev, T, H, D, q=q, q_scale=q_scale, k=k, k_scale=k_scale)
    _check_tensor(v, (T, H, D), torch.bfloat16, dev, "v")
    _check_offsets(offsets, dev)
    st = _torch_stream(stream)
    with torch.cuda.stream(st):
        out, lse = _outputs(q, out, lse, torch.bfloat16)
        rc = blockattn_mx_fwd(q.data_ptr(), q_scale.data_ptr(), k.data_ptr(),
                              k_scale.data_ptr(), v.data_ptr(), offsets.data_ptr(),
                              offsets.numel() - 1, T, H, D, block_size, window_blocks,
                              float(scale), out.data_ptr(), lse.data_ptr(), st.cuda_stream)
    if rc != OK:
        raise BlockAttnError("blockattn_mx_fwd", rc)
    return out, lse


def mxpv_fwd(q, q_scale, k, k_scale, v_t, v_scale, offsets, block_size: int,
             window_blocks: int, scale: float, out=None, lse=None, stream=None):
    """Forward with q, k and v in MXFP8 and the weights quantized for P.V
    (blockattn_mxpv_fwd): q, k uint8 [T, H, D] and q_scale, k_scale uint8
    [H, T, D/32] as for mx_fwd; v_t uint8 [H, D, 32 nb] (v transposed and
    blocked by user, padding with finite codes) and v_scale uint8 [H, nb, D]
    with nb = ceil(T/32) + batch (workloads.mx_v_device_layout builds them).
    Returns (out bf16 [T, H, D], lse fp32 [H, T])."""
    if not isinstance(q, torch.Tensor) or q.dim() != 3 or not q.is_cuda:
        raise ValueError("q must be a [T, H, D] device tensor")
    T, H, D = q.shape
    dev = q.device
    _check_offsets(offsets, dev)
    _check_mx_rows(dev, T, H, D, q=q, q_scale=q_scale, k=k, k_scale=k_scale)
    _check_mx_tok(dev, T, H, D, offsets.numel() - 1, v_t=v_t, v_scale=v_scale)
    st = _torch_stream(stream)
    with torch.cuda.stream(st):
        out, lse = _outputs(q, out, lse, torch.bfloat16)
        rc = blockattn_mxpv_fwd(q.data_ptr(), q_scale.data_ptr(), k.data_ptr(),
                                k_scale.data_ptr(), v_t.data_ptr(), v_scale.data_ptr(),
                                offsets.data_ptr(), offsets.numel() - 1, T, H, D, block_size,
                                window_blocks, float(scale), out.data_ptr(), lse.data_ptr(),
                                st.cuda_stream)
    if rc != OK:
        raise BlockAttnError("blockattn_mxpv_fwd", rc)
    return out, lse


def mx_bwd(q, q_scale, k, k_scale, v, v_scale, dout, dout_scale, q_t, q_t_scale, k_t,
           k_t_scale, dout_t, dout_t_scale, out, lse, offsets, block_size: int,
           window_blocks: int, scale: float, grads=None, workspace=None, stream=None):
    """MXFP8 backward (blockattn_mx_bwd).  q, k, v, dout uint8 [T, H, D] with
    scales uint8 [H, T, D/32] (head-dim blocks); q_t, k_t, dout_t uint8
    [H, D, 32 nb] with scales uint8 [H, nb, D] (token blocks, transposed,
    user-blocked: workloads.mx_v_device_layout builds them), nb =
    ceil(T/32) + batch; out bf16 [T, H, D] and lse fp32 [H, T] from the
    forward.  Returns (dq, dk, dv), bf16 [T, H, D]."""
    if not isinstance(q, torch.Tensor) or q.dim() != 3 or not q.is_cuda:
        raise ValueError("q must be a [T, H, D] device tensor")
    T, H, D = q.shape
    dev = q.device
    _check_offsets(offsets, dev)
    _check_mx_rows(dev, T, H, D, q=q, q_scale=q_scale, k=k, k_scale=k_scale, v=v,
                   v_scale=v_scale, dout=dout, dout_scale=dout_scale)
    _check_mx_tok(dev, T, H, D, offsets.numel() - 1, q_t=q_t, q_t_scale=q_t_scale, k_t=k_t,
                  k_t_scale=k_t_scale, dout_t=dout_t, dout_t_scale=dout_t_scale)
    _check_tensor(out, (T, H, D), torch.bfloat16, dev, "out")
    _check_lse(lse, H, T, dev)
    st = _torch_stream(stream)
    with torch.cuda.stream(st):
        dq, dk, dv = _grads(q, grads, torch.bfloat16)
        ws = _workspace(q, offsets, BF16, workspace)
        ws_ptr, ws_len = _ws_args(ws)
        rc = blockattn_mx_bwd(q.data_ptr(), q_scale.data_ptr(), k.data_ptr(), k_scale.data_ptr(),
                              v.data_ptr(), v_scale.data_ptr(), dout.data_ptr(),
                              dout_scale.data_ptr(), q_t.data_ptr(), q_t_scale.data_ptr(),
                              k_t.data_ptr(), k_t_scale.data_ptr(), dout_t.data_ptr(),
                              dout_t_scale.data_ptr(), out.data_ptr(), lse.data_ptr(),
                              offsets.data_ptr(), offsets.numel() - 1, T, H, D, block_size,
                              window_blocks, float(scale), dq.data_ptr(), dk.data_ptr(),
                              dv.data_ptr(), ws_ptr, ws_len, st.cuda_stream)
        del ws
    if rc != OK:
        raise BlockAttnError("blockattn_mx_bwd", rc)
    return dq, dk, dv
