"""The C-ABI library loads, exports every symbol include/blockattn.h declares,
and rejects invalid arguments before touching the GPU (no compute here)."""
import ctypes
import os
import re
import subprocess

import pytest

import long_sequence_block_amd as lsb
from long_sequence_block_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "blockattn.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(blockattn_[a-z_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = lsb.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", lsb.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(blockattn_\w+)", out))
    assert set(declared_functions()) <= exported


def test_version_and_status_strings():
    assert lsb.blockattn_abi_version() == 9
    names = [lsb.blockattn_status_string(s) for s in range(5)]
    assert len(set(names)) == 5 and names[0] == "ok"
    assert lsb.blockattn_status_string(99) == "unknown status"


FAKE = 0x1000  # aligned non-null pointer value; never dereferenced on these paths


def fwd_status(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, offsets=FAKE, batch=2, total_tokens=100,
             num_heads=2, head_dim=64, block_size=64, window_blocks=2, scale=0.125,
             dtype=lsb.BF16, out=FAKE, lse=FAKE, stream=None)
    a.update(kw)
    return lsb.blockattn_fwd(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), binding.ERR_INVALID_ARGUMENT),
    (dict(total_tokens=-5), binding.ERR_INVALID_ARGUMENT),
    (dict(num_heads=0), binding.ERR_INVALID_ARGUMENT),
    (dict(block_size=0), binding.ERR_INVALID_ARGUMENT),
    (dict(window_blocks=0), binding.ERR_INVALID_ARGUMENT),
    (dict(scale=float("nan")), binding.ERR_INVALID_ARGUMENT),
    (dict(scale=float("inf")), binding.ERR_INVALID_ARGUMENT),
    (dict(dtype=7), binding.ERR_INVALID_ARGUMENT),
    (dict(head_dim=48), binding.ERR_UNSUPPORTED),
    (dict(head_dim=256), binding.ERR_UNSUPPORTED),
    (dict(total_tokens=2**31, batch=1), binding.ERR_UNSUPPORTED),
    (dict(total_tokens=2**31 - 1000, batch=1), binding.ERR_UNSUPPORTED),
    # 128 rows of H * D elements must span less than 4 GiB (32-bit offsets)
    (dict(num_heads=200000, head_dim=128), binding.ERR_UNSUPPORTED),
    (dict(num_heads=2**31 - 1, head_dim=32), binding.ERR_UNSUPPORTED),
    # huge B and W are valid (clamped to T and ceil(T/B) without changing
    # the result); an empty call with them returns OK without launching
    (dict(block_size=2**31 - 1, window_blocks=2**31 - 1, total_tokens=0, q=None), binding.OK),
    (dict(q=None), binding.ERR_INVALID_ARGUMENT),
    (dict(lse=None), binding.ERR_INVALID_ARGUMENT),
    (dict(offsets=None), binding.ERR_INVALID_ARGUMENT),
    (dict(out=FAKE + 8), binding.ERR_INVALID_ARGUMENT),
    (dict(total_tokens=0, q=None, offsets=None), binding.OK),
    (dict(batch=0, q=None, offsets=None), binding.OK),
])
def test_fwd_argument_checks(kw, code):
    assert fwd_status(**kw) == code


def bwd_status(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, dout=FAKE, lse=FAKE, offsets=FAKE,
             batch=2, total_tokens=100, num_heads=2, head_dim=64, block_size=64,
             window_blocks=2, scale=0.125, dtype=lsb.BF16, dq=FAKE, dk=FAKE, dv=FAKE,
             workspace=FAKE, workspace_bytes=1 << 20, stream=None)
    a.update(kw)
    return lsb.blockattn_bwd(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(dout=None), binding.ERR_INVALID_ARGUMENT),
    (dict(dv=FAKE + 4), binding.ERR_INVALID_ARGUMENT),
    (dict(head_dim=16), binding.ERR_UNSUPPORTED),
    (dict(num_heads=200000, head_dim=128), binding.ERR_UNSUPPORTED),
    (dict(total_tokens=0, q=None, workspace=None), binding.OK),
])
def test_bwd_argument_checks(kw, code):
    assert bwd_status(**kw) == code


def test_noalloc_argument_checks():
    """blockattn_bwd_noalloc checks like blockattn_bwd, and a call whose
    workspace would exceed the static array returns the workspace error
    before any HIP call."""
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, dout=FAKE, lse=FAKE, offsets=FAKE,
             batch=2, total_tokens=100, num_heads=2, head_dim=48, block_size=64,
             window_blocks=2, scale=0.125, dtype=lsb.BF16, dq=FAKE, dk=FAKE, dv=FAKE,
             stream=None)
    assert lsb.blockattn_bwd_noalloc(*a.values()) == binding.ERR_UNSUPPORTED
    a.update(head_dim=64, dout=None)
    assert lsb.blockattn_bwd_noalloc(*a.values()) == binding.ERR_INVALID_ARGUMENT
    T = 4 << 20  # 2 * 4 B * 8 heads * T = 268 MB of row statistics > 64 MiB
    a.update(dout=FAKE, total_tokens=T, num_heads=8)
    assert lsb.blockattn_bwd_workspace_size(T, 2, 8, lsb.BF16) > lsb.NOALLOC_WORKSPACE_BYTES
    assert lsb.blockattn_bwd_noalloc(*a.values()) == binding.ERR_WORKSPACE
    a.update(total_tokens=0)
    assert lsb.blockattn_bwd_noalloc(*a.values()) == binding.OK


def test_sliding_window_argument_checks():
    """The sliding-window entry points check arguments like blockattn_fwd/bwd
    (window_tokens is the window in blocks of one token)."""
    a = dict(q=FAKE, k=FAKE, v=FAKE, offsets=FAKE, batch=2, total_tokens=100,
             num_heads=2, head_dim=64, window_tokens=0, scale=0.125, dtype=lsb.BF16,
             out=FAKE, lse=FAKE, stream=None)
    assert lsb.blockattn_swa_fwd(*a.values()) == binding.ERR_INVALID_ARGUMENT
    a.update(window_tokens=16, head_dim=96)
    assert lsb.blockattn_swa_fwd(*a.values()) == binding.ERR_UNSUPPORTED
    a.update(total_tokens=0, head_dim=64)
    assert lsb.blockattn_swa_fwd(*a.values()) == binding.OK
    b = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, dout=FAKE, lse=FAKE, offsets=FAKE,
             batch=2, total_tokens=100, num_heads=2, head_dim=64, window_tokens=-3,
             scale=0.125, dtype=lsb.BF16, dq=FAKE, dk=FAKE, dv=FAKE, workspace=FAKE,
             workspace_bytes=1 << 20, stream=None)
    assert lsb.blockattn_swa_bwd(*b.values()) == binding.ERR_INVALID_ARGUMENT
    b.update(window_tokens=8, workspace=None)
    assert lsb.blockattn_swa_bwd(*b.values()) == binding.ERR_WORKSPACE


def test_rope_argument_checks():
    a = dict(q=FAKE, k=FAKE, offsets=FAKE, batch=2, total_tokens=100, num_heads=2,
             head_dim=64, theta_base=0.0, dtype=lsb.BF16, q_rot=FAKE, k_rot=FAKE, stream=None)
    assert lsb.blockattn_rope(*a.values()) == binding.ERR_INVALID_ARGUMENT
    a.update(theta_base=float("inf"))
    assert lsb.blockattn_rope(*a.values()) == binding.ERR_INVALID_ARGUMENT
    a.update(theta_base=10000.0, head_dim=80)
    assert lsb.blockattn_rope(*a.values()) == binding.ERR_UNSUPPORTED
    a.update(head_dim=64, k_rot=FAKE + 2)
    assert lsb.blockattn_rope(*a.values()) == binding.ERR_INVALID_ARGUMENT
    a.update(k_rot=FAKE, total_tokens=0)
    assert lsb.blockattn_rope(*a.values()) == binding.OK
    b = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, dout=FAKE, lse=FAKE, offsets=FAKE,
             batch=2, total_tokens=100, num_heads=2, head_dim=64, block_size=64,
             window_blocks=2, scale=0.125, theta_base=-1.0, dtype=lsb.BF16, dq=FAKE,
             dk=FAKE, dv=FAKE, workspace=FAKE, workspace_bytes=1 << 20, stream=None)
    assert lsb.blockattn_rope_bwd(*b.values()) == binding.ERR_INVALID_ARGUMENT
    b.update(theta_base=10000.0, workspace=None)
    assert lsb.blockattn_rope_bwd(*b.values()) == binding.ERR_WORKSPACE


def test_gdpa_argument_checks():
    a = dict(q=FAKE, k=FAKE, v=FAKE, offsets=FAKE, batch=2, total_tokens=100, num_heads=2,
             head_dim=64, block_size=64, window_blocks=2, scale=0.125, activation=0,
             dtype=lsb.BF16, out=FAKE, stream=None)
    assert lsb.blockattn_gdpa_fwd(*a.values()) == binding.ERR_INVALID_ARGUMENT
    a.update(activation=3)
    assert lsb.blockattn_gdpa_fwd(*a.values()) == binding.ERR_INVALID_ARGUMENT
    a.update(activation=lsb.GDPA_GELU, out=None)
    assert lsb.blockattn_gdpa_fwd(*a.values()) == binding.ERR_INVALID_ARGUMENT
    a.update(out=FAKE, total_tokens=0)
    assert lsb.blockattn_gdpa_fwd(*a.values()) == binding.OK
    b = dict(q=FAKE, k=FAKE, v=FAKE, dout=FAKE, offsets=FAKE, batch=2, total_tokens=100,
             num_heads=2, head_dim=64, block_size=64, window_blocks=2, scale=0.125,
             activation=lsb.GDPA_SILU, dtype=lsb.BF16, dq=FAKE, dk=FAKE, dv=None,
             workspace=FAKE, workspace_bytes=1 << 20, stream=None)
    assert lsb.blockattn_gdpa_bwd(*b.values()) == binding.ERR_INVALID_ARGUMENT
    b.update(dv=FAKE, workspace=None)
    assert lsb.blockattn_gdpa_bwd(*b.values()) == binding.ERR_WORKSPACE


def test_mx_argument_checks():
    a = dict(q=FAKE, q_scale=FAKE, k=FAKE, k_scale=FAKE, v=FAKE, offsets=FAKE, batch=2,
             total_tokens=100, num_heads=2, head_dim=32, block_size=64, window_blocks=2,
             scale=0.125, out=FAKE, lse=FAKE, stream=None)
    assert lsb.blockattn_mx_fwd(*a.values()) == binding.ERR_UNSUPPORTED    # D = 32
    a.update(head_dim=64, k_scale=FAKE + 2)
    assert lsb.blockattn_mx_fwd(*a.values()) == binding.ERR_INVALID_ARGUMENT
    a.update(k_scale=FAKE, q=None)
    assert lsb.blockattn_mx_fwd(*a.values()) == binding.ERR_INVALID_ARGUMENT
    a.update(q=FAKE, total_tokens=0)
    assert lsb.blockattn_mx_fwd(*a.values()) == binding.OK


def test_workspace_size():
    r256 = lambda x: (x + 255) // 256 * 256
    assert lsb.blockattn_bwd_workspace_size(0, 4, 8, lsb.BF16) == 0
    assert lsb.blockattn_bwd_workspace_size(100, 0, 8, lsb.BF16) == 0
    assert lsb.blockattn_bwd_workspace_size(213551, 256, 8, lsb.FP32) == 0
    T, batch, H = 213551, 256, 8
    n = lsb.blockattn_bwd_workspace_size(T, batch, H, lsb.BF16)
    tiles = 2 * (-(-T // 128) + batch) * H
    assert n == 2 * r256(4 * H * T) + 256 + r256(4 * (batch + 1)) + r256(16 * tiles)
    bad = ctypes.c_size_t(-1).value
    assert lsb.blockattn_bwd_workspace_size(-1, 1, 8, lsb.BF16) == bad
    assert lsb.blockattn_bwd_workspace_size(10, -1, 8, lsb.BF16) == bad
    assert lsb.blockattn_bwd_workspace_size(10, 1, 0, lsb.BF16) == bad


def test_mxpv_argument_checks():
    """blockattn_mxpv_fwd: D 64 or 128, D * Tp below 2^32, v_t and v_scale
    present and aligned; empty calls succeed before any pointer is looked at."""
    a = dict(q=FAKE, q_scale=FAKE, k=FAKE, k_scale=FAKE, v_t=FAKE, v_scale=FAKE, offsets=FAKE,
             batch=2, total_tokens=100, num_heads=2, head_dim=32, block_size=64,
             window_blocks=2, scale=0.125, out=FAKE, lse=FAKE, stream=None)
    assert lsb.blockattn_mxpv_fwd(*a.values()) == binding.ERR_UNSUPPORTED    # D = 32
    a.update(head_dim=128, total_tokens=(1 << 25))     # 128 * 2^25 = 2^32
    assert lsb.blockattn_mxpv_fwd(*a.values()) == binding.ERR_UNSUPPORTED
    a.update(total_tokens=100, v_scale=FAKE + 2)
    assert lsb.blockattn_mxpv_fwd(*a.values()) == binding.ERR_INVALID_ARGUMENT
    a.update(v_scale=FAKE, v_t=FAKE + 8)
    assert lsb.blockattn_mxpv_fwd(*a.values()) == binding.ERR_INVALID_ARGUMENT
    a.update(v_t=None)
    assert lsb.blockattn_mxpv_fwd(*a.values()) == binding.ERR_INVALID_ARGUMENT
    a.update(v_t=FAKE, total_tokens=0)
    assert lsb.blockattn_mxpv_fwd(*a.values()) == binding.OK


def test_mx_bwd_argument_checks():
    """blockattn_mx_bwd: D 64 or 128, D * Tp below 2^32, every pointer present
    and aligned (16 bytes for codes, out, lse and gradients, 4 for scales),
    the workspace present, large enough and 256-byte aligned; empty calls
    succeed before any pointer is looked at."""
    a = dict(q=FAKE, q_scale=FAKE, k=FAKE, k_scale=FAKE, v=FAKE, v_scale=FAKE, dout=FAKE,
             dout_scale=FAKE, q_t=FAKE, q_t_scale=FAKE, k_t=FAKE, k_t_scale=FAKE, dout_t=FAKE,
             dout_t_scale=FAKE, out=FAKE, lse=FAKE, offsets=FAKE, batch=2, total_tokens=100,
             num_heads=2, head_dim=32, block_size=64, window_blocks=2, scale=0.125, dq=FAKE,
             dk=FAKE, dv=FAKE, workspace=FAKE, workspace_bytes=1 << 30, stream=None)
    call = lambda: lsb.blockattn_mx_bwd(*a.values())
    assert call() == binding.ERR_UNSUPPORTED                  # D = 32
    a.update(head_dim=128, total_tokens=(1 << 25))            # 128 * 2^25 = 2^32
    assert call() == binding.ERR_UNSUPPORTED
    a.update(total_tokens=100)
    for name, bad in (("dout_t_scale", FAKE + 2), ("k_t", FAKE + 8), ("q_t", None),
                      ("dv", FAKE + 4), ("lse", None), ("v_scale", FAKE + 1)):
        a[name] = bad
        assert call() == binding.ERR_INVALID_ARGUMENT, name
        a[name] = FAKE
    a.update(workspace=None)
    assert call() == binding.ERR_WORKSPACE
    a.update(workspace=FAKE, workspace_bytes=16)
    assert call() == binding.ERR_WORKSPACE
    a.update(workspace=FAKE + 16, workspace_bytes=1 << 30)
    assert call() == binding.ERR_WORKSPACE
    a.update(workspace=None, q=None, total_tokens=0)
    assert call() == binding.OK
