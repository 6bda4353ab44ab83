"""fp64 CPU oracle for block attention.

TEST INFRASTRUCTURE ONLY.  This package may be imported by the test suite,
by the smoke check and by the benchmark's CPU-baseline leg, and by nothing
else: the product path (the HIP library and its binding) never imports,
calls or links it, and the two share no code.

The arithmetic lives in ``blockattn_oracle.c`` (plain C, fp64, OpenMP over
(user, head) pairs); this module builds it with gcc and wraps it with ctypes.
What it computes, and the readings of the pages it rests on, are stated in
the header of that C file.  Pins that tie it to something other than itself
are in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "blockattn_oracle.c")
_LIB = os.path.join(_HERE, "libblockattn_oracle.so")
_lib = None


def build_oracle() -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build_oracle()
    lib = ctypes.CDLL(_LIB)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_fwd.argtypes = [dp, dp, dp, ip, i32, i64, i32, i32, i32, i32,
                               f64, dp, dp]
    lib.oracle_fwd.restype = ctypes.c_int
    lib.oracle_bwd.argtypes = [dp, dp, dp, dp, ip, i32, i64, i32, i32, i32,
                               i32, f64, dp, dp, dp]
    lib.oracle_bwd.restype = ctypes.c_int
    lib.oracle_probs.argtypes = [dp, dp, ip, i32, i64, i32, i32, i32, i32,
                                 f64, i32, i32, dp]
    lib.oracle_probs.restype = ctypes.c_int
    lib.oracle_gdpa_fwd.argtypes = [dp, dp, dp, ip, i32, i64, i32, i32, i32, i32,
                                    f64, i32, dp]
    lib.oracle_gdpa_fwd.restype = ctypes.c_int
    lib.oracle_gdpa_bwd.argtypes = [dp, dp, dp, dp, ip, i32, i64, i32, i32, i32,
                                    i32, f64, i32, dp, dp, dp]
    lib.oracle_gdpa_bwd.restype = ctypes.c_int
    lib.oracle_gdpa_fwd_abs.argtypes = lib.oracle_gdpa_fwd.argtypes
    lib.oracle_gdpa_fwd_abs.restype = ctypes.c_int
    lib.oracle_gdpa_bwd_abs.argtypes = lib.oracle_gdpa_bwd.argtypes
    lib.oracle_gdpa_bwd_abs.restype = ctypes.c_int
    lib.oracle_pair_count.argtypes = [ip, i32, i32, i32]
    lib.oracle_pair_count.restype = ctypes.c_int64
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
    lib.oracle_e4m3_round.argtypes = [f64]
    lib.oracle_e4m3_round.restype = ctypes.c_double
    lib.oracle_mxpv_fwd.argtypes = [dp, dp, dp, ip, i32, i64, i32, i32, i32, i32, f64, dp, dp]
    lib.oracle_mxpv_fwd.restype = ctypes.c_int
    lib.oracle_mxpv_slack.argtypes = [dp, dp, dp, ip, i32, i64, i32, i32, i32, i32, f64, dp,
                                      dp]
    lib.oracle_mxpv_slack.restype = ctypes.c_int
    lib.oracle_mx_bwd.argtypes = [dp] * 9 + [ip, i32, i64, i32, i32, i32, i32, f64, i32,
                                             dp, dp, dp]
    lib.oracle_mx_bwd.restype = ctypes.c_int
    lib.oracle_mx_bwd_bounds.argtypes = [dp] * 9 + [ip, i32, i64, i32, i32, i32, i32, f64,
                                                    f64] + [dp] * 9
    lib.oracle_mx_bwd_bounds.restype = ctypes.c_int
    lib.oracle_mx_quantize_block.argtypes = [dp, i64]
    lib.oracle_mx_quantize_block.restype = None
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _dp(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _ip(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def num_threads() -> int:
    """OpenMP threads the oracle runs with (OMP_NUM_THREADS or all cores)."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads of later oracle calls (results do not depend on it)."""
    _load().oracle_set_num_threads(int(n))


def pair_count(offsets, block_size: int, window_blocks: int) -> int:
    """Number of visible (query, key) pairs per head, summed over users."""
    off = _i32(offsets)
    r = _load().oracle_pair_count(_ip(off), len(off) - 1, int(block_size),
                                  int(window_blocks))
    if r < 0:
        raise ValueError("oracle_pair_count: invalid arguments")
    return int(r)


def fwd(q, k, v, offsets, block_size: int, window_blocks: int, scale: float):
    """Forward pass.  q, k, v: [T, H, D]; offsets: [batch+1].

    Returns (out [T, H, D] fp64, lse [H, T] fp64).
    """
    q, k, v, off = _f64(q), _f64(k), _f64(v), _i32(offsets)
    T, H, D = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [T, H, D] shape")
    out = np.zeros((T, H, D), np.float64)
    lse = np.zeros((H, T), np.float64)
    rc = _load().oracle_fwd(_dp(q), _dp(k), _dp(v), _ip(off), len(off) - 1, T,
                            H, D, int(block_size), int(window_blocks),
                            float(scale), _dp(out), _dp(lse))
    if rc != 0:
        raise ValueError(f"oracle_fwd failed with status {rc}")
    return out, lse


def bwd(q, k, v, dout, offsets, block_size: int, window_blocks: int,
        scale: float):
    """Backward pass.  Returns (dq, dk, dv), each [T, H, D] fp64."""
    q, k, v, do, off = _f64(q), _f64(k), _f64(v), _f64(dout), _i32(offsets)
    T, H, D = q.shape
    if k.shape != q.shape or v.shape != q.shape or do.shape != q.shape:
        raise ValueError("q, k, v, dout must share one [T, H, D] shape")
    dq = np.zeros((T, H, D), np.float64)
    dk = np.zeros((T, H, D), np.float64)
    dv = np.zeros((T, H, D), np.float64)
    rc = _load().oracle_bwd(_dp(q), _dp(k), _dp(v), _dp(do), _ip(off),
                            len(off) - 1, T, H, D, int(block_size),
                            int(window_blocks), float(scale), _dp(dq), _dp(dk),
                            _dp(dv))
    if rc != 0:
        raise ValueError(f"oracle_bwd failed with status {rc}")
    return dq, dk, dv


def probs(q, k, offsets, block_size: int, window_blocks: int, scale: float,
          user: int, head: int) -> np.ndarray:
    """Dense [L, L] attention-probability matrix of one (user, head)."""
    q, k, off = _f64(q), _f64(k), _i32(offsets)
    T, H, D = q.shape
    L = int(off[user + 1] - off[user])
    P = np.zeros((L, L), np.float64)
    rc = _load().oracle_probs(_dp(q), _dp(k), _ip(off), len(off) - 1, T, H, D,
                              int(block_size), int(window_blocks), float(scale),
                              int(user), int(head), _dp(P))
    if rc != 0:
        raise ValueError(f"oracle_probs failed with status {rc}")
    return P


# ------------------------------------ generalized dot-product attention
#
# The activation variant of the block pattern ("GEM (Meta)", section "Custom
# kernels": GDPA replaces the softmax by an activation such as GELU or SiLU).
# Definition and readings in blockattn_oracle.c.

GDPA_SILU, GDPA_GELU = 1, 2


def gdpa_fwd(q, k, v, offsets, block_size: int, window_blocks: int, scale: float,
             act: int, absolute: bool = False) -> np.ndarray:
    """out [T, H, D] fp64 of sum_j act(scale <q_i, k_j>) v_j over the block
    window (act 1 = SiLU, 2 = GELU).  absolute=True sums |terms| instead:
    sum_j |act(.)| |v_j|, the magnitude a per-term rounding error scales
    with."""
    q, k, v, off = _f64(q), _f64(k), _f64(v), _i32(offsets)
    T, H, D = q.shape
    out = np.zeros((T, H, D), np.float64)
    fn = _load().oracle_gdpa_fwd_abs if absolute else _load().oracle_gdpa_fwd
    rc = fn(_dp(q), _dp(k), _dp(v), _ip(off), len(off) - 1, T, H, D,
                                 int(block_size), int(window_blocks), float(scale), int(act),
                                 _dp(out))
    if rc != 0:
        raise ValueError(f"oracle_gdpa_fwd failed with status {rc}")
    return out


def gdpa_bwd(q, k, v, dout, offsets, block_size: int, window_blocks: int, scale: float,
             act: int, absolute: bool = False):
    """(dq, dk, dv) of sum(dout * gdpa_fwd(...)), each [T, H, D] fp64.
    absolute=True sums |terms| instead (|scale| sum_j |dS_ij| |k_j|, ...)."""
    q, k, v, do, off = _f64(q), _f64(k), _f64(v), _f64(dout), _i32(offsets)
    T, H, D = q.shape
    dq, dk, dv = (np.zeros((T, H, D), np.float64) for _ in range(3))
    fn = _load().oracle_gdpa_bwd_abs if absolute else _load().oracle_gdpa_bwd
    rc = fn(_dp(q), _dp(k), _dp(v), _dp(do), _ip(off), len(off) - 1, T,
                                 H, D, int(block_size), int(window_blocks), float(scale),
                                 int(act), _dp(dq), _dp(dk), _dp(dv))
    if rc != 0:
        raise ValueError(f"oracle_gdpa_bwd failed with status {rc}")
    return dq, dk, dv


# ------------------------------------------------------------------ MXFP8
#
# "GEM (Meta)", section "Custom kernels", says production attention runs in
# MXFP8, a block-scaled FP8 format, and names nothing more.  The reading is
# the OCP Microscaling format: elements are E4M3 bytes (sign, 4-bit exponent
# with bias 7, 3-bit mantissa; exponent field 0 is subnormal, m * 2^-9; the
# code with all exponent and mantissa bits set is NaN; no infinities), and
# every 32 consecutive elements along the head dim share one E8M0 scale
# byte, 2^(s - 127) (255 is NaN).  Decoding is exact in fp64.


def e4m3_value(code: int) -> float:
    """Value of one E4M3 byte, from its bit fields."""
    s, e, m = (code >> 7) & 1, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    v = m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


_E4M3 = np.array([e4m3_value(c) for c in range(256)], np.float64)


def mx_decode(codes, scales) -> np.ndarray:
    """fp64 values of MXFP8 data: codes uint8 [..., D], scales uint8
    [..., D/32] (scale j covers elements 32j .. 32j + 31)."""
    codes, scales = np.asarray(codes, np.uint8), np.asarray(scales, np.uint8)
    if codes.shape[-1] != 32 * scales.shape[-1] or codes.shape[:-1] != scales.shape[:-1]:
        raise ValueError("one scale per 32 elements of the last axis")
    f = np.where(scales == 255, np.nan, np.ldexp(1.0, scales.astype(np.int64) - 127))
    return _E4M3[codes] * np.repeat(f, 32, axis=-1)


def user_block_base(offsets) -> np.ndarray:
    """First 32-token block of each user in user-blocked MXFP8 data:
    ceil(offsets[u] / 32) + u, so user u's blocks (ceil(L_u / 32) of them)
    never meet the next user's; [batch] int64."""
    off = np.asarray(offsets, np.int64)
    return -(-off[:-1] // 32) + np.arange(len(off) - 1)


def mx_decode_user_blocks(codes, scales, offsets) -> np.ndarray:
    """fp64 values of MXFP8 data blocked along each user's tokens: codes
    uint8 [T, H, D], scales uint8 [nblocks, H, D]; local token j of user u
    has scale row user_block_base(offsets)[u] + j // 32."""
    codes, scales = np.asarray(codes, np.uint8), np.asarray(scales, np.uint8)
    off = np.asarray(offsets, np.int64)
    blk = np.zeros(codes.shape[0], np.int64)
    base = user_block_base(off)
    for u in range(len(off) - 1):
        blk[off[u]:off[u + 1]] = base[u] + np.arange(off[u + 1] - off[u]) // 32
    if len(blk) and (blk.max() >= scales.shape[0] or codes.shape[1:] != scales.shape[1:]):
        raise ValueError("scales [nblocks, H, D] cover every user's blocks")
    sc = scales[blk]
    f = np.where(sc == 255, np.nan, np.ldexp(1.0, sc.astype(np.int64) - 127))
    return _E4M3[codes] * f


def e4m3_round(x) -> np.ndarray:
    """Nearest E4M3 value (ties to even) of each x >= 0 below 2^8 + 2^4."""
    x = np.asarray(x, np.float64)
    f = _load().oracle_e4m3_round
    return np.array([f(float(v)) for v in x.ravel()], np.float64).reshape(x.shape)


def mxpv_fwd(q, k, v, offsets, block_size: int, window_blocks: int, scale: float):
    """Forward with the weights quantized to MXFP8 for the P.V product
    (blockattn_oracle.c: oracle_mxpv_fwd): (out [T, H, D], lse [H, T])."""
    q, k, v, off = _f64(q), _f64(k), _f64(v), _i32(offsets)
    T, H, D = q.shape
    out = np.zeros((T, H, D), np.float64)
    lse = np.zeros((H, T), np.float64)
    rc = _load().oracle_mxpv_fwd(_dp(q), _dp(k), _dp(v), _ip(off), len(off) - 1, T, H, D,
                                 int(block_size), int(window_blocks), float(scale), _dp(out),
                                 _dp(lse))
    if rc != 0:
        raise ValueError(f"oracle_mxpv_fwd failed with status {rc}")
    return out, lse


def mxpv_slack(q, k, v, offsets, block_size: int, window_blocks: int, scale: float, eps2):
    """Per-element parity allowance [T, H, D] of mxpv_fwd's out for a
    computation whose t_ij = s_ij log2(e) are off by at most eps2 [H, T]
    (blockattn_oracle.c: oracle_mxpv_slack).  Test support."""
    q, k, v, off = _f64(q), _f64(k), _f64(v), _i32(offsets)
    T, H, D = q.shape
    e = _f64(np.broadcast_to(np.asarray(eps2, np.float64), (H, T)))
    sl = np.zeros((T, H, D), np.float64)
    rc = _load().oracle_mxpv_slack(_dp(q), _dp(k), _dp(v), _ip(off), len(off) - 1, T, H, D,
                                   int(block_size), int(window_blocks), float(scale), _dp(e),
                                   _dp(sl))
    if rc != 0:
        raise ValueError(f"oracle_mxpv_slack failed with status {rc}")
    return sl


def _mx_bwd_inputs(q, k, v, dout, out, lse, q_t, k_t, dout_t):
    q, k, v, do, o = _f64(q), _f64(k), _f64(v), _f64(dout), _f64(out)
    qt, kt, dt = _f64(q_t), _f64(k_t), _f64(dout_t)
    T, H, D = q.shape
    for a in (k, v, do, o, qt, kt, dt):
        if a.shape != q.shape:
            raise ValueError("every tensor must share one [T, H, D] shape")
    ls = _f64(lse)
    if ls.shape != (H, T):
        raise ValueError("lse must be [H, T]")
    return (q, k, v, do, o, ls, qt, kt, dt), (T, H, D)


def mx_bwd(q, k, v, dout, out, lse, q_t, k_t, dout_t, offsets, block_size: int,
           window_blocks: int, scale: float, quantize: bool = True):
    """MXFP8 backward (blockattn_oracle.c: oracle_mx_bwd).  q, k, v, dout:
    decoded head-dim-blocked values; q_t, k_t, dout_t: decoded token-blocked
    values; out, lse: the forward's.  Returns (dq, dk, dv) [T, H, D] fp64.
    quantize=False skips the quantization of P and dS."""
    ins, (T, H, D) = _mx_bwd_inputs(q, k, v, dout, out, lse, q_t, k_t, dout_t)
    off = _i32(offsets)
    res = [np.zeros((T, H, D), np.float64) for _ in range(3)]
    rc = _load().oracle_mx_bwd(*[_dp(a) for a in ins], _ip(off), len(off) - 1, T, H, D,
                               int(block_size), int(window_blocks), float(scale),
                               int(bool(quantize)), *[_dp(a) for a in res])
    if rc != 0:
        raise ValueError(f"oracle_mx_bwd failed with status {rc}")
    return tuple(res)


def mx_quantize_block(x) -> np.ndarray:
    """The backward's block rule (blockattn_oracle.c: mx_block) on one block
    of values: returns the quantized copy."""
    y = _f64(x).copy()
    _load().oracle_mx_quantize_block(_dp(y), y.size)
    return y


def mx_bwd_bounds(q, k, v, dout, out, lse, q_t, k_t, dout_t, offsets, block_size: int,
                  window_blocks: int, scale: float, rho: float):
    """mx_bwd's (dq, dk, dv) with their parity allowances (test support;
    blockattn_oracle.c: oracle_mx_bwd_bounds): returns (ref, slack, absum),
    each a tuple (dq, dk, dv) of [T, H, D] fp64."""
    ins, (T, H, D) = _mx_bwd_inputs(q, k, v, dout, out, lse, q_t, k_t, dout_t)
    off = _i32(offsets)
    res = [np.zeros((T, H, D), np.float64) for _ in range(9)]
    rc = _load().oracle_mx_bwd_bounds(*[_dp(a) for a in ins], _ip(off), len(off) - 1, T, H,
                                      D, int(block_size), int(window_blocks), float(scale),
                                      float(rho), *[_dp(a) for a in res])
    if rc != 0:
        raise ValueError(f"oracle_mx_bwd_bounds failed with status {rc}")
    return tuple(res[0:3]), tuple(res[3:6]), tuple(res[6:9])


# ------------------------------------------------- rotary position embedding
#
# The production block-attention kernel fuses the backward of a rotary
# position embedding ("GEM (Meta)" on aiwiki.ai, section "Custom kernels").
# The pages name the embedding but not its variant, base or positions.  The
# readings taken: the rotate-half form (feature d pairs with d + D/2), the
# angle of pair d at position p is p * base**(-2d/D) with base 10000 unless
# given, and p is the token's index inside its own user (positions restart
# at every user, like the blocks).  Applied to Q and K only.  Plain numpy,
# fp64.


def rope_positions(offsets) -> np.ndarray:
    """Local index of every packed token inside its user, [T] int64."""
    off = _i32(offsets)
    pos = np.zeros(int(off[-1]), np.int64)
    for u in range(len(off) - 1):
        pos[off[u]:off[u + 1]] = np.arange(off[u + 1] - off[u])
    return pos


def rope_angles(offsets, head_dim: int, base: float = 10000.0) -> np.ndarray:
    """[T, D/2] rotation angles: position times base**(-2d/D)."""
    if head_dim % 2:
        raise ValueError("rotary embedding needs an even head dim")
    d = np.arange(head_dim // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * d / head_dim)
    return rope_positions(offsets).astype(np.float64)[:, None] * theta[None, :]


def _rotate(x, offsets, base, sign):
    x = _f64(x)
    T, H, D = x.shape
    a = rope_angles(offsets, D, base)[:, None, :]        # [T, 1, D/2]
    c, s = np.cos(a), sign * np.sin(a)
    lo, hi = x[..., :D // 2], x[..., D // 2:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def rope(x, offsets, base: float = 10000.0) -> np.ndarray:
    """Rotate every (token, head) row of x [T, H, D]: each pair
    (x_d, x_{d+D/2}) turns by its angle."""
    return _rotate(x, offsets, base, 1.0)


def rope_transpose(x, offsets, base: float = 10000.0) -> np.ndarray:
    """The transpose (inverse) rotation, which is the backward of rope."""
    return _rotate(x, offsets, base, -1.0)


def rope_bwd(q_rot, k_rot, v, dout, offsets, block_size: int, window_blocks: int,
             scale: float, base: float = 10000.0):
    """Gradients with respect to the unrotated q and k (and v) of
    sum(dout * attention(q_rot, k_rot, v)) where q_rot and k_rot are the
    rotated q and k: the attention backward on the rotated inputs, then the
    chain rule through the rotation, which is its transpose."""
    dqr, dkr, dv = bwd(q_rot, k_rot, v, dout, offsets, block_size, window_blocks, scale)
    return rope_transpose(dqr, offsets, base), rope_transpose(dkr, offsets, base), dv
