"""Seeded synthetic workloads for block attention.

This module only draws random numbers and lays them out; it holds none of
the attention arithmetic.  It is the one module that the oracle-side tests
and the GPU path both use, so that both see identical inputs.

The pages measure on production user-engagement histories ("GEM (Meta)",
sections "Architecture" and "Training infrastructure": histories from
hundreds to tens of thousands of events, jagged per user; section "Custom
kernels": 64-token blocks).  No public dataset is named, so seeded synthetic
sequences of those shapes stand in for them:

* lengths, for the jagged workloads: lognormal with median 600 (mu = ln 600)
  and sigma 0.8 in log space, rounded to the nearest integer and clipped to
  [16, 4096]; offsets are the int32 exclusive prefix sum;
* Q, K, V and the upstream gradient dO: i.i.d. standard normal float32 of
  shape [T, H, D]; the bf16 workloads round them to bf16 (round to nearest
  even) on the way to the device, and the oracle sees those rounded values;
* scale = 1/sqrt(D).

Random streams: numpy ``Generator(PCG64(SeedSequence([workload, stream])))``
with stream 0 = lengths, 1 = Q, 2 = K, 3 = V, 4 = dO.  The training-step
workload reuses the jagged workload's lengths and Q/K/V (workload id 3) and
draws dO from [5, 4]; the sliding-window training workload uses the same
inputs.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

STREAM_LENGTHS, STREAM_Q, STREAM_K, STREAM_V, STREAM_DO = 0, 1, 2, 3, 4
STREAM_QMX, STREAM_QSC, STREAM_KMX, STREAM_KSC = 5, 6, 7, 8
STREAM_VMX, STREAM_VSC = 9, 10
# the MXFP8 backward's head-dim-blocked v and dO, and token-blocked q, k, dO
STREAM_VHMX, STREAM_VHSC, STREAM_DOMX, STREAM_DOSC = 11, 12, 13, 14
STREAM_QTMX, STREAM_QTSC, STREAM_KTMX, STREAM_KTSC, STREAM_DOTMX, STREAM_DOTSC = range(15, 21)


def rng(workload: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([workload, stream])))


@dataclasses.dataclass(frozen=True)
class Workload:
    """A synthetic block-attention workload (sizes only; draws are lazy)."""
    wid: int                 # seed id of the lengths and Q/K/V streams
    name: str
    users: int
    heads: int
    head_dim: int
    block_size: int
    window_blocks: int
    dtype: str               # "fp32" or "bf16"
    backward: bool
    fixed_length: int = 0    # >0: every user has this length
    dout_wid: int = 0        # seed id of the dO stream (backward only)
    rope_base: float = 0.0   # >0: rotary embedding of q and k with this base
    act: int = 0             # 0 softmax; 1 SiLU, 2 GELU (generalized dot-product attention)
    mx: bool = False         # q and k as MXFP8 codes and block scales
    mx_v: bool = False       # v too (scales along tokens), weights quantized for P.V

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def lengths(self) -> np.ndarray:
        if self.fixed_length > 0:
            return np.full(self.users, self.fixed_length, dtype=np.int32)
        return lognormal_lengths(self.wid, self.users)

    def offsets(self) -> np.ndarray:
        return offsets_from_lengths(self.lengths())


def lognormal_lengths(wid: int, users: int, median: float = 600.0,
                      sigma: float = 0.8, lo: int = 16, hi: int = 4096) -> np.ndarray:
    g = rng(wid, STREAM_LENGTHS)
    x = g.lognormal(mean=math.log(median), sigma=sigma, size=users)
    return np.clip(np.rint(x), lo, hi).astype(np.int32)


def offsets_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    if off[-1] > np.iinfo(np.int32).max:
        raise ValueError("total token count does not fit int32 offsets")
    return off.astype(np.int32)


def mx_codes(wid: int, stream: int, shape) -> np.ndarray:
    """Random MXFP8 element codes (OCP E4M3 bytes: sign, 4-bit exponent field,
    3-bit mantissa).  Sign and mantissa uniform, exponent field uniform in
    [9, 15], the NaN code excluded: magnitudes 4 .. 448, the range an MX block
    of N(0, 1) values fills once its scale maps the block maximum near 448."""
    g = rng(wid, stream)
    sign = g.integers(0, 2, size=shape, dtype=np.uint8)
    expo = g.integers(9, 16, size=shape, dtype=np.uint8)
    mant = g.integers(0, 8, size=shape, dtype=np.uint8)
    mant = np.where((expo == 15) & (mant == 7), np.uint8(6), mant)
    return ((sign << 7) | (expo << 3) | mant).astype(np.uint8)


def mx_scales(wid: int, stream: int, shape, lo: int = 119, hi: int = 121) -> np.ndarray:
    """Random E8M0 block scales (biased exponents) uniform in lo .. hi; the
    default 119 .. 121 is 2^-8 .. 2^-6, which with the codes above gives
    values of magnitude 0.016 .. 3.5."""
    return rng(wid, stream).integers(lo, hi + 1, size=shape, dtype=np.uint8)


def mx_codes_all(wid: int, stream: int, shape) -> np.ndarray:
    """Random E4M3 codes uniform over all 254 finite codes: both zeros, the
    subnormals (exponent field 0) and every normal exponent up to 448; only
    the two NaN codes (0x7F, 0xFF) are left out."""
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    return finite[rng(wid, stream).integers(0, finite.size, size=shape)]


def normal(wid: int, stream: int, shape) -> np.ndarray:
    """i.i.d. N(0, 1) float32 draws for one tensor."""
    return rng(wid, stream).standard_normal(size=shape, dtype=np.float32)


WORKLOADS = {
    1: Workload(1, "tiny-fp32", users=2, heads=1, head_dim=32, block_size=32,
                window_blocks=1, dtype="fp32", backward=False, fixed_length=256),
    2: Workload(2, "fixed-bf16", users=64, heads=4, head_dim=64, block_size=64,
                window_blocks=2, dtype="bf16", backward=False, fixed_length=1024),
    3: Workload(3, "jagged-bf16", users=256, heads=8, head_dim=64, block_size=128,
                window_blocks=2, dtype="bf16", backward=False),
    4: Workload(4, "long-context-bf16", users=32, heads=8, head_dim=128,
                block_size=256, window_blocks=4, dtype="bf16", backward=False,
                fixed_length=16384),
    5: Workload(3, "jagged-bf16-train", users=256, heads=8, head_dim=64,
                block_size=128, window_blocks=2, dtype="bf16", backward=True,
                dout_wid=5),
    # The token sliding window (blocks of one token) on the training step's
    # inputs, with the window whose visible-pair count is closest to the
    # block pattern's (194 tokens: 36,689,648 pairs per head against
    # 36,616,647), so that both do the same algorithmic work.
    6: Workload(3, "sliding-window-bf16-train", users=256, heads=8, head_dim=64,
                block_size=1, window_blocks=194, dtype="bf16", backward=True,
                dout_wid=5),
    # The training step with the rotary embedding the production kernel
    # carries: rotate q and k, attend, and take the gradients through both.
    7: Workload(3, "jagged-bf16-train-rope", users=256, heads=8, head_dim=64,
                block_size=128, window_blocks=2, dtype="bf16", backward=True,
                dout_wid=5, rope_base=10000.0),
    # The long-context and jagged forwards with q and k in MXFP8 (the score
    # product on the block-scaled fp8 matrix cores; v stays bf16).
    9: Workload(4, "long-context-mxfp8qk", users=32, heads=8, head_dim=128,
                block_size=256, window_blocks=4, dtype="bf16", backward=False,
                fixed_length=16384, mx=True),
    10: Workload(3, "jagged-mxfp8qk", users=256, heads=8, head_dim=64, block_size=128,
                 window_blocks=2, dtype="bf16", backward=False, mx=True),
    # The long-context shape as a training step: forward and backward at
    # head dimension 128 (dO drawn from its own seed).
    11: Workload(4, "long-context-bf16-train", users=32, heads=8, head_dim=128,
                 block_size=256, window_blocks=4, dtype="bf16", backward=True,
                 fixed_length=16384, dout_wid=11),
    # The training step with SiLU scores in place of the softmax (generalized
    # dot-product attention on the block pattern).
    8: Workload(3, "jagged-bf16-train-gdpa-silu", users=256, heads=8, head_dim=64,
                block_size=128, window_blocks=2, dtype="bf16", backward=True,
                dout_wid=5, act=1),
    # The long-context and jagged forwards with q, k and v in MXFP8 and the
    # softmax weights quantized for a block-scaled P.V product.
    13: Workload(4, "long-context-mxfp8", users=32, heads=8, head_dim=128,
                 block_size=256, window_blocks=4, dtype="bf16", backward=False,
                 fixed_length=16384, mx=True, mx_v=True),
    14: Workload(3, "jagged-mxfp8", users=256, heads=8, head_dim=64, block_size=128,
                 window_blocks=2, dtype="bf16", backward=False, mx=True, mx_v=True),
    # The same two shapes as MXFP8 training steps: that forward, then the
    # backward with every product block-scaled (q, k, v and dO head-dim-
    # blocked, q, k and dO also token-blocked; mx_bwd_draw).
    15: Workload(3, "jagged-mxfp8-train", users=256, heads=8, head_dim=64, block_size=128,
                 window_blocks=2, dtype="bf16", backward=True, dout_wid=5, mx=True,
                 mx_v=True),
    16: Workload(4, "long-context-mxfp8-train", users=32, heads=8, head_dim=128,
                 block_size=256, window_blocks=4, dtype="bf16", backward=True,
                 fixed_length=16384, dout_wid=11, mx=True, mx_v=True),
    # The training step at a local batch of 1024 users (the pages put local
    # batches above 1,000 samples), same length law and shapes.
    12: Workload(12, "jagged-bf16-1024-train", users=1024, heads=8, head_dim=64,
                 block_size=128, window_blocks=2, dtype="bf16", backward=True,
                 dout_wid=12),
}

# Length sweep of the long-context workload (time should grow linearly).
LONG_CONTEXT_SWEEP = (2048, 4096, 8192, 16384)


def long_context(length: int) -> Workload:
    w = WORKLOADS[4]
    return dataclasses.replace(w, fixed_length=int(length),
                               name=f"long-context-bf16-L{length}")


def draw(w: Workload, users=None):
    """Draw the tensors of a workload.

    Returns a dict with ``offsets`` (int32 [batch+1]) and float32 numpy
    arrays ``q``, ``k``, ``v`` (and ``dout`` for backward workloads) of shape
    [T, H, D].  ``users`` (a slice) keeps only those users' rows; draws are
    made for the whole workload first so a subset matches the full run.
    """
    off = w.offsets()
    T = int(off[-1])
    shape = (T, w.heads, w.head_dim)
    if w.mx:
        sshape = (T, w.heads, w.head_dim // 32)
        out = {"offsets": off,
               "q_mx": mx_codes(w.wid, STREAM_QMX, shape),
               "q_sc": mx_scales(w.wid, STREAM_QSC, sshape),
               "k_mx": mx_codes(w.wid, STREAM_KMX, shape),
               "k_sc": mx_scales(w.wid, STREAM_KSC, sshape)}
        if w.mx_v:
            out.update(mx_v_draw(w.wid, off, w.heads, w.head_dim))
        else:
            out["v"] = normal(w.wid, STREAM_V, shape)
    else:
        out = {"offsets": off,
               "q": normal(w.wid, STREAM_Q, shape),
               "k": normal(w.wid, STREAM_K, shape),
               "v": normal(w.wid, STREAM_V, shape)}
    if w.backward and w.mx:
        out.update(mx_bwd_draw(w.wid, w.dout_wid, off, w.heads, w.head_dim))
    elif w.backward:
        out["dout"] = normal(w.dout_wid, STREAM_DO, shape)
    if users is not None:
        out = subset_users(out, users)
    return out


def user_block_base(offsets) -> np.ndarray:
    """First 32-token block of each user in user-blocked MXFP8 data:
    ceil(offsets[u] / 32) + u, so user u's ceil(L_u / 32) blocks never meet
    the next user's (index arithmetic only)."""
    off = np.asarray(offsets, np.int64)
    return -(-off[:-1] // 32) + np.arange(len(off) - 1)


def mx_v_blocks(offsets) -> int:
    """Block rows of user-blocked MXFP8 data: ceil(T / 32) + batch."""
    off = np.asarray(offsets, np.int64)
    return int(-(-off[-1] // 32)) + len(off) - 1


def mx_tok_draw(name: str, wid: int, streams, offsets, heads: int, head_dim: int,
                scales=(119, 121), codes=None):
    """A tensor as MXFP8 blocked along each user's tokens: codes
    ``<name>_mx`` uint8 [T, H, D] (the mx_codes draw, or ``codes`` =
    mx_codes_all) and block scales ``<name>_bsc`` uint8
    [ceil(T/32) + batch, H, D]; local token j of user u has scale row
    user_block_base(offsets)[u] + j // 32.  streams = (codes, scales)."""
    fn = mx_codes if codes is None else codes
    T = int(np.asarray(offsets)[-1])
    return {name + "_mx": fn(wid, streams[0], (T, heads, head_dim)),
            name + "_bsc": mx_scales(wid, streams[1], (mx_v_blocks(offsets), heads, head_dim),
                                     *scales)}


def mx_v_draw(wid: int, offsets, heads: int, head_dim: int, scales=(119, 121), codes=None):
    """v as MXFP8 blocked along each user's tokens (mx_tok_draw): ``v_mx``
    and ``v_bsc``."""
    return mx_tok_draw("v", wid, (STREAM_VMX, STREAM_VSC), offsets, heads, head_dim, scales,
                       codes)


def mx_bwd_draw(wid: int, dout_wid: int, offsets, heads: int, head_dim: int, wide=None):
    """The MXFP8 backward's further inputs, each an independent seeded draw
    (a producer would quantize one tensor twice; the draws stand in for both
    copies with the same code and scale ranges): head-dim-blocked v
    (``vh_mx``, ``vh_sc``) and dO (``do_mx``, ``do_sc``), codes [T, H, D] and
    scales [T, H, D/32]; token-blocked q, k and dO (``qt_``, ``kt_``,
    ``dot_`` + ``mx`` / ``bsc``, as mx_tok_draw).  dO's draws use dout_wid.
    wide: five scale ranges (vh, do, qt, kt, dot) with codes over every
    finite E4M3 code."""
    T = int(np.asarray(offsets)[-1])
    shape, sshape = (T, heads, head_dim), (T, heads, head_dim // 32)
    fn = mx_codes if wide is None else mx_codes_all
    rg = [(119, 121)] * 5 if wide is None else list(wide)
    out = {"vh_mx": fn(wid, STREAM_VHMX, shape),
           "vh_sc": mx_scales(wid, STREAM_VHSC, sshape, *rg[0]),
           "do_mx": fn(dout_wid, STREAM_DOMX, shape),
           "do_sc": mx_scales(dout_wid, STREAM_DOSC, sshape, *rg[1])}
    cf = None if wide is None else mx_codes_all
    out.update(mx_tok_draw("qt", wid, (STREAM_QTMX, STREAM_QTSC), offsets, heads, head_dim,
                           rg[2], cf))
    out.update(mx_tok_draw("kt", wid, (STREAM_KTMX, STREAM_KTSC), offsets, heads, head_dim,
                           rg[3], cf))
    out.update(mx_tok_draw("dot", dout_wid, (STREAM_DOTMX, STREAM_DOTSC), offsets, heads,
                           head_dim, rg[4], cf))
    return out


def mx_v_device_layout(v_mx: np.ndarray, v_bsc: np.ndarray, offsets):
    """The C ABI's layout of user-blocked MXFP8 v: codes transposed to
    [H, D, 32 (ceil(T/32) + batch)], user u's local token j at column
    32 user_block_base[u] + j (the rest: code 0, i.e. +0), and scales to
    [H, ceil(T/32) + batch, D]."""
    off = np.asarray(offsets, np.int64)
    T, H, D = v_mx.shape
    nb = mx_v_blocks(off)
    vt = np.zeros((H, D, 32 * nb), np.uint8)
    base = user_block_base(off)
    for u in range(len(off) - 1):
        a, b = int(off[u]), int(off[u + 1])
        vt[:, :, 32 * base[u]:32 * base[u] + b - a] = v_mx[a:b].transpose(1, 2, 0)
    return vt, np.ascontiguousarray(v_bsc.transpose(1, 0, 2))


def subset_users(tensors: dict, users: slice) -> dict:
    """Keep a contiguous range of users (rows and re-based offsets).  User
    block scales (keys ending in ``_bsc``) are re-indexed for the kept
    users' new positions."""
    off = tensors["offsets"]
    idx = np.arange(len(off) - 1)[users]
    if len(idx) == 0:
        lo = hi = 0
    else:
        if np.any(np.diff(idx) != 1):
            raise ValueError("subset_users needs a contiguous range")
        lo, hi = int(off[idx[0]]), int(off[idx[-1] + 1])
    res = {"offsets": (off[idx[0]: idx[-1] + 2] - lo).astype(np.int32)
           if len(idx) else np.zeros(1, np.int32)}
    for key, val in tensors.items():
        if key.endswith("_bsc"):
            new_off = res["offsets"]
            out = np.zeros((mx_v_blocks(new_off),) + val.shape[1:], val.dtype)
            old_base, new_base = user_block_base(off), user_block_base(new_off)
            for i, u in enumerate(idx):
                n = -(-int(off[u + 1] - off[u]) // 32)
                out[new_base[i]:new_base[i] + n] = val[old_base[u]:old_base[u] + n]
            res[key] = out
        elif key != "offsets":
            res[key] = val[lo:hi]
    return res


def random_case(seed: int, lengths, heads: int, head_dim: int, with_dout=True):
    """Small seeded case for tests: given per-user lengths, N(0,1) tensors."""
    off = offsets_from_lengths(lengths)
    T = int(off[-1])
    shape = (T, heads, head_dim)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000, seed])))
    out = {"offsets": off,
           "q": g.standard_normal(size=shape, dtype=np.float32),
           "k": g.standard_normal(size=shape, dtype=np.float32),
           "v": g.standard_normal(size=shape, dtype=np.float32)}
    if with_dout:
        out["dout"] = g.standard_normal(size=shape, dtype=np.float32)
    return out


def random_mx_case(seed: int, lengths, heads: int, head_dim: int, wide=None):
    """Small seeded case with q and k as MXFP8 codes and block scales (the
    draws of mx_codes / mx_scales) and v as N(0, 1).

    wide = ((q_lo, q_hi), (k_lo, k_hi)): codes from all finite E4M3 codes
    (mx_codes_all) and block scales uniform in those biased-exponent ranges
    instead."""
    off = offsets_from_lengths(lengths)
    T = int(off[-1])
    shape, sshape = (T, heads, head_dim), (T, heads, head_dim // 32)
    wid = 2000 + seed
    if wide is not None:
        (qlo, qhi), (klo, khi) = wide
        return {"offsets": off,
                "q_mx": mx_codes_all(wid, STREAM_QMX, shape),
                "q_sc": mx_scales(wid, STREAM_QSC, sshape, qlo, qhi),
                "k_mx": mx_codes_all(wid, STREAM_KMX, shape),
                "k_sc": mx_scales(wid, STREAM_KSC, sshape, klo, khi),
                "v": normal(wid, STREAM_V, shape)}
    return {"offsets": off,
            "q_mx": mx_codes(wid, STREAM_QMX, shape), "q_sc": mx_scales(wid, STREAM_QSC, sshape),
            "k_mx": mx_codes(wid, STREAM_KMX, shape), "k_sc": mx_scales(wid, STREAM_KSC, sshape),
            "v": normal(wid, STREAM_V, shape)}


def random_mxpv_case(seed: int, lengths, heads: int, head_dim: int, wide=None):
    """random_mx_case with v as user-blocked MXFP8 too (mx_v_draw) in place
    of the bf16 v; wide = ((q_lo, q_hi), (k_lo, k_hi), (v_lo, v_hi)) draws
    every finite code with those scale ranges."""
    c = random_mx_case(seed, lengths, heads, head_dim,
                       wide=None if wide is None else wide[:2])
    del c["v"]
    if wide is None:
        c.update(mx_v_draw(2000 + seed, c["offsets"], heads, head_dim))
    else:
        c.update(mx_v_draw(2000 + seed, c["offsets"], heads, head_dim, scales=wide[2],
                           codes=mx_codes_all))
    return c


def random_mxbwd_case(seed: int, lengths, heads: int, head_dim: int, wide=None):
    """random_mxpv_case plus the MXFP8 backward's inputs (mx_bwd_draw);
    wide = eight scale ranges (q, k, v, vh, do, qt, kt, dot), codes over
    every finite E4M3 code."""
    c = random_mxpv_case(seed, lengths, heads, head_dim,
                         wide=None if wide is None else tuple(wide[:3]))
    c.update(mx_bwd_draw(2000 + seed, 3000 + seed, c["offsets"], heads, head_dim,
                         wide=None if wide is None else tuple(wide[3:])))
    return c
