"""Helpers of the GPU parity tests: move seeded inputs to the device, run the
HIP path through the C ABI binding, and check it against the fp64 oracle.

Tolerances (from the arithmetic and the stated targets):
* bf16 workloads: O, dQ, dK, dV per element |gpu - oracle| <= 2e-2 of
  arithmetic error plus the rounding of the result to the bf16 output
  format, 2^-8 |oracle| (a correctly rounded bf16 value can sit that far from
  the exact one: 1/64 for values in [4, 8), 1/32 in [8, 16), so a plain 2e-2
  cannot hold for outputs of magnitude 8 and up); mean |gpu - oracle| <= 2e-3
  over each whole tensor; lse max <= 1e-3.  The oracle sees the bf16-rounded
  inputs.
* fp32 workloads: normwise ||gpu - oracle||_inf / ||oracle||_inf <= 1e-5 for
  every output tensor.

Full-size workloads are compared on every element too: the GPU runs the
whole workload once, in the launch configuration the benchmark times, and the
oracle recomputes it in contiguous user ranges (users are independent, so a
range re-based to its first token is an exact sub-problem).
"""
from __future__ import annotations

import numpy as np
import torch

import long_sequence_block_amd as lsb
import oracle

BF16_MAX, BF16_MEAN, LSE_MAX, FP32_REL = 2e-2, 2e-3, 1e-3, 1e-5
BF16_ROUND = 2.0 ** -8  # bound of round-to-nearest-even to bf16, relative


def to_device(case: dict, dtype: str, device="cuda"):
    """Device tensors (bf16 rounded RNE by torch, or fp32) and the exact fp64
    values the oracle must see."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev, host = {}, {}
    for key, val in case.items():
        if key == "offsets":
            dev[key] = torch.from_numpy(np.ascontiguousarray(val)).to(device)
            host[key] = np.asarray(val, np.int32)
        else:
            t = torch.from_numpy(np.ascontiguousarray(val)).to(tdt)
            host[key] = t.to(torch.float64).numpy()
            dev[key] = t.to(device)
    return dev, host


def to_device_lazy(case: dict, dtype: str, device="cuda"):
    """Like to_device, but the host side keeps the rounded values in their
    storage dtype (torch CPU tensors); chunks are widened to fp64 on demand
    (see host_rows).  For workloads whose fp64 copies would be large."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev, host = {}, {}
    for key, val in case.items():
        if key == "offsets":
            dev[key] = torch.from_numpy(np.ascontiguousarray(val)).to(device)
            host[key] = np.asarray(val, np.int32)
        else:
            t = torch.from_numpy(np.ascontiguousarray(val)).to(tdt)
            host[key] = t
            dev[key] = t.to(device)
    return dev, host


def host_rows(x, t0: int, t1: int) -> np.ndarray:
    """Token rows [t0, t1) of a host tensor as contiguous fp64 (integer
    arrays, such as MXFP8 codes and scales, keep their dtype)."""
    if isinstance(x, torch.Tensor):
        return x[t0:t1].to(torch.float64).numpy()
    x = np.asarray(x)
    if np.issubdtype(x.dtype, np.integer):
        return np.ascontiguousarray(x[t0:t1])
    return np.ascontiguousarray(x[t0:t1], dtype=np.float64)


def run_fwd(dev, B, W, scale):
    out, lse = lsb.fwd(dev["q"], dev["k"], dev["v"], dev["offsets"], B, W, scale)
    return out, lse


def run_bwd(dev, out, lse, B, W, scale):
    return lsb.bwd(dev["q"], dev["k"], dev["v"], out, dev["dout"], lse, dev["offsets"],
                   B, W, scale)


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


class Parity:
    """Accumulates the comparison of several output tensors, each possibly
    added in pieces (user ranges): per-element bounds are checked as pieces
    arrive, whole-tensor bounds (the bf16 mean, the fp32 normwise ratio) at
    finish().  Every element of every piece is compared."""

    def __init__(self, dtype: str):
        self.dtype = dtype
        self.acc = {}

    def add(self, name, got, ref, is_lse=False, tag="", extra=None):
        """extra: an additional per-element allowance (broadcast against ref)
        for a stated error source outside the bf16 arithmetic, such as the
        reduced-precision sums of the block-scaled fp8 products."""
        got = np.asarray(got, np.float64)
        ref = np.asarray(ref, np.float64)
        assert got.shape == ref.shape, (name, tag, got.shape, ref.shape)
        a = self.acc.setdefault(name, {"n": 0, "sum": 0.0, "max": 0.0, "refmax": 0.0,
                                       "arith": 0.0, "lse": is_lse})
        if got.size == 0:
            return
        assert np.all(np.isfinite(got)), f"{name} {tag}: non-finite values"
        err = np.abs(got - ref)
        emax = float(err.max())
        a["n"] += err.size
        a["sum"] += float(err.sum())
        a["max"] = max(a["max"], emax)
        a["refmax"] = max(a["refmax"], float(np.abs(ref).max()))
        if self.dtype == "fp32":
            return  # normwise: needs the whole tensor's reference magnitude
        if extra is not None:
            err = err - np.broadcast_to(np.asarray(extra, np.float64), err.shape)
            emax = float(err.max())
        if is_lse:
            assert emax <= LSE_MAX, f"{name} {tag}: max abs err {emax:.3e} > {LSE_MAX}"
        else:
            # the error beyond the output format's own rounding
            arith = err - BF16_ROUND * np.abs(ref)
            worst = int(np.argmax(arith))
            a["arith"] = max(a["arith"], float(arith.flat[worst]))
            assert arith.flat[worst] <= BF16_MAX, (
                f"{name} {tag}: err {err.flat[worst]:.3e} at ref {ref.flat[worst]:.3e} exceeds "
                f"{BF16_MAX} + 2^-8 |ref| by {arith.flat[worst] - BF16_MAX:.3e}")

    def finish(self):
        for name, a in self.acc.items():
            if a["n"] == 0:
                continue
            if self.dtype == "fp32":
                rel = a["max"] / max(a["refmax"], 1e-30)
                assert rel <= FP32_REL, f"{name}: normwise rel err {rel:.3e} > {FP32_REL}"
            elif not a["lse"]:
                mean = a["sum"] / a["n"]
                assert mean <= BF16_MEAN, f"{name}: mean abs err {mean:.3e} > {BF16_MEAN}"

    def summary(self) -> str:
        return ", ".join(f"{n} max {a['max']:.2e} (beyond rounding {a['arith']:.2e}) "
                         f"mean {a['sum'] / max(a['n'], 1):.1e}"
                         for n, a in self.acc.items())


# Generalized dot-product attention (activation scores, no normalisation):
# each output is an unnormalised sum of terms whose magnitudes are unrelated
# to the output's own size, so its bound is per element and scaled by
# A = the same sum over |terms| (oracle.gdpa_fwd/gdpa_bwd with absolute=True).
# The GPU rounds each term's weight (P, or dS) to bf16 before the matrix
# product, error <= 2^-8 |weight|, accumulates in fp32 and rounds the result
# to bf16, error <= 2^-8 |result|: |gpu - ref| <= 2^-8 (A + |ref|), plus fp32
# rounding of the scores and activations (GDPA_ATOL).  The mean over a
# tensor is held to a quarter of that bound's mean (rounding errors of many
# terms do not all align).
GDPA_REL, GDPA_ATOL, GDPA_MEAN_FRAC = 2.0 ** -8, 1e-5, 0.25


class GdpaParity:
    """Like Parity, with the GDPA bounds above for bf16 and the normwise
    FP32_REL for fp32 outputs."""

    def __init__(self, dtype: str):
        self.dtype = dtype
        self.acc = {}

    def add(self, name, got, ref, mag, tag=""):
        got, ref, mag = (np.asarray(x, np.float64) for x in (got, ref, mag))
        assert got.shape == ref.shape == mag.shape, (name, tag, got.shape, ref.shape)
        a = self.acc.setdefault(name, {"n": 0, "sum": 0.0, "bsum": 0.0, "max": 0.0,
                                       "refmax": 0.0, "ratio": 0.0})
        if got.size == 0:
            return
        assert np.all(np.isfinite(got)), f"{name} {tag}: non-finite values"
        err = np.abs(got - ref)
        bound = GDPA_REL * (mag + np.abs(ref)) + GDPA_ATOL
        a["n"] += err.size
        a["sum"] += float(err.sum())
        a["bsum"] += float(bound.sum())
        a["max"] = max(a["max"], float(err.max()))
        a["refmax"] = max(a["refmax"], float(np.abs(ref).max()))
        a["ratio"] = max(a["ratio"], float((err / bound).max()))
        if self.dtype == "bf16":
            worst = int(np.argmax(err - bound))
            assert err.flat[worst] <= bound.flat[worst], (
                f"{name} {tag}: err {err.flat[worst]:.3e} > bound {bound.flat[worst]:.3e} "
                f"(ref {ref.flat[worst]:.3e}, |terms| {mag.flat[worst]:.3e})")

    def finish(self):
        for name, a in self.acc.items():
            if a["n"] == 0:
                continue
            if self.dtype == "fp32":
                rel = a["max"] / max(a["refmax"], 1e-30)
                assert rel <= FP32_REL, f"{name}: normwise rel err {rel:.3e} > {FP32_REL}"
            else:
                assert a["sum"] <= GDPA_MEAN_FRAC * a["bsum"], (
                    f"{name}: mean err {a['sum'] / a['n']:.3e} > {GDPA_MEAN_FRAC} x mean bound "
                    f"{a['bsum'] / a['n']:.3e}")

    def summary(self) -> str:
        return ", ".join(f"{n} max {a['max']:.2e} max err/bound {a['ratio']:.2f} "
                         f"mean err/bound {a['sum'] / max(a['bsum'], 1e-300):.3f}"
                         for n, a in self.acc.items())


# MXFP8 backward (oracle.mx_bwd): per element, the oracle's slack for code
# flips (oracle.mx_bwd_bounds) plus the block-scaled products' own rounding,
# 2^-10 of A = the sum of |quantized operand| |other operand| (rho = 2^-11 of
# the fp8 instruction's sums, with a margin), plus the bf16 rounding of the
# result, plus 10^-6 of the piece's largest A.  The mean error over a tensor
# is held to a quarter of the bound's mean, so that a systematic error
# cannot hide inside the per-element slack.
MXB_RHO, MXB_ATOL, MXB_MEAN_FRAC = 2.0 ** -10, 1e-6, 0.25


class MxBwdParity:
    """Accumulates the MXFP8 backward's comparison (bounds above)."""

    def __init__(self):
        self.acc = {}

    def add(self, name, got, ref, slack, absum, tag=""):
        got, ref, slack, absum = (np.asarray(x, np.float64) for x in (got, ref, slack, absum))
        assert got.shape == ref.shape == slack.shape == absum.shape, (name, tag)
        a = self.acc.setdefault(name, {"n": 0, "sum": 0.0, "bsum": 0.0, "max": 0.0,
                                       "ratio": 0.0, "flip": 0})
        if got.size == 0:
            return
        assert np.all(np.isfinite(got)), f"{name} {tag}: non-finite values"
        err = np.abs(got - ref)
        bound = slack + MXB_RHO * absum + BF16_ROUND * np.abs(ref) + MXB_ATOL * absum.max()
        a["n"] += err.size
        a["sum"] += float(err.sum())
        a["bsum"] += float(bound.sum())
        a["max"] = max(a["max"], float(err.max()))
        a["ratio"] = max(a["ratio"], float((err / np.maximum(bound, 1e-300)).max()))
        a["flip"] += int(np.count_nonzero(slack > 0))
        worst = int(np.argmax(err - bound))
        assert err.flat[worst] <= bound.flat[worst], (
            f"{name} {tag}: err {err.flat[worst]:.3e} > bound {bound.flat[worst]:.3e} "
            f"(ref {ref.flat[worst]:.3e}, slack {slack.flat[worst]:.3e}, "
            f"|terms| {absum.flat[worst]:.3e}) at flat index {worst}")

    def finish(self):
        for name, a in self.acc.items():
            if a["n"] == 0:
                continue
            assert a["sum"] <= MXB_MEAN_FRAC * a["bsum"], (
                f"{name}: mean err {a['sum'] / a['n']:.3e} > {MXB_MEAN_FRAC} x mean bound "
                f"{a['bsum'] / a['n']:.3e}")

    def summary(self) -> str:
        return ", ".join(f"{n} max {a['max']:.2e} max err/bound {a['ratio']:.2f} "
                         f"mean err/bound {a['sum'] / max(a['bsum'], 1e-300):.3f} "
                         f"(elements with flip slack {a['flip'] / max(a['n'], 1):.1%})"
                         for n, a in self.acc.items())


def assert_close(name, got, ref, dtype, is_lse=False):
    """The stated bounds on one whole tensor."""
    p = Parity(dtype)
    p.add(name, got, ref, is_lse=is_lse)
    p.finish()


def check_full(case, dtype, B, W, scale, backward=True):
    """Whole-case parity: every output element against the oracle."""
    dev, host = to_device(case, dtype)
    out, lse = run_fwd(dev, B, W, scale)
    o_ref, l_ref = oracle.fwd(host["q"], host["k"], host["v"], host["offsets"], B, W, scale)
    p = Parity(dtype)
    p.add("out", np64(out), o_ref)
    p.add("lse", np64(lse), l_ref, is_lse=True)
    if backward:
        dq, dk, dv = run_bwd(dev, out, lse, B, W, scale)
        r = oracle.bwd(host["q"], host["k"], host["v"], host["dout"], host["offsets"], B, W,
                       scale)
        for name, g, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), r):
            p.add(name, np64(g), ref)
    torch.cuda.synchronize()
    p.finish()
    return p


def user_ranges(offsets, max_tokens: int):
    """Contiguous user ranges [u0, u1) holding at most max_tokens tokens each
    (a single longer user gets a range of its own)."""
    off = np.asarray(offsets, np.int64)
    batch = len(off) - 1
    u0 = 0
    while u0 < batch:
        u1 = u0 + 1
        while u1 < batch and off[u1 + 1] - off[u0] <= max_tokens:
            u1 += 1
        yield u0, u1
        u0 = u1


def compare_by_users(host, gpu, offsets, reference, dtype, max_tokens, log=None):
    """(reference may also return, under "extra:<name>", a per-element
    allowance for output <name>; see Parity.add.)"""
    return _compare_by_users(host, gpu, offsets, reference, dtype, max_tokens, log)


def _compare_by_users(host, gpu, offsets, reference, dtype, max_tokens, log=None):
    """Every element of the GPU outputs against the oracle, user range by
    user range.

    host: the inputs (host tensors or arrays, [T, H, D]); gpu: name -> GPU
    output already copied to the host ([T, H, D], or [H, T] for names that
    start with "lse"); reference(sub, rows) -> name -> oracle output of the
    range, given sub = {input name: fp64 rows of the range, "offsets": the
    re-based offsets, "range": (u0, u1, t0, t1), its users and tokens}."""
    off = np.asarray(offsets, np.int64)
    p = Parity(dtype)
    for u0, u1 in user_ranges(off, max_tokens):
        t0, t1 = int(off[u0]), int(off[u1])
        if t1 == t0:
            continue
        sub = {k: host_rows(v, t0, t1) for k, v in host.items() if k != "offsets"}
        sub["offsets"] = (off[u0:u1 + 1] - t0).astype(np.int32)
        sub["range"] = (u0, u1, t0, t1)
        ref = reference(sub)
        for name, g in gpu.items():
            is_lse = name.startswith("lse")
            got = g[:, t0:t1] if is_lse else g[t0:t1]
            got = got.to(torch.float64).numpy() if isinstance(got, torch.Tensor) else got
            p.add(name, got, ref[name], is_lse=is_lse, tag=f"users [{u0},{u1})",
                  extra=ref.get("extra:" + name))
        if log is not None:
            log(f"  users [{u0},{u1}) tokens [{t0},{t1}): {p.summary()}")
    p.finish()
    return p


def row_slice(L: int, a: int, b: int, B: int, W: int):
    """Token range [s0, e) of one user that holds everything rows [a, b) of
    the forward output and of dQ/dK/dV depend on.

    The visibility rule is causal and block-aligned, so a slice starting at a
    multiple of B keeps every block boundary: rows [a, b) see keys from
    (floor(a/B)-W+1)*B on, and keys in [a, b) are seen by queries below
    (floor((b-1)/B)+W)*B.
    """
    s0 = max(0, a // B - W + 1) * B
    e = min(L, ((b - 1) // B + W) * B)
    return s0, e


def random_shapes(n, seed, head_dims=(32, 64, 128), fp32_share=0.2):
    """n seeded shape sets (lengths, H, D, B, W, dtype, scale sign): 1-10
    users mixing empty, one- or two-token, short and multi-tile lengths,
    H 1-3, D from head_dims, B log-uniform in 1-300, W 1-8, a share in fp32
    and a quarter with a negative scale."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        users = int(rng.integers(1, 11))
        kind = rng.random(users)
        lengths = [int(x) for x in np.where(
            kind < 0.15, rng.integers(0, 3, users),
            np.where(kind < 0.6, rng.integers(3, 130, users), rng.integers(130, 700, users)))]
        H = int(rng.integers(1, 4))
        D = int(rng.choice(list(head_dims)))
        B = max(int(np.exp(rng.uniform(0.0, np.log(300.0)))), 1)
        W = int(rng.integers(1, 9))
        dtype = "fp32" if rng.random() < fp32_share else "bf16"
        sign = -1.0 if rng.random() < 0.25 else 1.0
        out.append((lengths, H, D, B, W, dtype, sign))
    return out
