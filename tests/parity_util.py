"""Helpers of the GPU parity tests: move seeded inputs to the device, run the
HIP path through the C ABI binding, and check it against the fp64 oracle.

Tolerances (from the arithmetic and the stated targets):
* bf16 workloads: O, dQ, dK, dV max |gpu - oracle| <= 2e-2 and mean <= 2e-3;
  lse max |gpu - oracle| <= 1e-3.  The oracle sees the bf16-rounded inputs.
* fp32 workloads: normwise ||gpu - oracle||_inf / ||oracle||_inf <= 1e-5 for
  every output.
"""
from __future__ import annotations

import numpy as np
import torch

import long_sequence_block_amd as lsb
import oracle

BF16_MAX, BF16_MEAN, LSE_MAX, FP32_REL = 2e-2, 2e-3, 1e-3, 1e-5
# GDPA (activation scores, no normalisation): outputs are not bounded by the
# values' magnitude as a softmax average is, so the bf16 bounds scale with
# the reference: max |err| <= 1e-2 max|ref|, mean |err| <= 1e-3 max|ref|
# (the ratio of the softmax bounds to those outputs' magnitude, about 2-4)
GDPA_MAX, GDPA_MEAN = 1e-2, 1e-3


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


def run_fwd(dev, B, W, scale):
    out, lse = lsb.fwd(dev["q"], dev["k"], dev["v"], dev["offsets"], B, W, scale)
    return out, lse


def run_bwd(dev, out, lse, B, W, scale):
    return lsb.bwd(dev["q"], dev["k"], dev["v"], out, dev["dout"], lse, dev["offsets"],
                   B, W, scale)


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def assert_close(name, got, ref, dtype, is_lse=False, ulp_slack=False):
    """The stated bounds.  ulp_slack (bf16 only) adds one bf16 ulp of the
    reference value (2^-7 relative) to the per-element bound, for stress
    cases whose gradients carry near-one-hot weights: there the backward's
    delta comes from the forward's bf16 O, and dS = P (dP - delta) passes that
    rounding on at full size."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if got.size == 0:
        return
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    if dtype == "fp32":
        rel = err.max() / max(np.abs(ref).max(), 1e-30)
        assert rel <= FP32_REL, f"{name}: normwise rel err {rel:.3e} > {FP32_REL}"
    elif is_lse:
        assert err.max() <= LSE_MAX, f"{name}: max abs err {err.max():.3e} > {LSE_MAX}"
    else:
        bound = BF16_MAX + (np.abs(ref) * 2.0 ** -7 if ulp_slack else 0.0)
        worst = (err - bound).max()
        assert worst <= 0, f"{name}: max abs err {err.max():.3e} exceeds its bound by {worst:.3e}"
        assert err.mean() <= BF16_MEAN, f"{name}: mean abs err {err.mean():.3e} > {BF16_MEAN}"


def check_full(case, dtype, B, W, scale, backward=True, ulp_slack=False):
    """Whole-case parity: every output element against the oracle."""
    dev, host = to_device(case, dtype)
    out, lse = run_fwd(dev, B, W, scale)
    o_ref, l_ref = oracle.fwd(host["q"], host["k"], host["v"], host["offsets"], B, W, scale)
    assert_close("out", np64(out), o_ref, dtype)
    assert_close("lse", np64(lse), l_ref, dtype, is_lse=True)
    if backward:
        dq, dk, dv = run_bwd(dev, out, lse, B, W, scale)
        r = oracle.bwd(host["q"], host["k"], host["v"], host["dout"], host["offsets"], B, W,
                       scale)
        for name, g, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), r):
            assert_close(name, np64(g), ref, dtype, ulp_slack=ulp_slack)
    torch.cuda.synchronize()


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


def check_sampled(dev, host, out, lse, grads, B, W, scale, dtype, samples):
    """Parity on sampled rows: samples = [(user, a, b)] local row ranges.
    The oracle runs on the slice of the user that those rows depend on."""
    off = host["offsets"]
    o_g, l_g = np64(out), np64(lse)
    g_g = [np64(g) for g in grads] if grads is not None else None
    for (u, a, b) in samples:
        t0, L = int(off[u]), int(off[u + 1] - off[u])
        a, b = min(a, L), min(b, L)
        if a >= b:
            continue
        s0, e = row_slice(L, a, b, B, W)
        sl = slice(t0 + s0, t0 + e)
        rows = slice(t0 + a, t0 + b)
        loc = slice(a - s0, b - s0)
        o_r, l_r = oracle.fwd(host["q"][sl], host["k"][sl], host["v"][sl],
                              [0, e - s0], B, W, scale)
        tag = f"user {u} rows [{a},{b})"
        assert_close(f"out {tag}", o_g[rows], o_r[loc], dtype)
        assert_close(f"lse {tag}", l_g[:, rows], l_r[:, loc], dtype, is_lse=True)
        if g_g is not None:
            r = oracle.bwd(host["q"][sl], host["k"][sl], host["v"][sl], host["dout"][sl],
                           [0, e - s0], B, W, scale)
            for name, g, ref in zip(("dq", "dk", "dv"), g_g, r):
                assert_close(f"{name} {tag}", g[rows], ref[loc], dtype)


def assert_close_scaled(name, got, ref, dtype):
    """The GDPA bounds (see GDPA_MAX): relative to the largest reference
    magnitude for bf16, normwise FP32_REL for fp32."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if got.size == 0:
        return
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    mag = max(np.abs(ref).max(), 1e-30)
    if dtype == "fp32":
        assert err.max() / mag <= FP32_REL, f"{name}: normwise rel err {err.max() / mag:.3e}"
        return
    assert err.max() <= GDPA_MAX * mag, f"{name}: max err {err.max():.3e} vs {GDPA_MAX * mag:.3e}"
    assert err.mean() <= GDPA_MEAN * mag, f"{name}: mean err {err.mean():.3e} vs {GDPA_MEAN * mag:.3e}"
