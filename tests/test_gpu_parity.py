"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle.

Small cases are compared element by element over every output; the five
workloads are run at their full sizes in the launch configuration the
benchmark times and compared on sampled rows that the oracle recomputes from
the slice of the user they depend on (tests/parity_util.py: row_slice).
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from long_sequence_block_amd import workloads as wl
from parity_util import (assert_close, check_full, check_sampled, np64, run_bwd, run_fwd,
                         to_device)

pytestmark = pytest.mark.gpu


def _print(msg):
    print(msg, flush=True)


SMALL = [
    # (lengths, H, D, B, W, dtype)
    ([256, 256], 1, 32, 32, 1, "fp32"),
    ([100, 37, 0, 300, 1], 2, 64, 64, 2, "bf16"),
    ([129, 255, 513, 7], 2, 64, 128, 2, "bf16"),
    ([1000, 16, 17], 1, 128, 256, 4, "bf16"),
    ([77, 300, 5], 3, 32, 16, 3, "bf16"),
    ([90, 200], 2, 64, 48, 2, "bf16"),
    ([333, 64, 65], 2, 128, 64, 1, "bf16"),
    ([500], 1, 64, 32, 20, "bf16"),       # window covers the whole user
    ([100, 37, 0, 300, 1], 2, 64, 64, 2, "fp32"),
    ([129, 600], 2, 128, 128, 3, "fp32"),
    ([45, 80], 2, 32, 16, 2, "fp32"),
]


@pytest.mark.parametrize("idx", range(len(SMALL)))
def test_small_cases_every_element(idx):
    lengths, H, D, B, W, dtype = SMALL[idx]
    _print(f"small case {idx}: lengths={lengths} H={H} D={D} B={B} W={W} {dtype}")
    case = wl.random_case(500 + idx, lengths, H, D)
    check_full(case, dtype, B, W, 1.0 / math.sqrt(D), backward=True)


def test_many_users_every_element():
    """1500 users of 0-40 tokens: the backward's tile-index scan runs over
    several 1024-user passes, and most tiles are one-chunk tiles.  Windows
    this short give near-one-hot weights, so the gradients are checked with
    one bf16 ulp of slack (parity_util.assert_close)."""
    rng = np.random.default_rng(77)
    lengths = [int(x) for x in rng.integers(0, 41, 1500)]
    _print(f"many users: {len(lengths)} users, T={sum(lengths)}")
    case = wl.random_case(601, lengths, 2, 64)
    check_full(case, "bf16", 32, 2, 0.125, backward=True, ulp_slack=True)


def test_empty_inputs():
    for lengths in ([], [0], [0, 0, 0]):
        case = wl.random_case(7, lengths, 2, 64)
        dev, _ = to_device(case, "bf16")
        out, lse = run_fwd(dev, 64, 2, 0.125)
        assert out.numel() == 0 and lse.numel() == 0
        dq, dk, dv = run_bwd(dev, out, lse, 64, 2, 0.125)
        assert dq.numel() == 0
    torch.cuda.synchronize()


def test_tiny_fp32_workload_full():
    w = wl.WORKLOADS[1]
    _print("workload 1 (tiny fp32), all elements")
    case = wl.draw(w)
    case["dout"] = wl.normal(1, wl.STREAM_DO, case["q"].shape)
    check_full(case, "fp32", w.block_size, w.window_blocks, w.scale, backward=True)


def _samples(off, B, rng, n_users=6):
    """Sampled row ranges: first, last and random users, plus block edges."""
    batch = len(off) - 1
    users = sorted(set([0, batch - 1, int(np.argmax(np.diff(off)))] +
                       list(rng.integers(0, batch, n_users))))
    out = []
    for u in users:
        L = int(off[u + 1] - off[u])
        out.append((u, 0, min(L, 2 * B)))                    # start of the user
        out.append((u, max(0, L - B - 5), L))                # ragged tail
        if L > 4 * B:
            a = int(rng.integers(B, L - 2 * B))
            out.append((u, a, a + B + 3))                    # interior, unaligned
    return out


@pytest.mark.parametrize("wid", [2, 3, 4, 5])
def test_workload_full_size_sampled(wid):
    w = wl.WORKLOADS[wid]
    _print(f"workload {wid} ({w.name}) full size, sampled rows")
    case = wl.draw(w)
    dev, host = to_device(case, w.dtype)
    del case
    out, lse = run_fwd(dev, w.block_size, w.window_blocks, w.scale)
    grads = run_bwd(dev, out, lse, w.block_size, w.window_blocks, w.scale) if w.backward else None
    torch.cuda.synchronize()
    rng = np.random.default_rng(wid)
    samples = _samples(host["offsets"], w.block_size, rng)
    check_sampled(dev, host, out, lse, grads, w.block_size, w.window_blocks, w.scale,
                  w.dtype, samples)
    # every row written: no NaN/garbage anywhere in the outputs
    assert torch.isfinite(out).all().item() and torch.isfinite(lse).all().item()
    if grads is not None:
        for g in grads:
            assert torch.isfinite(g).all().item()


@pytest.mark.parametrize("L", [2048, 4096, 8192])
def test_long_context_sweep_sampled(L):
    w = wl.long_context(L)
    _print(f"long-context sweep L={L}, sampled rows")
    w = dataclasses.replace(w, users=4)
    case = wl.draw(w)
    dev, host = to_device(case, w.dtype)
    out, lse = run_fwd(dev, w.block_size, w.window_blocks, w.scale)
    torch.cuda.synchronize()
    samples = [(u, a, a + 300) for u in range(4) for a in (0, L // 2 - 7, L - 300)]
    check_sampled(dev, host, out, lse, None, w.block_size, w.window_blocks, w.scale,
                  w.dtype, samples)


def test_lse_pin_zero_queries():
    """q = 0 on the GPU: lse_i = ln n_i exactly (up to fp32), O = window mean."""
    lengths = [300, 129, 64]
    B, W = 64, 2
    case = wl.random_case(9, lengths, 2, 64)
    case["q"][:] = 0
    dev, host = to_device(case, "bf16")
    out, lse = run_fwd(dev, B, W, 0.125)
    off = host["offsets"]
    for u, L in enumerate(lengths):
        i = np.arange(L)
        n = i - np.maximum(0, i // B - W + 1) * B + 1
        assert_close("lse", np64(lse)[:, off[u]:off[u + 1]], np.log(n)[None].repeat(2, 0),
                     "bf16", is_lse=True)
