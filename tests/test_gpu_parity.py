"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle.

Every output element is compared, in small cases and in the workloads at
their full sizes.  The full-size workloads run on the GPU in the launch
configuration the benchmark times; the oracle recomputes them in contiguous
user ranges (tests/parity_util.py: compare_by_users).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from long_sequence_block_amd import workloads as wl
import long_sequence_block_amd as lsb
from parity_util import (assert_close, check_full, compare_by_users, np64, run_bwd, run_fwd,
                         to_device, to_device_lazy)

pytestmark = pytest.mark.gpu


def _print(msg):
    print(msg, flush=True)


SMALL = [
    # (lengths, H, D, B, W, dtype)
    ([256, 256], 1, 32, 32, 1, "fp32"),
    ([100, 37, 0, 300, 1], 2, 64, 64, 2, "bf16"),
    ([129, 255, 513, 7], 2, 64, 128, 2, "bf16"),
    ([1000, 16, 17], 1, 128, 256, 4, "bf16"),
    ([256, 257, 511, 1100, 3, 0], 2, 128, 256, 2, "bf16"),
    ([700, 256, 40], 1, 128, 256, 1, "bf16"),
    ([77, 300, 5], 3, 32, 16, 3, "bf16"),
    ([90, 200], 2, 64, 48, 2, "bf16"),
    ([333, 64, 65], 2, 128, 64, 1, "bf16"),
    ([500], 1, 64, 32, 20, "bf16"),       # window covers the whole user
    ([100, 37, 0, 300, 1], 2, 64, 64, 2, "fp32"),
    ([129, 600], 2, 128, 128, 3, "fp32"),
    ([45, 80], 2, 32, 16, 2, "fp32"),
    # block sizes that are not multiples of 16, or above 256
    ([100, 37, 300], 2, 64, 7, 3, "bf16"),
    ([600, 5], 1, 128, 100, 2, "bf16"),
    ([513, 20], 2, 64, 300, 1, "bf16"),
    ([77, 130], 2, 32, 5, 4, "fp32"),
    # the largest block and window the ABI takes: one block per user, every
    # earlier key visible (the library clamps B to T and W to ceil(T/B))
    ([300, 77, 0, 5], 2, 64, 2**31 - 1, 2**31 - 1, "bf16"),
    ([100, 37], 1, 32, 2**31 - 1, 2**31 - 1, "fp32"),
    ([260, 1000], 1, 128, 64, 2**31 - 1, "bf16"),
    # windows of more than 1024 rows (W B after clamping): a key tile's
    # queries span up to 11 query tiles
    ([2000, 700], 1, 64, 256, 5, "bf16"),
    ([1500, 300, 40], 2, 128, 128, 10, "bf16"),
    ([1300, 9], 1, 32, 1200, 1, "bf16"),
]


@pytest.mark.parametrize("idx", range(len(SMALL)))
def test_small_cases_every_element(idx):
    lengths, H, D, B, W, dtype = SMALL[idx]
    _print(f"small case {idx}: lengths={lengths} H={H} D={D} B={B} W={W} {dtype}")
    case = wl.random_case(500 + idx, lengths, H, D)
    check_full(case, dtype, B, W, 1.0 / math.sqrt(D), backward=True)


SLIDING = [
    # (lengths, H, D, window_tokens, dtype): the token sliding window, i.e.
    # blocks of one token, through blockattn_swa_fwd / blockattn_swa_bwd
    ([300, 1, 0, 129], 2, 64, 1, "bf16"),
    ([500, 77], 2, 64, 37, "bf16"),
    ([700, 64, 3], 1, 128, 200, "bf16"),
    ([260, 31], 3, 32, 64, "bf16"),
    ([90, 300], 2, 64, 1000, "bf16"),   # longer than every user: causal attention
    ([200, 45], 2, 64, 19, "fp32"),
]


@pytest.mark.parametrize("idx", range(len(SLIDING)))
def test_sliding_window_every_element(idx):
    lengths, H, D, w, dtype = SLIDING[idx]
    _print(f"sliding window {idx}: lengths={lengths} H={H} D={D} w={w} {dtype}")
    case = wl.random_case(800 + idx, lengths, H, D)
    dev, host = to_device(case, dtype)
    scale = 1.0 / math.sqrt(D)
    out, lse = lsb.swa_fwd(dev["q"], dev["k"], dev["v"], dev["offsets"], w, scale)
    o_ref, l_ref = oracle.fwd(host["q"], host["k"], host["v"], host["offsets"], 1, w, scale)
    assert_close("out", np64(out), o_ref, dtype)
    assert_close("lse", np64(lse), l_ref, dtype, is_lse=True)
    grads = lsb.swa_bwd(dev["q"], dev["k"], dev["v"], out, dev["dout"], lse, dev["offsets"],
                        w, scale)
    refs = oracle.bwd(host["q"], host["k"], host["v"], host["dout"], host["offsets"], 1, w,
                      scale)
    for name, g, ref in zip(("dq", "dk", "dv"), grads, refs):
        assert_close(name, np64(g), ref, dtype)
    # the same call as block attention with blocks of one token
    out_b, lse_b = run_fwd(dev, 1, w, scale)
    assert torch.equal(out_b, out) and torch.equal(lse_b, lse)
    torch.cuda.synchronize()


NEG_SCALE = [
    # (lengths, H, D, B, W): a negative scale flips which key dominates
    ([300, 64, 129], 2, 64, 64, 2),
    ([600, 100], 1, 128, 256, 3),
]


@pytest.mark.parametrize("idx", range(len(NEG_SCALE)))
def test_negative_scale_every_element(idx):
    lengths, H, D, B, W = NEG_SCALE[idx]
    _print(f"negative scale {idx}: lengths={lengths} H={H} D={D} B={B} W={W}")
    case = wl.random_case(700 + idx, lengths, H, D)
    check_full(case, "bf16", B, W, -1.0 / math.sqrt(D), backward=True)


def test_many_users_every_element():
    """1500 users of 0-40 tokens: the backward's tile-index scan runs over
    several 1024-user passes, most tiles are one-chunk tiles, and windows this
    short give near-one-hot weights, the hardest case for the gradients'
    precision."""
    rng = np.random.default_rng(77)
    lengths = [int(x) for x in rng.integers(0, 41, 1500)]
    _print(f"many users: {len(lengths)} users, T={sum(lengths)}")
    case = wl.random_case(601, lengths, 2, 64)
    p = check_full(case, "bf16", 32, 2, 0.125, backward=True)
    _print("  " + p.summary())


LARGE_BATCH = [
    # (users, max tokens, H, D, B, W, seed): above 1024 users the forward's
    # tile decode reads four users per thread and pass; user counts that are
    # not multiples of four leave a ragged last group
    (4097, 70, 2, 64, 32, 2, 611),
    (5003, 24, 2, 128, 16, 3, 612),
]


@pytest.mark.parametrize("idx", range(len(LARGE_BATCH)))
def test_large_batch_every_element(idx):
    n, top, H, D, B, W, seed = LARGE_BATCH[idx]
    lengths = [int(x) for x in np.random.default_rng(seed).integers(0, top + 1, n)]
    _print(f"large batch {idx}: {n} users of 0-{top} tokens, T={sum(lengths)} H={H} D={D} "
           f"B={B} W={W}")
    case = wl.random_case(seed, lengths, H, D)
    p = check_full(case, "bf16", B, W, 1.0 / math.sqrt(D), backward=True)
    _print("  " + p.summary())


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


def full_size_every_element(w, max_tokens):
    """The whole workload on the GPU in the launch configuration bench.py
    times, then every element of out, lse (and dq, dk, dv) against the
    oracle, recomputed in user ranges of at most max_tokens tokens."""
    case = wl.draw(w)
    dev, host = to_device_lazy(case, w.dtype)
    del case
    B, W, sc = w.block_size, w.window_blocks, w.scale
    out, lse = run_fwd(dev, B, W, sc)
    gpu = {"out": out.cpu(), "lse": lse.cpu()}
    if w.backward:
        dq, dk, dv = run_bwd(dev, out, lse, B, W, sc)
        gpu.update(dq=dq.cpu(), dk=dk.cpu(), dv=dv.cpu())
        del dq, dk, dv
    torch.cuda.synchronize()
    del dev, out, lse

    def reference(sub):
        o, l = oracle.fwd(sub["q"], sub["k"], sub["v"], sub["offsets"], B, W, sc)
        r = {"out": o, "lse": l}
        if w.backward:
            r["dq"], r["dk"], r["dv"] = oracle.bwd(sub["q"], sub["k"], sub["v"], sub["dout"],
                                                   sub["offsets"], B, W, sc)
        return r

    p = compare_by_users(host, gpu, host["offsets"], reference, w.dtype, max_tokens, log=_print)
    _print("  " + p.summary())


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wid", [2, 3, 5, 6, 12])
def test_workload_full_size_every_element(wid):
    w = wl.WORKLOADS[wid]
    _print(f"workload {wid} ({w.name}) full size, every element")
    full_size_every_element(w, max_tokens=1 << 30)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wid", [4, 11])
def test_long_context_full_size_every_element(wid):
    """32 users of 16384 tokens (1 GiB per tensor): the oracle recomputes
    four users at a time."""
    w = wl.WORKLOADS[wid]
    _print(f"workload {wid} ({w.name}) full size, every element in 4-user ranges")
    full_size_every_element(w, max_tokens=4 * w.fixed_length)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("L", [2048, 4096, 8192])
def test_long_context_sweep_every_element(L):
    w = wl.long_context(L)
    _print(f"long-context sweep L={L}, all 32 users, every element")
    full_size_every_element(w, max_tokens=max(8 * L, 65536))


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
