"""GPU parity of generalized dot-product attention on the block pattern
(SiLU / GELU scores, no normalisation), through the C ABI, against the fp64
oracle.  The variant is the one "GEM (Meta)", section "Custom kernels",
describes (the softmax replaced by an activation); the readings are in the
oracle's C header and include/blockattn.h.
"""
import math

import numpy as np
import pytest
import torch

import long_sequence_block_amd as lsb
import oracle
from long_sequence_block_amd import workloads as wl
from parity_util import assert_close_scaled, np64, row_slice, to_device

pytestmark = pytest.mark.gpu


def _print(msg):
    print(msg, flush=True)


GDPA = [
    # (lengths, H, D, B, W, dtype, act, scale sign)
    ([300, 1, 0, 129], 2, 64, 64, 2, "bf16", 1, 1),
    ([700, 64], 1, 128, 256, 3, "bf16", 2, 1),
    ([260, 31], 3, 32, 16, 4, "bf16", 1, -1),
    ([500, 77], 2, 64, 1, 37, "bf16", 2, 1),    # sliding window of 37 tokens
    ([129, 255, 513, 7], 2, 64, 128, 2, "bf16", 2, -1),
    ([200, 45], 2, 64, 32, 2, "fp32", 1, 1),
    ([90, 130], 1, 128, 64, 2, "fp32", 2, -1),
]


@pytest.mark.parametrize("idx", range(len(GDPA)))
def test_gdpa_every_element(idx):
    lengths, H, D, B, W, dtype, act, sign = GDPA[idx]
    _print(f"gdpa {idx}: lengths={lengths} H={H} D={D} B={B} W={W} {dtype} act={act}")
    case = wl.random_case(1000 + idx, lengths, H, D)
    dev, host = to_device(case, dtype)
    scale = sign / math.sqrt(D)
    out = lsb.gdpa_fwd(dev["q"], dev["k"], dev["v"], dev["offsets"], B, W, scale, act)
    ref = oracle.gdpa_fwd(host["q"], host["k"], host["v"], host["offsets"], B, W, scale, act)
    assert_close_scaled("out", np64(out), ref, dtype)
    grads = lsb.gdpa_bwd(dev["q"], dev["k"], dev["v"], dev["dout"], dev["offsets"], B, W,
                         scale, act)
    refs = oracle.gdpa_bwd(host["q"], host["k"], host["v"], host["dout"], host["offsets"],
                           B, W, scale, act)
    for name, g, r in zip(("dq", "dk", "dv"), grads, refs):
        assert_close_scaled(name, np64(g), r, dtype)
    torch.cuda.synchronize()


def test_gdpa_training_workload_sampled():
    """The SiLU training step at full size, in the launch configuration
    bench.py times; sampled rows checked on the user slices they depend on."""
    w = wl.WORKLOADS[8]
    _print(f"workload 8 ({w.name}), sampled rows")
    c = wl.draw(w)
    dev, host = to_device(c, "bf16")
    B, W, sc, act = w.block_size, w.window_blocks, w.scale, w.act
    out = lsb.gdpa_fwd(dev["q"], dev["k"], dev["v"], dev["offsets"], B, W, sc, act)
    grads = lsb.gdpa_bwd(dev["q"], dev["k"], dev["v"], dev["dout"], dev["offsets"], B, W, sc,
                         act)
    o_g, g_g = np64(out), [np64(g) for g in grads]
    off = host["offsets"]
    L = np.diff(off)
    longest = int(np.argmax(L))
    for (u, a, b) in [(0, 0, 64), (longest, int(L[longest]) - 70, int(L[longest])),
                      (longest, 1000, 1100), (len(L) - 1, 0, int(L[-1]))]:
        t0, n = int(off[u]), int(L[u])
        a, b = min(a, n), min(b, n)
        s0, e = row_slice(n, a, b, B, W)
        sl, rows, loc = slice(t0 + s0, t0 + e), slice(t0 + a, t0 + b), slice(a - s0, b - s0)
        sub = [0, e - s0]
        o_r = oracle.gdpa_fwd(host["q"][sl], host["k"][sl], host["v"][sl], sub, B, W, sc, act)
        assert_close_scaled(f"out user {u} [{a},{b})", o_g[rows], o_r[loc], "bf16")
        r = oracle.gdpa_bwd(host["q"][sl], host["k"][sl], host["v"][sl], host["dout"][sl], sub,
                            B, W, sc, act)
        for name, g, ref in zip(("dq", "dk", "dv"), g_g, r):
            assert_close_scaled(f"{name} user {u} [{a},{b})", g[rows], ref[loc], "bf16")
    torch.cuda.synchronize()
