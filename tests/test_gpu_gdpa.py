"""GPU parity of generalized dot-product attention on the block pattern
(SiLU / GELU scores, no normalisation), through the C ABI, against the fp64
oracle.  The variant is the one "GEM (Meta)", section "Custom kernels",
describes (the softmax replaced by an activation); the readings are in the
oracle's C header and include/blockattn.h.

Bounds (tests/parity_util.py, GdpaParity): per element
|gpu - ref| <= 2^-8 (A + |ref|) + 1e-5, with A the same sum over |terms| from
the oracle, and the mean error at most a quarter of the mean bound; fp32
normwise 1e-5.  Every element is compared, including the training workload
at full size.
"""
import math

import pytest
import torch

import long_sequence_block_amd as lsb
import oracle
from long_sequence_block_amd import workloads as wl
from parity_util import (GdpaParity, host_rows, np64, random_shapes, to_device, to_device_lazy,
                         user_ranges)

pytestmark = pytest.mark.gpu


def _print(msg):
    print(msg, flush=True)


def add_gdpa(p, host, gpu, B, W, scale, act, t0=0, t1=None, tag=""):
    """Oracle outputs and their |term| sums for host rows [t0, t1) (a range
    of whole users, offsets re-based), compared with the GPU's."""
    out_g, grads_g = gpu
    t1 = host["offsets"][-1] if t1 is None else t1
    q, k, v, do = (host_rows(host[n], t0, t1) for n in ("q", "k", "v", "dout"))
    off = host["sub_offsets"]
    ref = oracle.gdpa_fwd(q, k, v, off, B, W, scale, act)
    mag = oracle.gdpa_fwd(q, k, v, off, B, W, scale, act, absolute=True)
    p.add("out", out_g[t0:t1], ref, mag, tag)
    refs = oracle.gdpa_bwd(q, k, v, do, off, B, W, scale, act)
    mags = oracle.gdpa_bwd(q, k, v, do, off, B, W, scale, act, absolute=True)
    for name, g, r, m in zip(("dq", "dk", "dv"), grads_g, refs, mags):
        p.add(name, g[t0:t1], r, m, tag)


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


def gdpa_case(seed, lengths, H, D, B, W, dtype, act, sign):
    """Forward and backward of one case, every element against the oracle."""
    case = wl.random_case(seed, lengths, H, D)
    dev, host = to_device(case, dtype)
    scale = sign / math.sqrt(D)
    out = lsb.gdpa_fwd(dev["q"], dev["k"], dev["v"], dev["offsets"], B, W, scale, act)
    grads = lsb.gdpa_bwd(dev["q"], dev["k"], dev["v"], dev["dout"], dev["offsets"], B, W,
                         scale, act)
    torch.cuda.synchronize()
    host["sub_offsets"] = host["offsets"]
    p = GdpaParity(dtype)
    add_gdpa(p, host, (np64(out), [np64(g) for g in grads]), B, W, scale, act)
    p.finish()
    _print("  " + p.summary())


@pytest.mark.parametrize("idx", range(len(GDPA)))
def test_gdpa_every_element(idx):
    lengths, H, D, B, W, dtype, act, sign = GDPA[idx]
    _print(f"gdpa {idx}: lengths={lengths} H={H} D={D} B={B} W={W} {dtype} act={act}")
    gdpa_case(1000 + idx, lengths, H, D, B, W, dtype, act, sign)


GDPA_RANDOM = random_shapes(10, 2029)


@pytest.mark.parametrize("idx", range(len(GDPA_RANDOM)))
def test_gdpa_random_shape_every_element(idx):
    """Seeded random shapes (parity_util.random_shapes), SiLU and GELU in turn."""
    lengths, H, D, B, W, dtype, sign = GDPA_RANDOM[idx]
    act = 1 + idx % 2
    _print(f"gdpa random {idx}: lengths={lengths} H={H} D={D} B={B} W={W} {dtype} act={act}")
    gdpa_case(1100 + idx, lengths, H, D, B, W, dtype, act, sign)


@pytest.mark.timeout(900)
def test_gdpa_training_workload_every_element():
    """The SiLU training step at full size, in the launch configuration
    bench.py times; every element of out, dq, dk and dv."""
    w = wl.WORKLOADS[8]
    _print(f"workload 8 ({w.name}), every element")
    dev, host = to_device_lazy(wl.draw(w), "bf16")
    B, W, sc, act = w.block_size, w.window_blocks, w.scale, w.act
    out = lsb.gdpa_fwd(dev["q"], dev["k"], dev["v"], dev["offsets"], B, W, sc, act)
    grads = lsb.gdpa_bwd(dev["q"], dev["k"], dev["v"], dev["dout"], dev["offsets"], B, W, sc,
                         act)
    torch.cuda.synchronize()
    gpu = (out.cpu().double().numpy(), [g.cpu().double().numpy() for g in grads])
    del dev, out, grads
    off = host["offsets"]
    p = GdpaParity("bf16")
    for u0, u1 in user_ranges(off, 1 << 16):
        t0, t1 = int(off[u0]), int(off[u1])
        host["sub_offsets"] = off[u0:u1 + 1] - t0
        add_gdpa(p, host, gpu, B, W, sc, act, t0, t1, tag=f"users [{u0},{u1})")
        _print(f"  users [{u0},{u1}): {p.summary()}")
    p.finish()
