"""GPU parity of the rotary position embedding and of the backward that has
its transpose fused in, through the C ABI, against the fp64 oracle.

The embedding is the one the production block-attention kernel carries
("GEM (Meta)", section "Custom kernels"), with the readings stated in the
oracle and in include/blockattn.h (rotate-half, base 10000 by default,
positions restarting at every user).
"""
import math

import numpy as np
import pytest
import torch

import long_sequence_block_amd as lsb
import oracle
from long_sequence_block_amd import workloads as wl
from parity_util import (assert_close, compare_by_users, np64, random_shapes, to_device,
                         to_device_lazy)

pytestmark = pytest.mark.gpu


def _print(msg):
    print(msg, flush=True)


def rotated_ref(host, base, dtype):
    """The oracle's rotation of q and k, stored in the call's dtype (RNE), as
    the GPU path stores its rotated q and k before attention."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    r = lambda x: torch.from_numpy(oracle.rope(x, host["offsets"], base)).to(tdt).double().numpy()
    return r(host["q"]), r(host["k"])


def assert_rotated(name, got, ref, dtype):
    """bf16: every element within RNE rounding of the result plus 1e-4;
    fp32: normwise 1e-6 (the angle is reduced in fp64)."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), name
    err = np.abs(got - ref)
    if dtype == "bf16":
        worst = (err - (2.0 ** -8 * np.abs(ref) + 1e-4)).max()
        assert worst <= 0, f"{name}: error exceeds rounding by {worst:.3e}"
    else:
        rel = err.max() / np.abs(ref).max()
        assert rel <= 1e-6, f"{name}: normwise rel err {rel:.3e}"


ROPE = [
    # (lengths, H, D, dtype, base)
    ([300, 0, 77, 1], 2, 64, "bf16", 10000.0),
    ([20000], 1, 128, "bf16", 10000.0),   # positions up to 20k: angles reduced in fp64
    ([513, 40], 3, 32, "bf16", 500.0),
    ([20000, 3], 1, 64, "fp32", 10000.0),
    ([129, 64], 2, 128, "fp32", 10000.0),
]


@pytest.mark.parametrize("idx", range(len(ROPE)))
def test_rope_every_element(idx):
    lengths, H, D, dtype, base = ROPE[idx]
    _print(f"rope {idx}: lengths={lengths} H={H} D={D} {dtype} base={base}")
    case = wl.random_case(900 + idx, lengths, H, D)
    dev, host = to_device(case, dtype)
    qr, kr = lsb.rope(dev["q"], dev["k"], dev["offsets"], base)
    assert_rotated("q_rot", np64(qr), oracle.rope(host["q"], host["offsets"], base), dtype)
    assert_rotated("k_rot", np64(kr), oracle.rope(host["k"], host["offsets"], base), dtype)
    # in place gives the same bits
    q2, k2 = dev["q"].clone(), dev["k"].clone()
    lsb.rope(q2, k2, dev["offsets"], base, q_rot=q2, k_rot=k2)
    assert torch.equal(q2, qr) and torch.equal(k2, kr)
    torch.cuda.synchronize()


ROPE_ATTN = [
    # (lengths, H, D, B, W, dtype, base)
    ([300, 1, 0, 129], 2, 64, 64, 2, "bf16", 10000.0),
    ([700, 64], 1, 128, 256, 3, "bf16", 10000.0),
    ([260, 31], 3, 32, 16, 4, "bf16", 100.0),
    ([500, 77], 2, 64, 1, 37, "bf16", 10000.0),   # sliding window of 37 tokens
    ([200, 45], 2, 64, 32, 2, "fp32", 10000.0),
    ([90, 130], 1, 128, 64, 2, "fp32", 10000.0),
]


def rope_attention_case(seed, lengths, H, D, B, W, dtype, base, scale):
    """rope, then the block-attention forward on the rotated q and k, then
    the backward with the rotation's transpose fused in: out, lse and the
    gradients with respect to the unrotated q, k and v.  The reference
    attends on the oracle's rotation stored in the call's dtype, as the GPU
    path stores its rotated q and k."""
    case = wl.random_case(seed, lengths, H, D)
    dev, host = to_device(case, dtype)
    qr, kr = lsb.rope(dev["q"], dev["k"], dev["offsets"], base)
    out, lse = lsb.fwd(qr, kr, dev["v"], dev["offsets"], B, W, scale)
    hq, hk = rotated_ref(host, base, dtype)
    o_ref, l_ref = oracle.fwd(hq, hk, host["v"], host["offsets"], B, W, scale)
    assert_close("out", np64(out), o_ref, dtype)
    assert_close("lse", np64(lse), l_ref, dtype, is_lse=True)
    grads = lsb.rope_bwd(qr, kr, dev["v"], out, dev["dout"], lse, dev["offsets"], B, W,
                         scale, base)
    refs = oracle.rope_bwd(hq, hk, host["v"], host["dout"], host["offsets"], B, W, scale,
                           base)
    for name, g, ref in zip(("dq", "dk", "dv"), grads, refs):
        assert_close(name, np64(g), ref, dtype)
    # dv does not see the rotation: the plain backward gives the same bits
    plain = lsb.bwd(qr, kr, dev["v"], out, dev["dout"], lse, dev["offsets"], B, W, scale)
    assert torch.equal(plain[2], grads[2])
    torch.cuda.synchronize()


@pytest.mark.parametrize("idx", range(len(ROPE_ATTN)))
def test_rope_attention_fwd_bwd_every_element(idx):
    lengths, H, D, B, W, dtype, base = ROPE_ATTN[idx]
    _print(f"rope attention {idx}: lengths={lengths} H={H} D={D} B={B} W={W} {dtype}")
    rope_attention_case(950 + idx, lengths, H, D, B, W, dtype, base, 1.0 / math.sqrt(D))


ROPE_RANDOM = random_shapes(8, 2030)


@pytest.mark.parametrize("idx", range(len(ROPE_RANDOM)))
def test_rope_attention_random_shape_every_element(idx):
    """Seeded random shapes (parity_util.random_shapes)."""
    lengths, H, D, B, W, dtype, sign = ROPE_RANDOM[idx]
    _print(f"rope random {idx}: lengths={lengths} H={H} D={D} B={B} W={W} {dtype}")
    rope_attention_case(1200 + idx, lengths, H, D, B, W, dtype, 10000.0, sign / math.sqrt(D))


@pytest.mark.timeout(900)
def test_rope_training_workload_every_element():
    """The training step with the rotary embedding at full size, in the
    launch configuration bench.py times, every element, in its two parts:

    1. the rope kernel on the workload's q and k against the oracle's
       rotation, within the RNE rounding of the result (its fp32 rotation and
       the oracle's fp64 one may round a value near a bf16 boundary to
       different neighbours, one ulp apart);
    2. the forward and the backward with the rotation's transpose fused in,
       run on the oracle's rotation stored in bf16, against the oracle on
       the same inputs: out, lse and the gradients with respect to the
       unrotated q, k (and v), at the block-attention bounds.

    (Feeding part 2 the GPU's own rotation would make the reference depend
    on which neighbour each one-ulp case took.)"""
    w = wl.WORKLOADS[7]
    _print(f"workload 7 ({w.name}), every element")
    c = wl.draw(w)
    dev, host = to_device_lazy(c, "bf16")
    B, W, sc, base = w.block_size, w.window_blocks, w.scale, w.rope_base
    off = host["offsets"]
    qr, kr = lsb.rope(dev["q"], dev["k"], dev["offsets"], base)
    torch.cuda.synchronize()
    T = int(off[-1])
    for name, g, x in (("q_rot", qr, host["q"]), ("k_rot", kr, host["k"])):
        ref = oracle.rope(x.double().numpy(), off, base)
        assert_rotated(name, np64(g), ref, "bf16")
        del ref
    _print("  rotation: every element within rounding")
    del qr, kr
    # the oracle's rotation, stored in bf16, as the attention inputs of both sides
    hq = torch.from_numpy(oracle.rope(host["q"].double().numpy(), off, base)).to(torch.bfloat16)
    hk = torch.from_numpy(oracle.rope(host["k"].double().numpy(), off, base)).to(torch.bfloat16)
    dq_, dk_ = hq.cuda(), hk.cuda()
    out, lse = lsb.fwd(dq_, dk_, dev["v"], dev["offsets"], B, W, sc)
    dq, dk, dv = lsb.rope_bwd(dq_, dk_, dev["v"], out, dev["dout"], lse, dev["offsets"], B, W,
                              sc, base)
    torch.cuda.synchronize()
    gpu = {"out": out.cpu(), "lse": lse.cpu(), "dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu()}
    del dev, dq_, dk_, out, lse, dq, dk, dv
    ins = {"offsets": off, "q": hq, "k": hk, "v": host["v"], "dout": host["dout"]}

    def reference(sub):
        o, l = oracle.fwd(sub["q"], sub["k"], sub["v"], sub["offsets"], B, W, sc)
        g = oracle.rope_bwd(sub["q"], sub["k"], sub["v"], sub["dout"], sub["offsets"], B, W,
                            sc, base)
        return {"out": o, "lse": l, "dq": g[0], "dk": g[1], "dv": g[2]}

    p = compare_by_users(ins, gpu, off, reference, "bf16", 1 << 30)
    _print("  " + p.summary())
