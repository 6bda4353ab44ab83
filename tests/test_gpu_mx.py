"""GPU parity of the forward with q and k in MXFP8 (block-scaled fp8 score
products), through the C ABI, against the fp64 oracle on the decoded values.

The format is read as the OCP MX format (E4M3 elements, one E8M0 scale per
32 head-dim elements; oracle.mx_decode), the one the pages' "MXFP8" names
("GEM (Meta)", section "Custom kernels").  Products of two E4M3 values are
exact and the scales are powers of two, so the scores are exact up to fp32
accumulation, and out and lse meet the bf16 bounds of block attention.
"""
import math

import numpy as np
import pytest
import torch

import long_sequence_block_amd as lsb
import oracle
from long_sequence_block_amd import workloads as wl
from parity_util import assert_close, check_sampled, np64

pytestmark = pytest.mark.gpu


def _print(msg):
    print(msg, flush=True)


def to_device_mx(c):
    """Device tensors: codes as is, scales head-major [H, T, D/32], v bf16;
    and the values the oracle sees (decoded q, k; bf16-rounded v)."""
    dev = {"offsets": torch.from_numpy(c["offsets"]).cuda()}
    for n in ("q", "k"):
        dev[n] = torch.from_numpy(c[n + "_mx"]).cuda()
        dev[n + "_sc"] = torch.from_numpy(np.ascontiguousarray(c[n + "_sc"].transpose(1, 0, 2))).cuda()
    vt = torch.from_numpy(c["v"]).to(torch.bfloat16)
    dev["v"] = vt.cuda()
    host = {"offsets": c["offsets"], "q": oracle.mx_decode(c["q_mx"], c["q_sc"]),
            "k": oracle.mx_decode(c["k_mx"], c["k_sc"]), "v": vt.double().numpy()}
    return dev, host


MX = [
    # (lengths, H, D, B, W, scale sign)
    ([300, 1, 0, 129], 2, 64, 64, 2, 1),
    ([700, 64, 3], 1, 128, 256, 3, 1),
    ([129, 255, 513, 7], 2, 64, 128, 2, -1),
    ([500, 77], 2, 128, 16, 4, 1),
    ([90, 300], 2, 64, 1, 37, 1),      # sliding window of 37 tokens
    ([1000, 16, 17], 1, 128, 256, 4, -1),
]


@pytest.mark.parametrize("idx", range(len(MX)))
def test_mx_fwd_every_element(idx):
    lengths, H, D, B, W, sign = MX[idx]
    _print(f"mx {idx}: lengths={lengths} H={H} D={D} B={B} W={W}")
    c = wl.random_mx_case(idx, lengths, H, D)
    dev, host = to_device_mx(c)
    scale = sign / math.sqrt(D)
    out, lse = lsb.mx_fwd(dev["q"], dev["q_sc"], dev["k"], dev["k_sc"], dev["v"],
                          dev["offsets"], B, W, scale)
    o_ref, l_ref = oracle.fwd(host["q"], host["k"], host["v"], host["offsets"], B, W, scale)
    assert_close("out", np64(out), o_ref, "bf16")
    assert_close("lse", np64(lse), l_ref, "bf16", is_lse=True)
    torch.cuda.synchronize()


@pytest.mark.parametrize("wid", [9, 10])
def test_mx_workload_full_size_sampled(wid):
    w = wl.WORKLOADS[wid]
    _print(f"workload {wid} ({w.name}), sampled rows")
    dev, host = to_device_mx(wl.draw(w))
    out, lse = lsb.mx_fwd(dev["q"], dev["q_sc"], dev["k"], dev["k_sc"], dev["v"],
                          dev["offsets"], w.block_size, w.window_blocks, w.scale)
    L = np.diff(host["offsets"])
    longest = int(np.argmax(L))
    samples = [(0, 0, 64), (longest, int(L[longest]) - 70, int(L[longest])),
               (longest, 3000, 3100), (len(L) - 1, 0, int(L[-1]))]
    check_sampled(dev, host, out, lse, None, w.block_size, w.window_blocks, w.scale, "bf16",
                  samples)
    torch.cuda.synchronize()
