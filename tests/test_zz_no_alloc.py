"""blockattn_bwd_noalloc (the backward with the library's static workspace)
against blockattn_bwd (a caller-owned workspace), through the C ABI: two
calls in a row on one GPU, the second with a smaller input, so the second
starts from the first call's leftovers in the shared array.  Both entry
points run the same kernels, so the outputs must agree bit for bit, which
is within the parity bounds."""
import math

import pytest
import torch

import long_sequence_block_amd as lsb
from long_sequence_block_amd import workloads as wl
from parity_util import to_device

pytestmark = pytest.mark.gpu

CALLS = [
    # (lengths, H, D, B, W, dtype): larger first, then smaller
    (([900, 33, 2000, 129, 0, 700], 4, 64, 128, 2, "bf16"),
     ([300, 17], 2, 64, 64, 3, "bf16")),
    (([1500, 64, 3], 2, 128, 256, 4, "bf16"),
     ([40, 0, 7], 1, 128, 16, 2, "bf16")),
    (([200, 45], 2, 32, 32, 2, "fp32"),
     ([30], 1, 32, 16, 1, "fp32")),
]


def _bwd_both(seed, lengths, H, D, B, W, dtype):
    case = wl.random_case(seed, lengths, H, D)
    dev, _ = to_device(case, dtype)
    scale = 1.0 / math.sqrt(D)
    out, lse = lsb.fwd(dev["q"], dev["k"], dev["v"], dev["offsets"], B, W, scale)
    ref = lsb.bwd(dev["q"], dev["k"], dev["v"], out, dev["dout"], lse, dev["offsets"], B, W,
                  scale)
    T = dev["q"].shape[0]
    got = tuple(torch.full_like(dev["q"], float("nan")) for _ in range(3))
    rc = lsb.blockattn_bwd_noalloc(
        dev["q"].data_ptr(), dev["k"].data_ptr(), dev["v"].data_ptr(), out.data_ptr(),
        dev["dout"].data_ptr(), lse.data_ptr(), dev["offsets"].data_ptr(), len(lengths), T, H,
        D, B, W, scale, lsb.BF16 if dtype == "bf16" else lsb.FP32, got[0].data_ptr(),
        got[1].data_ptr(), got[2].data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == lsb.binding.OK, lsb.blockattn_status_string(rc)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("idx", range(len(CALLS)))
def test_noalloc_matches_workspace_backward(idx):
    for n, (lengths, H, D, B, W, dtype) in enumerate(CALLS[idx]):
        print(f"noalloc case {idx} call {n}: lengths={lengths} H={H} D={D} B={B} W={W} {dtype}",
              flush=True)
        ref, got = _bwd_both(70 + 3 * idx + n, lengths, H, D, B, W, dtype)
        for name, r, g in zip(("dq", "dk", "dv"), ref, got):
            assert torch.equal(r, g), f"{name}: noalloc differs from the workspace backward"


def test_noalloc_rejects_sizes_beyond_the_array():
    T = 4 << 20
    assert lsb.blockattn_bwd_workspace_size(T, 2, 8, lsb.BF16) > lsb.NOALLOC_WORKSPACE_BYTES
    fake = 1 << 12
    rc = lsb.blockattn_bwd_noalloc(fake, fake, fake, fake, fake, fake, fake, 2, T, 8, 64, 64, 2,
                                   0.125, lsb.BF16, fake, fake, fake, None)
    assert rc == lsb.binding.ERR_WORKSPACE
