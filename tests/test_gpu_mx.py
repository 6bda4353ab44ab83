"""GPU parity of the forward with q and k in MXFP8 (block-scaled fp8 score
products), through the C ABI, against the fp64 oracle on the decoded values.

The format is read as the OCP MX format (E4M3 elements, one E8M0 scale per
32 head-dim elements; oracle.mx_decode), the one the pages' "MXFP8" names
("GEM (Meta)", section "Custom kernels").  The oracle attends in fp64 on the
exactly decoded values.

Bounds.  gfx950's block-scaled fp8 matrix instruction, which computes each
score, sums its 64 products with fewer bits than fp32: measured on the box
(scores of single-token users, where lse = the score), its error reaches
2^-12.0 of sum_d |q_d k_d| on draws over every finite code, against 2^-24
for an fp32 sum.  With rho = 2^-11 (twice that), each score of row i is off
by at most eps_i = rho * max_j |scale| sum_d |q_id k_jd|, bounded from above
by the oracle's lse of the same row on |q|, |k| and |scale| (an lse is at
least its largest term, and these terms are >= 0).  lse moves by at most
eps_i (an lse is 1-Lipschitz in each score), and every softmax weight by a
factor within exp(+-2 eps_i), so out moves by at most
(exp(2 eps_i) - 1) max|v|.  Those two allowances come on top of the
block-attention bounds (parity_util).  Every element is compared, in the
small cases and in both MXFP8 workloads at full size.
"""
import math

import numpy as np
import pytest
import torch

import long_sequence_block_amd as lsb
import oracle
from long_sequence_block_amd import workloads as wl
from parity_util import Parity, compare_by_users, np64, random_shapes

pytestmark = pytest.mark.gpu

MX_RHO = 2.0 ** -11  # score error relative to sum_d |q_d k_d| (see above)


def _print(msg):
    print(msg, flush=True)


def to_device_mx(c):
    """Device tensors: codes as is, scales head-major [H, T, D/32], v bf16.
    The host keeps the codes, the token-major scales and the bf16 v; the
    oracle decodes them (exactly, in fp64) range by range."""
    dev = {"offsets": torch.from_numpy(c["offsets"]).cuda()}
    for n in ("q", "k"):
        dev[n] = torch.from_numpy(c[n + "_mx"]).cuda()
        dev[n + "_sc"] = torch.from_numpy(np.ascontiguousarray(c[n + "_sc"].transpose(1, 0, 2))).cuda()
    vt = torch.from_numpy(c["v"]).to(torch.bfloat16)
    dev["v"] = vt.cuda()
    host = {"offsets": c["offsets"], "q_mx": c["q_mx"], "q_sc": c["q_sc"],
            "k_mx": c["k_mx"], "k_sc": c["k_sc"], "v": vt}
    return dev, host


def mx_parity(c, B, W, scale, max_tokens):
    dev, host = to_device_mx(c)
    out, lse = lsb.mx_fwd(dev["q"], dev["q_sc"], dev["k"], dev["k_sc"], dev["v"],
                          dev["offsets"], B, W, scale)
    torch.cuda.synchronize()
    gpu = {"out": out.cpu(), "lse": lse.cpu()}
    del dev, out, lse

    def reference(sub):
        q = oracle.mx_decode(sub["q_mx"], sub["q_sc"])
        k = oracle.mx_decode(sub["k_mx"], sub["k_sc"])
        o, l = oracle.fwd(q, k, sub["v"], sub["offsets"], B, W, scale)
        _, labs = oracle.fwd(np.abs(q), np.abs(k), sub["v"], sub["offsets"], B, W, abs(scale))
        eps = MX_RHO * labs                                   # [H, T]
        vmax = np.abs(sub["v"]).max() if sub["v"].size else 0.0
        return {"out": o, "lse": l, "extra:lse": eps,
                "extra:out": (np.expm1(2.0 * eps) * vmax).T[:, :, None]}

    return compare_by_users(host, gpu, host["offsets"], reference, "bf16", max_tokens)


MX = [
    # (lengths, H, D, B, W, scale sign)
    ([300, 1, 0, 129], 2, 64, 64, 2, 1),
    ([700, 64, 3], 1, 128, 256, 3, 1),
    ([129, 255, 513, 7], 2, 64, 128, 2, -1),
    ([500, 77], 2, 128, 16, 4, 1),
    ([90, 300], 2, 64, 1, 37, 1),      # sliding window of 37 tokens
    ([1000, 16, 17], 1, 128, 256, 4, -1),
    # T * H * D/32 not a multiple of 4: the last head's last key-scale window
    # ends inside a dword (read byte by byte)
    ([301, 0, 78], 1, 64, 64, 2, 1),
    ([129, 254], 3, 64, 16, 4, -1),
    # the largest block and window the ABI takes (clamped: every earlier key)
    ([300, 77, 0, 5, 130], 2, 128, 2**31 - 1, 2**31 - 1, -1),
    # 1101 users: the tile decode's four-users-per-thread form
    ([int(x) for x in np.random.default_rng(31).integers(0, 30, 1101)], 1, 64, 16, 2, 1),
]


@pytest.mark.parametrize("idx", range(len(MX)))
def test_mx_fwd_every_element(idx):
    lengths, H, D, B, W, sign = MX[idx]
    _print(f"mx {idx}: {len(lengths)} users, lengths={lengths[:8]} H={H} D={D} B={B} W={W}")
    c = wl.random_mx_case(idx, lengths, H, D)
    mx_parity(c, B, W, sign / math.sqrt(D), 1 << 30)


MX_RANDOM = random_shapes(10, 2031, head_dims=(64, 128), fp32_share=0.0)


@pytest.mark.parametrize("idx", range(len(MX_RANDOM)))
def test_mx_fwd_random_shape_every_element(idx):
    """Seeded random shapes (parity_util.random_shapes)."""
    lengths, H, D, B, W, _, sign = MX_RANDOM[idx]
    _print(f"mx random {idx}: lengths={lengths} H={H} D={D} B={B} W={W} sign {sign:+.0f}")
    c = wl.random_mx_case(200 + idx, lengths, H, D)
    mx_parity(c, B, W, sign / math.sqrt(D), 1 << 30)


# Codes over the whole finite E4M3 range (both zeros, subnormals, every
# exponent up to 448) with block scales far from 2^0: q blocks 2^-33 .. 2^-27
# and k blocks 2^13 .. 2^19, so each product of two scales is 2^-20 .. 2^-8
# and the scores stay in the range where fp32 resolves lse to 1e-3.
MX_WIDE = [
    # (lengths, H, D, B, W, scale sign, q scale range, k scale range)
    ([300, 1, 0, 129], 2, 64, 64, 2, 1, (94, 100), (140, 146)),
    ([700, 64, 3], 1, 128, 256, 3, -1, (94, 100), (140, 146)),
    ([200, 77], 2, 64, 16, 4, 1, (140, 146), (94, 100)),
]


@pytest.mark.parametrize("idx", range(len(MX_WIDE)))
def test_mx_fwd_full_code_range_every_element(idx):
    lengths, H, D, B, W, sign, qr, kr = MX_WIDE[idx]
    _print(f"mx wide {idx}: lengths={lengths} H={H} D={D} B={B} W={W} q sc {qr} k sc {kr}")
    c = wl.random_mx_case(100 + idx, lengths, H, D, wide=(qr, kr))
    # the draw exercises what it is meant to: zeros, subnormals, extreme scales
    assert (c["q_mx"] & 0x7F == 0).any() and ((c["k_mx"] & 0x78) == 0).any()
    # and its scores stay where fp32 lse keeps 1e-3 (|s| well below 2^10)
    q = oracle.mx_decode(c["q_mx"], c["q_sc"])
    k = oracle.mx_decode(c["k_mx"], c["k_sc"])
    s_max = np.abs(np.einsum("thd,thd->th", q[:64], k[:64])).max() / math.sqrt(D)
    assert s_max < 256, s_max
    p = mx_parity(c, B, W, sign / math.sqrt(D), 1 << 30)
    _print("  " + p.summary())


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wid", [9, 10])
def test_mx_workload_full_size_every_element(wid):
    w = wl.WORKLOADS[wid]
    _print(f"workload {wid} ({w.name}) full size, every element")
    c = wl.draw(w)
    max_tokens = 4 * w.fixed_length if w.fixed_length else 1 << 30
    p = mx_parity(c, w.block_size, w.window_blocks, w.scale, max_tokens)
    _print("  " + p.summary())


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("scales", [None, ((119, 121), (119, 121)), ((94, 100), (140, 146))])
def test_mx_score_precision_within_rho(D, scales):
    """The measurement the bounds above rest on.  Users of one token see only
    themselves, so lse_i = scale <q_i, k_i> exactly: on 8192 such rows, every
    GPU score is within MX_RHO * |scale| sum_d |q_d k_d| of the exact one
    (draws: the workloads' codes, or every finite code under two scale
    ranges)."""
    wide = None if scales is None else scales
    c = wl.random_mx_case(300 + D, [1] * 4096, 2, D, wide=wide)
    dev, _ = to_device_mx(c)
    scale = 1.0 / math.sqrt(D)
    _, lse = lsb.mx_fwd(dev["q"], dev["q_sc"], dev["k"], dev["k_sc"], dev["v"], dev["offsets"],
                        1, 1, scale)
    torch.cuda.synchronize()
    q = oracle.mx_decode(c["q_mx"], c["q_sc"])
    k = oracle.mx_decode(c["k_mx"], c["k_sc"])
    exact = scale * np.einsum("thd,thd->ht", q, k)
    mag = scale * np.einsum("thd,thd->ht", np.abs(q), np.abs(k))
    err = np.abs(np64(lse) - exact)
    worst = float((err / np.maximum(mag, 1e-300)).max())
    _print(f"D={D} scales={scales}: max err / sum|qk| = {worst:.3e} (2^{np.log2(worst + 1e-300):.1f})")
    assert np.all(err <= MX_RHO * mag + 1e-6)
