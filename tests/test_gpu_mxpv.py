"""GPU parity of the forward with q, k and v in MXFP8 and the softmax
weights quantized for a block-scaled P.V product (blockattn_mxpv_fwd),
through the C ABI, against the fp64 oracle (oracle.mxpv_fwd) on the decoded
values.  The reading of the quantization is oracle.mxpv_fwd's ("GEM (Meta)",
sections "Custom kernels" and "Ultra-low-precision training").

Bounds, on top of the block-attention bounds (parity_util):
  - the q.k scores come from the block-scaled fp8 instruction as in
    blockattn_mx_fwd: each score of row i is off by at most
    eps_i = rho * lse_i(|q|, |k|, |scale|) with rho = 2^-11 (see
    test_gpu_mx), which moves lse by at most eps_i and every normalised
    weight by a factor within exp(+-2 eps_i): out by at most
    (exp(2 eps_i) - 1) (1 + 2^-4) max|v| (a quantized weight is within 2^-4
    of its weight, plus a subnormal quantum);
  - a weight's E4M3 code depends only on its own block's scores, so the
    kernel and the oracle pick the same code unless the score error can
    carry the scaled weight across a rounding midpoint, or the block's
    maximum across an integer in the log2 domain; oracle.mxpv_slack adds,
    per output element, the largest change such flips allow (zero for
    every weight no flip can reach);
  - the P.V products sum with the same reduced precision as the scores:
    rho sum_j |Pq_ij v_j| / l_i <= rho (1 + 2^-4) sum_j P_ij |v_j| (the
    exact softmax on |v|, plus a little).
Every element is compared, in the small cases and in both workloads at
full size (user range by user range: a user's result does not depend on
the others).
"""
import math

import numpy as np
import pytest
import torch

import long_sequence_block_amd as lsb
import oracle
from long_sequence_block_amd import workloads as wl
from parity_util import compare_by_users, random_shapes

pytestmark = pytest.mark.gpu

RHO = 2.0 ** -11   # relative error of a block-scaled fp8 product sum (test_gpu_mx)


def _print(msg):
    print(msg, flush=True)


def mxpv_parity(c, B, W, scale, max_tokens):
    """Run blockattn_mxpv_fwd on case c (q_mx, q_sc, k_mx, k_sc as for the
    MX forward; v_mx [T, H, D] with user-block scales v_bsc) and compare
    every element with the oracle."""
    vt, vs = wl.mx_v_device_layout(c["v_mx"], c["v_bsc"], c["offsets"])
    dev = {"offsets": torch.from_numpy(c["offsets"]).cuda()}
    for n in ("q", "k"):
        dev[n] = torch.from_numpy(c[n + "_mx"]).cuda()
        dev[n + "_sc"] = torch.from_numpy(np.ascontiguousarray(c[n + "_sc"].transpose(1, 0, 2))).cuda()
    out, lse = lsb.mxpv_fwd(dev["q"], dev["q_sc"], dev["k"], dev["k_sc"],
                            torch.from_numpy(vt).cuda(), torch.from_numpy(vs).cuda(),
                            dev["offsets"], B, W, scale)
    torch.cuda.synchronize()
    gpu = {"out": out.cpu(), "lse": lse.cpu()}
    del dev, out, lse
    vfull = {"offsets": c["offsets"], "v_mx": c["v_mx"], "v_bsc": c["v_bsc"]}
    host = {"offsets": c["offsets"], "q_mx": c["q_mx"], "q_sc": c["q_sc"], "k_mx": c["k_mx"],
            "k_sc": c["k_sc"]}
    log2e = math.log2(math.e)

    def reference(sub):
        u0, u1 = sub["range"][:2]
        off = sub["offsets"]
        q = oracle.mx_decode(sub["q_mx"], sub["q_sc"])
        k = oracle.mx_decode(sub["k_mx"], sub["k_sc"])
        vs_ = wl.subset_users(vfull, slice(u0, u1))   # v's codes and re-indexed block scales
        v = oracle.mx_decode_user_blocks(vs_["v_mx"], vs_["v_bsc"], off)
        o, l = oracle.mxpv_fwd(q, k, v, off, B, W, scale)
        _, labs = oracle.fwd(np.abs(q), np.abs(k), v, off, B, W, abs(scale))
        eps = RHO * labs                                          # [H, T], natural log
        eps2 = (eps + 2.0 ** -20 * (labs + 1.0)) * log2e          # log2 domain, fp32 slack
        slack = oracle.mxpv_slack(q, k, v, off, B, W, scale, eps2)
        pabs, _ = oracle.fwd(q, k, np.abs(v), off, B, W, scale)   # sum_j P_ij |v_j|
        vmax = np.abs(v).max() if v.size else 0.0
        extra = (slack + (np.expm1(2.0 * eps) * 1.07 * vmax).T[:, :, None]
                 + RHO * 1.07 * pabs)
        return {"out": o, "lse": l, "extra:lse": eps, "extra:out": extra}

    return compare_by_users(host, gpu, c["offsets"], reference, "bf16", max_tokens)


MXPV = [
    # (lengths, H, D, B, W, scale sign)
    ([300, 1, 0, 129], 2, 64, 64, 2, 1),
    ([700, 64, 3], 1, 128, 256, 3, 1),
    ([129, 255, 513, 7], 2, 64, 128, 2, -1),
    ([500, 77], 2, 128, 16, 4, 1),
    ([90, 300], 2, 64, 1, 37, 1),      # sliding window of 37 tokens
    ([1000, 16, 17], 1, 128, 256, 4, -1),
    ([301, 0, 78], 1, 64, 64, 2, 1),
    ([129, 254], 3, 64, 16, 4, -1),
    # users that start off the packed 32-token grid, block sizes that are not
    # multiples of 32 (windows that start inside a 32-key block)
    ([45, 33, 70, 31, 64], 2, 64, 7, 5, 1),
    ([17, 600, 5], 2, 128, 100, 3, 1),
    # 1101 users: the tile decode's four-users-per-thread form
    ([int(x) for x in np.random.default_rng(32).integers(0, 30, 1101)], 1, 64, 16, 2, 1),
    # the largest block and window the ABI takes (clamped: every earlier key)
    ([300, 77, 0, 5, 130], 2, 64, 2**31 - 1, 2**31 - 1, 1),
]


@pytest.mark.parametrize("idx", range(len(MXPV)))
def test_mxpv_fwd_every_element(idx):
    lengths, H, D, B, W, sign = MXPV[idx]
    _print(f"mxpv {idx}: {len(lengths)} users, lengths={lengths[:8]} H={H} D={D} B={B} W={W}")
    c = wl.random_mxpv_case(300 + idx, lengths, H, D)
    p = mxpv_parity(c, B, W, sign / math.sqrt(D), 1 << 30)
    _print("  " + p.summary())


MXPV_RANDOM = random_shapes(12, 2028, head_dims=(64, 128), fp32_share=0.0)


@pytest.mark.parametrize("idx", range(len(MXPV_RANDOM)))
def test_mxpv_fwd_random_shape_every_element(idx):
    """Seeded random shapes (parity_util.random_shapes)."""
    lengths, H, D, B, W, _, sign = MXPV_RANDOM[idx]
    _print(f"mxpv random {idx}: lengths={lengths} H={H} D={D} B={B} W={W} sign {sign:+.0f}")
    c = wl.random_mxpv_case(450 + idx, lengths, H, D)
    p = mxpv_parity(c, B, W, sign / math.sqrt(D), 1 << 30)
    _print("  " + p.summary())


# Codes over the whole finite E4M3 range with block scales far from 2^0
# (q 2^-33 .. 2^-27, k 2^13 .. 2^19; v 2^-8 .. 2^-6, or v blocks 2^-17 ..
# 2^-7 apart by up to 2^10, |v| <= 3.5 so that the bf16 mean bound applies).
MXPV_WIDE = [
    ([300, 1, 0, 129], 2, 64, 64, 2, 1, ((94, 100), (140, 146), (119, 121))),
    ([700, 64, 3], 1, 128, 256, 3, -1, ((94, 100), (140, 146), (110, 120))),
]


@pytest.mark.parametrize("idx", range(len(MXPV_WIDE)))
def test_mxpv_fwd_full_code_range_every_element(idx):
    lengths, H, D, B, W, sign, wide = MXPV_WIDE[idx]
    _print(f"mxpv wide {idx}: lengths={lengths} H={H} D={D} B={B} W={W} scales {wide}")
    c = wl.random_mxpv_case(400 + idx, lengths, H, D, wide=wide)
    assert (c["v_mx"] & 0x7F == 0).any() and ((c["v_mx"] & 0x78) == 0).any()
    p = mxpv_parity(c, B, W, sign / math.sqrt(D), 1 << 30)
    _print("  " + p.summary())


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wid", [13, 14])
def test_mxpv_workload_full_size_every_element(wid):
    w = wl.WORKLOADS[wid]
    _print(f"workload {wid} ({w.name}) full size, every element")
    c = wl.draw(w)
    p = mxpv_parity(c, w.block_size, w.window_blocks, w.scale, 4 * 16384)
    _print("  " + p.summary())


def _concat_users(a, b):
    """Case a's users followed by case b's, each user's v block scales moved
    to its new blocks."""
    off = np.concatenate([a["offsets"], a["offsets"][-1] + b["offsets"][1:]]).astype(np.int32)
    c = {"offsets": off}
    for n in ("q_mx", "q_sc", "k_mx", "k_sc", "v_mx"):
        c[n] = np.concatenate([a[n], b[n]])
    bsc = np.zeros((wl.mx_v_blocks(off),) + a["v_bsc"].shape[1:], np.uint8)
    nbase = wl.user_block_base(off)
    i = 0
    for part in (a, b):
        base = wl.user_block_base(part["offsets"])
        for u in range(len(part["offsets"]) - 1):
            n = -(-int(part["offsets"][u + 1] - part["offsets"][u]) // 32)
            bsc[nbase[i]:nbase[i] + n] = part["v_bsc"][base[u]:base[u] + n]
            i += 1
    c["v_bsc"] = bsc
    return c


def _run(c, B, W, scale):
    vt, vs = wl.mx_v_device_layout(c["v_mx"], c["v_bsc"], c["offsets"])
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    out, lse = lsb.mxpv_fwd(d(c["q_mx"]), d(c["q_sc"].transpose(1, 0, 2)), d(c["k_mx"]),
                            d(c["k_sc"].transpose(1, 0, 2)), d(vt), d(vs), d(c["offsets"]),
                            B, W, scale)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def test_mxpv_users_are_independent():
    """A user's output and lse are bitwise the same with other users in
    front of it (a different packed position, other block bases)."""
    users = wl.random_mxpv_case(510, [45, 70, 0, 33], 2, 64)
    pre = wl.random_mxpv_case(511, [3, 29, 1], 2, 64)
    B, W, scale = 16, 3, 0.125
    o1, l1 = _run(users, B, W, scale)
    o2, l2 = _run(_concat_users(pre, users), B, W, scale)
    n = int(pre["offsets"][-1])
    assert torch.equal(o1.view(torch.int16), o2[n:].view(torch.int16))
    assert torch.equal(l1, l2[:, n:])
