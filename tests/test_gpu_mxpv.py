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
full size (user range by user range, each with its packed first token).
"""
import math

import numpy as np
import pytest
import torch

import long_sequence_block_amd as lsb
import oracle
from long_sequence_block_amd import workloads as wl
from parity_util import compare_by_users

pytestmark = pytest.mark.gpu

RHO = 2.0 ** -11   # relative error of a block-scaled fp8 product sum (test_gpu_mx)


def _print(msg):
    print(msg, flush=True)


def mxpv_parity(c, B, W, scale, max_tokens):
    """Run blockattn_mxpv_fwd on case c (q_mx, q_sc, k_mx, k_sc as for the
    MX forward; v_mx [T, H, D] with token-block scales v_bsc) and compare
    every element with the oracle."""
    T = int(c["offsets"][-1])
    vt, vs = wl.mx_v_device_layout(c["v_mx"], c["v_bsc"])
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
    v_bsc = c["v_bsc"]
    host = {"offsets": c["offsets"], "q_mx": c["q_mx"], "q_sc": c["q_sc"], "k_mx": c["k_mx"],
            "k_sc": c["k_sc"], "v_mx": c["v_mx"], "tok": np.arange(T, dtype=np.int64)}
    log2e = math.log2(math.e)

    def reference(sub):
        t0 = int(sub["tok"][0])
        off = sub["offsets"]
        q = oracle.mx_decode(sub["q_mx"], sub["q_sc"])
        k = oracle.mx_decode(sub["k_mx"], sub["k_sc"])
        v = oracle.mx_decode_tokens(sub["v_mx"], v_bsc, t0)
        o, l = oracle.mxpv_fwd(q, k, v, off, B, W, scale, first_token=t0)
        _, labs = oracle.fwd(np.abs(q), np.abs(k), v, off, B, W, abs(scale))
        eps = RHO * labs                                          # [H, T], natural log
        eps2 = (eps + 2.0 ** -20 * (labs + 1.0)) * log2e          # log2 domain, fp32 slack
        slack = oracle.mxpv_slack(q, k, v, off, B, W, scale, eps2, first_token=t0)
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
    # users that start off the 32-token grid, a block size not a multiple of 16
    ([45, 33, 70, 31, 64], 2, 64, 7, 5, 1),
    ([17, 600, 5], 2, 128, 100, 3, 1),
    # 1101 users: the tile decode's four-users-per-thread form
    ([int(x) for x in np.random.default_rng(32).integers(0, 30, 1101)], 1, 64, 16, 2, 1),
]


@pytest.mark.parametrize("idx", range(len(MXPV)))
def test_mxpv_fwd_every_element(idx):
    lengths, H, D, B, W, sign = MXPV[idx]
    _print(f"mxpv {idx}: {len(lengths)} users, lengths={lengths[:8]} H={H} D={D} B={B} W={W}")
    c = wl.random_mxpv_case(300 + idx, lengths, H, D)
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
