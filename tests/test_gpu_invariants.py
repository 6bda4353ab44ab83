"""Invariants of the definition checked bitwise on the GPU path.

Block attention is exact with respect to its definition, so properties that
hold for the definition must hold bit for bit for a kernel that only ever
touches visible keys and treats every (user, head) independently:
determinism, locality (keys outside a query's window do not matter), jagged
semantics (users can be split, permuted, or padded with empty users) and
head independence.
"""
import numpy as np
import pytest
import torch

import long_sequence_block_amd as lsb
from long_sequence_block_amd import workloads as wl
from parity_util import run_bwd, run_fwd, to_device

pytestmark = pytest.mark.gpu

CONFIGS = [(64, 64, 2, "bf16"), (128, 128, 2, "bf16"), (32, 32, 1, "fp32"),
           (128, 256, 4, "bf16"), (64, 48, 3, "bf16")]


def _run(case, dtype, B, W, backward=True):
    dev, _ = to_device(case, dtype)
    out, lse = run_fwd(dev, B, W, 0.125)
    res = [out, lse]
    if backward:
        res += list(run_bwd(dev, out, lse, B, W, 0.125))
    torch.cuda.synchronize()
    return [r.cpu() for r in res]


@pytest.mark.parametrize("D,B,W,dtype", CONFIGS)
def test_determinism(D, B, W, dtype):
    print(f"determinism D={D} B={B} W={W} {dtype}", flush=True)
    case = wl.random_case(31, [700, 33, 260], 2, D)
    a = _run(case, dtype, B, W)
    b = _run(case, dtype, B, W)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("D,B,W,dtype", CONFIGS)
def test_locality_outside_window(D, B, W, dtype):
    """Perturbing K/V rows that row i cannot see leaves O_i, lse_i bitwise."""
    print(f"locality D={D} B={B} W={W} {dtype}", flush=True)
    L = 6 * B + 11
    case = wl.random_case(32, [L], 1, D, with_dout=False)
    base = _run(case, dtype, B, W, backward=False)
    i = 4 * B + 5                                   # a query in block 4
    lo = max(0, i // B - W + 1) * B
    pert = {k: v.copy() for k, v in case.items()}
    rng = np.random.default_rng(0)
    for name in ("k", "v"):
        pert[name][:lo] = rng.standard_normal(pert[name][:lo].shape) * 3
        pert[name][i + 1:] = rng.standard_normal(pert[name][i + 1:].shape) * 3
    got = _run(pert, dtype, B, W, backward=False)
    assert torch.equal(got[0][i], base[0][i])
    assert torch.equal(got[1][:, i], base[1][:, i])


@pytest.mark.parametrize("D,B,W,dtype", CONFIGS)
def test_jagged_split_permute_empty_users(D, B, W, dtype):
    print(f"jagged D={D} B={B} W={W} {dtype}", flush=True)
    lengths = [3 * B + 1, 17, 0, 2 * B, B - 1]
    case = wl.random_case(33, lengths, 2, D)
    full = _run(case, dtype, B, W)
    off = case["offsets"]
    perm = [4, 1, 2, 0, 3]
    rows = np.concatenate([np.arange(off[u], off[u + 1]) for u in perm])
    new = {k: (v[rows] if k != "offsets" else None) for k, v in case.items()}
    new["offsets"] = wl.offsets_from_lengths([0] + [lengths[u] for u in perm] + [0, 0])
    got = _run(new, dtype, B, W)
    r = torch.from_numpy(rows)
    for x, y in zip(got[:1] + got[2:], full[:1] + full[2:]):
        assert torch.equal(x, y[r])
    assert torch.equal(got[1], full[1][:, r])
    # one user on its own
    a, b = off[0], off[1]
    one = {k: (v[a:b] if k != "offsets" else np.array([0, b - a], np.int32))
           for k, v in case.items()}
    got1 = _run(one, dtype, B, W)
    assert torch.equal(got1[0], full[0][a:b]) and torch.equal(got1[2], full[2][a:b])


@pytest.mark.parametrize("D,B,W,dtype", CONFIGS[:2])
def test_heads_independent(D, B, W, dtype):
    case = wl.random_case(34, [400, 90], 3, D)
    base = _run(case, dtype, B, W)
    pert = {k: v.copy() for k, v in case.items()}
    for name in ("q", "k", "v", "dout"):
        pert[name][:, 1] *= -2.0
    got = _run(pert, dtype, B, W)
    for x, y in zip(got[:1] + got[2:], base[:1] + base[2:]):
        assert torch.equal(x[:, [0, 2]], y[:, [0, 2]])
    assert torch.equal(got[1][[0, 2]], base[1][[0, 2]])


def _variants(case, mxcase):
    """One call of every variant entry point (bf16): sliding window, rotary
    embedding with its fused backward, both GDPA activations, MXFP8."""
    import long_sequence_block_amd as lsb
    dev, _ = to_device(case, "bf16")
    q, k, v, do, off = dev["q"], dev["k"], dev["v"], dev["dout"], dev["offsets"]
    res = []
    o, l = lsb.swa_fwd(q, k, v, off, 45, 0.125)
    res += [o, l, *lsb.swa_bwd(q, k, v, o, do, l, off, 45, 0.125)]
    qr, kr = lsb.rope(q, k, off, 10000.0)
    o, l = lsb.fwd(qr, kr, v, off, 64, 2, 0.125)
    res += [qr, kr, o, l, *lsb.rope_bwd(qr, kr, v, o, do, l, off, 64, 2, 0.125)]
    for act in (lsb.GDPA_SILU, lsb.GDPA_GELU):
        o = lsb.gdpa_fwd(q, k, v, off, 64, 2, 0.125, act)
        res += [o, *lsb.gdpa_bwd(q, k, v, do, off, 64, 2, 0.125, act)]
    m = {n: torch.from_numpy(np.ascontiguousarray(mxcase[n].transpose(1, 0, 2)) if n.endswith("_sc")
                             else mxcase[n]).cuda() for n in ("q_mx", "q_sc", "k_mx", "k_sc")}
    vm = torch.from_numpy(mxcase["v"]).to(torch.bfloat16).cuda()
    om = torch.from_numpy(mxcase["offsets"]).cuda()
    res += list(lsb.mx_fwd(m["q_mx"], m["q_sc"], m["k_mx"], m["k_sc"], vm, om, 64, 2, 0.125))
    torch.cuda.synchronize()
    return [r.cpu() for r in res]


def test_variant_entry_points_are_deterministic():
    """Every variant entry point gives the same bits on a second call (the
    header's determinism promise covers them all)."""
    print("variant determinism", flush=True)
    case = wl.random_case(32, [700, 33, 260], 2, 64)
    mxcase = wl.random_mx_case(7, [700, 33, 260], 2, 64)
    a, b = _variants(case, mxcase), _variants(case, mxcase)
    for i, (x, y) in enumerate(zip(a, b)):
        assert torch.equal(x, y), i


def test_gdpa_locality_outside_window():
    """GDPA on the block pattern: keys and values outside every window of a
    set of queries do not change their outputs, bit for bit."""
    import long_sequence_block_amd as lsb
    print("gdpa locality", flush=True)
    B, W, L = 64, 2, 600
    case = wl.random_case(33, [L], 2, 64)
    dev, _ = to_device(case, "bf16")
    o1 = lsb.gdpa_fwd(dev["q"], dev["k"], dev["v"], dev["offsets"], B, W, 0.125, lsb.GDPA_GELU)
    k2, v2 = dev["k"].clone(), dev["v"].clone()
    # rows 448.. (blocks 7, 8, 9) see keys from block 6 on: perturb blocks 0..5
    k2[:384] += 1.0
    v2[:384] -= 2.0
    o2 = lsb.gdpa_fwd(dev["q"], k2, v2, dev["offsets"], B, W, 0.125, lsb.GDPA_GELU)
    torch.cuda.synchronize()
    assert torch.equal(o1[448:], o2[448:])
    assert not torch.equal(o1[:448], o2[:448])


def test_side_stream_calls_match_current_stream():
    """fwd and bwd issued on a side stream (outputs and workspace allocated by
    the binding on that stream) give the same bits as on the current stream,
    while the current stream keeps allocating and writing memory of the
    workspace's size: a workspace handed back to the allocator too early
    would be overwritten under the backward's kernels."""
    print("side stream", flush=True)
    case = wl.random_case(41, [900, 33, 2000, 129], 4, 64)
    dev, _ = to_device(case, "bf16")
    ref = _run(case, "bf16", 128, 2)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out, lse = lsb.fwd(dev["q"], dev["k"], dev["v"], dev["offsets"], 128, 2, 0.125, stream=side)
    grads = lsb.bwd(dev["q"], dev["k"], dev["v"], out, dev["dout"], lse, dev["offsets"], 128, 2,
                    0.125, stream=side)
    T, H, _ = case["q"].shape
    n = lsb.blockattn_bwd_workspace_size(T, len(case["offsets"]) - 1, H, lsb.BF16)
    for i in range(64):  # churn on the current stream meanwhile
        junk = torch.empty(n, dtype=torch.uint8, device="cuda")
        junk.fill_(i)
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for x, y in zip(ref, [out, lse, *grads]):
        assert torch.equal(x, y.cpu())
