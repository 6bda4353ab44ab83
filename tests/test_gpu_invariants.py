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
