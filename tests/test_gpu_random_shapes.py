"""GPU parity on seeded random shapes: forward and backward, every element,
against the fp64 oracle, over block sizes, windows, head dims, head counts,
user counts and length mixes drawn from one fixed generator (a net for
combinations the listed cases do not name: short and empty users next to
long ones, blocks that do not divide a user or a tile, windows wider than a
user, negative scales)."""
import math

import numpy as np
import pytest

from long_sequence_block_amd import workloads as wl
from parity_util import check_full

pytestmark = pytest.mark.gpu


def _shapes(n, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        users = int(rng.integers(1, 11))
        kind = rng.random(users)
        lengths = [int(x) for x in np.where(
            kind < 0.15, rng.integers(0, 3, users),           # empty and one- or two-token users
            np.where(kind < 0.6, rng.integers(3, 130, users),  # short users
                     rng.integers(130, 700, users)))]          # users over several tiles
        H = int(rng.integers(1, 4))
        D = int(rng.choice([32, 64, 128]))
        B = int(np.exp(rng.uniform(0.0, math.log(300.0))))    # 1 .. 300, log-uniform
        W = int(rng.integers(1, 9))
        dtype = "fp32" if rng.random() < 0.2 else "bf16"
        sign = -1.0 if rng.random() < 0.25 else 1.0
        out.append((lengths, H, D, max(B, 1), W, dtype, sign))
    return out


SHAPES = _shapes(24)


@pytest.mark.parametrize("idx", range(len(SHAPES)))
def test_random_shape_every_element(idx):
    lengths, H, D, B, W, dtype, sign = SHAPES[idx]
    print(f"random shape {idx}: lengths={lengths} H={H} D={D} B={B} W={W} {dtype} "
          f"scale sign {sign:+.0f}", flush=True)
    case = wl.random_case(900 + idx, lengths, H, D)
    p = check_full(case, dtype, B, W, sign / math.sqrt(D), backward=True)
    print("  " + p.summary(), flush=True)
