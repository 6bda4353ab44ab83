"""Pins of the fp64 oracle against things other than itself.

Each test ties the oracle to a closed form, a library routine, brute force
on tiny inputs, an invariant of the definition, or a value worked out by
hand (tests/golden/hand_cases.json).  Together they are chosen so that a
dropped term, a wrong sign or index, a shifted window or a transposed
operand in the oracle fails at least one of them.

The definition being pinned is block attention as described by "GEM (Meta)"
(aiwiki.ai), section "Custom kernels", and the ai.info news item, section
"Kunlun changes how GEM scales", with the readings stated in the oracle's
header (window of W blocks including the query's own, causal, blocks
left-aligned per user).
"""
import json
import math
import os
import subprocess
import sys

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from long_sequence_block_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def visible_mask(L, B, W):
    """Predicate form of the visibility rule, materialised densely."""
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    return (j <= i) & ((i // B) - (j // B) <= W - 1)


def brute_force_user(q, k, v, B, W, scale):
    """Dense masked attention of one user, all heads: [L,H,D] inputs.

    Uses torch's scaled_dot_product_attention (fp64, CPU, boolean mask) for
    the output and scipy's logsumexp over masked scores for lse.
    """
    L, H, D = q.shape
    mask = visible_mask(L, B, W)
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.from_numpy(mask), scale=scale)
    s = np.einsum("hid,hjd->hij", qt.numpy(), kt.numpy()) * scale
    s = np.where(mask[None], s, -np.inf)
    lse = logsumexp(s, axis=-1)
    return o.numpy().transpose(1, 0, 2), lse


def case(seed, lengths, H=2, D=4):
    c = wl.random_case(seed, lengths, H, D)
    return {k: (v.astype(np.float64) if k != "offsets" else v) for k, v in c.items()}


# ---------------------------------------------------------------- golden


def test_golden_hand_cases():
    data = json.load(open(GOLDEN))
    for c in data["cases"]:
        off = wl.offsets_from_lengths(c["lengths"])
        T = int(off[-1])
        shp = (T, 1, 1)
        q, k, v = (np.array(c[n], np.float64).reshape(shp) for n in "qkv")
        out, lse = oracle.fwd(q, k, v, off, c["block_size"], c["window_blocks"], c["scale"])
        np.testing.assert_allclose(out.ravel(), c["out"], rtol=0, atol=1e-12, err_msg=c["name"])
        np.testing.assert_allclose(lse.ravel(), c["lse"], rtol=0, atol=1e-12, err_msg=c["name"])
        if "dout" in c:
            do = np.array(c["dout"], np.float64).reshape(shp)
            dq, dk, dv = oracle.bwd(q, k, v, do, off, c["block_size"], c["window_blocks"], c["scale"])
            for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
                np.testing.assert_allclose(got.ravel(), c[name], rtol=0, atol=1e-12,
                                           err_msg=f"{c['name']}:{name}")


# ----------------------------------------------------------- closed forms


@pytest.mark.parametrize("B,W", [(4, 1), (4, 2), (8, 3), (5, 2), (1, 1), (3, 4)])
def test_zero_query_uniform_weights(B, W):
    """q = 0 makes all visible weights equal: lse_i = ln n_i, O_i = mean v_j.

    n_i is counted here from the dense predicate mask, independently of the
    oracle's own range arithmetic.
    """
    lengths = [1, 7, 16, 23, 0, 9]
    c = case(11, lengths, H=2, D=3)
    q = np.zeros_like(c["q"])
    out, lse = oracle.fwd(q, c["k"], c["v"], c["offsets"], B, W, 0.7)
    off = c["offsets"]
    for u in range(len(lengths)):
        a, b = off[u], off[u + 1]
        mask = visible_mask(b - a, B, W)
        n = mask.sum(1)
        for h in range(2):
            np.testing.assert_allclose(lse[h, a:b], np.log(n), atol=1e-13, rtol=0)
            mean = (mask.astype(np.float64) @ c["v"][a:b, h, :]) / n[:, None]
            np.testing.assert_allclose(out[a:b, h, :], mean, atol=1e-13, rtol=0)


def test_constant_v_gives_constant_output_and_zero_qk_grads():
    lengths = [13, 5, 30]
    c = case(12, lengths)
    v = np.full_like(c["v"], 0.0)
    v[..., :] = np.array([1.5, -2.0, 0.25, 3.0])
    out, _ = oracle.fwd(c["q"], c["k"], v, c["offsets"], 4, 2, 0.5)
    np.testing.assert_allclose(out, v, atol=1e-13, rtol=0)
    dq, dk, dv = oracle.bwd(c["q"], c["k"], v, c["dout"], c["offsets"], 4, 2, 0.5)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
    assert np.abs(dv).max() > 0.1


# ------------------------------------------------- library special cases


@pytest.mark.parametrize("lengths", [[17], [1, 40, 33], [64, 3]])
def test_whole_window_is_dense_causal_attention(lengths):
    """W >= number of blocks: each user gets plain causal attention
    (torch SDPA with is_causal=True, fp64)."""
    B = 8
    c = case(13, lengths, H=3, D=5)
    W = max(math.ceil(L / B) for L in lengths) + 1
    scale = 0.37
    out, _ = oracle.fwd(c["q"], c["k"], c["v"], c["offsets"], B, W, scale)
    off = c["offsets"]
    for u in range(len(lengths)):
        a, b = off[u], off[u + 1]
        t = [torch.from_numpy(np.ascontiguousarray(c[n][a:b].transpose(1, 0, 2))) for n in "qkv"]
        ref = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=True, scale=scale)
        np.testing.assert_allclose(out[a:b], ref.numpy().transpose(1, 0, 2), atol=1e-13, rtol=0)


def test_window_one_is_independent_causal_blocks():
    """W = 1 with B dividing L: reshape each user to [L/B, B] blocks and run
    causal SDPA on every block on its own."""
    B = 8
    lengths = [32, 16, 8]
    c = case(14, lengths, H=2, D=6)
    out, _ = oracle.fwd(c["q"], c["k"], c["v"], c["offsets"], B, 1, 0.41)
    off = c["offsets"]
    for u, L in enumerate(lengths):
        a = off[u]
        blk = [torch.from_numpy(np.ascontiguousarray(
            c[n][a:a + L].reshape(L // B, B, 2, 6).transpose(0, 2, 1, 3))) for n in "qkv"]
        ref = torch.nn.functional.scaled_dot_product_attention(*blk, is_causal=True, scale=0.41)
        ref = ref.numpy().transpose(0, 2, 1, 3).reshape(L, 2, 6)
        np.testing.assert_allclose(out[a:a + L], ref, atol=1e-13, rtol=0)


def test_one_block_sequence_is_ordinary_attention():
    """L <= B: one (partial) block, so the result is causal softmax attention."""
    c = case(15, [7], H=1, D=4)
    out, lse = oracle.fwd(c["q"], c["k"], c["v"], c["offsets"], 16, 1, 0.9)
    q, k, v = c["q"][:, 0], c["k"][:, 0], c["v"][:, 0]
    s = 0.9 * q @ k.T
    s[np.triu_indices(7, 1)] = -np.inf
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    np.testing.assert_allclose(out[:, 0], p @ v, atol=1e-13, rtol=0)


# ------------------------------------------------------------ brute force


@pytest.mark.parametrize("B", [4, 8])
@pytest.mark.parametrize("W", [1, 2, 3])
def test_brute_force_general_window(B, W):
    lengths = [0, 1, 3, 4, 9, 17, 70, 26]
    c = case(100 + 10 * B + W, lengths, H=2, D=8)
    out, lse = oracle.fwd(c["q"], c["k"], c["v"], c["offsets"], B, W, 0.3)
    off = c["offsets"]
    for u in range(len(lengths)):
        a, b = off[u], off[u + 1]
        if a == b:
            continue
        o_ref, lse_ref = brute_force_user(c["q"][a:b], c["k"][a:b], c["v"][a:b], B, W, 0.3)
        np.testing.assert_allclose(out[a:b], o_ref, atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse[:, a:b], lse_ref, atol=1e-12, rtol=0)


# -------------------------------------------- token sliding window (B = 1)
#
# The sliding window that block attention replaced ("GEM (Meta)", section
# "Custom kernels") is computed as blocks of one token with a window of w
# blocks.  These pins tie that path to the token band written directly.


def band_mask(L, w):
    """The token band i - w < j <= i, with no block index in it."""
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    return (j <= i) & (i - j < w)


@pytest.mark.parametrize("w", [1, 2, 5, 16, 100])
def test_sliding_window_is_a_token_band(w):
    lengths = [0, 1, 7, 30, 64]
    c = case(300 + w, lengths, H=2, D=6)
    sc = 0.45
    out, lse = oracle.fwd(c["q"], c["k"], c["v"], c["offsets"], 1, w, sc)
    off = c["offsets"]
    for u, L in enumerate(lengths):
        a, b = off[u], off[u + 1]
        if L == 0:
            continue
        mask = band_mask(L, w)
        t = [torch.from_numpy(np.ascontiguousarray(c[n][a:b].transpose(1, 0, 2))) for n in "qk"]
        vt = torch.from_numpy(np.ascontiguousarray(c["v"][a:b].transpose(1, 0, 2)))
        ref = torch.nn.functional.scaled_dot_product_attention(
            t[0], t[1], vt, attn_mask=torch.from_numpy(mask), scale=sc)
        np.testing.assert_allclose(out[a:b], ref.numpy().transpose(1, 0, 2), atol=1e-12, rtol=0)
        s = np.einsum("hid,hjd->hij", t[0].numpy(), t[1].numpy()) * sc
        lse_ref = logsumexp(np.where(mask[None], s, -np.inf), axis=-1)
        np.testing.assert_allclose(lse[:, a:b], lse_ref, atol=1e-12, rtol=0)


def test_sliding_window_of_one_token():
    """w = 1: every query sees only itself, so out = v, lse = scale <q_i, k_i>,
    dV = dO, and dQ = dK = 0 (a softmax over a single key is constant)."""
    c = case(320, [9, 0, 4], H=2, D=5)
    sc = 0.8
    out, lse = oracle.fwd(c["q"], c["k"], c["v"], c["offsets"], 1, 1, sc)
    np.testing.assert_allclose(out, c["v"], atol=1e-15, rtol=0)
    np.testing.assert_allclose(lse, sc * np.sum(c["q"] * c["k"], axis=2).T, atol=1e-14, rtol=0)
    dq, dk, dv = oracle.bwd(c["q"], c["k"], c["v"], c["dout"], c["offsets"], 1, 1, sc)
    np.testing.assert_allclose(dv, c["dout"], atol=1e-15, rtol=0)
    np.testing.assert_allclose(dq, 0.0, atol=1e-14)
    np.testing.assert_allclose(dk, 0.0, atol=1e-14)


def test_pair_count_against_mask_and_closed_form():
    rs = np.random.default_rng(0)
    for _ in range(30):
        lengths = rs.integers(0, 90, size=rs.integers(1, 6))
        B, W = int(rs.integers(1, 12)), int(rs.integers(1, 5))
        off = wl.offsets_from_lengths(lengths)
        brute = sum(int(visible_mask(int(L), B, W).sum()) for L in lengths)
        assert oracle.pair_count(off, B, W) == brute
    # L a multiple of B with at least W blocks: nb(B(B+1)/2 + (W-1)B^2) - B^2 W(W-1)/2
    for B, W, nb in [(4, 2, 5), (8, 3, 3), (16, 1, 7), (3, 4, 9)]:
        closed = nb * (B * (B + 1) // 2 + (W - 1) * B * B) - B * B * W * (W - 1) // 2
        assert oracle.pair_count(wl.offsets_from_lengths([nb * B]), B, W) == closed


# ------------------------------------------------------------- invariants


def test_probability_rows_sum_to_one_and_respect_mask():
    lengths = [21, 10]
    c = case(16, lengths, H=2, D=4)
    for u, L in enumerate(lengths):
        for h in range(2):
            P = oracle.probs(c["q"], c["k"], c["offsets"], 4, 2, 0.8, u, h)
            np.testing.assert_allclose(P.sum(1), 1.0, atol=1e-14, rtol=0)
            assert np.all(P[~visible_mask(L, 4, 2)] == 0.0)
            assert np.all(P[visible_mask(L, 4, 2)] > 0.0)


def test_locality_outside_window_is_bitwise_irrelevant():
    """Changing K/V rows a query cannot see leaves its O and lse bitwise equal."""
    B, W, L = 4, 2, 29
    c = case(17, [L], H=1, D=4)
    out, lse = oracle.fwd(c["q"], c["k"], c["v"], c["offsets"], B, W, 0.5)
    mask = visible_mask(L, B, W)
    rs = np.random.default_rng(1)
    for i in [0, 5, 11, 17, 28]:
        k2, v2 = c["k"].copy(), c["v"].copy()
        hidden = ~mask[i]
        k2[hidden] = rs.normal(size=k2[hidden].shape) * 10
        v2[hidden] = rs.normal(size=v2[hidden].shape) * 10
        o2, l2 = oracle.fwd(c["q"], k2, v2, c["offsets"], B, W, 0.5)
        assert np.array_equal(o2[i], out[i]) and np.array_equal(l2[:, i], lse[:, i])
        if hidden.any():
            assert not np.array_equal(o2, out)  # some other row did change


def test_jagged_concat_permute_empty_users_and_heads():
    lengths = [9, 0, 14, 3]
    c = case(18, lengths, H=3, D=4)
    B, W, sc = 4, 2, 0.6
    out, lse = oracle.fwd(c["q"], c["k"], c["v"], c["offsets"], B, W, sc)
    off = c["offsets"]
    # each user alone
    for u in range(len(lengths)):
        a, b = off[u], off[u + 1]
        o1, l1 = oracle.fwd(c["q"][a:b], c["k"][a:b], c["v"][a:b], [0, b - a], B, W, sc)
        assert np.array_equal(o1, out[a:b]) and np.array_equal(l1, lse[:, a:b])
    # permuted users with extra empty users
    perm = [3, 1, 0, 2]
    rows = np.concatenate([np.arange(off[u], off[u + 1]) for u in perm])
    new_len = [0] + [lengths[u] for u in perm] + [0]
    o2, l2 = oracle.fwd(c["q"][rows], c["k"][rows], c["v"][rows],
                        wl.offsets_from_lengths(new_len), B, W, sc)
    assert np.array_equal(o2, out[rows]) and np.array_equal(l2, lse[:, rows])
    # heads are independent
    q3 = c["q"].copy()
    q3[:, 1] += 5.0
    o3, l3 = oracle.fwd(q3, c["k"], c["v"], off, B, W, sc)
    assert np.array_equal(o3[:, [0, 2]], out[:, [0, 2]])
    assert not np.array_equal(o3[:, 1], out[:, 1])


def test_key_shift_invariance():
    """k_j + c shifts every score of row i by <q_i, c>*scale: O and lse - shift
    are unchanged up to rounding."""
    c = case(19, [25, 12], H=2, D=4)
    shift = np.array([0.3, -1.1, 2.0, 0.7])
    o1, l1 = oracle.fwd(c["q"], c["k"], c["v"], c["offsets"], 4, 3, 0.5)
    o2, l2 = oracle.fwd(c["q"], c["k"] + shift, c["v"], c["offsets"], 4, 3, 0.5)
    np.testing.assert_allclose(o2, o1, atol=1e-12, rtol=0)
    np.testing.assert_allclose(l2, l1 + 0.5 * np.einsum("thd,d->ht", c["q"], shift),
                               atol=1e-12, rtol=0)


def test_thread_count_does_not_change_results():
    code = (
        "import numpy as np, oracle;"
        "from long_sequence_block_amd import workloads as wl;"
        "c=wl.random_case(20,[30,0,17,45],3,8);"
        "o,l=oracle.fwd(c['q'],c['k'],c['v'],c['offsets'],8,2,0.35);"
        "g=oracle.bwd(c['q'],c['k'],c['v'],c['dout'],c['offsets'],8,2,0.35);"
        "import hashlib;h=hashlib.sha256();"
        "[h.update(np.ascontiguousarray(a).tobytes()) for a in (o,l)+g];print(h.hexdigest())")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    digests = []
    for n in ("1", "3"):
        env = dict(os.environ, OMP_NUM_THREADS=n, PYTHONPATH=root)
        r = subprocess.run([sys.executable, "-c", code], env=env, cwd=root,
                           capture_output=True, text=True, check=True)
        digests.append(r.stdout.strip())
    assert digests[0] == digests[1]


# --------------------------------------------------------------- backward


def _loss(c, q, k, v, B, W, sc):
    out, _ = oracle.fwd(q, k, v, c["offsets"], B, W, sc)
    return float(np.sum(out * c["dout"]))


@pytest.mark.parametrize("B,W", [(4, 1), (4, 2), (3, 3), (1, 4)])
def test_backward_matches_central_finite_differences(B, W):
    c = case(21 + B + W, [11, 0, 6], H=2, D=3)
    sc, eps = 0.7, 1e-6
    dq, dk, dv = oracle.bwd(c["q"], c["k"], c["v"], c["dout"], c["offsets"], B, W, sc)
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        num = np.zeros_like(grad)
        it = np.nditer(grad, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            args = {n: c[n].copy() for n in "qkv"}
            args[name][idx] += eps
            fp = _loss(c, args["q"], args["k"], args["v"], B, W, sc)
            args[name][idx] -= 2 * eps
            fm = _loss(c, args["q"], args["k"], args["v"], B, W, sc)
            num[idx] = (fp - fm) / (2 * eps)
        err = np.abs(num - grad).max() / max(np.abs(grad).max(), 1e-30)
        assert err <= 1e-6, (name, err)


def test_backward_sum_identities_and_delta_shortcut():
    lengths = [40, 7, 19]
    c = case(22, lengths, H=2, D=5)
    B, W, sc = 4, 3, 0.45
    dq, dk, dv = oracle.bwd(c["q"], c["k"], c["v"], c["dout"], c["offsets"], B, W, sc)
    out, _ = oracle.fwd(c["q"], c["k"], c["v"], c["offsets"], B, W, sc)
    off = c["offsets"]
    for u in range(len(lengths)):
        a, b = off[u], off[u + 1]
        for h in range(2):
            # sum_j dV_j = sum_i dO_i  (rows of P sum to one)
            np.testing.assert_allclose(dv[a:b, h].sum(0), c["dout"][a:b, h].sum(0), atol=1e-12)
            # sum_j dK_j = 0           (rows of dS sum to zero)
            np.testing.assert_allclose(dk[a:b, h].sum(0), 0.0, atol=1e-12)
            # sum_i <q_i,dQ_i> = sum_j <k_j,dK_j>  (both equal scale*sum dS_ij s_ij/scale)
            np.testing.assert_allclose(np.sum(c["q"][a:b, h] * dq[a:b, h]),
                                       np.sum(c["k"][a:b, h] * dk[a:b, h]), atol=1e-12)
            # delta_i = sum_j P_ij dP_ij equals <dO_i, O_i>
            P = oracle.probs(c["q"], c["k"], off, B, W, sc, u, h)
            dP = c["dout"][a:b, h] @ c["v"][a:b, h].T
            np.testing.assert_allclose((P * dP).sum(1),
                                       np.sum(c["dout"][a:b, h] * out[a:b, h], axis=1),
                                       atol=1e-12)


def test_invalid_offsets_rejected():
    c = case(23, [4, 4], H=1, D=2)
    with pytest.raises(ValueError):
        oracle.fwd(c["q"], c["k"], c["v"], np.array([0, 5, 4], np.int32), 2, 1, 1.0)
    with pytest.raises(ValueError):
        oracle.fwd(c["q"], c["k"], c["v"], np.array([0, 4, 9], np.int32), 2, 1, 1.0)
    with pytest.raises(ValueError):
        oracle.fwd(c["q"], c["k"], c["v"], c["offsets"], 0, 1, 1.0)


def test_workload_generator_shapes():
    """The jagged workload's lengths follow the stated recipe and seed."""
    w = wl.WORKLOADS[3]
    L = w.lengths()
    assert len(L) == 256 and L.min() >= 16 and L.max() <= 4096
    off = w.offsets()
    assert off[0] == 0 and off[-1] == L.sum() and off.dtype == np.int32
    assert wl.WORKLOADS[5].offsets().tolist() == off.tolist()
    assert wl.WORKLOADS[6].offsets().tolist() == off.tolist()
    # the sliding window of workload 6 matches the block pattern's work to 0.2%
    blk, swa = oracle.pair_count(off, 128, 2), oracle.pair_count(off, 1, 194)
    assert abs(swa / blk - 1) < 2.1e-3
    # the long-context training step shares the long-context forward's inputs
    lc, lct = wl.WORKLOADS[4], wl.WORKLOADS[11]
    assert lct.backward and lct.offsets().tolist() == lc.offsets().tolist()
    assert (lct.wid, lct.heads, lct.head_dim, lct.block_size, lct.window_blocks) == \
        (lc.wid, lc.heads, lc.head_dim, lc.block_size, lc.window_blocks)
    # median of a lognormal(ln 600, 0.8) sample of 256 sits near 600
    assert 450 < np.median(L) < 750


# ---------------------------------------------------- rotary embedding
#
# The rotate-half rotary embedding the production kernel's backward fuses
# ("GEM (Meta)", section "Custom kernels"), with the readings stated in the
# oracle (angle p * base**(-2d/D), p the index inside the user).


def test_rope_single_pair_turns_by_the_position():
    """D = 2: the only frequency is base**0 = 1, so the token at position p
    turns (x0, x1) by p radians (math.cos / math.sin)."""
    off = np.array([0, 6], np.int32)
    x = np.zeros((6, 1, 2))
    x[:, 0, 0], x[:, 0, 1] = 1.0, 0.5
    r = oracle.rope(x, off)
    for p in range(6):
        c, s = math.cos(p), math.sin(p)
        assert abs(r[p, 0, 0] - (c - 0.5 * s)) < 1e-15
        assert abs(r[p, 0, 1] - (0.5 * c + s)) < 1e-15


def test_rope_second_frequency_follows_the_base():
    """D = 4: the second pair (features 1 and 3) turns by base**(-1/2) per
    position: 0.01 rad for base 10000 (position 100 turns it by 1 rad) and
    0.1 rad for base 100 (position 30 turns it by 3 rad)."""
    for base, p, ang in ((10000.0, 100, 1.0), (100.0, 30, 3.0)):
        off = np.array([0, p + 1], np.int32)
        x = np.zeros((p + 1, 1, 4))
        x[:, 0, 1] = 1.0
        r = oracle.rope(x, off, base)
        np.testing.assert_allclose(r[p, 0], [0.0, math.cos(ang), 0.0, math.sin(ang)],
                                   atol=1e-13)
        # the first pair has zero input and stays zero; the turn is p, not p+1
        np.testing.assert_allclose(r[1, 0, [1, 3]],
                                   [math.cos(ang / p), math.sin(ang / p)], atol=1e-15)


def test_rope_is_complex_multiplication():
    """As complex numbers z_d = x_d + i x_{d+D/2}, the embedding multiplies
    z_d by exp(i p theta_d) (numpy complex exponential)."""
    c = case(400, [9, 0, 13], H=2, D=8)
    r = oracle.rope(c["q"], c["offsets"], 500.0)
    z = c["q"][..., :4] + 1j * c["q"][..., 4:]
    pos = np.concatenate([np.arange(9), np.arange(13)]).astype(np.float64)
    theta = 500.0 ** (-np.arange(4) / 4.0)
    zr = z * np.exp(1j * pos[:, None, None] * theta[None, None, :])
    np.testing.assert_allclose(r[..., :4], zr.real, atol=1e-13)
    np.testing.assert_allclose(r[..., 4:], zr.imag, atol=1e-13)


def test_rope_scores_depend_only_on_the_offset():
    """One q and one k vector repeated at every position: the rotated scores
    <rope(q)_i, rope(k)_j> form a Toeplitz matrix (they depend on i - j only),
    in every user, since positions restart per user."""
    rs = np.random.default_rng(5)
    qv, kv = rs.standard_normal(16), rs.standard_normal(16)
    lengths = [20, 7]
    off = wl.offsets_from_lengths(lengths)
    T = sum(lengths)
    q = np.tile(qv, (T, 1, 1))
    k = np.tile(kv, (T, 1, 1))
    qr, kr = oracle.rope(q, off), oracle.rope(k, off)
    for u, L in enumerate(lengths):
        a = off[u]
        S = qr[a:a + L, 0] @ kr[a:a + L, 0].T
        for dlt in range(-L + 1, L):
            diag = np.diagonal(S, dlt)
            np.testing.assert_allclose(diag, diag[0], atol=1e-12)
    # and the first user's scores equal the second's for the same offsets
    S0 = qr[:7, 0] @ kr[:7, 0].T
    S1 = qr[20:27, 0] @ kr[20:27, 0].T
    np.testing.assert_allclose(S0, S1, atol=1e-12)


def test_rope_is_a_rotation():
    c = case(401, [30, 4], H=3, D=16)
    r = oracle.rope(c["k"], c["offsets"])
    np.testing.assert_allclose(np.linalg.norm(r, axis=2), np.linalg.norm(c["k"], axis=2),
                               atol=1e-12)
    np.testing.assert_array_equal(r[0], c["k"][0])      # position 0 of user 0
    np.testing.assert_array_equal(r[30], c["k"][30])    # position 0 of user 1
    np.testing.assert_allclose(oracle.rope_transpose(r, c["offsets"]), c["k"], atol=1e-12)


def test_rope_backward_matches_central_finite_differences():
    """Gradients of sum(dO * attention(rope(q), rope(k), v)) with respect to
    the unrotated q, k and v."""
    c = case(402, [9, 5], H=1, D=4)
    B, W, sc, base, eps = 2, 2, 0.6, 50.0, 1e-6

    def loss(q, k, v):
        o, _ = oracle.fwd(oracle.rope(q, c["offsets"], base), oracle.rope(k, c["offsets"], base),
                          v, c["offsets"], B, W, sc)
        return float(np.sum(o * c["dout"]))

    grads = oracle.rope_bwd(oracle.rope(c["q"], c["offsets"], base),
                            oracle.rope(c["k"], c["offsets"], base), c["v"], c["dout"],
                            c["offsets"], B, W, sc, base)
    for name, grad in zip("qkv", grads):
        num = np.zeros_like(grad)
        it = np.nditer(grad, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            args = {n: c[n].copy() for n in "qkv"}
            args[name][idx] += eps
            fp = loss(args["q"], args["k"], args["v"])
            args[name][idx] -= 2 * eps
            fm = loss(args["q"], args["k"], args["v"])
            num[idx] = (fp - fm) / (2 * eps)
        err = np.abs(num - grad).max() / max(np.abs(grad).max(), 1e-30)
        assert err <= 1e-6, (name, err)


# ------------------------------------------ generalized dot-product attention
#
# GDPA replaces the softmax by an activation ("GEM (Meta)", section "Custom
# kernels"); the reading is no normalisation (the oracle's header).


def _gdpa_torch(q, k, v, L, B, W, scale, act):
    """Dense fp64 reference of one user with torch's own SiLU / GELU (exact
    erf form) and the predicate mask; returns out [L, H, D] as a tensor."""
    mask = torch.from_numpy(visible_mask(L, B, W))
    s = torch.einsum("ihd,jhd->hij", q, k) * scale
    a = torch.nn.functional.silu(s) if act == oracle.GDPA_SILU else \
        torch.nn.functional.gelu(s, approximate="none")
    p = torch.where(mask[None], a, torch.zeros_like(a))
    return torch.einsum("hij,jhd->ihd", p, v)


@pytest.mark.parametrize("act", [1, 2])
@pytest.mark.parametrize("B,W", [(4, 2), (1, 5), (8, 1)])
def test_gdpa_matches_torch_activations_and_autograd(act, B, W):
    lengths = [0, 1, 9, 23, 40]
    c = case(500 + 10 * act + B + W, lengths, H=2, D=6)
    sc = 0.55
    out = oracle.gdpa_fwd(c["q"], c["k"], c["v"], c["offsets"], B, W, sc, act)
    dq, dk, dv = oracle.gdpa_bwd(c["q"], c["k"], c["v"], c["dout"], c["offsets"], B, W, sc, act)
    off = c["offsets"]
    for u, L in enumerate(lengths):
        a, b = off[u], off[u + 1]
        if L == 0:
            continue
        t = {n: torch.from_numpy(c[n][a:b].copy()).requires_grad_(n in "qkv") for n in
             ("q", "k", "v", "dout")}
        ref = _gdpa_torch(t["q"], t["k"], t["v"], L, B, W, sc, act)
        np.testing.assert_allclose(out[a:b], ref.detach().numpy(), atol=1e-12, rtol=0)
        (ref * t["dout"]).sum().backward()
        np.testing.assert_allclose(dq[a:b], t["q"].grad.numpy(), atol=1e-12, rtol=0)
        np.testing.assert_allclose(dk[a:b], t["k"].grad.numpy(), atol=1e-12, rtol=0)
        np.testing.assert_allclose(dv[a:b], t["v"].grad.numpy(), atol=1e-12, rtol=0)


def test_gdpa_constant_scores_weight_the_window_sum():
    """All keys of a user equal and all queries equal: every visible score is
    the same x, so out_i = act(x) times the sum of the visible v_j (prefix
    sums), with act written from its definition via math.exp / math.erf."""
    L, B, W, D = 37, 8, 2, 4
    rs = np.random.default_rng(9)
    qv, kv = rs.standard_normal(D), rs.standard_normal(D)
    v = rs.standard_normal((L, 1, D))
    q, k = np.tile(qv, (L, 1, 1)), np.tile(kv, (L, 1, 1))
    off = np.array([0, L], np.int32)
    x = 0.7 * float(qv @ kv)
    silu = x / (1 + math.exp(-x))
    gelu = 0.5 * x * (1 + math.erf(x / math.sqrt(2)))
    csum = np.concatenate([np.zeros((1, D)), np.cumsum(v[:, 0], axis=0)])
    for act, a in ((1, silu), (2, gelu)):
        out = oracle.gdpa_fwd(q, k, v, off, B, W, 0.7, act)
        for i in range(L):
            j0 = max(0, i // B - W + 1) * B
            np.testing.assert_allclose(out[i, 0], a * (csum[i + 1] - csum[j0]), atol=1e-12)


# --------------------------------------------------------------- MXFP8
#
# MXFP8 inputs ("GEM (Meta)", section "Custom kernels": production attention
# runs in a block-scaled FP8 format), read as the OCP MX format (oracle).


def test_mx_decode_matches_torch_fp8_types():
    """Every E4M3 code under several E8M0 scales decodes as torch's own
    float8_e4m3fn and float8_e8m0fnu types do."""
    codes = np.tile(np.arange(256, dtype=np.uint8), 4).reshape(2, 16, 32)
    scales = np.array([[0, 119, 127, 254]] * 2, np.uint8).reshape(2, 4, 1)
    scales = np.repeat(scales, 4, axis=1).reshape(2, 16, 1)
    got = oracle.mx_decode(codes, scales)
    c = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64)
    f = torch.from_numpy(scales).view(torch.float8_e8m0fnu).to(torch.float64)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(c.numpy()))
    ok = ~np.isnan(got)
    np.testing.assert_array_equal(got[ok], (c * f).numpy()[ok])


def test_mx_decode_known_values():
    """1.0 = 0x38, 448 = 0x7E (largest), 2^-6 = 0x08 (smallest normal), 2^-9
    = 0x01 (smallest subnormal), -0 = 0x80; a scale byte of 127 is 1 and of
    120 is 2^-7; each scale covers its own 32 elements."""
    codes = np.zeros((1, 64), np.uint8)
    codes[0, :6] = [0x38, 0x7E, 0x08, 0x01, 0x80, 0xB8]
    codes[0, 32] = 0x38
    v = oracle.mx_decode(codes, np.array([[127, 120]], np.uint8))
    np.testing.assert_array_equal(v[0, :6], [1.0, 448.0, 2.0 ** -6, 2.0 ** -9, -0.0, -1.0])
    assert v[0, 32] == 2.0 ** -7 and np.signbit(v[0, 4])


def test_mx_workload_draws():
    """The MX draws are finite E4M3 codes of magnitude 4 .. 448 and scales
    2^-8 .. 2^-6, one per 32 head-dim elements."""
    c = wl.random_mx_case(3, [50, 7], 2, 64)
    assert c["q_mx"].shape == (57, 2, 64) and c["q_sc"].shape == (57, 2, 2)
    v = np.abs(oracle.mx_decode(c["q_mx"], np.full(c["q_sc"].shape, 127, np.uint8)))
    assert np.all(np.isfinite(v)) and v.min() >= 4 and v.max() <= 448
    assert set(np.unique(c["k_sc"])) <= {119, 120, 121}


def test_gdpa_absolute_sums_against_torch():
    """The oracle's sums of |terms| (the magnitude the GPU parity bounds of
    GDPA scale with) against the same dense torch reference with every term
    made non-negative: |act(s)| |v| forward; |scale act'(s) dP| |k|,
    |scale act'(s) dP| |q| and |act(s)| |dO| backward, with dP = dO . v."""
    lengths = [0, 1, 9, 23]
    c = case(640, lengths, H=2, D=6)
    off = c["offsets"]
    for act in (1, 2):
        for B, W, sc in ((4, 2, 0.55), (1, 5, -0.8)):
            out = oracle.gdpa_fwd(c["q"], c["k"], c["v"], off, B, W, sc, act, absolute=True)
            g = oracle.gdpa_bwd(c["q"], c["k"], c["v"], c["dout"], off, B, W, sc, act,
                                absolute=True)
            for u, L in enumerate(lengths):
                a, b = off[u], off[u + 1]
                if L == 0:
                    continue
                q, k, v, do = (torch.from_numpy(c[n][a:b].copy()) for n in ("q", "k", "v", "dout"))
                s = torch.einsum("ihd,jhd->hij", q, k) * sc
                m = torch.from_numpy(visible_mask(L, B, W))[None]
                if act == 1:
                    p, slope = torch.nn.functional.silu(s), torch.sigmoid(s) * (1 + s * (1 - torch.sigmoid(s)))
                else:
                    cdf = 0.5 * (1 + torch.erf(s / math.sqrt(2)))
                    p = s * cdf
                    slope = cdf + s * torch.exp(-0.5 * s * s) / math.sqrt(2 * math.pi)
                p = torch.where(m, p, torch.zeros_like(p)).abs()
                dp = torch.einsum("ihd,jhd->hij", do, v)
                ds = torch.where(m, (sc * slope * dp).abs(), torch.zeros_like(s))
                np.testing.assert_allclose(out[a:b], torch.einsum("hij,jhd->ihd", p, v.abs()).numpy(),
                                           atol=1e-12, rtol=1e-12)
                np.testing.assert_allclose(g[0][a:b], torch.einsum("hij,jhd->ihd", ds, k.abs()).numpy(),
                                           atol=1e-12, rtol=1e-12)
                np.testing.assert_allclose(g[1][a:b], torch.einsum("hij,ihd->jhd", ds, q.abs()).numpy(),
                                           atol=1e-12, rtol=1e-12)
                np.testing.assert_allclose(g[2][a:b], torch.einsum("hij,ihd->jhd", p, do.abs()).numpy(),
                                           atol=1e-12, rtol=1e-12)


def test_gdpa_absolute_sums_bound_the_sums():
    """Triangle inequality: every plain sum is at most its sum of |terms|,
    and the two agree where every term is non-negative (q = k with positive
    entries and scale > 0 make every score, activation and slope positive;
    v, dO positive)."""
    c = case(641, [30, 17], H=2, D=5)
    off = c["offsets"]
    for act in (1, 2):
        o = oracle.gdpa_fwd(c["q"], c["k"], c["v"], off, 8, 2, 0.6, act)
        oa = oracle.gdpa_fwd(c["q"], c["k"], c["v"], off, 8, 2, 0.6, act, absolute=True)
        assert np.all(np.abs(o) <= oa + 1e-12)
        g = oracle.gdpa_bwd(c["q"], c["k"], c["v"], c["dout"], off, 8, 2, 0.6, act)
        ga = oracle.gdpa_bwd(c["q"], c["k"], c["v"], c["dout"], off, 8, 2, 0.6, act, absolute=True)
        for x, xa in zip(g, ga):
            assert np.all(np.abs(x) <= xa + 1e-12)
        pos = {n: np.abs(c[n]) + 0.1 for n in ("q", "v", "dout")}
        o = oracle.gdpa_fwd(pos["q"], pos["q"], pos["v"], off, 8, 2, 0.6, act)
        oa = oracle.gdpa_fwd(pos["q"], pos["q"], pos["v"], off, 8, 2, 0.6, act, absolute=True)
        np.testing.assert_allclose(o, oa, rtol=1e-13, atol=0)
        g = oracle.gdpa_bwd(pos["q"], pos["q"], pos["v"], pos["dout"], off, 8, 2, 0.6, act)
        ga = oracle.gdpa_bwd(pos["q"], pos["q"], pos["v"], pos["dout"], off, 8, 2, 0.6, act,
                             absolute=True)
        for x, xa in zip(g, ga):
            np.testing.assert_allclose(x, xa, rtol=1e-13, atol=0)


def test_huge_block_and_window_are_causal_attention():
    """B and W as large as int32 allows: one block per user, every earlier
    key visible, i.e. causal attention (torch SDPA, fp64); the oracle's
    scratch is sized by the longest visible range, not by W * B."""
    lengths = [40, 0, 13]
    c = case(642, lengths, H=2, D=4)
    big = 2 ** 31 - 1
    out, lse = oracle.fwd(c["q"], c["k"], c["v"], c["offsets"], big, big, 0.5)
    g = oracle.bwd(c["q"], c["k"], c["v"], c["dout"], c["offsets"], big, big, 0.5)
    ref = oracle.fwd(c["q"], c["k"], c["v"], c["offsets"], 64, 1, 0.5)
    refg = oracle.bwd(c["q"], c["k"], c["v"], c["dout"], c["offsets"], 64, 1, 0.5)
    np.testing.assert_array_equal(out, ref[0])
    np.testing.assert_array_equal(lse, ref[1])
    for x, y in zip(g, refg):
        np.testing.assert_array_equal(x, y)
    off = c["offsets"]
    for u in (0, 2):
        a, b = off[u], off[u + 1]
        t = [torch.from_numpy(np.ascontiguousarray(c[n][a:b].transpose(1, 0, 2))) for n in "qkv"]
        sd = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=True, scale=0.5)
        np.testing.assert_allclose(out[a:b], sd.numpy().transpose(1, 0, 2), atol=1e-13, rtol=0)


def test_mx_all_codes_draw():
    """The full-range MX draw covers all 254 finite E4M3 codes (both zeros,
    every subnormal), never a NaN code, and scales in the requested range."""
    c = wl.random_mx_case(7, [400, 300], 2, 64, wide=((94, 100), (140, 146)))
    codes = np.concatenate([c["q_mx"].ravel(), c["k_mx"].ravel()])
    assert len(np.unique(codes)) == 254
    assert not np.any((codes & 0x7F) == 0x7F)
    assert c["q_sc"].min() >= 94 and c["q_sc"].max() <= 100
    assert c["k_sc"].min() >= 140 and c["k_sc"].max() <= 146


# ------------------------------------------- MXFP8 weights for the P.V product


def test_e4m3_round_matches_torch():
    """oracle's E4M3 rounding (nearest, ties to the even code) against
    torch's float8_e4m3fn conversion: every code value, every midpoint
    between neighbouring codes (the ties), their fp32 neighbours, and
    log-uniform values from below the smallest subnormal to 2^8.  All
    inputs are fp32 values: torch converts through fp32, so an fp64 input
    one ulp from a midpoint would be rounded twice there."""
    vals = np.array(sorted({oracle.e4m3_value(c) for c in range(127)}), np.float32)  # 0 .. 448
    vals = vals[vals <= 256.0]
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(5)
    x = np.concatenate([vals, mids, np.nextafter(mids, np.float32(0)),
                        np.nextafter(mids, np.float32(np.inf)),
                        np.exp2(rng.uniform(-12, 8, 20000)).astype(np.float32)])
    x = x[x < 2 ** 8 + 2 ** 3]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).double().numpy()
    x = x.astype(np.float64)
    np.testing.assert_array_equal(oracle.e4m3_round(x), ref)


def _mx_rows(seed, lengths, D, lo=-1, hi=2):
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    q = rng.integers(lo, hi, (T, 1, D)).astype(np.float64)
    k = rng.integers(lo, hi, (T, 1, D)).astype(np.float64)
    v = rng.standard_normal((T, 1, D))
    return q, k, v, wl.offsets_from_lengths(lengths)


def test_mxpv_integer_scores_are_exact():
    """With scale = ln 2 and integer q, k every t_ij = s_ij log2(e) is an
    integer, so every weight is a power of two (within 2^16 of its block's
    largest here) and exactly representable: the quantized forward equals
    the plain softmax forward."""
    q, k, v, off = _mx_rows(11, [70, 33, 1, 40], 4)
    out, lse = oracle.mxpv_fwd(q, k, v, off, 16, 3, math.log(2))
    ref, lref = oracle.fwd(q, k, v, off, 16, 3, math.log(2))
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lref, rtol=1e-14, atol=1e-14)


def test_mxpv_integer_row_shift_changes_nothing():
    """A bias column adds the same amount to every t_ij of a row.  An
    integer amount moves every block's F by that integer and leaves every
    code, hence out, unchanged; half an integer moves the codes."""
    lengths = [90, 37, 64]
    c = case(12, lengths, H=2, D=16)
    scale = 0.3

    def with_bias(n):
        q = np.concatenate([c["q"], np.ones(c["q"].shape[:2] + (1,))], axis=2)
        b = n / (scale * math.log2(math.e))
        k = np.concatenate([c["k"], np.full(c["k"].shape[:2] + (1,), b)], axis=2)
        v = np.concatenate([c["v"], np.zeros(c["v"].shape[:2] + (1,))], axis=2)
        return oracle.mxpv_fwd(q, k, v, c["offsets"], 32, 2, scale)[0]

    base = with_bias(0)
    for n in (3, -5, 17):
        np.testing.assert_allclose(with_bias(n), base, rtol=1e-12, atol=1e-13)
    assert np.abs(with_bias(0.5) - base).max() > 1e-4


def test_mxpv_normal_weights_round_to_four_significant_bits():
    """Where no weight falls below 2^-13 of its block's largest (the E4M3
    subnormal range), each quantized weight is the weight rounded to four
    significant bits (ties to even): out = sum_j sig4(w_ij) v_j / sum_j w_ij,
    written here from frexp and numpy's half-even rounding, with no block
    exponent and no E4M3 table (the weights in a power-of-two unit, since
    four-bit rounding commutes only with power-of-two scaling)."""
    lengths = [100, 45]
    c = case(13, lengths, H=2, D=8)
    scale = 0.15   # t spans well under 13 within any block
    B, W = 32, 2
    out, _ = oracle.mxpv_fwd(c["q"], c["k"], c["v"], c["offsets"], B, W, scale)
    off = c["offsets"]
    ref = np.zeros_like(out)
    for u in range(len(lengths)):
        t0 = off[u]
        for h in range(2):
            for i in range(off[u + 1] - t0):
                j0 = max(0, (i // B - W + 1) * B)
                kk = c["k"][t0 + j0:t0 + i + 1, h]
                s = scale * kk @ c["q"][t0 + i, h]
                t = s * math.log2(math.e)
                w = np.exp2(t - np.floor(t.max()))   # a power-of-two unit
                assert w.min() > 2.0 ** -12
                m, e = np.frexp(w)
                sig4 = np.ldexp(np.round(m * 16) / 16, e)
                ref[t0 + i, h] = sig4 @ c["v"][t0 + j0:t0 + i + 1, h] / w.sum()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_mxpv_small_weights_use_their_blocks_exponent():
    """Hand case, scale = ln 2 so t_ij = <q_i, k_j>: query 32 of a user at
    token 0 sees keys 0..32; key 0 has t = 0, keys 1..31 t = -100 and key
    32 t = -14.3.  Key 32 is alone in block 1 (tokens 32..63), so F = -15 and
    2^(t - F + 7) = 2^7.7 = 207.9 rounds to 208: weight 208 * 2^-22.  Moved
    to token 1, inside block 0 (F = 0), the same t gives 2^-7.3 = 0.00635,
    in the subnormal range: 3 * 2^-9, weight 3 * 2^-16.  With key 0 at
    t = -0.5 the block's F is floor(-0.5) = -1, and key 1 at t = -14.8 gives
    2^-6.8 = 0.00897, i.e. 5 * 2^-9 (4.59 quanta), weight 5 * 2^-17 (F = 0
    would give 2 quanta at 2^-7: 4 * 2^-17).  Blocks count from the user's
    first token: behind a 5-token user, local key 27 still shares block 0
    with key 0, and local key 32 is still alone in block 1."""
    def run(pos, t0, tp, pre=0):
        # (pre: tokens of an earlier user, which move the packed positions)
        q = np.zeros((pre + 33, 1, 2))
        k = np.zeros((pre + 33, 1, 2))
        v = np.zeros((pre + 33, 1, 2))
        q[:, 0, 0] = 1.0
        k[pre + 1:, 0, 0] = -100.0
        k[pre, 0, 0] = t0
        k[pre + pos, 0, 0] = tp
        v[pre + pos, 0, 1] = 1.0
        off = [0, pre, pre + 33] if pre else [0, 33]
        out, _ = oracle.mxpv_fwd(q, k, v, off, 64, 1, math.log(2))
        l = 2.0 ** t0 + 31 * 2.0 ** -100 + 2.0 ** tp
        return out[pre + 32, 0, 1] * l

    assert run(32, 0.0, -14.3) == pytest.approx(208 * 2.0 ** -22, rel=1e-12)
    assert run(1, 0.0, -14.3) == pytest.approx(3 * 2.0 ** -16, rel=1e-12)
    assert run(1, -0.5, -14.8) == pytest.approx(5 * 2.0 ** -17, rel=1e-12)
    assert run(27, 0.0, -14.3, pre=5) == pytest.approx(3 * 2.0 ** -16, rel=1e-12)
    assert run(32, 0.0, -14.3, pre=5) == pytest.approx(208 * 2.0 ** -22, rel=1e-12)


def test_mxpv_keys_outside_the_window_do_not_matter():
    """Keys no query of a user sees (here: another user's, and later keys)
    may take any value: out and lse of the others are unchanged, so block
    maxima are taken over visible keys only."""
    lengths = [80, 50]
    c = case(14, lengths, H=1, D=8)
    a = oracle.mxpv_fwd(c["q"], c["k"], c["v"], c["offsets"], 16, 2, 0.4)
    k2 = c["k"].copy()
    k2[80:] = 50.0          # user 1's keys: user 0 never sees them
    b = oracle.mxpv_fwd(c["q"], k2, c["v"], c["offsets"], 16, 2, 0.4)
    np.testing.assert_array_equal(a[0][:80], b[0][:80])
    np.testing.assert_array_equal(a[1][:, :80], b[1][:, :80])


def test_mxpv_slack_covers_perturbed_scores():
    """The parity allowance is zero for exact scores and covers what a
    computation with scores off by up to eps does: perturb q so every t_ij
    moves by at most eps (|dt| <= |scale| |dq|_1 max|k| log2 e) and check
    |out' - out| <= slack + (2^(2 eps) - 1) max|v| (the second term: the
    unquantized weights' own change)."""
    lengths = [120, 64, 7]
    c = case(15, lengths, H=2, D=16)
    scale, B, W = 0.25, 32, 2
    T = sum(lengths)
    z = oracle.mxpv_slack(c["q"], c["k"], c["v"], c["offsets"], B, W, scale, np.zeros((2, T)))
    assert not z.any()
    out, _ = oracle.mxpv_fwd(c["q"], c["k"], c["v"], c["offsets"], B, W, scale)
    rng = np.random.default_rng(3)
    kmax = np.abs(c["k"]).max()
    hits = 0
    for rep in range(6):
        dq = rng.uniform(-1, 1, c["q"].shape) * 1e-3
        eps = abs(scale) * np.abs(dq).sum(axis=2).T * kmax * math.log2(math.e)  # [H, T]
        sl = oracle.mxpv_slack(c["q"], c["k"], c["v"], c["offsets"], B, W, scale, eps)
        o2, _ = oracle.mxpv_fwd(c["q"] + dq, c["k"], c["v"], c["offsets"], B, W, scale)
        extra = (np.exp2(2 * eps) - 1).T[:, :, None] * np.abs(c["v"]).max()
        assert np.all(np.abs(o2 - out) <= sl + extra + 1e-12)
        hits += int(np.sum(np.abs(o2 - out) > extra))
    assert hits > 0   # some codes did flip, and the slack covered them


def test_mxpv_users_are_independent():
    """A user's quantized forward does not depend on the rest of the batch:
    users 1..2 checked on their own (re-based offsets) give the whole run's
    values, and so do the same users behind other users."""
    lengths = [45, 70, 33]
    c = case(16, lengths, H=2, D=8)
    full, lfull = oracle.mxpv_fwd(c["q"], c["k"], c["v"], c["offsets"], 16, 3, 0.7)
    lo, hi = 45, 148
    sub = wl.subset_users(c, slice(1, 3))
    part, lpart = oracle.mxpv_fwd(sub["q"], sub["k"], sub["v"], sub["offsets"], 16, 3, 0.7)
    np.testing.assert_array_equal(part, full[lo:hi])
    np.testing.assert_array_equal(lpart, lfull[:, lo:hi])
    pre = case(17, [3, 29], H=2, D=8)
    cat = {n: np.concatenate([pre[n], sub[n]]) for n in ("q", "k", "v")}
    off = wl.offsets_from_lengths([3, 29] + lengths[1:])
    moved, _ = oracle.mxpv_fwd(cat["q"], cat["k"], cat["v"], off, 16, 3, 0.7)
    np.testing.assert_array_equal(moved[32:], full[lo:hi])


def test_mx_decode_user_blocks():
    """User-blocked decode: code 0x38 (1.0) with scale byte 127 + r on scale
    row r gives 2^r; user u's local token j reads row
    ceil(off[u] / 32) + u + j // 32."""
    off = np.array([0, 40, 40, 105], np.int32)
    base = oracle.user_block_base(off)
    np.testing.assert_array_equal(base, [0, 3, 4])   # ceil(0/32)+0, ceil(40/32)+1, +2
    codes = np.full((105, 1, 2), 0x38, np.uint8)
    scales = (127 + np.arange(8, dtype=np.uint8))[:, None, None].repeat(2, axis=2)
    v = oracle.mx_decode_user_blocks(codes, scales, off)
    expect = np.concatenate([np.arange(40) // 32, 4 + np.arange(65) // 32])
    np.testing.assert_array_equal(v[:, 0, 0], 2.0 ** expect)


# ------------------------------------------------------------ MXFP8 backward


def _mxb_case(seed, lengths, H=2, D=32, B=16, W=2, scale=0.3):
    """Random inputs of the MXFP8 backward oracle with the exact forward's
    O and lse, and token-blocked copies equal to the head-dim-blocked ones
    (the oracle takes decoded values; which quantization produced them does
    not matter to it)."""
    rng = np.random.default_rng(seed)
    off = wl.offsets_from_lengths(lengths)
    T = int(off[-1])
    q, k, v, do = (rng.standard_normal((T, H, D)) for _ in range(4))
    o, lse = oracle.fwd(q, k, v, off, B, W, scale)
    return dict(q=q, k=k, v=v, dout=do, out=o, lse=lse, q_t=q.copy(), k_t=k.copy(),
                dout_t=do.copy(), offsets=off, block_size=B, window_blocks=W, scale=scale)


def _mxb(c, **kw):
    args = dict(c)
    args.update(kw)
    return oracle.mx_bwd(**args)


@pytest.mark.parametrize("B,W", [(16, 2), (5, 3), (1, 1), (64, 1)])
def test_mx_bwd_unquantized_is_the_exact_backward(B, W):
    """Without the quantization step, given the exact forward's O and lse
    and the same values for both quantizations of q, k and dO, the MXFP8
    backward's steps (P from lse, delta from <dO, O>, dS, the three
    products) give the exact backward, itself pinned to finite differences
    and the sum identities."""
    c = _mxb_case(1, [40, 7, 73, 1], B=B, W=W)
    got = _mxb(c, quantize=False)
    ref = oracle.bwd(c["q"], c["k"], c["v"], c["dout"], c["offsets"], B, W, c["scale"])
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-12 * np.abs(r).max())


@pytest.mark.parametrize("quantize", [False, True])
def test_mx_bwd_token_blocked_operands_feed_their_own_products(quantize):
    """dQ takes k_t, dK takes q_t and dV takes dout_t, linearly, and nothing
    else does: scaling one of them by 4 scales exactly its gradient, bit for
    bit.  (The quantized operands P and dS do not depend on them.)"""
    c = _mxb_case(2, [45, 20])
    dq, dk, dv = _mxb(c, quantize=quantize)
    for name, idx in (("k_t", 0), ("q_t", 1), ("dout_t", 2)):
        got = _mxb(c, quantize=quantize, **{name: 4.0 * c[name]})
        for j, (g, r) in enumerate(zip(got, (dq, dk, dv))):
            if j == idx:
                np.testing.assert_array_equal(g, 4.0 * r)
            else:
                np.testing.assert_array_equal(g, r)


def test_mx_block_rule_matches_torch_fp8():
    """The block rule: with E = floor(log2 max|x|) - 7, each value becomes
    2^E times torch's float8_e4m3fn conversion of x 2^-E (nearest, ties to
    even, sign kept), for blocks of mixed signs, zeros, magnitudes from 2^-40
    to 2^40 and spreads up to 2^30 inside a block, fp32 inputs (torch
    converts through fp32); blocks whose maximum is tiny clamp E at -127;
    an all-zero block stays zero."""
    rng = np.random.default_rng(7)
    for _ in range(400):
        n = int(rng.integers(1, 33))
        mag = rng.uniform(-40, 40)
        x = (np.exp2(mag - rng.uniform(0, 30, n)) * rng.choice([-1, 1], n)).astype(np.float32)
        x[rng.random(n) < 0.1] = 0
        x = x.astype(np.float64)
        got = oracle.mx_quantize_block(x)
        a = np.abs(x).max()
        if a == 0:
            np.testing.assert_array_equal(got, 0 * x)
            continue
        E = max(math.frexp(a)[1] - 8, -127)
        y = torch.from_numpy(np.ldexp(x, -E).astype(np.float32))
        ref = np.ldexp(y.to(torch.float8_e4m3fn).double().numpy(), E)
        np.testing.assert_array_equal(got, ref)
    x = np.array([2.0 ** -130, -(2.0 ** -131), 2.0 ** -140])
    E = -127
    y = torch.from_numpy(np.ldexp(x, -E).astype(np.float32))
    np.testing.assert_array_equal(oracle.mx_quantize_block(x),
                                  np.ldexp(y.to(torch.float8_e4m3fn).double().numpy(), E))
    np.testing.assert_array_equal(oracle.mx_quantize_block(np.zeros(5)), np.zeros(5))


def test_mx_bwd_dq_blocks_run_along_the_row():
    """dS is quantized along each query's keys for dQ: scaling query i's dO
    (hence its dP, delta and whole dS row) by 2^5 scales dQ_i by exactly 2^5
    and leaves every other query's dQ bit-for-bit unchanged.  Blocks along
    queries would mix row i into other rows' codes."""
    c = _mxb_case(3, [70, 50], B=8, W=3)
    dq, _, _ = _mxb(c)
    for row in (0, 33, 69, 70 + 41):
        d2 = c["dout"].copy()
        d2[row] *= 32.0
        got, _, _ = _mxb(c, dout=d2)
        np.testing.assert_array_equal(got[row], 32.0 * dq[row])
        other = np.ones(len(dq), bool)
        other[row] = False
        np.testing.assert_array_equal(got[other], dq[other])


def _only_rows(x, rows):
    y = np.zeros_like(x)
    y[rows] = x[rows]
    return y


@pytest.mark.parametrize("user,blk", [(1, 1), (1, 0), (2, 2)])
def test_mx_bwd_dk_dv_blocks_run_along_each_keys_queries(user, blk):
    """P and dS are quantized along each key's queries in blocks of 32
    counted from the user's first token (users here start at 37 and 100,
    off the packed axis's multiples of 32).  Scaling the dO of the queries
    of one such block by 2^3 scales their dS entries exactly, so
    dK = dK + 7 dK_b, with dK_b the block's own share (q_t zeroed outside
    it); shifting their lse by 2 ln 2 scales their P and dS by 2^-2, so
    dV = dV - (3/4) dV_b and dK = dK - (3/4) dK_b.  Blocks cut anywhere else
    would change other queries' codes."""
    c = _mxb_case(4, [37, 63, 101], B=16, W=3)
    off = c["offsets"]
    rows = np.arange(off[user] + 32 * blk, min(off[user] + 32 * blk + 32, off[user + 1]))
    dq, dk, dv = _mxb(c)
    _, dk_b, _ = _mxb(c, q_t=_only_rows(c["q_t"], rows))
    _, _, dv_b = _mxb(c, dout_t=_only_rows(c["dout_t"], rows))
    d2 = c["dout"].copy()
    d2[rows] *= 8.0
    _, got_dk, got_dv = _mxb(c, dout=d2)
    np.testing.assert_allclose(got_dk, dk + 7.0 * dk_b, rtol=0, atol=1e-12 * np.abs(dk).max())
    np.testing.assert_array_equal(got_dv, dv)
    l2 = c["lse"].copy()
    l2[:, rows] += 2.0 * math.log(2.0)
    _, got_dk, got_dv = _mxb(c, lse=l2)
    np.testing.assert_allclose(got_dv, dv - 0.75 * dv_b, rtol=0, atol=1e-12 * np.abs(dv).max())
    np.testing.assert_allclose(got_dk, dk - 0.75 * dk_b, rtol=0, atol=1e-12 * np.abs(dk).max())


def test_mx_bwd_single_token_window_closed_form():
    """B = W = 1: each query sees only itself, P_ii = 1 (stored exactly),
    O_i = v_i, so dS_ii = <dO_i, v_i> - <dO_i, O_i> = 0: dQ = dK = 0 and
    dV = dout_t exactly."""
    c = _mxb_case(5, [9, 1, 30], B=1, W=1)
    np.testing.assert_array_equal(c["out"], c["v"])
    dq, dk, dv = _mxb(c)
    np.testing.assert_array_equal(dq, 0 * dq)
    np.testing.assert_array_equal(dk, 0 * dk)
    np.testing.assert_array_equal(dv, c["dout_t"])


def test_mx_bwd_users_are_independent():
    """A user's gradients are the same alone and inside a batch (blocks
    start at each user's first token)."""
    lengths = [37, 70, 5]
    c = _mxb_case(6, lengths, B=8, W=4)
    full = _mxb(c)
    off = c["offsets"]
    for u in range(len(lengths)):
        sl = slice(off[u], off[u + 1])
        cu = {n: (x[sl] if isinstance(x, np.ndarray) and x.shape[:1] == (off[-1],) else x)
              for n, x in c.items()}
        cu["lse"] = c["lse"][:, sl]
        cu["offsets"] = np.array([0, off[u + 1] - off[u]], np.int32)
        for g, r in zip(oracle.mx_bwd(**cu), full):
            np.testing.assert_array_equal(g, r[sl])


def test_mx_bwd_bounds_cover_perturbed_products():
    """The allowance of mx_bwd_bounds covers real flips: scores and dP taken
    from q and v perturbed elementwise by up to rho relative (so each moves
    by at most rho times its magnitude sum, the allowed error) change the
    quantized gradients by no more than the slack.  Also the absolute sums
    bound the gradients."""
    rho = 2.0 ** -11
    c = _mxb_case(8, [80, 45], B=16, W=3)
    (dq, dk, dv), sl, ab = oracle.mx_bwd_bounds(**c, rho=rho)
    for g, a in zip((dq, dk, dv), ab):
        assert np.all(np.abs(g) <= a * (1 + 1e-12))
    rng = np.random.default_rng(9)
    flipped = 0
    for t in range(4):
        qp = c["q"] * (1 + rho * rng.uniform(-1, 1, c["q"].shape))
        vp = c["v"] * (1 + rho * rng.uniform(-1, 1, c["v"].shape))
        got = _mxb(c, q=qp, v=vp)
        for g, r, s in zip(got, (dq, dk, dv), sl):
            d = np.abs(g - r)
            flipped += int(np.count_nonzero(d > 1e-12 * np.abs(r).max()))
            assert np.all(d <= s + 1e-12 * np.abs(r).max())
    assert flipped > 0  # the perturbations did move codes


def test_mx_bwd_p_and_ds_blocks_hold_one_keys_queries():
    """Scaling one key's column of P by 4 (q has a constant unit feature,
    and that key's k moves by 2 ln 2 / scale along it, so every s_ij of the
    key grows by 2 ln 2) scales the key's P and dS entries and hence its dV
    and dK by 4, and leaves every other key's dV and dK bit-for-bit
    unchanged: each key's queries form its own blocks.  Blocks along a
    query's keys would move other keys' codes."""
    c = _mxb_case(10, [70, 45], B=16, W=3)
    for name in ("q", "q_t"):
        c[name][:, :, 0] = 1.0
    c["out"], c["lse"] = oracle.fwd(c["q"], c["k"], c["v"], c["offsets"], 16, 3, c["scale"])
    _, dk, dv = _mxb(c)
    for key in (3, 40, 70 + 17):
        k2 = c["k"].copy()
        k2[key, :, 0] += 2.0 * math.log(2.0) / c["scale"]
        _, got_dk, got_dv = _mxb(c, k=k2)
        other = np.ones(len(dk), bool)
        other[key] = False
        np.testing.assert_array_equal(got_dv[other], dv[other])
        np.testing.assert_array_equal(got_dk[other], dk[other])
        np.testing.assert_allclose(got_dv[key], 4.0 * dv[key], rtol=1e-12)
        np.testing.assert_allclose(got_dk[key], 4.0 * dk[key], rtol=1e-9,
                                   atol=1e-12 * np.abs(dk).max())


def _mx_quantize(x, off, axis):
    """x quantized with the block rule along head dims (axis 'd', 32-element
    blocks) or along each user's tokens (axis 't', 32-token blocks from the
    user's first token)."""
    y = x.copy()
    T, H, D = x.shape
    if axis == "d":
        for t in range(T):
            for h in range(H):
                for b in range(D // 32):
                    y[t, h, 32 * b:32 * b + 32] = oracle.mx_quantize_block(x[t, h, 32 * b:32 * b + 32])
        return y
    for u in range(len(off) - 1):
        for t0 in range(int(off[u]), int(off[u + 1]), 32):
            t1 = min(t0 + 32, int(off[u + 1]))
            for h in range(H):
                for d in range(D):
                    y[t0:t1, h, d] = oracle.mx_quantize_block(x[t0:t1, h, d])
    return y


def test_mx_bwd_error_against_the_exact_gradient():
    """A property, not a pin: on N(0,1) inputs quantized along each product's
    contraction, the MXFP8 backward stays within 10% (relative L2 norm) of
    the exact gradient of the unquantized inputs, and quantizing P and dS in
    the backward adds at most 4% (three mantissa bits round a value by about
    2-4%).  A wrong block exponent or axis would land far outside."""
    rng = np.random.default_rng(12)
    off = wl.offsets_from_lengths([200, 37, 130])
    T, H, D, B, W = int(off[-1]), 2, 64, 32, 3
    sc = 1 / math.sqrt(D)
    q, k, v, do = (rng.standard_normal((T, H, D)) for _ in range(4))
    exact = oracle.bwd(q, k, v, do, off, B, W, sc)
    qd, kd, vd, dd = (_mx_quantize(x, off, "d") for x in (q, k, v, do))
    qt, kt, dt = (_mx_quantize(x, off, "t") for x in (q, k, do))
    o, lse = oracle.fwd(qd, kd, vd, off, B, W, sc)
    args = (qd, kd, vd, dd, o, lse, qt, kt, dt, off, B, W, sc)
    got = oracle.mx_bwd(*args)
    unq = oracle.mx_bwd(*args, quantize=False)
    rel = lambda a, b: np.linalg.norm(a - b) / np.linalg.norm(b)
    for g, e, u in zip(got, exact, unq):
        assert 0.01 < rel(g, e) < 0.10
        assert 0.005 < rel(g, u) < 0.04
