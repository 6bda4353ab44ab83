#!/usr/bin/env python3
"""Benchmark of jagged block attention on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
the forward kernel (scores, mask, online softmax, PV, epilogue) and, for
training workloads, the fused backward kernel (dQ, dK, dV).  The default
workload is the jagged bf16 training step: 256 users with lognormal lengths
(median 600, sigma 0.8, clipped to [16, 4096]), 8 heads, head_dim 64,
block 128, window 2 blocks, forward plus backward.

Prints ONE JSON line.  ``value`` is algorithmic TFLOP/s over unmasked
(query, key) pairs: 4*D flops per pair forward, 8*D backward.  Inputs are
resident in HBM before the timed region.  ``roofline`` describes the
dominant kernel (each entry point is a single kernel launch), timed with HIP
events on the stream the kernels run on; ``cpu_baseline`` times the fp64
oracle on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0  # dense fp8 MFMA, MI355X
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "block-attention TFLOP/s and tokens/s (fwd+bwd, jagged bf16) and % of MFMA peak"
KERNEL_SOURCES = ("common.h", "kernels.h", "mfma_util.h", "lds_tile.h", "api.hip",
                  "scalar_kernels.hip", "mfma_fwd.hip", "mfma_bwd.hip", "mfma_bwd_mx.hip",
                  "rope.hip")


def pairs_per_head(offsets: np.ndarray, B: int, W: int) -> int:
    """Number of visible (query, key) pairs per head: the FLOP count basis."""
    total = 0
    for L in np.diff(offsets.astype(np.int64)):
        i = np.arange(L, dtype=np.int64)
        total += int(np.sum(i - np.maximum(0, i // B - W + 1) * B + 1))
    return total


def cpu_sample_users(w, offsets: np.ndarray, budget: float = 1.5e12) -> int:
    """Users [0, n) whose oracle work (forward, and backward for training
    workloads) stays within `budget` flops, at least one: about 30 s on 16
    host threads for the plain oracle.  The MXFP8 oracle quantizes every
    weight and dS element in scalar code, so it gets a quarter of that."""
    per = 4.0 * w.head_dim + (8.0 * w.head_dim if w.backward else 0.0)
    budget = budget / 4 if w.mx else budget
    spent, n = 0.0, 0
    for u in range(len(offsets) - 1):
        spent += per * w.heads * pairs_per_head(offsets[u:u + 2] - offsets[u], w.block_size,
                                                w.window_blocks)
        if n > 0 and spent > budget:
            break
        n += 1
    return max(n, 1)


def source_code(text: str) -> str:
    """C/HIP source without its comments, trailing blanks and empty lines:
    what the compiler sees (the sources hold no string literals with comment
    markers), so an edit to a comment leaves the hash of the kernels alone."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(l.rstrip() for l in text.splitlines() if l.strip())


def kernel_source_hash() -> str:
    """Hash of the kernel and ABI sources' code (comments excluded), which
    the committed profile summaries record."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        p = os.path.join(ROOT, "long_sequence_block_amd", "csrc", name)
        if os.path.exists(p):
            h.update(name.encode())
            h.update(source_code(open(p).read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if there is none for the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"kernel_source_hash:\s*([0-9a-f]+)", text)
    m_val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_src or not m_val or m_src.group(1) != kernel_source_hash():
        return None
    return float(m_val.group(1))


def measured_counters(kernel: str, workload: str):
    """Shader clock and MFMA busy share of the dominant kernel from the
    committed rocprofv3 counter summary (fwd_mfma for the forward; for the
    backward, each of its passes, bf16 or MXFP8), or None if there is none for the
    current kernel sources."""
    files = ([f"fwd_{workload}_counters.md", f"fwd-bwd_{workload}_counters.md"]
             if kernel == "fwd" else [f"fwd-bwd_{workload}_counters.md"])
    row_key = ("fwd_mfma",) if kernel == "fwd" else ("bwd_mfma", "bwd_mx")
    for f in files:
        path = os.path.join(ROOT, "profiles", f)
        if not os.path.exists(path):
            continue
        text = open(path).read()
        m_src = re.search(r"kernel_source_hash\s*([0-9a-f]{16})", text)
        if not m_src or m_src.group(1) != kernel_source_hash():
            return None
        rows = []
        for line in text.splitlines():
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if cells and cells[0].startswith(row_key) and len(cells) > 4:
                rows.append({"kernel": cells[0], "clock_ghz": float(cells[3]),
                             "mfma_busy_pct": float(cells[4]),
                             "source": os.path.join("profiles", f)})
        if rows:
            return rows[0] if kernel == "fwd" else rows
    return None


def _oracle_inputs(w, users):
    """Users [0, users) of the workload as the oracle sees them: fp64 values
    of the bf16-rounded inputs (or decoded MXFP8)."""
    import oracle
    import torch
    from long_sequence_block_amd import workloads as wl
    c = wl.draw(w, users=slice(0, users))
    host = {}
    for key, val in c.items():
        if key == "offsets" or key.endswith(("_mx", "_sc", "_bsc")):
            host[key] = val
        else:
            t = torch.from_numpy(val)
            if w.dtype == "bf16":
                t = t.to(torch.bfloat16)
            host[key] = t.to(torch.float64).numpy()
    if w.mx:  # the oracle attends on the decoded MXFP8 values
        host["q"] = oracle.mx_decode(host.pop("q_mx"), host.pop("q_sc"))
        host["k"] = oracle.mx_decode(host.pop("k_mx"), host.pop("k_sc"))
    if w.mx_v:
        host["v"] = oracle.mx_decode_user_blocks(host.pop("v_mx"), host.pop("v_bsc"),
                                                 host["offsets"])
    if w.mx and w.backward:  # the MXFP8 backward's head-dim- and token-blocked copies
        host["v_h"] = oracle.mx_decode(host.pop("vh_mx"), host.pop("vh_sc"))
        host["dout"] = oracle.mx_decode(host.pop("do_mx"), host.pop("do_sc"))
        for n in ("qt", "kt", "dot"):
            host[n] = oracle.mx_decode_user_blocks(host.pop(n + "_mx"), host.pop(n + "_bsc"),
                                                   host["offsets"])
    return host


def _oracle_run(w, host):
    """The oracle's whole path for the workload: forward (and backward)."""
    import oracle
    off = host["offsets"]
    q, k, v = host["q"], host["k"], host["v"]
    B, W, sc = w.block_size, w.window_blocks, w.scale
    if w.act:  # activation scores
        oracle.gdpa_fwd(q, k, v, off, B, W, sc, w.act)
        if w.backward:
            oracle.gdpa_bwd(q, k, v, host["dout"], off, B, W, sc, w.act)
        return
    if w.mx_v:  # the weights quantized for P.V
        o, l = oracle.mxpv_fwd(q, k, v, off, B, W, sc)
        if w.backward:  # every product block-scaled
            oracle.mx_bwd(q, k, host["v_h"], host["dout"], o, l, host["qt"], host["kt"],
                          host["dot"], off, B, W, sc)
        return
    if w.rope_base:
        q, k = oracle.rope(q, off, w.rope_base), oracle.rope(k, off, w.rope_base)
    oracle.fwd(q, k, v, off, B, W, sc)
    if w.backward and w.rope_base:
        oracle.rope_bwd(q, k, v, host["dout"], off, B, W, sc, w.rope_base)
    elif w.backward:
        oracle.bwd(q, k, v, host["dout"], off, B, W, sc)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, users: int, flops_per_pair_head: float):
    """The fp64 oracle, as it stands, on users [0, users) of the workload, on
    all host threads; plus single-thread times of the forward on bounded
    samples of the tiny, fixed-length and jagged workloads."""
    import oracle
    from long_sequence_block_amd import workloads as wl
    host = _oracle_inputs(w, users)
    off = host["offsets"]
    t0 = time.perf_counter()
    _oracle_run(w, host)
    dt = time.perf_counter() - t0
    flops = flops_per_pair_head * pairs_per_head(off, w.block_size, w.window_blocks) * w.heads
    threads = oracle.num_threads()
    single = []
    oracle.set_num_threads(1)
    try:
        for wid, nu in ((1, 2), (2, 8), (3, 32)):
            ws = dataclasses.replace(wl.WORKLOADS[wid], backward=False)
            hs = _oracle_inputs(ws, nu)
            t1 = time.perf_counter()
            _oracle_run(ws, hs)
            d1 = time.perf_counter() - t1
            f1 = 4.0 * ws.head_dim * pairs_per_head(hs["offsets"], ws.block_size,
                                                    ws.window_blocks) * ws.heads
            single.append({"workload": ws.name, "sample": f"users 0-{nu - 1} of {ws.users}, fwd",
                           "seconds": round(d1, 3), "GFLOP/s": round(f1 / d1 / 1e9, 3)})
    finally:
        oracle.set_num_threads(threads)
    try:
        nproc = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        nproc = os.cpu_count()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"users 0-{users - 1} of {w.name} ({int(off[-1])} tokens, "
                       f"{'fwd+bwd' if w.backward else 'fwd'}, fp64), {dt:.1f} s"),
            "seconds": dt, "threads": threads, "nproc": nproc, "cpu_count": os.cpu_count(),
            "cpu_model": cpu_model(), "single_thread": single}


WARM_SECONDS = 0.5  # least wall time of untimed steps before a timed region


def warm_up(fn, steps: int, seconds: float = WARM_SECONDS) -> int:
    """Runs fn back to back at least `steps` times and for at least `seconds`
    of wall time, then waits for the GPU.  The GPU raises its clocks over its
    first tens of milliseconds under load, so a timed region that starts
    earlier measures that ramp: in one run of the jagged training step, 20
    timed steps after 5 warm-up steps took 0.92 ms each, and every later
    group of 20 about 0.84 ms.  Returns how many times fn ran."""
    import torch
    n, t_end = 0, time.perf_counter() + seconds
    while n < steps or time.perf_counter() < t_end:
        fn()
        n += 1
        if n % 4 == 0:  # keep the host within a few calls of the GPU
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def copy_calibration(mib: int, steps: int, warmup: int):
    """Times torch's device-to-device copy of a known size: its HBM byte
    counters (read mib MiB, write mib MiB per launch) calibrate the counters
    taken on the attention kernels."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    warm_up(lambda: dst.copy_(src), warmup)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms_per_copy": ms,
                      "GB_per_s": 2 * n / (ms * 1e-3) / 1e9}), flush=True)


def length_sweep(steps: int, warmup: int):
    """The long-context shape (32 users of L tokens, 8 heads, head_dim 128,
    block 256) at every sweep length, forward, with the block window (W = 4)
    and with a window of L/256 blocks (plain causal attention), on the same
    kernels: one JSON line per (L, window) with the median call time, then
    the affine fit of the block-window times against the visible-pair count
    and the log-log slopes of both against L.  Inputs: seeded N(0,1) draws
    made on the device (the values do not change the work)."""
    import torch
    import long_sequence_block_amd as lsb
    from long_sequence_block_amd import workloads as wl
    dev = torch.device("cuda:0")
    rows = []
    for L in wl.LONG_CONTEXT_SWEEP:
        w = wl.long_context(L)
        T, H, D, B = w.users * L, w.heads, w.head_dim, w.block_size
        g = torch.Generator(device=dev)
        g.manual_seed(L)
        q, k, v = (torch.randn(T, H, D, generator=g, device=dev).to(torch.bfloat16)
                   for _ in range(3))
        off = torch.arange(0, T + 1, L, dtype=torch.int32, device=dev)
        out = torch.empty_like(q)
        lse = torch.empty((H, T), dtype=torch.float32, device=dev)
        for W, kind in ((w.window_blocks, "block window"), (L // B, "full causal")):
            warm_up(lambda: lsb.fwd(q, k, v, off, B, W, w.scale, out=out, lse=lse), warmup,
                    0.2)
            times = []
            for _ in range(steps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                lsb.fwd(q, k, v, off, B, W, w.scale, out=out, lse=lse)
                e1.record()
                e1.synchronize()
                times.append(e0.elapsed_time(e1))
            times.sort()
            npair = pairs_per_head(off.cpu().numpy(), B, W)
            row = {"length": L, "window": kind, "window_blocks": W, "pairs_per_head": npair,
                   "median_ms": round(times[len(times) // 2], 4), "min_ms": round(times[0], 4),
                   "TFLOP/s": round(4.0 * D * npair * H / (times[len(times) // 2] * 1e-3) / 1e12,
                                    1)}
            rows.append(row)
            print(json.dumps(row), flush=True)
        del q, k, v, out, lse
    blk = [r for r in rows if r["window"] == "block window"]
    cau = [r for r in rows if r["window"] == "full causal"]
    x = np.array([r["pairs_per_head"] for r in blk], np.float64)
    y = np.array([r["median_ms"] for r in blk], np.float64)
    a, c = np.polyfit(x, y, 1)
    r2 = 1.0 - np.sum((y - (a * x + c)) ** 2) / np.sum((y - y.mean()) ** 2)
    lens = np.log([r["length"] for r in blk])
    slope = lambda rs: float(np.polyfit(lens, np.log([r["median_ms"] for r in rs]), 1)[0])
    print(json.dumps({"fit": "block-window median_ms = a * pairs_per_head + c",
                      "a_ms_per_pair": a, "c_ms": round(c, 4), "r2": round(r2, 5),
                      "loglog_slope_block": round(slope(blk), 3),
                      "loglog_slope_causal": round(slope(cau), 3)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=5,
                    help="1 tiny fp32, 2 fixed bf16, 3 jagged bf16, 4 long context, "
                         "5 jagged bf16 training step (default), 6 the same step with a "
                         "194-token sliding window (same visible-pair count), 7 the training "
                         "step with the rotary embedding (rope, fwd, fused rope backward), 8 the "
                         "training step with SiLU scores (generalized dot-product attention), "
                         "9 and 10 the long-context and jagged forwards with q, k in MXFP8, "
                         "11 the long-context shape as a training step, 12 the training step "
                         "at 1024 users, 13 and 14 the long-context and jagged forwards with "
                         "q, k, v in MXFP8 and the weights quantized for a block-scaled P.V, "
                         "15 and 16 the jagged and long-context MXFP8 training steps (that "
                         "forward, then the backward with every product block-scaled)")
    ap.add_argument("--length", type=int, default=0,
                    help="long-context workload: per-user length (sweep)")
    ap.add_argument("--window-blocks", type=int, default=0,
                    help="override the workload's window W (e.g. L/B: full causal attention)")
    ap.add_argument("--block-size", type=int, default=0,
                    help="override the workload's block size B (tokens)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold pass (steps after an L2 / Infinity Cache flush)")
    ap.add_argument("--cpu-users", type=int, default=0,
                    help="users timed for the oracle baseline (default: all)")
    ap.add_argument("--length-sweep", action="store_true",
                    help="instead of the workload, time the long-context forward at each sweep "
                         "length with the block window and with full causal attention")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the workload, time a plain device copy of MIB MiB "
                         "(reference kernel for scaling HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py measures one GPU only: this build has no multi-GPU path "
                  "(users and heads would shard across GPUs with no exchange). "
                  "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import long_sequence_block_amd as lsb
    from long_sequence_block_amd import workloads as wl

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps, args.warmup)
        return
    if args.length_sweep:
        length_sweep(args.steps, args.warmup)
        return

    w = wl.WORKLOADS[args.workload]
    if args.length:
        w = wl.long_context(args.length)
    if args.block_size:
        w = dataclasses.replace(w, block_size=args.block_size,
                                name=f"{w.name}-B{args.block_size}")
    if args.window_blocks:
        w = dataclasses.replace(w, window_blocks=args.window_blocks,
                                name=f"{w.name}-W{args.window_blocks}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    c = wl.draw(w)
    off_np = c["offsets"]
    T = int(off_np[-1])
    if w.mx:  # fp8 codes as is, scales head-major [H, T, D/32]
        d = {k: torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)) if k.endswith("_sc")
                                 else v).to(dev)
             for k, v in c.items() if k in ("offsets", "q_mx", "q_sc", "k_mx", "k_sc")}
        d["q"], d["k"] = d.pop("q_mx"), d.pop("k_mx")
        if w.mx_v:  # v transposed, user-blocked [H, D, 32 nb], scales [H, nb, D]
            vt, vs = wl.mx_v_device_layout(c["v_mx"], c["v_bsc"], c["offsets"])
            d["v_t"], d["v_bsc"] = torch.from_numpy(vt).to(dev), torch.from_numpy(vs).to(dev)
            if w.backward:  # the MXFP8 backward's v, dO and token-blocked q, k, dO
                for n in ("vh", "do"):
                    d[n] = torch.from_numpy(c[n + "_mx"]).to(dev)
                    d[n + "_sc"] = torch.from_numpy(
                        np.ascontiguousarray(c[n + "_sc"].transpose(1, 0, 2))).to(dev)
                for n in ("qt", "kt", "dot"):
                    xt, xs = wl.mx_v_device_layout(c[n + "_mx"], c[n + "_bsc"], c["offsets"])
                    d[n], d[n + "_bsc"] = (torch.from_numpy(xt).to(dev),
                                           torch.from_numpy(xs).to(dev))
        else:
            d["v"] = torch.from_numpy(c["v"]).to(tdt).to(dev)
    else:
        d = {k: torch.from_numpy(v).to(dev) if k == "offsets" else
             torch.from_numpy(v).to(tdt).to(dev) for k, v in c.items()}
    del c
    B, W, sc = w.block_size, w.window_blocks, w.scale
    H, D = w.heads, w.head_dim
    out = torch.empty((T, H, D), dtype=tdt, device=dev)
    lse = torch.empty((H, T), dtype=torch.float32, device=dev)
    grads = tuple(torch.empty_like(out) for _ in range(3)) if w.backward else None
    ws_n = lsb.blockattn_bwd_workspace_size(T, d["offsets"].numel() - 1, H,
                                           lsb.BF16 if w.dtype == "bf16" else lsb.FP32)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n else None
    rb = w.rope_base
    qa, ka = (torch.empty_like(d["q"]), torch.empty_like(d["k"])) if rb else (d["q"], d["k"])

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        if rb:  # rotary embedding of q and k into qa, ka
            lsb.rope(d["q"], d["k"], d["offsets"], rb, q_rot=qa, k_rot=ka)
        if w.mx_v:  # q, k, v in MXFP8, the weights quantized for P.V
            lsb.mxpv_fwd(qa, d["q_sc"], ka, d["k_sc"], d["v_t"], d["v_bsc"], d["offsets"], B, W,
                         sc, out=out, lse=lse)
        elif w.mx:  # q, k in MXFP8
            lsb.mx_fwd(qa, d["q_sc"], ka, d["k_sc"], d["v"], d["offsets"], B, W, sc, out=out,
                       lse=lse)
        elif w.act:  # activation scores (GDPA): no lse
            lsb.gdpa_fwd(qa, ka, d["v"], d["offsets"], B, W, sc, w.act, out=out)
        else:
            lsb.fwd(qa, ka, d["v"], d["offsets"], B, W, sc, out=out, lse=lse)
        if ev is not None:
            ev[1].record()
        if w.backward and w.act:
            lsb.gdpa_bwd(qa, ka, d["v"], d["dout"], d["offsets"], B, W, sc, w.act, grads=grads,
                         workspace=ws)
        elif w.backward and rb:  # gradients through attention and the rotation
            lsb.rope_bwd(qa, ka, d["v"], out, d["dout"], lse, d["offsets"], B, W, sc, rb,
                         grads=grads, workspace=ws)
        elif w.backward and w.mx:  # every product block-scaled
            lsb.mx_bwd(qa, d["q_sc"], ka, d["k_sc"], d["vh"], d["vh_sc"], d["do"], d["do_sc"],
                       d["qt"], d["qt_bsc"], d["kt"], d["kt_bsc"], d["dot"], d["dot_bsc"], out,
                       lse, d["offsets"], B, W, sc, grads=grads, workspace=ws)
        elif w.backward:
            lsb.bwd(qa, ka, d["v"], out, d["dout"], lse, d["offsets"], B, W, sc,
                    grads=grads, workspace=ws)
        if w.backward and ev is not None:
            ev[2].record()

    warm_steps = warm_up(step, args.warmup)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(evs[i])
    stop.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(stop) / args.steps
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    bwd_ms = (sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps) if w.backward else 0.0

    def spread(times):
        t = sorted(times)
        return {"median": round(t[len(t) // 2], 4), "min": round(t[0], 4)}

    # Per-call medians and minima: warm (the back-to-back steps above) and
    # cold (each step after a 512 MiB write that evicts L2 and the
    # Infinity Cache; the write is outside the events).
    calls = {"warm": {"fwd_ms": spread([e[0].elapsed_time(e[1]) for e in evs])}}
    if w.backward:
        calls["warm"]["bwd_ms"] = spread([e[1].elapsed_time(e[2]) for e in evs])
    if not args.no_cold:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cold = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
                for _ in range(args.steps)]
        for i in range(args.steps):
            flush.fill_(i & 0xFF)
            step(cold[i])
        torch.cuda.synchronize()
        del flush
        calls["cold"] = {"fwd_ms": spread([e[0].elapsed_time(e[1]) for e in cold])}
        if w.backward:
            calls["cold"]["bwd_ms"] = spread([e[1].elapsed_time(e[2]) for e in cold])

    npair = pairs_per_head(off_np, B, W)
    e = 2 if w.dtype == "bf16" else 4
    fwd_flops = 4.0 * D * npair * H
    bwd_flops = 8.0 * D * npair * H if w.backward else 0.0
    fwd_bytes = T * H * (4.0 * D * e + (0 if w.act else 4)) + (4.0 * T * H * D * e if rb else 0.0)
    if w.mx:  # q, k one byte per element plus one scale byte per 32
        fwd_bytes = T * H * (2.0 * D * (1 + 1 / 32) + 2.0 * D * e + 4)
    if w.mx_v:  # v one byte per element too
        fwd_bytes = T * H * (3.0 * D * (1 + 1 / 32) + 2.0 * D + 4)
    # GDPA's backward reads q, k, v, dO and writes dq, dk, dv (no out, no lse)
    bwd_bytes = (T * H * ((7.0 * D * e) if w.act else (8.0 * D * e + 4))) if w.backward else 0.0
    if w.mx and w.backward:  # seven MXFP8 inputs (one byte + a scale per 32), O, lse in;
        bwd_bytes = T * H * (7.0 * D * (1 + 1 / 32) + 2.0 * D + 4 + 6.0 * D)  # dq, dk, dv out
    flops = fwd_flops + bwd_flops
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    if w.mx:  # half the products at the fp8 rate, half (P.V) at the bf16 rate
        peak = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
    if w.mx_v:  # both products at the fp8 rate
        peak = PEAK_FP8_TFLOPS

    # dominant kernel: the entry point (one launch each) with the larger time
    if w.backward and bwd_ms >= fwd_ms:
        kname, k_ms, k_flops, k_bytes = "bwd", bwd_ms, bwd_flops, bwd_bytes
    else:
        kname, k_ms, k_flops, k_bytes = "fwd", fwd_ms, fwd_flops, fwd_bytes
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    if k_flops / k_bytes < ridge:
        ach = k_bytes / (k_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4)}
    else:
        ach = k_flops / (k_ms * 1e-3) / 1e12
        roof = {"bound": "mfma" if w.dtype == "bf16" else "alu", "achieved": round(ach, 2),
                "peak": peak, "unit": "TFLOP/s", "frac": round(ach / peak, 4)}
    roof["traffic"] = measured_traffic(kname, w.name)
    # measured HBM rate of the dominant kernel: counted bytes per launch over
    # this run's average launch time (null without a traffic measurement)
    roof["traffic_gbs"] = (round(roof["traffic"] / (k_ms * 1e-3) / 1e9, 1)
                           if roof["traffic"] else None)
    roof["counters"] = measured_counters(kname, w.name)
    roof["kernel"] = kname
    roof["avg_launch_ms"] = round(k_ms, 4)
    roof["algorithmic_bytes"] = k_bytes
    roof["algorithmic_flops"] = k_flops

    res = {
        "metric": METRIC, "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_steps_run": warm_steps,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp8" if w.mx_v else "mxfp8(qk)+bf16" if w.mx else w.dtype,
        "data": "synthetic (seeded; lognormal jagged lengths, N(0,1) values"
                + ("; random E4M3 codes and E8M0 scales for q, k, v, dO and the backward's "
                   "second copies)" if w.mx_v and w.backward else
                   "; random E4M3 codes and E8M0 scales for q, k, v)" if w.mx_v else
                   "; random E4M3 codes and E8M0 scales for q, k)" if w.mx else ")"),
        "config": {"workload": w.name, "users": w.users, "tokens": T, "heads": H,
                   "head_dim": D, "block_size": B, "window_blocks": W,
                   "backward": w.backward, "pairs_per_head": npair,
                   **({"rope_base": rb} if rb else {}),
                   **({"activation": {1: "silu", 2: "gelu"}[w.act]} if w.act else {}),
                   "parallelism": "single GPU"},
        "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
        "pct_mfma_peak": round(100.0 * tflops / peak, 3),
        "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
        "timing": ("value and ms_per_step: warm, the timed steps run back to back with "
                   "inputs resident in HBM, after at least `warmup` untimed steps and "
                   f"{WARM_SECONDS} s of them (warmup_steps_run), so that the GPU's clocks "
                   "have settled under the load; calls.cold: per-call medians after a 512 MiB "
                   "write that evicts L2 and the Infinity Cache"),
        "calls": calls,
        "roofline": roof,
        "cpu_baseline": None,
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        users = (min(args.cpu_users, w.users) if args.cpu_users > 0
                 else cpu_sample_users(w, off_np))
        res["cpu_baseline"] = cpu_baseline(w, users, 4.0 * D + (8.0 * D if w.backward else 0))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
