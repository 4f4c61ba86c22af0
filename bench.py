#!/usr/bin/env python3
"""Verify-step benchmark on one MI355X.

One step is one verification-attention call over the 32k-context, 64-node
tree workload (batch 1, 32/8 heads, head_dim 128, bf16): the ancestor mask,
the split prefix attention, the masked tree attention and the log-sum-exp
merge, all in the HIP library.  Inputs are resident in HBM before timing.
Several copies of the KV cache (standing for the caches of successive
layers) are rotated so that a step never finds its cache in the 256 MB
Infinity Cache left over from the previous step.

Timing protocol (every figure on the line): W warm-up steps, then whole steps
replayed back to back from one captured HIP graph for at least 50 ms so the
shader clock settles at its sustained value, then EXACTLY K steps as one
replay of the graph of K steps, between synchronisations.  ms_per_step is
that wall time over K; HIP events on the replay's stream give the same within
a few per cent (reported under ``timing`` with the eager per-call figure).

Prints ONE JSON line (rank 0):
  value = KV-read GB/s of the whole step; ms_per_step = time per step;
  roofline = the dominant kernel (the attention partials), its average
  duration from HIP events around a replay of a graph of K back-to-back
  launches on its stream (settled the same way); traffic = its HBM bytes per
  launch from the committed rocprofv3 counter summary, when that summary was
  taken on the current kernel source; workloads = the other four workloads'
  whole-step figures under the same protocol; cpu_baseline = the fp64
  oracle timed on the host cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

from __future__ import annotations

import argparse
import functools
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verify-step µs and KV-read GB/s (% HBM peak) at 32k ctx, 64-node tree"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
INFINITY_CACHE_BYTES = 256 * 2 ** 20
# Counter summary of the dominant kernel (written from rocprofv3 --pmc runs)
# and the sources whose hash it records.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "attn_partial_dma_tree32k_counters.md")
KERNEL_SOURCES = ("long_context_tree_verify_amd/csrc/attn_dma.hip",
                  "long_context_tree_verify_amd/csrc/common.hpp",
                  "long_context_tree_verify_amd/csrc/plan.h")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kv_bytes(inp) -> int:
    """Algorithmic KV bytes of one step: every (b, kv head) reads K and V rows of
    its prefix (or its index set) and of the draft block once."""
    wl = inp.wl
    row = 2 * wl.head_dim * (2 if wl.dtype == "bf16" else 4)  # K + V row
    if inp.kv_idx is not None:
        keys = wl.batch * wl.n_kv_heads * (wl.n_sel + wl.n_draft)
    else:
        keys = int((inp.ctx_lens.astype(int) + wl.n_draft).sum()) * wl.n_kv_heads
    return keys * row


def step_flops(inp) -> int:
    """QK^T and PV multiply-adds over the same key sets, 2 FLOP each."""
    wl = inp.wl
    per_key_row = 2 * 2 * wl.head_dim * wl.group * wl.n_draft   # per key per kv head
    row = 2 * wl.head_dim * (2 if wl.dtype == "bf16" else 4)
    return kv_bytes(inp) // row * per_key_row


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload: str):
    """HBM bytes per launch of the partial kernel from the committed counter
    summary, or None if there is none for this workload or the kernel source
    changed since it was taken."""
    if workload != "tree32k" or not os.path.exists(TRAFFIC_PROFILE):
        return None
    fields = {}
    with open(TRAFFIC_PROFILE) as f:
        for line in f:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp, target_s: float):
    """Time the fp64 oracle on a bounded sample of output rows and scale."""
    import numpy as np

    import oracle
    wl = inp.wl
    B, N, Hq = wl.batch, wl.n_draft, wl.n_q_heads
    total = B * N * Hq
    rng = np.random.default_rng(0)
    order = rng.permutation(total)

    def run(n):
        idx = order[:n]
        rows = [(int(r // (N * Hq)), int((r // Hq) % N), int(r % Hq)) for r in idx]
        t = time.perf_counter()
        oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent,
                           kv_idx=inp.kv_idx, bf16=inp.is_bf16, rows=rows)
        return time.perf_counter() - t

    threads = oracle.num_threads()
    n = min(total, max(threads, 8))
    t = run(n)
    if t < target_s and n < total:
        n2 = min(total, max(n + 1, int(n * target_s / max(t, 1e-3))))
        t = run(n2)
        n = n2
    reps = 1
    if n == total:  # the whole step fits: repeat it for a stable figure
        while t < target_s:
            t += run(n)
            reps += 1
    step_s = t / reps * total / n
    gbs = kv_bytes(inp) / step_s / 1e9
    what = (f"{n} of {total}" if n < total else f"all {total}") + \
        f" (b, node, head) rows of the {wl.name} step, each over its full key set, fp64"
    # the same oracle on one thread, over the first 8 rows of the sample
    n1 = min(total, 8)
    oracle.set_num_threads(1)
    try:
        t1 = run(n1)
    finally:
        oracle.set_num_threads(threads)
    step1_s = t1 * total / n1
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model,
            "sample": f"{what}; {reps} run(s), {t:.2f} s measured"
                      + (f", scaled by {total}/{n}" if n < total else ""),
            "step_s": round(step_s, 4),
            "one_thread": {"value": round(kv_bytes(inp) / step1_s / 1e9, 4), "unit": "GB/s",
                           "step_s": round(step1_s, 6),
                           "sample": f"{n1} rows on one thread, {t1:.4f} s, scaled by "
                                     f"{total}/{n1}"}}


# Verification index-set selection on the sparse workload's shape: 8
# sequences x 8 KV heads, 65536-position importance maps, a 4096-entry set
# of 4 sinks, a 512-token window, 1790 by the draft map, the rest by the
# target map.
SELECT_SHAPE = dict(batch=8, n_kv_heads=8, score_len=65536, n_sel=4096, n_sink=4,
                    n_recent=512, n_draft_top=1790, seed=505)


def measure_selection(hsv, dev, steps: int, warmup: int):
    """Average duration of one hsv_select_kv_idx call (the settled graph
    protocol of `settled_timing`) and the algorithmic
    bytes it moves: each candidate score of both maps read once, the index
    set written once."""
    import numpy as np
    import torch

    import synth
    sh = SELECT_SHAPE
    B, H, L = sh["batch"], sh["n_kv_heads"], sh["score_len"]
    rng = np.random.Generator(np.random.PCG64(sh["seed"]))
    ctx_np = np.full(B, L, np.int32)
    draft_np, target_np = synth.importance_maps(rng, ctx_np, H, L)
    draft, target = torch.from_numpy(draft_np).to(dev), torch.from_numpy(target_np).to(dev)
    ctx = torch.from_numpy(ctx_np).to(dev)
    kv_idx = torch.empty((B, H, sh["n_sel"]), dtype=torch.int32, device=dev)
    ws = torch.empty(hsv.hsv_select_workspace_bytes(B, H, L), dtype=torch.uint8, device=dev)
    kw = dict(n_sel=sh["n_sel"], n_sink=sh["n_sink"], n_recent=sh["n_recent"],
              n_draft_top=sh["n_draft_top"], kv_idx=kv_idx, workspace=ws)
    us = settled_timing(lambda j: hsv.hsv_select_kv_idx(draft, target, ctx, **kw), steps,
                        warmup, dev, eager=False)["us"]
    n_cand = L - sh["n_sink"] - sh["n_recent"]
    nbytes = B * H * (2 * 4 * n_cand + 4 * sh["n_sel"])
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"kernel": "select_floor (sample floors per sequence and KV head) + select_filter "
                      "(every CU streams the maps) + select_lists (exact radix select per "
                      "sequence and KV head)",
            "workload": f"B{B} Hkv{H} L{L} n_sel {sh['n_sel']} (sinks {sh['n_sink']}, "
                        f"window {sh['n_recent']}, draft top {sh['n_draft_top']})",
            "call_us": round(us, 2), "algorithmic_bytes_per_call": nbytes,
            "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4)}


def measure_accept(hsv, dev, inp, steps: int):
    """Accepted-path cache update on the workload's own shape and trees, the
    deepest node of each tree accepted.  The context lengths are restored
    before every call (the update grows them); HIP events on the current
    stream bracket each call alone.  Bytes: every moved K and V row read
    and written once."""
    import numpy as np
    import torch

    wl = inp.wl
    B, H, N, D = wl.batch, wl.n_kv_heads, wl.n_draft, wl.head_dim
    S = wl.kv_capacity
    dt = torch.bfloat16 if inp.is_bf16 else torch.float32
    k = torch.zeros((B, H, S, D), dtype=dt, device=dev)
    v = torch.zeros_like(k)
    parent = torch.from_numpy(inp.parent).to(dev)
    # the path of node i is its ancestor-or-self mask; the deepest node has
    # the most bits; rows 0, 1, ... at the path's start are already in place
    anc = hsv.hsv_tree_ancestor_mask(parent).cpu().numpy().view(np.uint64)
    bits = np.array([[bin(int(x)).count("1") for x in row] for row in anc])
    node_np = bits.argmax(axis=1).astype(np.int32)
    node = torch.from_numpy(node_np).to(dev)
    ctx0 = torch.from_numpy(inp.ctx_lens).to(dev)
    ctx = ctx0.clone()
    moved = 0
    for b in range(B):
        m = int(anc[b, node_np[b]])
        lead = (~m & (m + 1)).bit_length() - 1      # trailing ones of m
        moved += bin(m).count("1") - lead
    nbytes = 2 * 2 * moved * H * D * k.element_size()
    # K (restore lengths, update) pairs in one graph, less a graph of the K
    # restores alone; HIP events on the capture stream bracket each replay
    side = torch.cuda.Stream(dev)

    def timed(with_update):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for _ in range(steps):
                ctx.copy_(ctx0)
                if with_update:
                    hsv.hsv_accept_path(k, v, ctx, parent, node)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(side):
            e0.record()
            g.replay()
            e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

    us = max(timed(True) - timed(False), 1e-3)
    return {"kernel": "accept_copy + accept_bump (one workgroup per sequence and KV head)",
            "workload": f"{wl.name} shape, deepest node accepted: {moved} rows moved per KV head",
            "call_us": round(us, 2), "algorithmic_bytes_per_call": nbytes,
            "achieved": round(nbytes / (us * 1e-6) / 1e9, 2), "unit": "GB/s",
            "note": "two launches (copy, then the length update), timed in a graph; "
                    "launch-bound at this size"}


PAGED_BLOCK = 128


def eager_us(call, steps: int) -> float:
    """K calls issued one at a time from Python, between synchronisations."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(steps):
        call(j)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e6 / steps


SETTLE_MS = 50.0  # back-to-back replays before any timed region (clock settling)


def settled_timing(call, steps: int, warmup: int, dev, settle_ms: float = SETTLE_MS,
                   eager: bool = True):
    """Time `call(j)` (one whole step on cache copy j) under sustained load.

    W eager warm-up calls; a graph of K calls captured on a side stream;
    replays of it back to back until at least `settle_ms` of GPU work has run
    (the shader clock falls by 10-15 % over the first milliseconds of
    sustained load and then holds); then ONE timed replay of the K calls,
    between synchronisations, with HIP events on the replay's stream.
    Returns wall and event microseconds per call (and, if asked, K eager calls
    timed between synchronisations, for reference only)."""
    import torch
    for j in range(warmup):
        call(j)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for j in range(steps):
            call(j)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(side):
        g.replay()
    torch.cuda.synchronize()
    one_ms = (time.perf_counter() - t0) * 1e3
    # further replays back to back (no host wait inside a batch) until the
    # settling time has passed
    n_settle = 1
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        left = settle_ms - (time.perf_counter() - t0) * 1e3
        n = max(1, math.ceil(left / max(one_ms, 1e-3)))
        with torch.cuda.stream(side):
            for _ in range(n):
                g.replay()
        torch.cuda.synchronize()
        n_settle += n
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    with torch.cuda.stream(side):
        e0.record()
        g.replay()
        e1.record()
    torch.cuda.synchronize()
    wall_us = (time.perf_counter() - w0) * 1e6 / steps
    ev_us = e0.elapsed_time(e1) * 1e3 / steps
    out = {"us": wall_us, "event_us": ev_us, "settle_replays": n_settle,
           "settle_ms": round((w0 - t0) * 1e3, 1)}
    if eager:
        out["eager_us"] = eager_us(call, steps)
    del g
    return out


def _smi_sample():
    """(socket power W, mean gfx clock MHz) from amd-smi, or None."""
    import re
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True,
                           text=True, timeout=10)
    except (OSError, subprocess.SubprocessError):
        return None
    m = re.search(r'"socket_power": \{\s*"value": (\d+)', r.stdout)
    c = re.findall(r'"gfx_\d+": \{\s*"clk": \{\s*"value": (\d+)', r.stdout)
    if not m:
        return None
    return int(m.group(1)), (sum(int(x) for x in c) / len(c) if c else None)


def idle_power():
    """Mean socket power over a second with the GPU idle (taken before any
    work in the process), or None."""
    xs = []
    for _ in range(10):
        x = _smi_sample()
        if x:
            xs.append(x[0])
        time.sleep(0.1)
    return sum(xs) / len(xs) if xs else None


def measure_power(call, steps: int, dev, p_idle, seconds: float = 2.0):
    """Socket power and shader clock (amd-smi, sampled from a second thread)
    while `call` replays back to back from a graph of `steps` calls for
    `seconds`, against the idle reading just before.  The energy per call is
    (power - idle) x the call's duration in that run.  None if amd-smi gives
    no reading."""
    import threading
    import torch
    if p_idle is None:
        return None
    side = torch.cuda.Stream(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for j in range(steps):
            call(j)
    torch.cuda.synchronize()
    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            x = _smi_sample()
            if x:
                samples.append(x)
            time.sleep(0.05)

    th = threading.Thread(target=poll)
    th.start()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        with torch.cuda.stream(side):
            for _ in range(5):
                g.replay()
        torch.cuda.synchronize()
        n += 5
    dt = time.perf_counter() - t0
    stop.set()
    th.join()
    del g
    steady = samples[len(samples) // 3:]
    if not steady:
        return None
    p = sum(x for x, _ in steady) / len(steady)
    clk = [c for _, c in steady if c]
    us = dt * 1e6 / (n * steps)
    return {"socket_w": round(p, 1), "idle_w": round(p_idle, 1),
            "gfx_mhz": round(sum(clk) / len(clk)) if clk else None,
            "us_per_call": round(us, 2),
            "dynamic_mj_per_call": round((p - p_idle) * us * 1e-3, 2),
            "samples": len(steady), "seconds": round(dt, 2)}


def measure_hbm_copy(dev, reps: int = 5):
    """The HBM rate a plain device-to-device copy reaches in this run (1 GiB
    read + 1 GiB written per copy, HIP events on the copy's stream): the
    practical ceiling the step's share is also quoted against."""
    import torch
    n = 2 ** 28  # fp32 elements: 1 GiB
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    moved = 2 * n * 4
    del src, dst
    torch.cuda.empty_cache()
    return {"what": "torch device-to-device copy, 1 GiB read + 1 GiB written",
            "bytes_moved": moved, "us": round(us, 1),
            "gbs": round(moved / (us * 1e-6) / 1e9, 1)}


def measure_paged(hsv, dev, inp, steps: int, warmup: int, out_dtype):
    """The same verify step (dense, or sparse over the workload's index sets)
    over a paged copy of the cache (pool blocks of PAGED_BLOCK tokens in
    seeded random order, a block table), pool copies rotated like the
    contiguous measurement, under the settled graph protocol of
    `settled_timing`."""
    import numpy as np
    import torch

    import synth
    wl = inp.wl
    bs = PAGED_BLOCK
    S = inp.k.shape[2]
    cap = -(-S // bs) * bs
    pad = ((0, 0), (0, 0), (0, cap - S), (0, 0))
    kp, vp, table = synth.to_paged(np.pad(inp.k, pad), np.pad(inp.v, pad), bs,
                                   np.random.Generator(np.random.PCG64(7)))

    def up(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    k0, v0 = up(kp), up(vp)
    # the bytes one step reads (a sparse step reads only its index sets' rows)
    step_bytes = kv_bytes(inp)
    copies = max(1, math.ceil(2 * INFINITY_CACHE_BYTES / step_bytes) + 1) if step_bytes < \
        2 * INFINITY_CACHE_BYTES else 1
    ks, vs = [k0] + [k0.clone() for _ in range(copies - 1)], [v0] + [v0.clone()
                                                                      for _ in range(copies - 1)]
    q = torch.from_numpy(inp.q.view(np.int16)).view(torch.bfloat16).to(dev)
    tab = torch.from_numpy(table).to(dev)
    ctx = torch.from_numpy(inp.ctx_lens).to(dev)
    parent = torch.from_numpy(inp.parent).to(dev)
    kv_idx = None if inp.kv_idx is None else torch.from_numpy(inp.kv_idx).to(dev)
    B, N, Hq, D = q.shape
    o = torch.empty((B, N, Hq, D), dtype=out_dtype, device=dev)
    lse = torch.empty((B, N, Hq), dtype=torch.float32, device=dev)
    max_ctx = int(inp.ctx_lens.max())
    desc = hsv.make_desc(batch=B, n_draft=N, n_q_heads=Hq, n_kv_heads=wl.n_kv_heads,
                         head_dim=D, kv_capacity=cap, max_ctx=max_ctx,
                         n_sel=0 if kv_idx is None else kv_idx.shape[2], in_dtype=hsv.HSV_BF16,
                         out_dtype=hsv.HSV_BF16 if out_dtype == torch.bfloat16 else hsv.HSV_F32,
                         block_size=bs)
    ws = torch.empty(hsv.hsv_verify_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    kw = dict(max_ctx=max_ctx, out_dtype=out_dtype, o=o, lse=lse, workspace=ws, stream=None)
    entry = "hsv_verify_attn_paged" if kv_idx is None else "hsv_verify_attn_sparse_paged"

    def call(j):
        if kv_idx is None:
            hsv.hsv_verify_attn_paged(q, ks[j % copies], vs[j % copies], tab, ctx, parent, **kw)
        else:
            hsv.hsv_verify_attn_sparse_paged(q, ks[j % copies], vs[j % copies], tab, ctx,
                                             parent, None, kv_idx, **kw)

    t = settled_timing(call, steps, warmup, dev)
    us = t["us"]
    nbytes = step_bytes
    del ks, vs, k0, v0
    torch.cuda.empty_cache()
    return {"entry": entry, "block_size": bs,
            "workload": f"{wl.name}, pool blocks in random order, {copies} pool copies",
            "us_per_step": round(us, 2), "event_us_per_step": round(t["event_us"], 2),
            "eager_us_per_step": round(t["eager_us"], 2), "kv_read_bytes": nbytes,
            "achieved": round(nbytes / (us * 1e-6) / 1e9, 2), "unit": "GB/s"}


def measure_recall(hsv, dev, steps: int, warmup: int):
    """Returns (recall, sparse_vs_dense).

    recall: the attention recall rate of the selected index sets (Dustin page,
    methodology 2 names the rate; reading: the share of the full prefix's
    softmax mass the set keeps, exp(lse_set - lse_full) per query row) on
    the workload with 256 planted heavy-hitter keys per (sequence, KV head):
    importance maps that flag most of those keys -> hsv_select_kv_idx ->
    prefix-only sparse attention over the set, against prefix-only dense
    attention.  A random Zipf-ranked set of the same size is the contrast.

    sparse_vs_dense: whole verify steps on the same inputs (prefix or index
    set, draft block, merge), the dense step over the full caches against the
    sparse step over the selected sets, each under the settled graph protocol
    of `settled_timing`.  Three copies of K and V are rotated, so the
    sparse step's gathered rows (134 MB per step) are not left in the 256 MB
    Infinity Cache by the step before."""
    import numpy as np
    import torch

    import synth
    sh = SELECT_SHAPE
    log("bench: generating the heavy-hitter workload for the recall rate")
    inp = synth.make_inputs("sparse64k_hh")
    wl = inp.wl
    B, H, L = wl.batch, wl.n_kv_heads, inp.k.shape[2]
    rng = np.random.Generator(np.random.PCG64(sh["seed"]))
    draft_np, target_np = synth.heavy_importance_maps(rng, inp, L)

    def up(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = up(inp.q), up(inp.k), up(inp.v)
    ctx = torch.from_numpy(inp.ctx_lens).to(dev)
    parent = torch.from_numpy(inp.parent).to(dev)
    draft, target = torch.from_numpy(draft_np).to(dev), torch.from_numpy(target_np).to(dev)
    kv_idx = torch.empty((B, H, wl.n_sel), dtype=torch.int32, device=dev)
    ws = torch.empty(hsv.hsv_select_workspace_bytes(B, H, L), dtype=torch.uint8, device=dev)
    kw = dict(n_sel=wl.n_sel, n_sink=wl.n_sink, n_recent=wl.n_recent,
              n_draft_top=sh["n_draft_top"], kv_idx=kv_idx, workspace=ws)
    hsv.hsv_select_kv_idx(draft, target, ctx, **kw)
    max_ctx = int(inp.ctx_lens.max())
    flags = hsv.HSV_FLAG_NO_TREE
    _, lse_full = hsv.hsv_verify_attn(q, k, v, ctx, parent, max_ctx=max_ctx, flags=flags)
    _, lse_sel = hsv.hsv_verify_attn_sparse(q, k, v, ctx, parent, None, kv_idx,
                                            max_ctx=max_ctx, flags=flags)
    rand_idx = torch.from_numpy(inp.kv_idx).to(dev)
    _, lse_rand = hsv.hsv_verify_attn_sparse(q, k, v, ctx, parent, None, rand_idx,
                                             max_ctx=max_ctx, flags=flags)
    torch.cuda.synchronize()
    arr = torch.exp(lse_sel.double() - lse_full.double())
    arr_rand = torch.exp(lse_rand.double() - lse_full.double())

    copies = 3
    ks = [k] + [k.clone() for _ in range(copies - 1)]
    vs = [v] + [v.clone() for _ in range(copies - 1)]
    B_, N_, Hq_, D_ = q.shape
    o = torch.empty((B_, N_, Hq_, D_), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B_, N_, Hq_), dtype=torch.float32, device=dev)
    desc = hsv.make_desc(batch=B_, n_draft=N_, n_q_heads=Hq_, n_kv_heads=H, head_dim=D_,
                         kv_capacity=k.shape[2], max_ctx=max_ctx, n_sel=wl.n_sel,
                         in_dtype=hsv.HSV_BF16, out_dtype=hsv.HSV_BF16)
    vws = torch.empty(hsv.hsv_verify_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    desc.n_sel = 0
    dws = torch.empty(hsv.hsv_verify_workspace_bytes(desc), dtype=torch.uint8, device=dev)

    def dense(j):
        hsv.hsv_verify_attn(q, ks[j % copies], vs[j % copies], ctx, parent, max_ctx=max_ctx,
                            out_dtype=torch.bfloat16, o=o, lse=lse, workspace=dws, stream=None)

    def sparse(j):
        hsv.hsv_verify_attn_sparse(q, ks[j % copies], vs[j % copies], ctx, parent, None, kv_idx,
                                   max_ctx=max_ctx, out_dtype=torch.bfloat16, o=o, lse=lse,
                                   workspace=vws, stream=None)

    def graph_us(fn):
        return settled_timing(fn, steps, warmup, dev, eager=False)["us"]

    dense_us, sparse_us = graph_us(dense), graph_us(sparse)
    dense_bytes = int((inp.ctx_lens.astype(np.int64) + wl.n_draft).sum()) * H * 2 * wl.head_dim * 2
    sparse_bytes = B * H * (wl.n_sel + wl.n_draft) * 2 * wl.head_dim * 2
    speed = {"workload": f"{wl.name}, whole verify steps (prefix or index set, draft block, "
                         f"merge), bf16 output, {copies} cache copies rotated",
             "dense_us_per_step": round(dense_us, 2), "sparse_us_per_step": round(sparse_us, 2),
             "speedup": round(dense_us / sparse_us, 2),
             "dense_kv_gbs": round(dense_bytes / (dense_us * 1e-6) / 1e9, 1),
             "sparse_kv_gbs": round(sparse_bytes / (sparse_us * 1e-6) / 1e9, 1),
             "kv_bytes_ratio": round(dense_bytes / sparse_bytes, 2)}
    del ks, vs
    recall = {"workload": f"{wl.name}: {wl.description}",
              "set": f"{wl.n_sel} positions (sinks {wl.n_sink}, window {wl.n_recent}, draft "
                     f"top {sh['n_draft_top']}) from maps flagging 70 % (draft) / 80 % "
                     f"(target) of the planted keys",
              "arr_mean": round(float(arr.mean()), 4), "arr_min": round(float(arr.min()), 4),
              "arr_random_set_mean": round(float(arr_rand.mean()), 4),
              "rows": int(arr.numel())}
    return recall, speed


def measure_wide_tree(hsv, dev, steps: int, warmup: int, out_dtype):
    """The 32k-context step with a 256-node draft tree (masks of four 64-bit
    words, 1024 grouped rows per KV head) under the settled graph protocol
    of `settled_timing`.  At 1024 rows the step does 4x the MFMA work per
    KV byte of the 64-node tree, so the matrix cores bound it."""
    import numpy as np
    import torch

    import synth
    inp = synth.make_inputs("tree32k", n_draft=256, max_depth=16)
    wl = inp.wl

    def up(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k0, v0 = up(inp.q), up(inp.k), up(inp.v)
    cache_bytes = 2 * k0.numel() * k0.element_size()
    copies = max(1, math.ceil(2 * INFINITY_CACHE_BYTES / cache_bytes) + 1)
    ks, vs = [k0] + [k0.clone() for _ in range(copies - 1)], [v0] + [v0.clone()
                                                                      for _ in range(copies - 1)]
    ctx = torch.from_numpy(inp.ctx_lens).to(dev)
    parent = torch.from_numpy(inp.parent).to(dev)
    B, N, Hq, D = q.shape
    o = torch.empty((B, N, Hq, D), dtype=out_dtype, device=dev)
    lse = torch.empty((B, N, Hq), dtype=torch.float32, device=dev)
    max_ctx = int(inp.ctx_lens.max())
    desc = hsv.make_desc(batch=B, n_draft=N, n_q_heads=Hq, n_kv_heads=wl.n_kv_heads,
                         head_dim=D, kv_capacity=k0.shape[2], max_ctx=max_ctx,
                         in_dtype=hsv.HSV_BF16,
                         out_dtype=hsv.HSV_BF16 if out_dtype == torch.bfloat16 else hsv.HSV_F32)
    ws = torch.empty(hsv.hsv_verify_workspace_bytes(desc), dtype=torch.uint8, device=dev)

    def call(j):
        hsv.hsv_verify_attn(q, ks[j % copies], vs[j % copies], ctx, parent, max_ctx=max_ctx,
                            out_dtype=out_dtype, o=o, lse=lse, workspace=ws, stream=None)

    t = settled_timing(call, steps, warmup, dev)
    us = t["us"]
    nbytes, flops = kv_bytes(inp), step_flops(inp)
    return {"workload": f"tree32k with a 256-node tree (depth <= 16, branching <= 4), "
                        f"{wl.group * N} grouped rows per KV head",
            "us_per_step": round(us, 2), "event_us_per_step": round(t["event_us"], 2),
            "eager_us_per_step": round(t["eager_us"], 2), "kv_read_bytes": nbytes, "flop": flops,
            "kv_gbs": round(nbytes / (us * 1e-6) / 1e9, 2),
            "tflops": round(flops / (us * 1e-6) / 1e12, 1),
            "mfma_util": round(flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}


@functools.lru_cache(maxsize=2)
def workload_inputs(name: str):
    """The seeded host inputs of a workload (kept: the paged measurement
    reuses the 64k sparse workload's)."""
    import synth
    log(f"bench: generating workload {name}")
    return synth.make_inputs(name)


def setup_workload(hsv, dev, name: str, out_dtype, num_splits: int = 0):
    """Inputs of one workload on the device, with enough cache copies that a
    step never finds its K/V bytes in the Infinity Cache, and a step callable
    call(j, flags) on copy j (torch's current stream: the capture stream
    inside a graph)."""
    import numpy as np
    import torch

    inp = workload_inputs(name)
    wl = inp.wl
    bf = inp.is_bf16

    def up(a):
        if bf and a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    q, k0, v0 = up(inp.q), up(inp.k), up(inp.v)
    ctx = torch.from_numpy(inp.ctx_lens).to(dev)
    parent = torch.from_numpy(inp.parent).to(dev)
    kv_idx = None if inp.kv_idx is None else torch.from_numpy(inp.kv_idx).to(dev)
    # the bytes one step reads must not fit the cache twice over
    step_bytes = kv_bytes(inp)
    copies = max(1, math.ceil(2 * INFINITY_CACHE_BYTES / step_bytes) + 1) if step_bytes < \
        2 * INFINITY_CACHE_BYTES else 1
    ks, vs = [k0], [v0]
    for _ in range(copies - 1):
        ks.append(k0.clone())
        vs.append(v0.clone())
    B, N, Hq, D = q.shape
    o = torch.empty((B, N, Hq, D), dtype=out_dtype, device=dev)
    lse = torch.empty((B, N, Hq), dtype=torch.float32, device=dev)
    max_ctx = int(inp.ctx_lens.max())
    desc = hsv.make_desc(batch=B, n_draft=N, n_q_heads=Hq, n_kv_heads=wl.n_kv_heads,
                         head_dim=D, kv_capacity=k0.shape[2], max_ctx=max_ctx,
                         n_sel=0 if kv_idx is None else kv_idx.shape[2],
                         in_dtype=hsv.HSV_BF16 if bf else hsv.HSV_F32,
                         out_dtype=hsv.HSV_BF16 if out_dtype == torch.bfloat16 else hsv.HSV_F32,
                         num_splits=num_splits)
    ws = torch.empty(hsv.hsv_verify_workspace_bytes(desc), dtype=torch.uint8, device=dev)

    def call(j, flags=0):
        kw = dict(max_ctx=max_ctx, out_dtype=out_dtype, num_splits=num_splits,
                  flags=flags, o=o, lse=lse, workspace=ws, stream=None)
        c = j % copies
        if kv_idx is None:
            hsv.hsv_verify_attn(q, ks[c], vs[c], ctx, parent, **kw)
        else:
            hsv.hsv_verify_attn_sparse(q, ks[c], vs[c], ctx, parent, None, kv_idx, **kw)

    cache_bytes = 2 * k0.numel() * k0.element_size()
    log(f"bench: {name}: {copies} cache copies of {cache_bytes / 2**20:.1f} MiB")
    return inp, call, copies


def kernel_name_of(inp) -> str:
    wl = inp.wl
    rows = wl.group * wl.n_draft
    if not inp.is_bf16:
        return "attn_partial_valu"
    if inp.kv_idx is None and wl.head_dim == 128 and rows > 128:
        return "attn_partial_dma (prefix + draft rows, split along keys)"
    if wl.head_dim == 128 and rows <= 32:
        return ("attn_partial_dma_small<sparse> (index set + draft rows, per-wave DMA)"
                if inp.kv_idx is not None else
                "attn_partial_dma_small<dense> (prefix + draft rows, per-wave DMA)")
    return "attn_partial_mfma (prefix or index-set splits, draft slot)"


def measure_step_and_kernel(hsv, call, steps: int, warmup: int, dev):
    """Whole steps and the partial kernel alone, each under the settled
    protocol; the kernel is a strict part of the step, so its time must not
    exceed the step's."""
    step = settled_timing(lambda j: call(j), steps, warmup, dev)
    part = settled_timing(lambda j: call(j, hsv.HSV_FLAG_PHASE_PARTIALS), steps, 0, dev,
                          eager=False)
    return step, part


def measure_other_workload(hsv, dev, name: str, steps: int, warmup: int, out_dtype):
    """One of the other four workloads under the same protocol: whole-step
    µs, its KV rate, and the share of the step the partial kernel takes."""
    import torch
    inp, call, copies = setup_workload(hsv, dev, name, out_dtype)
    step, part = measure_step_and_kernel(hsv, call, steps, warmup, dev)
    nbytes = kv_bytes(inp)
    wl = inp.wl
    res = {"desc": wl.description, "us_per_step": round(step["us"], 2),
           "event_us_per_step": round(step["event_us"], 2),
           "eager_us_per_step": round(step["eager_us"], 2),
           "kv_read_bytes": nbytes, "flop": step_flops(inp),
           "kv_gbs": round(nbytes / (step["us"] * 1e-6) / 1e9, 1),
           "pct_hbm_peak": round(100 * nbytes / (step["us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
           "kernel": kernel_name_of(inp), "kernel_us": round(part["event_us"], 2),
           "kernel_gbs": round(nbytes / (part["event_us"] * 1e-6) / 1e9, 1),
           "kernel_share_of_step": round(part["event_us"] / step["us"], 4),
           "cache_copies": copies, "steps": steps}
    if part["event_us"] > step["us"] * 1.02:
        raise AssertionError(f"{name}: partial kernel {part['event_us']:.2f} us exceeds the "
                             f"step {step['us']:.2f} us")
    del call
    torch.cuda.empty_cache()
    return res


OTHER_WORKLOADS = ("tiny_tree", "chain_b16", "tree128k", "sparse64k")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="tree32k")
    ap.add_argument("--out-dtype", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-wide", action="store_true",
                    help="skip the 256-node tree measurement")
    ap.add_argument("--no-paged", action="store_true",
                    help="skip the paged-cache measurement")
    ap.add_argument("--no-selection", action="store_true",
                    help="skip the index-set selection measurement")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the other four workloads")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(json.dumps({"error": "hsv runs on one GPU (no collectives); --gpus must be 1",
                          "n_gpus": args.gpus}))
        log("bench.py: only --gpus 1 is supported: the library runs on one GPU and has no "
            "collectives")
        return 2
    if args.steps < 1 or args.warmup < 0:
        log("bench.py: --steps must be >= 1 and --warmup >= 0")
        return 2

    import torch

    import long_context_tree_verify_amd as hsv

    p_idle = idle_power()  # before this process puts any load on the GPU
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    out_dtype = torch.bfloat16 if args.out_dtype == "bf16" else torch.float32
    inp, call, copies = setup_workload(hsv, dev, args.workload, out_dtype, args.num_splits)
    wl = inp.wl
    bf = inp.is_bf16
    max_ctx = int(inp.ctx_lens.max())

    log(f"bench: {args.workload}: warm-up {args.warmup}, settle >= {SETTLE_MS:.0f} ms, "
        f"then {args.steps} timed steps")
    step, part = measure_step_and_kernel(hsv, call, args.steps, args.warmup, dev)
    us = step["us"]
    kern_us = part["event_us"]

    # Single steps, each between its own pair of HIP events on the stream the
    # call runs on: the spread of the step time, and (labelled cache-assisted)
    # the same with one cache copy reused, so the 256 MB Infinity Cache holds
    # much of it.
    cur = torch.cuda.current_stream(dev)

    def single_steps(copy_of):
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(args.steps)]
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(pairs):
            a.record(cur)
            call(copy_of(j))
            b.record(cur)
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) * 1e3 for a, b in pairs)

    def pct(xs, q):
        return xs[min(len(xs) - 1, int(round(q * (len(xs) - 1))))]

    flushed = single_steps(lambda j: j)
    warm = single_steps(lambda j: 0)

    if args.copy_probe:
        src = torch.empty(2 ** 26, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    nbytes = kv_bytes(inp)
    flops = step_flops(inp)
    traffic = recorded_traffic(wl.name) if inp.kv_idx is None and bf else None
    gbs = nbytes / (us * 1e-6) / 1e9
    kern_gbs = nbytes / (kern_us * 1e-6) / 1e9
    if kern_us > us * 1.02:
        raise AssertionError(f"partial kernel {kern_us:.2f} us exceeds the whole step "
                             f"{us:.2f} us: the timing is not steady")
    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us * 1e-3, 5),
        "us_per_step": round(us, 2),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "desc": wl.description, "batch": wl.batch,
                   "ctx": int(max_ctx), "n_draft": wl.n_draft, "q_heads": wl.n_q_heads,
                   "kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim,
                   "n_sel": wl.n_sel, "out_dtype": args.out_dtype,
                   "kv_read_bytes": nbytes, "flop": flops, "cache_copies": copies},
        "roofline": {"bound": "hbm", "achieved": round(kern_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(kern_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                     "copy-calibrated)",
                     "algorithmic_bytes_per_launch": nbytes,
                     "kernel": kernel_name_of(inp),
                     "kernel_us": round(kern_us, 2),
                     "kernel_share_of_step": round(kern_us / us, 4),
                     "mfma_util": round(flops / (kern_us * 1e-6) / 1e12 /
                                        MFMA_BF16_PEAK_TFLOPS, 4)},
        "step_us_p10_p50_p90": [round(pct(flushed, q), 2) for q in (0.1, 0.5, 0.9)],
        "cache_assisted_step_us_p50": round(pct(warm, 0.5), 2),
        "timing": {"protocol": f"{args.warmup} warm-up steps, graph replays of "
                               f"{args.steps} steps back to back for >= {SETTLE_MS:.0f} ms "
                               f"({step['settle_replays']} replays, {step['settle_ms']} ms), "
                               f"then one timed replay of {args.steps} steps between "
                               f"synchronisations",
                   "wall_us_per_step": round(us, 2),
                   "event_us_per_step": round(step["event_us"], 2),
                   "eager_us_per_step": round(step["eager_us"], 2),
                   "kernel_settle_replays": part["settle_replays"]},
    }
    log("bench: socket power and shader clock under back-to-back partial-kernel launches")
    result["roofline"]["power"] = measure_power(
        lambda j: call(j, hsv.HSV_FLAG_PHASE_PARTIALS), args.steps, dev, p_idle)
    del call
    torch.cuda.empty_cache()
    log("bench: timing a 1 GiB device copy (a plain stream for comparison)")
    hbm = measure_hbm_copy(dev)
    result["hbm_copy"] = hbm
    streams = {"hbm_copy": hbm["gbs"], f"{wl.name}_step": gbs, f"{wl.name}_kernel": kern_gbs}
    if wl.name == "tree32k" and not args.no_others:
        result["workloads"] = {}
        for other in OTHER_WORKLOADS:
            log(f"bench: timing workload {other}")
            res = measure_other_workload(hsv, dev, other, min(args.steps, 200),
                                         args.warmup, out_dtype)
            result["workloads"][other] = res
            if other != "tiny_tree":
                streams[f"{other}_step"] = res["kv_gbs"]
                streams[f"{other}_kernel"] = res["kernel_gbs"]
    if inp.kv_idx is None and bf and wl.head_dim == 128 and not args.no_paged:
        log("bench: timing the paged-cache step")
        result["paged"] = measure_paged(hsv, dev, inp, args.steps, args.warmup, out_dtype)
    if wl.name == "tree32k" and not args.no_paged and not args.no_others:
        log("bench: timing the paged sparse step (sparse64k)")
        result["paged_sparse"] = measure_paged(hsv, dev, workload_inputs("sparse64k"),
                                               min(args.steps, 200), args.warmup, out_dtype)
    if wl.name == "tree32k" and not args.no_wide:
        log("bench: timing the 256-node tree step")
        result["wide_tree"] = measure_wide_tree(hsv, dev, min(args.steps, 100), args.warmup,
                                                out_dtype)
    log("bench: timing the accepted-path cache update")
    result["accept"] = measure_accept(hsv, dev, inp, args.steps)
    if not args.no_selection:
        log("bench: timing the index-set selection")
        result["selection"] = measure_selection(hsv, dev, args.steps, args.warmup)
        result["selection"]["recall"], result["sparse_vs_dense"] = measure_recall(
            hsv, dev, min(args.steps, 100), args.warmup)
        streams["sparse_vs_dense_dense_step"] = result["sparse_vs_dense"]["dense_kv_gbs"]
    # The fastest stream this run reached (a plain copy, or any step or
    # kernel above): the measured ceiling the step's rate is also quoted
    # against.
    best = max(streams, key=streams.get)
    result["best_stream"] = {"what": best, "gbs": round(streams[best], 1)}
    result["pct_best_stream"] = round(100 * gbs / streams[best], 2)
    if not args.no_cpu_baseline:
        log("bench: timing the fp64 oracle on a row sample")
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
