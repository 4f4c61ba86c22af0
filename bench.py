#!/usr/bin/env python3
"""Verify-step benchmark on one MI355X.

One step is one verification-attention call over the 32k-context, 64-node
tree workload (batch 1, 32/8 heads, head_dim 128, bf16): the ancestor mask,
the split prefix attention, the masked tree attention and the log-sum-exp
merge, all in the HIP library.  Inputs are resident in HBM before timing.
Several copies of the KV cache (standing for the caches of successive
layers) are rotated so that a step never finds its cache in the 256 MB
Infinity Cache left over from the previous step.

The K timed steps are issued two ways: one Python call per step, and replayed
from one captured HIP graph (no host work between kernels); each is K whole
steps between synchronisations, and the faster is the step time.

Prints ONE JSON line (rank 0):
  value = KV-read GB/s of the whole step; ms_per_step = time per step;
  roofline = the dominant kernel (the attention partials), its average
  duration from HIP events around five replays of a graph of K back-to-back
  launches on its stream; traffic = its HBM bytes per launch from the committed rocprofv3
  counter summary, when that summary was taken on the current kernel source;
  cpu_baseline = the fp64 oracle timed on the host cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

from __future__ import annotations

import argparse
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
PART_REPLAYS = 5  # timed replays of the graph of partial-kernel launches
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
    """Average duration of one hsv_select_kv_idx launch (HIP events around a
    graph of `steps` launches on the stream they run on) and the algorithmic
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
    for _ in range(warmup):
        hsv.hsv_select_kv_idx(draft, target, ctx, **kw)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for _ in range(steps):
            hsv.hsv_select_kv_idx(draft, target, ctx, **kw)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    n_cand = L - sh["n_sink"] - sh["n_recent"]
    nbytes = B * H * (2 * 4 * n_cand + 4 * sh["n_sel"])
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"kernel": "select_filter (every CU streams the maps) + select_lists (exact radix "
                      "select per sequence and KV head)",
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


def measure_hbm_read(dev, reps: int = 5):
    """The HBM rate a plain read-only stream of 16-byte loads reaches in this
    run (the probe kernel of libhsv_probe.so over 2 GiB, HIP events on its
    stream): the measured ceiling for a kernel that mostly reads."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "long_context_tree_verify_amd", "libhsv_probe.so")
    if not os.path.exists(path):
        log(f"bench: {path} is not built; no read-only ceiling in this run")
        return None
    lib = ctypes.CDLL(path)
    lib.hsv_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                   ctypes.c_void_p]
    lib.hsv_probe_read.restype = ctypes.c_int
    lib.hsv_probe_blocks.restype = ctypes.c_int
    nbytes = 2 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(lib.hsv_probe_blocks(), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def launch():
        rc = lib.hsv_probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                ctypes.c_void_p(sink.data_ptr()),
                                ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hsv_probe_read failed: {rc}")

    launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del buf, sink
    torch.cuda.empty_cache()
    return {"what": "read-only stream of 16-byte loads (libhsv_probe), 2 GiB per pass",
            "bytes_read": nbytes, "us": round(us, 1), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1)}


def measure_paged(hsv, dev, inp, steps: int, out_dtype):
    """The same verify step over a paged copy of the cache (pool blocks of
    PAGED_BLOCK tokens in seeded random order, a block table), K steps in a
    graph with the pool copies rotated like the contiguous measurement
    (HIP events on the capture stream bracket the replay) and K eager calls;
    like the contiguous step, the faster of the two is the step time."""
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
    pool_bytes = 2 * k0.numel() * k0.element_size()
    copies = max(1, math.ceil(2 * INFINITY_CACHE_BYTES / pool_bytes) + 1) if pool_bytes < \
        2 * INFINITY_CACHE_BYTES else 1
    ks, vs = [k0] + [k0.clone() for _ in range(copies - 1)], [v0] + [v0.clone()
                                                                      for _ in range(copies - 1)]
    q = torch.from_numpy(inp.q.view(np.int16)).view(torch.bfloat16).to(dev)
    tab = torch.from_numpy(table).to(dev)
    ctx = torch.from_numpy(inp.ctx_lens).to(dev)
    parent = torch.from_numpy(inp.parent).to(dev)
    B, N, Hq, D = q.shape
    o = torch.empty((B, N, Hq, D), dtype=out_dtype, device=dev)
    lse = torch.empty((B, N, Hq), dtype=torch.float32, device=dev)
    max_ctx = int(inp.ctx_lens.max())
    desc = hsv.make_desc(batch=B, n_draft=N, n_q_heads=Hq, n_kv_heads=wl.n_kv_heads,
                         head_dim=D, kv_capacity=cap, max_ctx=max_ctx, in_dtype=hsv.HSV_BF16,
                         out_dtype=hsv.HSV_BF16 if out_dtype == torch.bfloat16 else hsv.HSV_F32,
                         block_size=bs)
    ws = torch.empty(hsv.hsv_verify_workspace_bytes(desc), dtype=torch.uint8, device=dev)

    def call(j):
        hsv.hsv_verify_attn_paged(q, ks[j % copies], vs[j % copies], tab, ctx, parent,
                                  max_ctx=max_ctx, out_dtype=out_dtype, o=o, lse=lse,
                                  workspace=ws, stream=None)

    for j in range(3):
        call(j)
    side = torch.cuda.Stream(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for j in range(steps):
            call(j)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(side):
        e0.record()
        g.replay()
        e1.record()
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / steps
    eager = eager_us(call, steps)
    us = min(graph_us, eager)
    nbytes = kv_bytes(inp)
    return {"entry": "hsv_verify_attn_paged", "block_size": bs,
            "workload": f"{wl.name}, pool blocks in random order, {copies} pool copies",
            "us_per_step": round(us, 2), "graph_us_per_step": round(graph_us, 2),
            "eager_us_per_step": round(eager, 2), "kv_read_bytes": nbytes,
            "achieved": round(nbytes / (us * 1e-6) / 1e9, 2), "unit": "GB/s"}


def measure_recall(hsv, dev, steps: int):
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
    sparse step over the selected sets, each K steps in a graph timed with HIP
    events on the capture stream.  Three copies of K and V are rotated, so the
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
        for j in range(3):
            fn(j)
        side = torch.cuda.Stream(dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for j in range(steps):
                fn(j)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(side):
            e0.record()
            g.replay()
            e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

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


def measure_wide_tree(hsv, dev, steps: int, out_dtype):
    """The 32k-context step with a 256-node draft tree (masks of four 64-bit
    words, 1024 grouped rows per KV head): whole steps in a graph (HIP events
    on the capture stream) and K eager calls, the faster of the two.  At 1024 rows the step does 4x the MFMA work per
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

    for j in range(3):
        call(j)
    side = torch.cuda.Stream(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for j in range(steps):
            call(j)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(side):
        e0.record()
        g.replay()
        e1.record()
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / steps
    eager = eager_us(call, steps)
    us = min(graph_us, eager)
    nbytes, flops = kv_bytes(inp), step_flops(inp)
    return {"workload": f"tree32k with a 256-node tree (depth <= 16, branching <= 4), "
                        f"{wl.group * N} grouped rows per KV head",
            "us_per_step": round(us, 2), "graph_us_per_step": round(graph_us, 2),
            "eager_us_per_step": round(eager, 2), "kv_read_bytes": nbytes, "flop": flops,
            "kv_gbs": round(nbytes / (us * 1e-6) / 1e9, 2),
            "tflops": round(flops / (us * 1e-6) / 1e12, 1),
            "mfma_util": round(flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
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
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        log("bench.py: only --gpus 1 is supported (single-GPU build; no collectives)")
        return 2

    import numpy as np
    import torch

    import synth
    import long_context_tree_verify_amd as hsv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"bench: generating workload {args.workload}")
    inp = synth.make_inputs(args.workload)
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
    cache_bytes = 2 * k0.numel() * k0.element_size()
    copies = max(1, math.ceil(2 * INFINITY_CACHE_BYTES / cache_bytes) + 1) if cache_bytes < \
        2 * INFINITY_CACHE_BYTES else 1
    ks, vs = [k0], [v0]
    for _ in range(copies - 1):
        ks.append(k0.clone())
        vs.append(v0.clone())
    out_dtype = torch.bfloat16 if args.out_dtype == "bf16" else torch.float32
    B, N, Hq, D = q.shape
    o = torch.empty((B, N, Hq, D), dtype=out_dtype, device=dev)
    lse = torch.empty((B, N, Hq), dtype=torch.float32, device=dev)
    max_ctx = int(inp.ctx_lens.max())
    desc = hsv.make_desc(batch=B, n_draft=N, n_q_heads=Hq, n_kv_heads=wl.n_kv_heads,
                         head_dim=D, kv_capacity=k0.shape[2], max_ctx=max_ctx,
                         n_sel=0 if kv_idx is None else kv_idx.shape[2],
                         in_dtype=hsv.HSV_BF16 if bf else hsv.HSV_F32,
                         out_dtype=hsv.HSV_BF16 if out_dtype == torch.bfloat16 else hsv.HSV_F32,
                         num_splits=args.num_splits)
    ws = torch.empty(hsv.hsv_verify_workspace_bytes(desc), dtype=torch.uint8, device=dev)

    def call(j, flags=0):
        # stream=None: torch's current stream (the capture stream inside a graph)
        kw = dict(max_ctx=max_ctx, out_dtype=out_dtype, num_splits=args.num_splits,
                  flags=flags, o=o, lse=lse, workspace=ws, stream=None)
        c = j % copies
        if kv_idx is None:
            hsv.hsv_verify_attn(q, ks[c], vs[c], ctx, parent, **kw)
        else:
            hsv.hsv_verify_attn_sparse(q, ks[c], vs[c], ctx, parent, None, kv_idx, **kw)

    log(f"bench: {copies} cache copies of {cache_bytes / 2**20:.1f} MiB; warmup {args.warmup}")
    for j in range(args.warmup):
        call(j)
    torch.cuda.synchronize()

    # K steps issued one Python call at a time (reported alongside)
    t2 = time.perf_counter()
    for j in range(args.steps):
        call(j)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t2) * 1e3 / args.steps

    # The K timed steps as one captured graph (steps j = 0..K-1, cache copy
    # j % copies), replayed once untimed, then once timed.
    side = torch.cuda.Stream(dev)
    g_step = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_step, stream=side):
        for j in range(args.steps):
            call(j)
    g_step.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    g_step.replay()
    ev1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    graph_ms = ev0.elapsed_time(ev1) / args.steps
    # Both are whole-job times of the same K steps; report the faster issue mode.
    ms = min(wall_ms, eager_ms)

    # The dominant kernel alone: K back-to-back launches of the partial phase
    # in one graph, replayed once untimed and then PART_REPLAYS times, each
    # replay bracketed by HIP events on the stream it runs on.  The duration
    # is the mean over all timed launches: the chip's clock moves by about
    # 10 % over the first few milliseconds of sustained load, so one replay
    # alone would say more about where the clock stood than about the kernel.
    g_part = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_part, stream=side):
        for j in range(args.steps):
            call(j, hsv.HSV_FLAG_PHASE_PARTIALS)
    g_part.replay()
    torch.cuda.synchronize()
    part_ms = []
    for _ in range(PART_REPLAYS):
        ek0, ek1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ek0.record()
        g_part.replay()
        ek1.record()
        torch.cuda.synchronize()
        part_ms.append(ek0.elapsed_time(ek1) / args.steps)
    kern_ms = sum(part_ms) / len(part_ms)

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
    traffic = recorded_traffic(wl.name) if kv_idx is None and bf else None
    rows = wl.group * wl.n_draft
    if not bf:
        kernel_name = "attn_partial_valu"
    elif kv_idx is None and wl.head_dim == 128 and rows > 128:
        kernel_name = "attn_partial_dma (prefix + draft rows, split along keys)"
    elif wl.head_dim == 128 and rows <= 32:
        kernel_name = ("attn_partial_dma_small<sparse> (index set + draft rows, per-wave DMA)"
                       if kv_idx is not None else
                       "attn_partial_dma_small<dense> (prefix + draft rows, per-wave DMA)")
    else:
        kernel_name = "attn_partial_mfma (prefix or index-set splits, draft slot)"
    gbs = nbytes / (ms * 1e-3) / 1e9
    kern_gbs = nbytes / (kern_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 2),
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
                     "kernel": kernel_name,
                     "kernel_us": round(kern_ms * 1e3, 2),
                     "kernel_us_per_replay": [round(x * 1e3, 2) for x in part_ms],
                     "mfma_util": round(flops / (kern_ms * 1e-3) / 1e12 /
                                        MFMA_BF16_PEAK_TFLOPS, 4)},
        "step_us_p10_p50_p90": [round(pct(flushed, q), 2) for q in (0.1, 0.5, 0.9)],
        "cache_assisted_step_us_p50": round(pct(warm, 0.5), 2),
        "timing": {"graph_ms_per_step_wall": round(wall_ms, 5),
                   "graph_ms_per_step_events": round(graph_ms, 5),
                   "eager_ms_per_step": round(eager_ms, 5)},
    }
    log("bench: timing a plain read-only stream and a 1 GiB copy (measured HBM ceilings)")
    hbm_read = measure_hbm_read(dev)
    hbm = measure_hbm_copy(dev)
    result["hbm_read"] = hbm_read
    result["hbm_copy"] = hbm
    ceiling = hbm_read["gbs"] if hbm_read else hbm["gbs"]
    result["pct_measured_hbm"] = round(100 * gbs / ceiling, 2)
    result["roofline"]["frac_of_measured_read"] = (round(kern_gbs / hbm_read["gbs"], 4)
                                                   if hbm_read else None)
    result["roofline"]["frac_of_measured_copy"] = round(kern_gbs / hbm["gbs"], 4)
    if inp.kv_idx is None and bf and wl.head_dim == 128 and not args.no_paged:
        log("bench: timing the paged-cache step")
        result["paged"] = measure_paged(hsv, dev, inp, args.steps, out_dtype)
    if wl.name == "tree32k" and not args.no_wide:
        log("bench: timing the 256-node tree step")
        result["wide_tree"] = measure_wide_tree(hsv, dev, args.steps, out_dtype)
    log("bench: timing the accepted-path cache update")
    result["accept"] = measure_accept(hsv, dev, inp, args.steps)
    if not args.no_selection:
        log("bench: timing the index-set selection")
        result["selection"] = measure_selection(hsv, dev, args.steps, args.warmup)
        result["selection"]["recall"], result["sparse_vs_dense"] = measure_recall(
            hsv, dev, args.steps)
    if not args.no_cpu_baseline:
        log("bench: timing the fp64 oracle on a row sample")
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
