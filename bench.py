#!/usr/bin/env python3
"""Verify-step benchmark on one MI355X.

One step is one verification-attention call over the 32k-context, 64-node
tree workload (batch 1, 32/8 heads, head_dim 128, bf16): the ancestor mask,
the split prefix attention, the masked tree attention and the log-sum-exp
merge, all in the HIP library.  Inputs are resident in HBM before timing.
Several copies of the KV cache (standing for the caches of successive
layers) are rotated so that a step never finds its cache in the 256 MB
Infinity Cache left over from the previous step.

Prints ONE JSON line (rank 0):
  value = KV-read GB/s of the whole step; ms_per_step = wall time per step;
  roofline = the dominant kernel (prefix/tree partials) timed with HIP events
  on its own stream; cpu_baseline = the fp64 oracle on a bounded row sample.

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
    step_s = t * total / n
    gbs = kv_bytes(inp) / step_s / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {total} (b, node, head) rows of the {wl.name} step, each over "
                      f"its full key set, fp64; {t:.2f} s measured, scaled by {total}/{n}",
            "step_s": round(step_s, 3)}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="tree32k")
    ap.add_argument("--out-dtype", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    stream = torch.cuda.current_stream(dev)

    def call(j, flags=0):
        kw = dict(max_ctx=max_ctx, out_dtype=out_dtype, num_splits=args.num_splits,
                  flags=flags, o=o, lse=lse, workspace=ws, stream=stream)
        c = j % copies
        if kv_idx is None:
            hsv.hsv_verify_attn(q, ks[c], vs[c], ctx, parent, **kw)
        else:
            hsv.hsv_verify_attn_sparse(q, ks[c], vs[c], ctx, parent, None, kv_idx, **kw)

    log(f"bench: {copies} cache copies of {cache_bytes / 2**20:.1f} MiB; warmup {args.warmup}")
    for j in range(args.warmup):
        call(j)
    torch.cuda.synchronize()

    # timed region: K whole steps; the partial-attention phase (the dominant
    # kernel) is bracketed by events on the stream it runs on
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(args.steps):
        ev[j][0].record(stream)
        call(j, hsv.HSV_FLAG_PHASE_PARTIALS)
        ev[j][1].record(stream)
        call(j, hsv.HSV_FLAG_PHASE_MERGE)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / args.steps
    kern_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps

    # the same steps without events, each call both phases (the product call)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for j in range(args.steps):
        call(j)
    torch.cuda.synchronize()
    plain_ms = (time.perf_counter() - t2) * 1e3 / args.steps
    ms = min(wall_ms, plain_ms)

    if args.copy_probe:
        src = torch.empty(2 ** 26, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    nbytes = kv_bytes(inp)
    flops = step_flops(inp)
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
                     "traffic": None, "kernel": "attention partials (prefix splits + tree)",
                     "kernel_us": round(kern_ms * 1e3, 2),
                     "mfma_util": round(flops / (kern_ms * 1e-3) / 1e12 /
                                        MFMA_BF16_PEAK_TFLOPS, 4)},
        "timing": {"wall_ms_with_phase_events": round(wall_ms, 5),
                   "wall_ms_plain": round(plain_ms, 5)},
    }
    if not args.no_cpu_baseline:
        log("bench: timing the fp64 oracle on a row sample")
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
