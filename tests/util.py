"""Helpers shared by the GPU tests: moving seeded inputs to the device,
running the C-ABI path, and the parity bar."""

from __future__ import annotations

import functools
import sys

import numpy as np

import synth

# Parity bar for bf16 inputs with fp32 accumulation: max-abs error on O and
# max relative error on the row LSE, |lse - ref| / max(|ref|, 1).
O_ATOL = 1e-2
LSE_RTOL = 1e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, bf16: bool, device):
    import torch
    if bf16 and a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def device_inputs(inp: synth.VerifyInputs, device):
    import torch
    bf = inp.is_bf16
    out = dict(q=to_dev(inp.q, bf, device), k=to_dev(inp.k, bf, device),
               v=to_dev(inp.v, bf, device),
               ctx=torch.from_numpy(inp.ctx_lens).to(device),
               parent=torch.from_numpy(inp.parent).to(device))
    out["kv_idx"] = None if inp.kv_idx is None else torch.from_numpy(inp.kv_idx).to(device)
    return out


def run_hip(hsv, inp: synth.VerifyInputs, dev, *, sparse=None, out_dtype=None, **kw):
    import torch
    if sparse is None:
        sparse = inp.kv_idx is not None
    out_dtype = out_dtype or torch.float32
    max_ctx = int(inp.ctx_lens.max())
    if sparse:
        o, lse = hsv.hsv_verify_attn_sparse(dev["q"], dev["k"], dev["v"], dev["ctx"],
                                            kw.pop("parent", dev["parent"]), kw.pop("anc", None),
                                            dev["kv_idx"], max_ctx=max_ctx, out_dtype=out_dtype,
                                            **kw)
    else:
        o, lse = hsv.hsv_verify_attn(dev["q"], dev["k"], dev["v"], dev["ctx"],
                                     kw.pop("parent", dev["parent"]), kw.pop("anc", None),
                                     max_ctx=max_ctx, out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return o, lse


def errors(o_gpu, lse_gpu, o_ref, lse_ref):
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    o_err = float(np.max(np.abs(o_gpu - o_ref))) if o_ref.size else 0.0
    fin = np.isfinite(lse_ref)
    assert (np.isneginf(lse_gpu) == np.isneginf(lse_ref)).all(), "empty-row pattern differs"
    denom = np.maximum(np.abs(lse_ref[fin]), 1.0)
    l_err = float(np.max(np.abs(lse_gpu[fin] - lse_ref[fin]) / denom)) if fin.any() else 0.0
    return o_err, l_err


def assert_parity(o_gpu, lse_gpu, o_ref, lse_ref, what="", o_atol=O_ATOL, lse_rtol=LSE_RTOL):
    assert np.isfinite(np.asarray(o_gpu)).all(), f"{what}: non-finite output"
    o_err, l_err = errors(o_gpu, lse_gpu, o_ref, lse_ref)
    log(f"  parity {what}: max|dO|={o_err:.3e} max rel dLSE={l_err:.3e}")
    assert o_err <= o_atol, f"{what}: O error {o_err} > {o_atol}"
    assert l_err <= lse_rtol, f"{what}: LSE error {l_err} > {lse_rtol}"
    return o_err, l_err


@functools.lru_cache(maxsize=4)
def cached_inputs(name: str, overrides: tuple = (), poison: bool = False):
    return synth.make_inputs(name, poison_unselected=poison, **dict(overrides))


def assert_all_rows(o_gpu, lse_gpu, inp: synth.VerifyInputs, what: str, o_ref=None, lse_ref=None,
                    **oracle_kw):
    """Every output row of a full-size call against the fp64 oracle, element
    by element (the oracle runs on every host core over all B*N*Hq rows).
    Logs the all-row maximum errors."""
    import time

    import oracle
    if o_ref is None:
        t = time.perf_counter()
        kw = dict(parent=inp.parent, kv_idx=inp.kv_idx)
        kw.update(oracle_kw)
        o_ref, lse_ref = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens,
                                            bf16=inp.is_bf16, **kw)
        log(f"  {what}: oracle over all {lse_ref.size} rows in "
            f"{time.perf_counter() - t:.1f} s on {oracle.num_threads()} threads")
    o_gpu = np.asarray(o_gpu)
    lse_gpu = np.asarray(lse_gpu)
    assert o_gpu.shape == o_ref.shape and lse_gpu.shape == lse_ref.shape
    o_err, l_err = assert_parity(o_gpu, lse_gpu, o_ref, lse_ref, f"{what}, all rows")
    return o_err, l_err


@functools.lru_cache(maxsize=2)
def oracle_full(name: str, overrides: tuple = ()):
    """The oracle's output over every row of a workload (cached: several
    full-size tests share the 32k-context tree)."""
    import oracle
    inp = cached_inputs(name, overrides)
    return oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent,
                              kv_idx=inp.kv_idx, bf16=inp.is_bf16)
