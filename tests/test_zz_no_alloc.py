"""hsv_verify_attn_noalloc, the workspace-free variant of hsv_verify_attn
(its scratch is a library-owned array on each GPU): through the C ABI it
gives the workspace entry point's result bit for bit, on two calls in a row
whose second input is smaller than the first, and it rejects descriptors
whose scratch would not fit."""

import ctypes

import numpy as np
import pytest

from util import cached_inputs, device_inputs, log, run_hip


@pytest.fixture(scope="module")
def hsv():
    import long_context_tree_verify_amd as m
    return m


def test_noalloc_rejects_what_does_not_fit(hsv):
    # host-side checks only: these return before any device work
    big = hsv.make_desc(batch=64, n_draft=64, n_q_heads=32, n_kv_heads=8, head_dim=128,
                        kv_capacity=32832, max_ctx=32768)
    n = hsv.hsv_verify_workspace_bytes(big)
    assert n > hsv.HSV_NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: the call fails first
    code = hsv.lib.hsv_verify_attn_noalloc(ctypes.byref(big), fake, fake, fake, fake, fake, None,
                                           fake, fake, None)
    assert code == hsv.HSV_ERR_WORKSPACE
    sparse = hsv.make_desc(batch=1, n_draft=8, n_q_heads=32, n_kv_heads=8, head_dim=128,
                           kv_capacity=4096, max_ctx=4000, n_sel=512)
    code = hsv.lib.hsv_verify_attn_noalloc(ctypes.byref(sparse), fake, fake, fake, fake, fake,
                                           None, fake, fake, None)
    assert code == hsv.HSV_ERR_SHAPE
    assert hsv.lib.hsv_verify_attn_noalloc(None, fake, fake, fake, fake, fake, None, fake, fake,
                                           None) == hsv.HSV_ERR_NULL


# the first call's plan fills most of the scratch (32 splits x 8 KV heads of
# 256 rows); the second is a smaller ragged batch of 8-token chains
CALLS = [
    ("tree32k", (("ctx", (32768, 32768)),)),
    ("chain_b16", (("ctx", (700, 2100)), ("batch", 3))),
]


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point(hsv, gpu):
    import torch
    for out_dtype in (torch.float32, torch.bfloat16):
        for name, over in CALLS:
            log(f"noalloc: {name} {dict(over)} out {out_dtype}")
            inp = cached_inputs(name, over)
            dev = device_inputs(inp, gpu)
            o_ref, l_ref = run_hip(hsv, inp, dev, out_dtype=out_dtype)
            o = torch.full_like(o_ref, float("nan"))
            lse = torch.full_like(l_ref, float("nan"))
            hsv.hsv_verify_attn_noalloc(dev["q"], dev["k"], dev["v"], dev["ctx"], dev["parent"],
                                        max_ctx=int(inp.ctx_lens.max()), o=o, lse=lse)
            torch.cuda.synchronize()
            assert torch.equal(o, o_ref), f"{name}: o differs"
            assert torch.equal(lse, l_ref), f"{name}: lse differs"
            assert np.isfinite(o.float().cpu().numpy()).all()
            del dev
    torch.cuda.empty_cache()
