"""HSV_FLAG_VALIDATE over random shapes (failure handling forced from the
host; every kernel exits normally).  On valid inputs a validating call
returns the results of the plain call bit for bit; each corrupted input the
check covers -- a context past max_ctx, a negative context, a parent at or
after its node or below -1, an index-set entry at or past the context or out
of order -- returns HSV_ERR_DEVICE_CHECK.  The check kernel only compares
these values, so the corrupted calls read nothing out of range.  Shapes are
the first cases of the random shape sweep that pass parent arrays.
"""

import numpy as np
import pytest

import synth
from test_gpu_random import draw_case
from util import device_inputs

pytestmark = pytest.mark.gpu

CASES = [k for k in range(40) if draw_case(k)[1]["mask"] is None][:30]


@pytest.fixture(scope="module")
def hsv(gpu):
    import long_context_tree_verify_amd as m
    return m


def _call(hsv, inp, dev, max_ctx, ctx=None, parent=None, kv_idx=None, flags=0):
    import torch
    kw = dict(max_ctx=max_ctx, out_dtype=torch.float32, flags=flags)
    ctx = dev["ctx"] if ctx is None else ctx
    parent = dev["parent"] if parent is None else parent
    if inp.kv_idx is not None:
        kv_idx = dev["kv_idx"] if kv_idx is None else kv_idx
        return hsv.hsv_verify_attn_sparse(dev["q"], dev["k"], dev["v"], ctx, parent, None,
                                          kv_idx, **kw)
    return hsv.hsv_verify_attn(dev["q"], dev["k"], dev["v"], ctx, parent, None, **kw)


@pytest.mark.parametrize("k", CASES)
def test_validate_random(hsv, gpu, k):
    import torch
    over, run, seed = draw_case(k)
    base = "tree32k" if over["dtype"] == "bf16" else "tiny_tree"
    inp = synth.make_inputs(base, seed=seed, **over)
    dev = device_inputs(inp, gpu)
    max_ctx = int(inp.ctx_lens.max())
    o1, l1 = _call(hsv, inp, dev, max_ctx)
    o2, l2 = _call(hsv, inp, dev, max_ctx, flags=hsv.HSV_FLAG_VALIDATE)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), f"case {k}: validated result differs"

    rng = np.random.default_rng(seed)
    B, N = inp.wl.batch, inp.wl.n_draft
    b = int(rng.integers(B))
    bad = []
    for c in (max_ctx + 1, -1):
        ctx = dev["ctx"].clone()
        ctx[b] = c
        bad.append((f"context {c}", dict(ctx=ctx)))
    if N > 1:
        i = int(rng.integers(1, N))
        for p in (i, -2):
            par = dev["parent"].clone()
            par[b, i] = p
            bad.append((f"parent[{i}] = {p}", dict(parent=par)))
    if inp.kv_idx is not None:
        g = int(rng.integers(inp.wl.n_kv_heads))
        c_b = int(inp.ctx_lens[b])
        row = inp.kv_idx[b, g]
        n_valid = int((row >= 0).sum())
        if n_valid:
            idx = dev["kv_idx"].clone()
            idx[b, g, n_valid - 1] = c_b                  # at the context: outside the prefix
            bad.append(("index at the context", dict(kv_idx=idx)))
        if n_valid > 1:
            idx = dev["kv_idx"].clone()
            idx[b, g, 1] = idx[b, g, 0]                   # not strictly increasing
            bad.append(("repeated index", dict(kv_idx=idx)))
    for what, kw in bad:
        with pytest.raises(hsv.HsvError) as e:
            _call(hsv, inp, dev, max_ctx, flags=hsv.HSV_FLAG_VALIDATE, **kw)
        assert e.value.code == hsv.HSV_ERR_DEVICE_CHECK, f"case {k}: {what}"
    torch.cuda.synchronize()
