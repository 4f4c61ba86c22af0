"""Calls on several HIP streams at once, each with its own workspace and
outputs, give bit for bit what they give one after another on one stream:
every launch of a call goes to the caller's stream, and calls share no
device state.  (hsv_verify_attn_noalloc shares its scratch on purpose and is
left out.)  The verify workloads cover the 256-row DMA kernel, the
small-group kernel on a ragged dense batch and on a sparse set, and the
fp32 VALU kernel; an index-set selection runs beside them.  Before every
round each call's outputs are overwritten on its own stream, so a call
that wrote nothing cannot pass.
"""

import numpy as np
import pytest

import synth
from util import device_inputs

pytestmark = pytest.mark.gpu

CASES = [
    ("tree32k", (("ctx", (3000, 3000)),)),
    ("chain_b16", (("ctx", (500, 2100)), ("batch", 4))),
    ("sparse64k", (("ctx", (3000, 3000)), ("batch", 2), ("n_sel", 1000), ("n_recent", 200))),
    ("tiny_tree", ()),
]


@pytest.fixture(scope="module")
def hsv(gpu):
    import long_context_tree_verify_amd as m
    return m


def _verify_call(hsv, gpu, name, over):
    """A verify call on preallocated workspace and outputs: (launch, outputs)."""
    import torch
    inp = synth.make_inputs(name, **dict(over))
    dev = device_inputs(inp, gpu)
    sparse = inp.kv_idx is not None
    B, N, Hq, D = inp.q.shape
    max_ctx = int(inp.ctx_lens.max())
    desc = hsv.make_desc(batch=B, n_draft=N, n_q_heads=Hq, n_kv_heads=inp.wl.n_kv_heads,
                         head_dim=D, kv_capacity=inp.k.shape[2], max_ctx=max_ctx,
                         n_sel=inp.kv_idx.shape[2] if sparse else 0,
                         in_dtype=hsv.HSV_BF16 if inp.is_bf16 else hsv.HSV_F32,
                         out_dtype=hsv.HSV_F32)
    ws = torch.empty(max(256, hsv.hsv_verify_workspace_bytes(desc)), dtype=torch.uint8,
                     device=gpu)
    o = torch.empty((B, N, Hq, D), dtype=torch.float32, device=gpu)
    lse = torch.empty((B, N, Hq), dtype=torch.float32, device=gpu)

    def launch(stream):
        kw = dict(max_ctx=max_ctx, o=o, lse=lse, workspace=ws, stream=stream)
        if sparse:
            hsv.hsv_verify_attn_sparse(dev["q"], dev["k"], dev["v"], dev["ctx"], dev["parent"],
                                       None, dev["kv_idx"], **kw)
        else:
            hsv.hsv_verify_attn(dev["q"], dev["k"], dev["v"], dev["ctx"], dev["parent"], **kw)
    return launch, (o, lse)


def _select_call(hsv, gpu):
    import torch
    rng = np.random.Generator(np.random.PCG64(71))
    ctx = np.array([20000, 7000, 19000], np.int32)
    draft, target = synth.importance_maps(rng, ctx, 4, 20000)
    d_t, t_t = torch.from_numpy(draft).to(gpu), torch.from_numpy(target).to(gpu)
    c_t = torch.from_numpy(ctx).to(gpu)
    ws = torch.empty(hsv.hsv_select_workspace_bytes(3, 4, 20000), dtype=torch.uint8, device=gpu)
    idx = torch.empty((3, 4, 4096), dtype=torch.int32, device=gpu)

    def launch(stream):
        hsv.hsv_select_kv_idx(d_t, t_t, c_t, n_sel=4096, n_sink=4, n_recent=512,
                              n_draft_top=1000, kv_idx=idx, workspace=ws, stream=stream)
    return launch, (idx,)


def test_concurrent_streams_match_serial(hsv, gpu):
    import torch
    calls = [_verify_call(hsv, gpu, name, over) for name, over in CASES]
    calls.append(_select_call(hsv, gpu))
    main = torch.cuda.current_stream(gpu)
    for launch, _ in calls:
        launch(main)
    torch.cuda.synchronize()
    ref = [tuple(t.clone() for t in outs) for _, outs in calls]
    streams = [torch.cuda.Stream(gpu) for _ in calls]
    for rep in range(10):
        for (launch, outs), s in zip(calls, streams):
            s.wait_stream(main)
            with torch.cuda.stream(s):
                for t in outs:
                    t.fill_(-7)
                launch(s)
        torch.cuda.synchronize()
        for i, ((_, outs), r) in enumerate(zip(calls, ref)):
            for t, u in zip(outs, r):
                assert torch.equal(t, u), f"round {rep}: call {i} differs from its serial result"
