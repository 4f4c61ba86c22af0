"""Captured HIP graphs of the newer entry points, replayed several times with
eager work and synchronisations in between: every replay must give the eager
result bit for bit (the benchmark times graph replays).  Covers the
two-launch selection (workspace lists between the launches), the paged
attention, the 256-node tree (masks built in the workspace), the
accepted-path update (two launches; the lengths restored before each) and
the entry point without a workspace (its scratch is the library's own)."""

import numpy as np
import pytest

import synth
from util import cached_inputs, device_inputs, log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hsv(gpu):
    import long_context_tree_verify_amd as m
    return m


def _replay(gpu, call, outputs, reset=None, reps=3):
    """Capture call(), replay `reps` times (outputs poisoned, an eager call
    of torch work and a sync between replays); return each replay's outputs."""
    import torch
    side = torch.cuda.Stream(gpu)
    g = torch.cuda.CUDAGraph()
    if reset:
        reset()
    with torch.cuda.graph(g, stream=side):
        call()
    got = []
    for _ in range(reps):
        for t in outputs:
            t.fill_(-1 if not t.is_floating_point() else float("nan"))
        if reset:
            reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got.append([t.clone() for t in outputs])
        _ = torch.ones(1024, device=gpu).sum()   # eager work between replays
        torch.cuda.synchronize()
    return got


def test_selection_graph(hsv, gpu):
    import torch
    rng = np.random.Generator(np.random.PCG64(130))
    ctx_np = np.array([65536, 40000, 1000, 70], np.int32)
    draft_np, target_np = synth.importance_maps(rng, ctx_np, 2, 65536)
    draft, target = torch.from_numpy(draft_np).to(gpu), torch.from_numpy(target_np).to(gpu)
    ctx = torch.from_numpy(ctx_np).to(gpu)
    kw = dict(n_sel=4096, n_sink=4, n_recent=512, n_draft_top=1790)
    ref = hsv.hsv_select_kv_idx(draft, target, ctx, **kw).clone()
    out = torch.empty_like(ref)
    ws = torch.empty(hsv.hsv_select_workspace_bytes(4, 2, 65536), dtype=torch.uint8, device=gpu)
    for i, (o,) in enumerate(_replay(gpu, lambda: hsv.hsv_select_kv_idx(
            draft, target, ctx, kv_idx=out, workspace=ws, **kw), [out])):
        assert torch.equal(o, ref), f"selection replay {i}"
    log("  selection: 3 replays identical")


def test_paged_graph(hsv, gpu):
    import torch
    inp = cached_inputs("tree32k", (("ctx", (3000, 3000)),))
    rng = np.random.Generator(np.random.PCG64(131))
    S = inp.k.shape[2]
    cap = -(-S // 64) * 64
    pad = ((0, 0), (0, 0), (0, cap - S), (0, 0))
    kp, vp, table = synth.to_paged(np.pad(inp.k, pad), np.pad(inp.v, pad), 64, rng)
    args = (to_dev(inp.q, True, gpu), to_dev(kp, True, gpu), to_dev(vp, True, gpu),
            torch.from_numpy(table).to(gpu), torch.from_numpy(inp.ctx_lens).to(gpu),
            torch.from_numpy(inp.parent).to(gpu))
    max_ctx = int(inp.ctx_lens.max())
    o_ref, l_ref = hsv.hsv_verify_attn_paged(*args, max_ctx=max_ctx)
    o, lse = torch.empty_like(o_ref), torch.empty_like(l_ref)
    desc = hsv.make_desc(batch=1, n_draft=64, n_q_heads=32, n_kv_heads=8, head_dim=128,
                         kv_capacity=cap, max_ctx=max_ctx, block_size=64)
    ws = torch.empty(hsv.hsv_verify_workspace_bytes(desc), dtype=torch.uint8, device=gpu)
    for i, (a, b) in enumerate(_replay(gpu, lambda: hsv.hsv_verify_attn_paged(
            *args, max_ctx=max_ctx, o=o, lse=lse, workspace=ws), [o, lse])):
        assert torch.equal(a, o_ref) and torch.equal(b, l_ref), f"paged replay {i}"
    log("  paged: 3 replays identical")


def test_wide_tree_graph(hsv, gpu):
    import torch
    inp = cached_inputs("tree32k", (("ctx", (2000, 2000)), ("n_draft", 256), ("max_depth", 16)))
    dev = device_inputs(inp, gpu)
    max_ctx = int(inp.ctx_lens.max())
    o_ref, l_ref = hsv.hsv_verify_attn(dev["q"], dev["k"], dev["v"], dev["ctx"], dev["parent"],
                                       max_ctx=max_ctx)
    o, lse = torch.empty_like(o_ref), torch.empty_like(l_ref)
    desc = hsv.make_desc(batch=1, n_draft=256, n_q_heads=32, n_kv_heads=8, head_dim=128,
                         kv_capacity=inp.k.shape[2], max_ctx=max_ctx)
    ws = torch.empty(hsv.hsv_verify_workspace_bytes(desc), dtype=torch.uint8, device=gpu)
    for i, (a, b) in enumerate(_replay(gpu, lambda: hsv.hsv_verify_attn(
            dev["q"], dev["k"], dev["v"], dev["ctx"], dev["parent"], max_ctx=max_ctx, o=o,
            lse=lse, workspace=ws), [o, lse])):
        assert torch.equal(a, o_ref) and torch.equal(b, l_ref), f"wide tree replay {i}"
    log("  256-node tree: 3 replays identical")


def test_accept_graph(hsv, gpu):
    import torch
    rng = np.random.Generator(np.random.PCG64(132))
    B, H, N, S, D = 4, 8, 64, 2000, 128
    par = np.stack([synth.random_tree_parents(rng, N, 6, 4) for _ in range(B)]).astype(np.int32)
    ctx0 = torch.from_numpy(rng.integers(100, S - N, B).astype(np.int32)).to(gpu)
    node = torch.from_numpy(rng.integers(0, N, B).astype(np.int32)).to(gpu)
    parent = torch.from_numpy(par).to(gpu)
    k0 = torch.randn((B, H, S, D), device=gpu).to(torch.bfloat16)
    v0 = torch.randn((B, H, S, D), device=gpu).to(torch.bfloat16)
    k, v, ctx = k0.clone(), v0.clone(), ctx0.clone()
    hsv.hsv_accept_path(k, v, ctx, parent, node)
    torch.cuda.synchronize()
    k_ref, v_ref, c_ref = k.clone(), v.clone(), ctx.clone()

    def reset():
        k.copy_(k0)
        v.copy_(v0)
        ctx.copy_(ctx0)

    # the update is in place: capture it, then per replay restore the inputs
    side = torch.cuda.Stream(gpu)
    g = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        hsv.hsv_accept_path(k, v, ctx, parent, node)
    for rep in range(3):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(k, k_ref) and torch.equal(v, v_ref) and torch.equal(ctx, c_ref), \
            f"accept replay {rep}"
        _ = torch.ones(1024, device=gpu).sum()
        torch.cuda.synchronize()
    log("  accepted-path update: 3 replays identical")


def test_noalloc_graph(hsv, gpu):
    # the call callers under graph capture use: its scratch is a library-owned
    # per-GPU array, looked up by the first (eager) call
    import torch
    inp = cached_inputs("tree32k", (("ctx", (4000, 4000)),))
    dev = device_inputs(inp, gpu)
    mc = int(inp.ctx_lens.max())
    o_ref, l_ref = hsv.hsv_verify_attn(dev["q"], dev["k"], dev["v"], dev["ctx"], dev["parent"],
                                       max_ctx=mc)
    o, lse = torch.empty_like(o_ref), torch.empty_like(l_ref)
    call = lambda: hsv.hsv_verify_attn_noalloc(dev["q"], dev["k"], dev["v"], dev["ctx"],
                                               dev["parent"], max_ctx=mc, o=o, lse=lse)
    call()
    torch.cuda.synchronize()
    for i, (o_g, l_g) in enumerate(_replay(gpu, call, [o, lse])):
        assert torch.equal(o_g, o_ref) and torch.equal(l_g, l_ref), f"replay {i} differs"
    log("  no-alloc call in a graph: every replay identical to the eager workspace call")
