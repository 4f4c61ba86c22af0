"""A seeded random sweep over the shapes the verify calls accept, each case
against the fp64 oracle on every output row.

The hand-picked parity cases cover each kernel at its edges; this sweep
draws combinations nobody picked -- batch, draft nodes, query and KV heads,
head dim, input and output dtype, dense or sparse, tree shape, ragged
contexts, split count, partial format -- so that a planner decision or a
work mapping that only fails on some pairing is still met.  Every draw is
fixed by its case number; sizes are kept where the oracle takes about a
second.  (Random trees branch at most 4 ways, so a depth of at least 4 holds
256 nodes.)  Dense cases whose workspace fits the library's scratch also run
hsv_verify_attn_noalloc, which must give identical results.  A case with
bf16 output is checked through the same call's fp32 output (parity against
the oracle), and its bf16 output must be that output's round to nearest
even, bit for bit.
"""

import numpy as np
import pytest

import oracle
import synth
from util import assert_parity, device_inputs, log, run_hip

N_CASES = 400
ROW_KEY_BUDGET = 2e7   # (output rows) x (keys per row) the oracle is given


@pytest.fixture(scope="module")
def hsv(gpu):
    import long_context_tree_verify_amd as m
    return m


def draw_case(k: int):
    rng = np.random.default_rng(1000 + k)
    pick = lambda xs: xs[int(rng.integers(len(xs)))]
    dtype = "bf16" if rng.random() < 0.75 else "f32"
    D = pick([64, 128])
    Hkv = pick([1, 2, 4, 8])
    G = pick([1, 2, 4, 8])
    N = pick([1, 2, 5, 8, 16, 31, 64, 65, 100, 256])
    B = pick([1, 2, 3, 5, 8, 17])
    tree = pick(["uniform", "tree", "chain"])
    hi = pick([0, 1, 33, 100, 700, 3000])
    lo = int(rng.integers(0, hi + 1)) if rng.random() < 0.7 else hi
    n_sel = 0
    if dtype == "bf16" and rng.random() < 0.3:
        n_sel = pick([1, 7, 64, 300])
        hi = max(hi, n_sel + 10)
        lo = max(lo, n_sel)
    # keep the oracle's work bounded
    while B * N * G * Hkv * (hi + N) > ROW_KEY_BUDGET and (B > 1 or hi > n_sel + 10):
        if B > 1:
            B = max(1, B // 2)
        else:
            hi = max(n_sel + 10, hi // 2)
            lo = min(lo, hi)
    over = dict(batch=B, n_draft=N, n_q_heads=G * Hkv, n_kv_heads=Hkv, head_dim=D,
                ctx=(lo, hi), dtype=dtype, tree=tree,
                max_depth=int(rng.integers(4, max(5, N) + 1)) if tree == "tree" else 0)
    if n_sel:
        n_sink = min(4, n_sel // 4)
        over.update(n_sel=n_sel, n_sink=n_sink, n_recent=min(n_sel - n_sink, n_sel // 2))
    run = dict(num_splits=pick([0, 0, 1, 3, 64]),
               out_bf16=bool(rng.random() < 0.25),
               f32_partials=bool(rng.random() < 0.2))
    # an explicit visibility mask instead of the parents in a quarter of the
    # cases: random bits (rows may see nothing of the draft block) or the
    # block-parallel masks of FlexDraft
    u = rng.random()
    run["mask"] = None if u < 0.75 else ("random" if u < 0.875 and N <= 64 else "block")
    run["mask_arg"] = float(rng.uniform(0.05, 0.9)) if run["mask"] == "random" else int(
        rng.integers(1, N + 1))
    # index sets cut short by -1 slots; one part alone; a score scale of the
    # caller's; the partials and the merge as two calls on one workspace
    run["tail_seed"] = int(rng.integers(1 << 30)) if n_sel and rng.random() < 0.3 else None
    run["part"] = pick([None] * 8 + ["prefix", "tree"])
    run["scale"] = float(np.float32(rng.uniform(0.02, 0.3))) if rng.random() < 0.2 else 0.0
    run["phase_split"] = bool(rng.random() < 0.2)
    return over, run, int(1000 + k)


def cut_tails(kv_idx, seed):
    """kv_idx with the sets of some sequences cut short by -1 slots."""
    rng = np.random.default_rng(seed)
    idx = kv_idx.copy()
    for b in range(idx.shape[0]):
        if rng.random() < 0.6:
            idx[b, :, int(rng.integers(0, idx.shape[2] + 1)):] = -1
    return idx


def make_mask(run, B, N, seed):
    if run["mask"] == "random":
        return synth.random_masks(np.random.default_rng(seed), B, N, run["mask_arg"])
    m = synth.block_masks(N, run["mask_arg"])
    return np.broadcast_to(m, (B,) + m.shape).copy()


@pytest.mark.gpu
@pytest.mark.parametrize("k", range(N_CASES))
def test_random_shape(hsv, gpu, k):
    import torch
    over, run, seed = draw_case(k)
    base = "tree32k" if over["dtype"] == "bf16" else "tiny_tree"
    inp = synth.make_inputs(base, seed=seed, **over)
    log(f"random case {k}: {over} {run} ctx={inp.ctx_lens.tolist()[:8]}")
    dev = device_inputs(inp, gpu)
    flags = hsv.HSV_FLAG_F32_PARTIALS if run["f32_partials"] else 0
    parts = oracle.PART_BOTH
    if run["part"] == "prefix":
        flags |= hsv.HSV_FLAG_NO_TREE
        parts = oracle.PART_PREFIX
    elif run["part"] == "tree":
        flags |= hsv.HSV_FLAG_NO_PREFIX
        parts = oracle.PART_TREE
    out = torch.bfloat16 if run["out_bf16"] else torch.float32
    anc = anc_t = None
    if run["mask"]:
        anc = make_mask(run, inp.wl.batch, inp.wl.n_draft, seed)
        anc_t = torch.from_numpy(anc.view(np.int64)).to(gpu)
        dev = dict(dev, parent=None)
    kv_idx = inp.kv_idx
    if run["tail_seed"] is not None:
        kv_idx = cut_tails(kv_idx, run["tail_seed"])
        dev = dict(dev, kv_idx=torch.from_numpy(kv_idx).to(gpu))
    o, lse = run_hip(hsv, inp, dev, num_splits=run["num_splits"], flags=flags, out_dtype=out,
                     anc=anc_t, scale=run["scale"])
    o_ref, l_ref = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens,
                                      parent=None if anc is not None else inp.parent,
                                      anc_mask=anc, kv_idx=kv_idx, bf16=inp.is_bf16,
                                      scale=run["scale"] or None, parts=parts)
    o_chk = o
    if run["out_bf16"]:
        # parity is on the fp32 output; the bf16 output is its round to
        # nearest even, bit for bit (rounding alone moves an |O| above 2.56
        # by more than the 1e-2 bar)
        o32, l32 = run_hip(hsv, inp, dev, num_splits=run["num_splits"], flags=flags,
                           out_dtype=torch.float32, anc=anc_t, scale=run["scale"])
        assert torch.equal(l32, lse), f"case {k}: lse depends on the output dtype"
        rne = synth.f32_to_bf16_bits(o32.cpu().numpy())
        np.testing.assert_array_equal(o.cpu().view(torch.int16).numpy().view(np.uint16), rne,
                                      err_msg=f"case {k}: bf16 output is not the RNE of fp32")
        o_chk = o32
    assert_parity(o_chk.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"random case {k}")
    if run["phase_split"]:
        # the partials, then the merge, as two calls on one workspace
        d = hsv.make_desc(batch=inp.wl.batch, n_draft=inp.wl.n_draft, n_q_heads=inp.wl.n_q_heads,
                          n_kv_heads=inp.wl.n_kv_heads, head_dim=inp.wl.head_dim,
                          kv_capacity=inp.k.shape[2], max_ctx=int(inp.ctx_lens.max()),
                          n_sel=0 if kv_idx is None else kv_idx.shape[2],
                          in_dtype=hsv.HSV_BF16 if inp.is_bf16 else hsv.HSV_F32,
                          out_dtype=hsv.HSV_BF16 if run["out_bf16"] else hsv.HSV_F32,
                          num_splits=run["num_splits"], flags=flags, scale=run["scale"])
        ws = torch.empty(max(256, hsv.hsv_verify_workspace_bytes(d)), dtype=torch.uint8,
                         device=gpu)
        o3, l3 = torch.empty_like(o), torch.empty_like(lse)
        for phase in (hsv.HSV_FLAG_PHASE_PARTIALS, hsv.HSV_FLAG_PHASE_MERGE):
            run_hip(hsv, inp, dev, num_splits=run["num_splits"], flags=flags | phase,
                    out_dtype=out, anc=anc_t, scale=run["scale"], o=o3, lse=l3, workspace=ws)
        assert torch.equal(o3, o) and torch.equal(l3, lse), f"case {k}: two-phase call differs"
    # the entry point that allocates nothing runs the same plan on the
    # library's scratch: identical results where the workspace fits it
    if inp.kv_idx is None and run["scale"] == 0.0:
        d = hsv.make_desc(batch=inp.wl.batch, n_draft=inp.wl.n_draft, n_q_heads=inp.wl.n_q_heads,
                          n_kv_heads=inp.wl.n_kv_heads, head_dim=inp.wl.head_dim,
                          kv_capacity=inp.k.shape[2], max_ctx=int(inp.ctx_lens.max()),
                          in_dtype=hsv.HSV_BF16 if inp.is_bf16 else hsv.HSV_F32,
                          out_dtype=hsv.HSV_BF16 if run["out_bf16"] else hsv.HSV_F32,
                          num_splits=run["num_splits"], flags=flags)
        if hsv.hsv_verify_workspace_bytes(d) <= hsv.HSV_NOALLOC_SCRATCH_BYTES:
            o2, l2 = torch.empty_like(o), torch.empty_like(lse)
            hsv.hsv_verify_attn_noalloc(dev["q"], dev["k"], dev["v"], dev["ctx"], dev["parent"],
                                        anc_t, max_ctx=int(inp.ctx_lens.max()), o=o2, lse=l2,
                                        num_splits=run["num_splits"], flags=flags)
            assert torch.equal(o2, o) and torch.equal(l2, lse), f"case {k}: no-alloc differs"


# Large grids, beyond the sweep's sizes: many sequences (past the 64 that
# share slots by key range), many KV heads (MHA with 64 heads), and query
# groups of 512 and 1024 rows (several 256-row chunks per KV head, on the
# XCD-aware chunk order and off it), with short contexts for the oracle.
LARGE_CASES = [
    dict(batch=128, n_draft=8, n_q_heads=4, n_kv_heads=1, head_dim=128, ctx=(20, 200), dtype="bf16", tree="chain"),
    dict(batch=70, n_draft=4, n_q_heads=16, n_kv_heads=8, head_dim=128, ctx=(0, 300), dtype="bf16", tree="uniform"),
    dict(batch=3, n_draft=16, n_q_heads=64, n_kv_heads=64, head_dim=128, ctx=(100, 400), dtype="bf16", tree="tree", max_depth=6),
    dict(batch=2, n_draft=64, n_q_heads=64, n_kv_heads=8, head_dim=128, ctx=(300, 500), dtype="bf16", tree="tree", max_depth=8),
    dict(batch=1, n_draft=128, n_q_heads=64, n_kv_heads=8, head_dim=128, ctx=(700, 700), dtype="bf16", tree="tree", max_depth=10),
    dict(batch=5, n_draft=128, n_q_heads=24, n_kv_heads=3, head_dim=128, ctx=(50, 400), dtype="bf16", tree="uniform"),
    dict(batch=40, n_draft=8, n_q_heads=32, n_kv_heads=32, head_dim=64, ctx=(0, 150), dtype="f32", tree="chain"),
    dict(batch=96, n_draft=8, n_q_heads=32, n_kv_heads=8, head_dim=128, ctx=(100, 200), dtype="bf16",
         tree="chain", n_sel=64, n_sink=4, n_recent=16),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(len(LARGE_CASES)))
def test_large_grid(hsv, gpu, case):
    over = LARGE_CASES[case]
    base = "tree32k" if over["dtype"] == "bf16" else "tiny_tree"
    inp = synth.make_inputs(base, seed=9000 + case, **over)
    log(f"large grid case {case}: {over}")
    dev = device_inputs(inp, gpu)
    o, lse = run_hip(hsv, inp, dev)
    o_ref, l_ref = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent,
                                      kv_idx=inp.kv_idx, bf16=inp.is_bf16)
    assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"large grid case {case}")
