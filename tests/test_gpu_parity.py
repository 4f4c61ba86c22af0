"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small cases compare every output element; the full-size workloads (in the
launch configuration the benchmark times) compare sampled rows, which the
oracle computes one by one.  Mask, index and gather handling must be
bit-exact; O within 1e-2 max-abs and the LSE within 1e-3 relative.
"""

import dataclasses

import numpy as np
import pytest

import oracle
import synth
from util import (assert_parity, cached_inputs, device_inputs, errors, log, run_hip, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hsv(gpu):
    import long_context_tree_verify_amd as m
    return m


def _oracle_all(inp, **kw):
    return oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent,
                              kv_idx=inp.kv_idx, bf16=inp.is_bf16, **kw)


# ----------------------------------------------------------------------------
# a1: ancestor bitmask, bit-exact
# ----------------------------------------------------------------------------

def test_tree_mask_all_small_trees_bit_exact(hsv, gpu):
    import itertools
    import torch
    for n in range(1, 7):
        trees = np.array(list(itertools.product(*[range(-1, i) for i in range(n)])),
                         dtype=np.int32)
        ref = oracle.ancestor_mask(trees)
        got = hsv.hsv_tree_ancestor_mask(torch.from_numpy(trees).to(gpu))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.cpu().numpy().view(np.uint64), ref)
    log(f"  all parent arrays with N <= 6 match")


def test_tree_mask_large_trees_and_bad_parents(hsv, gpu):
    import torch
    rng = np.random.Generator(np.random.PCG64(77))
    trees = [synth.random_tree_parents(rng, 64, max_depth=d, max_branch=64 if d <= 2 else 4)
             for d in (1, 2, 6, 8, 64)]
    trees += [synth.chain_parents(64), np.full(64, -1, np.int32),
              synth.uniform_parents(rng, 64)]
    trees = np.stack(trees).astype(np.int32)
    got = hsv.hsv_tree_ancestor_mask(torch.from_numpy(trees).to(gpu)).cpu().numpy()
    np.testing.assert_array_equal(got.view(np.uint64), oracle.ancestor_mask(trees))
    bad = trees.copy()
    bad[2, 10] = 10        # self-parent: invalid
    got = hsv.hsv_tree_ancestor_mask(torch.from_numpy(bad).to(gpu)).cpu().numpy()
    assert (got[2] == 0).all()
    np.testing.assert_array_equal(got[[0, 1, 3]].view(np.uint64),
                                  oracle.ancestor_mask(trees[[0, 1, 3]]))


# ----------------------------------------------------------------------------
# a2-a4: dense verification attention, small cases, every element
# ----------------------------------------------------------------------------

SMALL_CASES = [
    ("tiny_tree", ()),                                                   # full size
    ("tree32k", (("ctx", (3000, 3000)),)),                               # ragged tail
    ("tree32k", (("ctx", (700, 700)), ("n_draft", 37), ("max_depth", 5))),
    ("chain_b16", (("ctx", (500, 2100)), ("batch", 4))),
    ("tree128k", (("ctx", (5000, 5000)),)),                              # x8 sinks
    ("tree32k", (("ctx", (1000, 1000)), ("n_q_heads", 8), ("n_kv_heads", 8))),  # MHA, G=1
    ("tree32k", (("ctx", (1500, 1500)), ("head_dim", 64), ("n_draft", 16))),
    ("chain_b16", (("ctx", (0, 300)), ("batch", 6), ("n_draft", 1))),    # may hit c = 0
]


@pytest.mark.parametrize("name,over", SMALL_CASES)
def test_dense_parity_small(hsv, gpu, name, over):
    inp = cached_inputs(name, over)
    log(f"case {name} {dict(over)} ctx={inp.ctx_lens.tolist()[:6]}")
    dev = device_inputs(inp, gpu)
    o, lse = run_hip(hsv, inp, dev)
    o_ref, l_ref = _oracle_all(inp)
    assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, name)


# The 256-row kernel walks prefix and draft rows as one key range: contexts
# around its 32-key block and 64-key tile boundaries put the draft rows
# across blocks; c = 0 leaves only the draft block; ragged batches give
# sequences whose later splits are empty.
DMA_EDGE_CASES = [
    (("ctx", (c, c)), ("batch", 1)) for c in (0, 1, 31, 32, 33, 63, 64, 65, 100, 1056)
] + [
    (("ctx", (0, 200)), ("batch", 3)),
    (("ctx", (60, 2000)), ("batch", 3), ("n_draft", 50)),
]


@pytest.mark.parametrize("over", DMA_EDGE_CASES)
@pytest.mark.parametrize("wl", ["tree32k", "chain_b16"])   # 256 and 32 grouped rows
def test_dma_path_edges(hsv, gpu, over, wl):
    inp = cached_inputs(wl, over)
    log(f"dma edge {wl} {dict(over)} ctx={inp.ctx_lens.tolist()}")
    dev = device_inputs(inp, gpu)
    o_ref, l_ref = _oracle_all(inp)
    for splits in (0, 3, 64):
        o, lse = run_hip(hsv, inp, dev, num_splits=splits)
        assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"splits={splits}")



# Dense batches of several sequences on the small-group kernel share
# n_splits * B slots among the sequences by key range: a long sequence among
# short or empty ones asks for more than twice the split count and is capped
# there, tiny ones still take one slot, empty ones (no keys without the tree)
# take one that writes nothing; 64 sequences is the largest batch shared
# that way and 65 falls back to equal slots.
BALANCED_CASES = [
    ("skewed", 12, (3000, 0, 5, 1, 0, 31, 2, 0, 0, 7, 3, 0)),
    ("one long", 6, (2900, 40, 40, 40, 40, 40)),
    ("b64", 64, None),   # contexts drawn from [0, 600]
    ("b65", 65, None),
]


@pytest.mark.parametrize("label,batch,ctx", BALANCED_CASES)
def test_small_kernel_balanced_slots(hsv, gpu, label, batch, ctx):
    if ctx is None:
        inp = cached_inputs("chain_b16", (("ctx", (0, 600)), ("batch", batch)))
    else:
        # every sequence drawn at the longest context, then cut to its own
        # length, with the rows past c + N poisoned again
        inp = cached_inputs("chain_b16", (("ctx", (max(ctx), max(ctx))), ("batch", batch)))
        c = np.array(ctx, dtype=np.int32)
        nan = np.uint16(0x7FC0) if inp.k.dtype == np.uint16 else np.float32(np.nan)
        k, v = inp.k.copy(), inp.v.copy()
        for b in range(batch):
            k[b, :, c[b] + inp.wl.n_draft:] = nan
            v[b, :, c[b] + inp.wl.n_draft:] = nan
        inp = dataclasses.replace(inp, ctx_lens=c, k=k, v=v)
    log(f"balanced {label} B={batch} ctx={inp.ctx_lens.tolist()[:12]}")
    dev = device_inputs(inp, gpu)
    o_ref, l_ref = _oracle_all(inp)
    for splits in (0, 3, 64):
        o, lse = run_hip(hsv, inp, dev, num_splits=splits)
        assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"{label} splits={splits}")
    for flag, part in ((hsv.HSV_FLAG_NO_TREE, oracle.PART_PREFIX),
                       (hsv.HSV_FLAG_NO_PREFIX, oracle.PART_TREE)):
        o, lse = run_hip(hsv, inp, dev, flags=flag)
        o_ref, l_ref = _oracle_all(inp, parts=part)
        assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"{label} flag={flag}")

# Keys scored far above everything before them (32x the row, so the score
# jumps by many log2 units), placed mid-range, at the last row of a 32-key
# block, in the last prefix block and among the draft rows: the softmax's slow
# path then rescales accumulators that already hold the P.V of earlier blocks,
# including the block just before, whose P.V the 256-row kernel adds one step
# late.
def test_dma_rescale_mid_range(hsv, gpu):
    import dataclasses
    inp = cached_inputs("tree32k", (("ctx", (3000, 3000)),))
    assert inp.k.dtype == np.uint16
    c = int(inp.ctx_lens[0])
    rows = [37, 700, 1055, 1535, c - 1, c + 5]
    k = inp.k.copy()
    f = (k[:, :, rows, :].astype(np.uint32) << 16).view(np.float32) * np.float32(32.0)
    k[:, :, rows, :] = (f.view(np.uint32) >> 16).astype(np.uint16)
    spiked = dataclasses.replace(inp, k=k)
    dev = device_inputs(spiked, gpu)
    o_ref, l_ref = _oracle_all(spiked)
    base_ref = _oracle_all(inp)[1]
    assert float(np.max(l_ref - base_ref)) > 10.0   # the spikes dominate many rows
    for splits in (1, 3, 0):
        o, lse = run_hip(hsv, spiked, dev, num_splits=splits)
        assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"splits={splits}")


def test_tiny_fp32_is_tight(hsv, gpu):
    inp = cached_inputs("tiny_tree")
    dev = device_inputs(inp, gpu)
    o, lse = run_hip(hsv, inp, dev)
    o_ref, l_ref = _oracle_all(inp)
    o_err, l_err = errors(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref)
    assert o_err < 1e-5 and l_err < 1e-6


@pytest.mark.parametrize("splits", [1, 2, 7, 32, 0])
def test_split_count_invariance(hsv, gpu, splits):
    import torch
    inp = cached_inputs("tree32k", (("ctx", (3000, 3000)),))
    dev = device_inputs(inp, gpu)
    o, lse = run_hip(hsv, inp, dev, num_splits=splits)
    o1, l1 = run_hip(hsv, inp, dev, num_splits=1)
    # P is rounded to bf16 (unit roundoff 2^-8) relative to each split's own
    # running reference, so different split counts round P differently: O may
    # move by up to about 2^-8 * max|V| in the worst case, typically ~1e-4.
    # The LSE comes from fp32 sums of unrounded P and moves only by fp32
    # rounding.
    d_o = float((o - o1).abs().max())
    d_l = float(((lse - l1).abs() / l1.abs().clamp(min=1)).max())
    log(f"  splits={splits}: max|O - O(1 split)| = {d_o:.2e}, rel dLSE = {d_l:.2e}")
    assert d_o <= 1e-3
    assert d_l <= 1e-6
    o_ref, l_ref = _oracle_all(inp)
    assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"splits={splits}")
    assert torch.isfinite(o).all()


def test_deterministic_and_bf16_output_is_rne_of_fp32(hsv, gpu):
    import torch
    inp = cached_inputs("tree32k", (("ctx", (3000, 3000)),))
    dev = device_inputs(inp, gpu)
    o1, l1 = run_hip(hsv, inp, dev)
    o2, l2 = run_hip(hsv, inp, dev)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ob, lb = run_hip(hsv, inp, dev, out_dtype=torch.bfloat16)
    assert torch.equal(lb, l1)
    rne = synth.f32_to_bf16_bits(o1.cpu().numpy())
    np.testing.assert_array_equal(ob.cpu().view(torch.int16).numpy().view(np.uint16), rne)


def test_parts_alone_match_oracle_parts(hsv, gpu):
    inp = cached_inputs("tree32k", (("ctx", (3000, 3000)),))
    dev = device_inputs(inp, gpu)
    for flag, part in ((hsv.HSV_FLAG_NO_TREE, oracle.PART_PREFIX),
                       (hsv.HSV_FLAG_NO_PREFIX, oracle.PART_TREE)):
        o, lse = run_hip(hsv, inp, dev, flags=flag)
        o_ref, l_ref = _oracle_all(inp, parts=part)
        assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"flag={flag}")


def test_ancestor_mask_input_and_general_masks(hsv, gpu):
    import torch
    inp = cached_inputs("tree32k", (("ctx", (3000, 3000)),))
    dev = device_inputs(inp, gpu)
    anc = oracle.ancestor_mask(inp.parent)
    anc_dev = torch.from_numpy(anc.view(np.int64)).to(gpu)
    o1, l1 = run_hip(hsv, inp, dev)
    o2, l2 = run_hip(hsv, inp, dev, parent=None, anc=anc_dev)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # block-bidirectional masks (not a tree): 16-node blocks see each other
    N = inp.wl.n_draft
    blk = np.arange(N) // 16
    anc2 = np.array([[sum(1 << j for j in range(N) if blk[j] == blk[i]) for i in range(N)]],
                    dtype=np.uint64)
    o3, l3 = run_hip(hsv, inp, dev, parent=None,
                     anc=torch.from_numpy(anc2.view(np.int64)).to(gpu))
    o_ref, l_ref = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, anc_mask=anc2,
                                      bf16=True)
    assert_parity(o3.cpu().numpy(), l3.cpu().numpy(), o_ref, l_ref, "block mask")


# ----------------------------------------------------------------------------
# a5: sparse verification attention and the gather
# ----------------------------------------------------------------------------

SPARSE_CASES = [
    (("ctx", (8000, 8000)), ("batch", 2), ("n_sel", 1000), ("n_recent", 200)),
    (("ctx", (3000, 3000)), ("batch", 3), ("n_sel", 77), ("n_recent", 10), ("n_draft", 5)),
    (("ctx", (600, 600)), ("batch", 1), ("n_sel", 600), ("n_recent", 96)),   # all selected
    (("ctx", (500, 900)), ("batch", 2), ("n_sel", 1), ("n_sink", 0), ("n_recent", 1)),
    (("ctx", (500, 900)), ("batch", 2), ("n_sel", 33), ("n_sink", 4), ("n_recent", 8)),
    (("ctx", (300, 300)), ("batch", 1), ("n_sel", 100), ("n_recent", 20), ("n_draft", 3)),
]


@pytest.mark.parametrize("over", SPARSE_CASES[3:])
def test_sparse_splits_and_parts(hsv, gpu, over):
    inp = cached_inputs("sparse64k", over, poison=True)
    log(f"sparse splits/parts {dict(over)}")
    dev = device_inputs(inp, gpu)
    o_ref, l_ref = _oracle_all(inp)
    for splits in (0, 2, 5):
        o, lse = run_hip(hsv, inp, dev, num_splits=splits)
        assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"splits={splits}")
    for flag, part in ((hsv.HSV_FLAG_NO_TREE, oracle.PART_PREFIX),
                       (hsv.HSV_FLAG_NO_PREFIX, oracle.PART_TREE)):
        o, lse = run_hip(hsv, inp, dev, flags=flag)
        o_p, l_p = _oracle_all(inp, parts=part)
        assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_p, l_p, f"flags={flag}")


@pytest.mark.parametrize("over", SPARSE_CASES)
def test_sparse_parity_small_poisoned(hsv, gpu, over):
    inp = cached_inputs("sparse64k", over, poison=True)
    log(f"sparse case {dict(over)}")
    dev = device_inputs(inp, gpu)
    o, lse = run_hip(hsv, inp, dev)
    o_ref, l_ref = _oracle_all(inp)
    assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "sparse")


# fp32 inputs take the vector-ALU kernel.  With no sinks, row 0 is left out of
# almost every index set and holds NaN after poisoning; the kernel's lanes
# past a chunk's end read row 0 and must keep it out of the scores and P.V.
@pytest.mark.parametrize("D", [64, 128])
def test_fp32_sparse_poisoned(hsv, gpu, D):
    over = (("ctx", (700, 700)), ("batch", 2), ("n_sel", 50), ("n_sink", 0),
            ("n_recent", 8), ("dtype", "f32"), ("head_dim", D))
    inp = cached_inputs("sparse64k", over, poison=True)
    assert not inp.is_bf16 and (inp.kv_idx[..., 0] != 0).any()
    assert np.isnan(inp.k[:, :, 0, :]).any()
    dev = device_inputs(inp, gpu)
    o_ref, l_ref = _oracle_all(inp)
    for splits in (0, 3):
        o, lse = run_hip(hsv, inp, dev, num_splits=splits)
        assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref,
                      f"fp32 sparse poisoned D={D} splits={splits}")


def test_gather_kv_bit_exact(hsv, gpu):
    import torch
    inp = cached_inputs("sparse64k", SPARSE_CASES[0], poison=True)
    dev = device_inputs(inp, gpu)
    kg, vg = hsv.hsv_gather_kv(dev["k"], dev["v"], dev["kv_idx"])
    torch.cuda.synchronize()
    rk, rv = oracle.gather_kv(inp.k, inp.v, inp.kv_idx)
    np.testing.assert_array_equal(kg.cpu().view(torch.int16).numpy().view(np.uint16), rk)
    np.testing.assert_array_equal(vg.cpu().view(torch.int16).numpy().view(np.uint16), rv)


# ----------------------------------------------------------------------------
# a4 alone: the exported merge
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("P,D", [(1, 64), (3, 128), (33, 128), (130, 64)])
def test_lse_merge_matches_oracle(hsv, gpu, P, D):
    import torch
    rng = np.random.default_rng(P * 1000 + D)
    R = 50
    o_parts = rng.standard_normal((P, R, D)).astype(np.float32)
    lse_parts = (rng.standard_normal((P, R)) * 3).astype(np.float32)
    lse_parts[rng.random((P, R)) < 0.2] = -np.inf
    lse_parts[:, 0] = -np.inf                     # an empty row
    o_parts[np.isneginf(lse_parts)] = np.nan      # never read
    o, lse = hsv.hsv_lse_merge(torch.from_numpy(o_parts).to(gpu),
                               torch.from_numpy(lse_parts).to(gpu))
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    for r in range(R):
        ro, rl = oracle.lse_merge(lse_parts[:, r].astype(np.float64),
                                  np.nan_to_num(o_parts[:, r].astype(np.float64)))
        if np.isneginf(rl):
            assert np.isneginf(lse[r]) and (o[r] == 0).all()
            continue
        assert abs(lse[r] - rl) <= 1e-5 * max(1, abs(rl))
        np.testing.assert_allclose(o[r], ro, rtol=0, atol=1e-5)


# ----------------------------------------------------------------------------
# validation flag (failure handling forced from the host; kernels exit normally)
# ----------------------------------------------------------------------------

def test_validate_flag(hsv, gpu):
    import torch
    inp = cached_inputs("chain_b16", (("ctx", (500, 2100)), ("batch", 4)))
    dev = device_inputs(inp, gpu)
    run_hip(hsv, inp, dev, flags=hsv.HSV_FLAG_VALIDATE)        # good data passes
    bad_parent = dev["parent"].clone()
    bad_parent[1, 3] = 5
    with pytest.raises(hsv.HsvError) as e:
        run_hip(hsv, inp, dev, parent=bad_parent, flags=hsv.HSV_FLAG_VALIDATE)
    assert e.value.code == hsv.HSV_ERR_DEVICE_CHECK
    sp = cached_inputs("sparse64k", SPARSE_CASES[1], poison=True)
    sdev = device_inputs(sp, gpu)
    run_hip(hsv, sp, sdev, flags=hsv.HSV_FLAG_VALIDATE)
    bad_idx = sdev["kv_idx"].clone()
    bad_idx[0, 0, 5] = bad_idx[0, 0, 4]                        # duplicate
    sdev2 = dict(sdev, kv_idx=bad_idx)
    with pytest.raises(hsv.HsvError) as e:
        run_hip(hsv, sp, sdev2, flags=hsv.HSV_FLAG_VALIDATE)
    assert e.value.code == hsv.HSV_ERR_DEVICE_CHECK
    torch.cuda.synchronize()


def test_graph_replays_match_eager(hsv, gpu):
    """A captured call replayed several times, with eager calls and
    synchronisations in between, gives the eager result bit for bit each time
    (the benchmark times graph replays)."""
    import torch
    for wl, over in (("tree32k", (("ctx", (3000, 3000)),)),
                     ("chain_b16", (("ctx", (700, 2000)), ("batch", 3))),
                     ("sparse64k", SPARSE_CASES[1])):
        inp = cached_inputs(wl, over, poison=wl == "sparse64k")
        log(f"graph replay case {wl} {dict(over)}")
        dev = device_inputs(inp, gpu)
        o_ref, l_ref = run_hip(hsv, inp, dev)
        o = torch.empty_like(o_ref)
        lse = torch.empty_like(l_ref)
        max_ctx = int(inp.ctx_lens.max())
        sparse = inp.kv_idx is not None
        n = hsv.hsv_verify_workspace_bytes(hsv.make_desc(
            batch=inp.wl.batch, n_draft=inp.wl.n_draft, n_q_heads=inp.wl.n_q_heads,
            n_kv_heads=inp.wl.n_kv_heads, head_dim=inp.wl.head_dim,
            kv_capacity=inp.k.shape[2], max_ctx=max_ctx,
            n_sel=inp.kv_idx.shape[2] if sparse else 0,
            in_dtype=hsv.HSV_BF16 if inp.is_bf16 else hsv.HSV_F32, out_dtype=hsv.HSV_F32))
        ws = torch.empty(n, dtype=torch.uint8, device=gpu)

        def call():
            kw = dict(max_ctx=max_ctx, out_dtype=torch.float32, o=o, lse=lse, workspace=ws)
            if sparse:
                hsv.hsv_verify_attn_sparse(dev["q"], dev["k"], dev["v"], dev["ctx"],
                                           dev["parent"], None, dev["kv_idx"], **kw)
            else:
                hsv.hsv_verify_attn(dev["q"], dev["k"], dev["v"], dev["ctx"], dev["parent"],
                                    None, **kw)

        side = torch.cuda.Stream(gpu)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            call()
        for rep in range(3):
            o.fill_(float("nan"))
            lse.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), f"replay {rep}"
            o2, l2 = run_hip(hsv, inp, dev)      # eager work between replays
            assert torch.equal(o2, o_ref) and torch.equal(l2, l_ref)


@pytest.mark.parametrize("dtype", ["bf16_256rows", "bf16_32rows", "bf16_mfma", "f32"])
def test_empty_key_set_without_partials(hsv, gpu, dtype):
    """No prefix keys (max_ctx 0) and no tree part: the plan has no partial
    results at all, and the merge writes the empty-set result (o = 0,
    lse = -inf) without reading the workspace."""
    import torch
    heads = {"bf16_256rows": (32, 8, 64, 128), "bf16_32rows": (32, 8, 8, 128),
             "bf16_mfma": (16, 8, 32, 64), "f32": (1, 1, 8, 64)}[dtype]
    Hq, Hkv, N, D = heads
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    B, cap = 2, 64
    q = torch.randn((B, N, Hq, D), device=gpu).to(dt)
    k = torch.randn((B, Hkv, cap, D), device=gpu).to(dt)
    v = torch.randn((B, Hkv, cap, D), device=gpu).to(dt)
    ctx = torch.zeros(B, dtype=torch.int32, device=gpu)
    for out_dtype in (torch.float32, torch.bfloat16):
        o = torch.full((B, N, Hq, D), float("nan"), dtype=out_dtype, device=gpu)
        lse = torch.full((B, N, Hq), float("nan"), dtype=torch.float32, device=gpu)
        # the smallest legal workspace for this plan (no partial rows)
        desc = hsv.make_desc(batch=B, n_draft=N, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D,
                             kv_capacity=cap, max_ctx=0,
                             in_dtype=hsv.HSV_F32 if dt == torch.float32 else hsv.HSV_BF16,
                             out_dtype=hsv.HSV_F32 if out_dtype == torch.float32
                             else hsv.HSV_BF16, flags=hsv.HSV_FLAG_NO_TREE)
        ws = torch.empty(hsv.hsv_verify_workspace_bytes(desc), dtype=torch.uint8, device=gpu)
        hsv.hsv_verify_attn(q, k, v, ctx, None, None, max_ctx=0, out_dtype=out_dtype,
                            flags=hsv.HSV_FLAG_NO_TREE, o=o, lse=lse, workspace=ws)
        torch.cuda.synchronize()
        assert (o.float() == 0).all(), dtype
        assert torch.isneginf(lse).all(), dtype


@pytest.mark.parametrize("wl", ["tree32k", "chain_b16", "sparse64k"])
def test_f32_partials_small(hsv, gpu, wl):
    """HSV_FLAG_F32_PARTIALS on both DMA kernels (256-row and small-group,
    dense and gathered): parity against the oracle for several split counts,
    and the two phases run apart give the combined call's result bit for
    bit."""
    import torch
    over = {"tree32k": (("ctx", (3000, 3000)),),
            "chain_b16": (("ctx", (500, 2100)), ("batch", 4)),
            "sparse64k": SPARSE_CASES[1]}[wl]
    inp = cached_inputs(wl, over, poison=wl == "sparse64k")
    dev = device_inputs(inp, gpu)
    o_ref, l_ref = _oracle_all(inp)
    F = hsv.HSV_FLAG_F32_PARTIALS
    for splits in (0, 1, 7):
        o, lse = run_hip(hsv, inp, dev, num_splits=splits, flags=F)
        assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref,
                      f"{wl} fp32 partials splits={splits}")
    o, lse = run_hip(hsv, inp, dev, flags=F)
    o2, l2 = torch.empty_like(o), torch.empty_like(lse)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=gpu)
    run_hip(hsv, inp, dev, flags=F | hsv.HSV_FLAG_PHASE_PARTIALS, o=o2, lse=l2, workspace=ws)
    run_hip(hsv, inp, dev, flags=F | hsv.HSV_FLAG_PHASE_MERGE, o=o2, lse=l2, workspace=ws)
    assert torch.equal(o, o2) and torch.equal(lse, l2)


# Index-set entries outside [0, c) -- negative, at or just past the context,
# past the cache, the int32 extremes -- take no part and are never read (the
# kernels turn them into a masked in-set row before forming an address):
# the result is that of the set without them.  Runs the small-group kernel
# (bf16, D 128, 20 grouped rows), the register-staged MFMA kernel (D 64) and
# the fp32 kernel; unselected rows hold NaN.
def _garbage_indices(kv_idx, ctx, cap, seed):
    """kv_idx with about 15 % of its valid entries replaced by out-of-range
    values, and the same set with those entries removed (-1 tail)."""
    rng = np.random.default_rng(seed)
    bad = kv_idx.copy()
    clean = np.full_like(kv_idx, -1)
    B, H, n = kv_idx.shape
    for b in range(B):
        junk = np.array([-3, ctx[b], ctx[b] + 1, cap + 100, 1 << 30, -(1 << 31)], np.int64)
        for g in range(H):
            row = bad[b, g]
            hit = (row >= 0) & (rng.random(n) < 0.15)
            row[hit] = junk[rng.integers(0, len(junk), int(hit.sum()))].astype(np.int32)
            keep = row[(row >= 0) & (row < ctx[b])]
            clean[b, g, :keep.size] = keep
    return bad, clean


@pytest.mark.parametrize("over", [(), (("head_dim", 64),), (("dtype", "f32"),)])
def test_sparse_out_of_range_indices_are_masked(hsv, gpu, over):
    import torch
    inp = cached_inputs("sparse64k", SPARSE_CASES[1] + tuple(over), poison=True)
    bad, clean = _garbage_indices(inp.kv_idx, inp.ctx_lens, inp.k.shape[2], 150)
    dev = dict(device_inputs(inp, gpu), kv_idx=torch.from_numpy(bad).to(gpu))
    o, lse = run_hip(hsv, inp, dev)
    o_ref, l_ref = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent,
                                      kv_idx=clean, bf16=inp.is_bf16)
    assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"garbage indices {over}")


# Valid index sets ending in -1 slots (the selection writes them when the
# context is shorter than the set) on every sparse kernel: the small-group
# kernel, the register-staged MFMA kernel (D 64; 64 grouped rows) and the
# fp32 kernel.  Sequence 0 keeps its first 30 entries, sequence 1 none.
@pytest.mark.parametrize("over", [(), (("head_dim", 64),), (("n_draft", 16),),
                                  (("dtype", "f32"),)])
def test_sparse_minus_one_tails_every_kernel(hsv, gpu, over):
    import torch
    inp = cached_inputs("sparse64k", SPARSE_CASES[1] + tuple(over), poison=True)
    idx = inp.kv_idx.copy()
    idx[0, :, 30:] = -1
    idx[1] = -1
    dev = dict(device_inputs(inp, gpu), kv_idx=torch.from_numpy(idx).to(gpu))
    o, lse = run_hip(hsv, inp, dev)
    o_ref, l_ref = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent,
                                      kv_idx=idx, bf16=inp.is_bf16)
    assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"-1 tails {over}")
