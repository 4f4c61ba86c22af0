"""Draft trees of more than 64 nodes (masks of ceil(N/64) 64-bit words) on
the GPU against the fp64 oracle: the multi-word ancestor masks bit for bit,
and verification attention through the 256-row kernel with the masks built
from parents (in the workspace) or given, block-parallel masks, forced
split counts, a paged cache and the full 32k context."""

import numpy as np
import pytest

import oracle
import synth
from util import (assert_all_rows, assert_parity, cached_inputs, device_inputs, log, run_hip,
                  to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hsv(gpu):
    import long_context_tree_verify_amd as m
    return m


def test_wide_ancestor_masks_bit_exact(hsv, gpu):
    import torch
    rng = np.random.Generator(np.random.PCG64(120))
    for n in (65, 128, 200, 256):
        par = np.stack([synth.chain_parents(n), np.full(n, -1, np.int32),
                        synth.uniform_parents(rng, n),
                        synth.random_tree_parents(rng, n, max_depth=16, max_branch=4),
                        synth.random_tree_parents(rng, n, max_depth=n, max_branch=2)]).astype(np.int32)
        bad = par.copy()
        bad[2, n - 1] = n                      # out of range: that sequence is all zero
        got = hsv.hsv_tree_ancestor_mask(torch.from_numpy(bad).to(gpu)).cpu().numpy()
        assert got.shape == (5, n, oracle.mask_words(n))
        ok = [0, 1, 3, 4]
        np.testing.assert_array_equal(got[ok].view(np.uint64), oracle.ancestor_mask(par[ok]))
        assert (got[2] == 0).all()
    log("  ancestor masks identical for N = 65, 128, 200, 256")


CASES = [
    (("ctx", (2000, 2000)), ("n_draft", 96), ("max_depth", 12)),
    (("ctx", (1500, 2500)), ("batch", 2), ("n_draft", 128), ("max_depth", 16)),
    (("ctx", (3000, 3000)), ("n_draft", 200), ("max_depth", 24)),
    (("ctx", (2000, 2000)), ("n_draft", 256), ("max_depth", 16)),
    # two KV heads, two 256-row chunks per head: the automatic split count
    # gives a multiple of eight (split, KV head) units, whose row chunks share
    # an XCD; 1 and 7 splits give 2 and 14 units, in the plain order
    (("ctx", (1800, 1800)), ("n_q_heads", 8), ("n_kv_heads", 2), ("n_draft", 96),
     ("max_depth", 12)),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_wide_tree_attention(hsv, gpu, case):
    import torch
    over = CASES[case]
    inp = cached_inputs("tree32k", over)
    dev = device_inputs(inp, gpu)
    o_ref, l_ref = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent,
                                      bf16=True)
    for splits in (0, 1, 7):
        o, lse = run_hip(hsv, inp, dev, num_splits=splits)
        assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref,
                      f"N={inp.wl.n_draft} parents splits={splits}")
    anc = oracle.ancestor_mask(inp.parent)
    o, lse = run_hip(hsv, inp, dev, parent=None,
                     anc=torch.from_numpy(anc.view(np.int64)).to(gpu))
    assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref,
                  f"N={inp.wl.n_draft} mask words")


def test_wide_block_masks(hsv, gpu):
    import torch
    inp = cached_inputs("tree32k", (("ctx", (2000, 2000)), ("n_draft", 256), ("max_depth", 16)))
    dev = device_inputs(inp, gpu)
    for block in (32, 100):
        anc = synth.block_masks(256, block)[None]
        o, lse = run_hip(hsv, inp, dev, parent=None,
                         anc=torch.from_numpy(np.ascontiguousarray(anc).view(np.int64)).to(gpu))
        o_ref, l_ref = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, anc_mask=anc,
                                          bf16=True)
        assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref,
                      f"N=256 blocks of {block}")


def test_wide_tree_paged(hsv, gpu):
    import torch
    inp = cached_inputs("tree32k", (("ctx", (1500, 2500)), ("batch", 2), ("n_draft", 128),
                                    ("max_depth", 16)))
    rng = np.random.Generator(np.random.PCG64(121))
    S = inp.k.shape[2]
    cap = -(-S // 128) * 128
    pad = ((0, 0), (0, 0), (0, cap - S), (0, 0))
    kp, vp, table = synth.to_paged(np.pad(inp.k, pad), np.pad(inp.v, pad), 128, rng)
    o, lse = hsv.hsv_verify_attn_paged(
        to_dev(inp.q, True, gpu), to_dev(kp, True, gpu), to_dev(vp, True, gpu),
        torch.from_numpy(table).to(gpu), torch.from_numpy(inp.ctx_lens).to(gpu),
        torch.from_numpy(inp.parent).to(gpu), max_ctx=int(inp.ctx_lens.max()))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent,
                                      bf16=True)
    assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "N=128 paged")


def test_wide_tree_full_size(hsv, gpu):
    import torch
    inp = synth.make_inputs("tree32k", n_draft=256, max_depth=16, ctx=(32768, 32768))
    dev = device_inputs(inp, gpu)
    o, lse = run_hip(hsv, inp, dev)
    o_np, l_np = o.cpu().numpy(), lse.cpu().numpy()
    del dev
    torch.cuda.empty_cache()
    o_err, l_err = assert_all_rows(o_np, l_np, inp, "N=256 full size")
    log(f"  N=256 at 32k: all {l_np.size} rows max|dO| = {o_err:.3e}, "
        f"max rel dLSE = {l_err:.3e}")


# Trees of more than 64 nodes on the kernels other than the 256-row DMA one:
# the MFMA kernels (D = 64, or 33 to 128 grouped rows) read a 32-bit chunk of
# the row's mask words per key block, the fp32 kernel one word per 64 keys.
OTHER_KERNEL_CASES = [
    ("tree32k", (("ctx", (500, 500)), ("n_draft", 80), ("head_dim", 64), ("max_depth", 12))),
    ("tree32k", (("ctx", (700, 900)), ("batch", 2), ("n_draft", 100), ("n_q_heads", 8),
                 ("n_kv_heads", 8), ("max_depth", 20))),
    ("tree32k", (("ctx", (600, 600)), ("n_draft", 200), ("n_q_heads", 8), ("n_kv_heads", 8),
                 ("head_dim", 64), ("max_depth", 24))),
    ("tree32k", (("ctx", (400, 400)), ("n_draft", 120), ("n_q_heads", 2), ("n_kv_heads", 2),
                 ("max_depth", 16))),
    ("tiny_tree", (("ctx", (300, 300)), ("n_draft", 96))),
    ("tiny_tree", (("ctx", (200, 200)), ("n_draft", 256), ("head_dim", 128))),
]


@pytest.mark.parametrize("case", range(len(OTHER_KERNEL_CASES)))
def test_wide_tree_other_kernels(hsv, gpu, case):
    import torch
    name, over = OTHER_KERNEL_CASES[case]
    inp = cached_inputs(name, over)
    dev = device_inputs(inp, gpu)
    o_ref, l_ref = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent,
                                      bf16=inp.is_bf16)
    what = f"{name} {dict(over)}"
    for splits in (0, 3):
        o, lse = run_hip(hsv, inp, dev, num_splits=splits)
        assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"{what} splits={splits}")
    anc = oracle.ancestor_mask(inp.parent)
    o, lse = run_hip(hsv, inp, dev, parent=None,
                     anc=torch.from_numpy(np.ascontiguousarray(anc).view(np.int64)).to(gpu))
    assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"{what} mask words")
    # block-parallel masks (bits above the row's own index)
    N = inp.wl.n_draft
    blk = np.broadcast_to(synth.block_masks(N, 40), (inp.wl.batch,) + synth.block_masks(N, 40).shape)
    blk = np.array(blk, order="C", copy=True)  # writable, C-ordered (not the broadcast view)
    o, lse = run_hip(hsv, inp, dev, parent=None,
                     anc=torch.from_numpy(blk.view(np.int64)).to(gpu))
    ob, lb = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, anc_mask=blk, bf16=inp.is_bf16)
    assert_parity(o.cpu().numpy(), lse.cpu().numpy(), ob, lb, f"{what} blocks of 40")
