"""A seeded random sweep of the paged verify calls (HiSpec page: paged
attention with block tables; Dustin page: verification over a selected
subset), each case against the fp64 oracle on the contiguous view of the
same cache, and for sparse calls also bit for bit against the contiguous
sparse call.

Draws stay within the shapes the paged calls accept (bf16, head dim 128,
the 256-row kernel's more than 128 grouped rows or the small-group kernel's
at most 32; sparse only on the latter): batch, draft nodes, query and KV
heads, block size 64 to 1024, ragged contexts including 0, index-set size
split count and, for a third of the dense calls, an explicit visibility
mask (random bits or block-parallel) instead of the parents.  Pool blocks
are in a seeded random order and the spare ones hold NaN.  Every draw is fixed by its case number.
"""

import numpy as np
import pytest

import oracle
import synth
from test_gpu_paged import _paged, _run, _run_sparse, _run_sparse_contiguous
from util import assert_parity, log

pytestmark = pytest.mark.gpu

N_CASES = 150


@pytest.fixture(scope="module")
def hsv(gpu):
    import long_context_tree_verify_amd as m
    return m


def draw_case(k: int):
    rng = np.random.default_rng(3000 + k)
    pick = lambda xs: xs[int(rng.integers(len(xs)))]
    sparse = rng.random() < 0.4
    if sparse or rng.random() < 0.5:      # small-group kernel: G * N <= 32
        G = pick([1, 2, 4])
        N = pick([n for n in (1, 2, 5, 8, 16, 32) if G * n <= 32])
    else:                                  # 256-row kernel: G * N > 128
        G = pick([4, 8])
        N = pick([n for n in (17, 33, 64, 65, 100, 256) if G * n > 128])
    Hkv = pick([1, 2, 4, 8])
    B = pick([1, 2, 3, 6])
    bs = pick([64, 128, 256, 512, 1024])
    hi = pick([0, 100, 700, 3000, 5000])
    lo = int(rng.integers(0, hi + 1)) if rng.random() < 0.7 else hi
    over = dict(batch=B, n_draft=N, n_q_heads=G * Hkv, n_kv_heads=Hkv, head_dim=128,
                dtype="bf16", tree=pick(["uniform", "chain"]))
    if sparse:
        n_sel = pick([1, 64, 300])
        hi, lo = max(hi, n_sel + 10), max(lo, n_sel)
        n_sink = min(4, n_sel // 4)
        over.update(n_sel=n_sel, n_sink=n_sink, n_recent=min(n_sel - n_sink, n_sel // 2))
    while B * N * G * Hkv * (hi + N) > 2e7 and B > 1:
        B = over["batch"] = max(1, B // 2)
    over["ctx"] = (lo, hi)
    # an explicit visibility mask instead of the parents in a third of the
    # cases (dense calls): random bits up to 64 nodes, else block-parallel
    u = rng.random()
    mask = None if sparse or u < 0.67 else ("random" if N <= 64 and u < 0.85 else "block")
    over["_mask"] = (mask, int(rng.integers(1, N + 1)))
    return over, bs, pick([0, 1, 5]), 3000 + k


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_paged(hsv, gpu, k):
    import torch
    over, bs, splits, seed = draw_case(k)
    mask, arg = over.pop("_mask")
    inp = synth.make_inputs("tree32k", seed=seed, **over)
    kp, vp, table = _paged(inp, bs, seed)
    log(f"paged case {k}: {over} bs={bs} splits={splits} ctx={inp.ctx_lens.tolist()}")
    anc = None
    if mask == "random":
        anc = synth.random_masks(np.random.default_rng(seed), inp.wl.batch, inp.wl.n_draft,
                                 0.1 + 0.8 * (arg % 8) / 8)
    elif mask == "block":
        m = synth.block_masks(inp.wl.n_draft, arg)
        anc = np.broadcast_to(m, (inp.wl.batch,) + m.shape).copy()
    o_ref, l_ref = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens,
                                      parent=None if anc is not None else inp.parent,
                                      anc_mask=anc, kv_idx=inp.kv_idx, bf16=True)
    if inp.kv_idx is None and anc is not None:
        o, lse = _run(hsv, gpu, inp, kp, vp, table, num_splits=splits, parent=None,
                      anc=torch.from_numpy(anc.view(np.int64)).to(gpu))
    elif inp.kv_idx is None:
        o, lse = _run(hsv, gpu, inp, kp, vp, table, num_splits=splits)
    else:
        o, lse = _run_sparse(hsv, gpu, inp, kp, vp, table, inp.kv_idx, num_splits=splits)
        o_c, l_c = _run_sparse_contiguous(hsv, gpu, inp, inp.kv_idx, num_splits=splits)
        assert np.array_equal(o, o_c) and np.array_equal(lse, l_c), f"case {k}: paged != contiguous"
    assert_parity(o, lse, o_ref, l_ref, f"paged case {k}")
