"""A seeded random sweep of hsv_select_kv_idx against oracle.select_kv_idx,
bit-exact (Dustin page, methodology 1).

Each case draws the batch, KV heads, score-row length (across the 8192-
position chunks, the 73728-position bound of the list path and the
streaming path beyond it), per-sequence contexts anywhere in [0, L], the
budget (sinks, window, draft share -- also beyond the budget) and one of
four score families: bf16-precision importance maps (many equal scores),
full-precision fp32 scores, a few distinct values only (huge ties), and
importance maps with NaN, +-0 and +-inf mixed in.  Every draw is fixed by
its case number.
"""

import numpy as np
import pytest

import oracle
import synth
from util import log

pytestmark = pytest.mark.gpu

N_CASES = 400
LENGTHS = [1, 7, 100, 2000, 8192, 8193, 20000, 65536, 65544, 73728, 73729, 100000]


@pytest.fixture(scope="module")
def hsv(gpu):
    import long_context_tree_verify_amd as m
    return m


def draw_case(k: int):
    rng = np.random.Generator(np.random.PCG64(2000 + k))
    B = int(rng.integers(1, 7))
    H = int(rng.choice([1, 2, 4, 8]))
    L = int(rng.choice(LENGTHS))
    ctx = rng.integers(0, L + 1, size=B).astype(np.int32)
    ctx[rng.random(B) < 0.3] = L
    n_sel = int(rng.choice([1, 16, 300, 1000, 4096]))
    n_sink = int(rng.integers(0, min(8, n_sel) + 1))
    n_recent = int(rng.integers(0, n_sel - n_sink + 1))
    n_draft_top = int(rng.integers(0, n_sel + 11))
    kind = int(rng.integers(0, 4))
    if kind == 1:
        draft = rng.random((B, H, L), dtype=np.float32)
        target = rng.random((B, H, L), dtype=np.float32)
    elif kind == 2:
        draft = rng.integers(0, 4, size=(B, H, L)).astype(np.float32)
        target = rng.integers(0, 3, size=(B, H, L)).astype(np.float32)
    else:
        draft, target = synth.importance_maps(rng, np.minimum(ctx, L), H, L)
        if kind == 3:
            specials = np.array([np.nan, 0.0, -0.0, np.inf, -np.inf], np.float32)
            for m in (draft, target):
                hit = rng.random(m.shape) < 0.02
                m[hit] = specials[rng.integers(0, len(specials), size=int(hit.sum()))]
    budget = dict(n_sel=n_sel, n_sink=n_sink, n_recent=n_recent, n_draft_top=n_draft_top)
    return draft, target, ctx, budget, kind


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_selection(hsv, gpu, k):
    import torch
    draft, target, ctx, budget, kind = draw_case(k)
    log(f"selection case {k}: maps {draft.shape} kind {kind} ctx {ctx.tolist()} {budget}")
    got = hsv.hsv_select_kv_idx(torch.from_numpy(draft).to(gpu), torch.from_numpy(target).to(gpu),
                                torch.from_numpy(ctx).to(gpu), **budget)
    torch.cuda.synchronize()
    ref = oracle.select_kv_idx(draft, target, ctx, **budget)
    got = got.cpu().numpy()
    bad = np.argwhere((got != ref).any(axis=-1))
    assert bad.size == 0, f"case {k}: (b, g) rows differ: {bad[:4].tolist()}"
