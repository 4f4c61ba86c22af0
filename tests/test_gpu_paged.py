"""GPU parity of verification attention over a paged cache (pool blocks and a
block table; HiSpec page: paged attention with block tables) against the
fp64 oracle on the contiguous view of the same cache.

The pool order is a seeded random permutation and the spare pool blocks hold
NaN, so a kernel that follows a wrong table entry fails parity.  Cases cover
both kernels that take a paged cache (256-row chunks and the small-group
kernel), block sizes 64 to 1024, ragged contexts including c = 0, forced
split counts, explicit masks, and the 32k-context tree at full size.
"""

import numpy as np
import pytest

import oracle
import synth
from util import assert_all_rows, assert_parity, cached_inputs, log, oracle_full, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hsv(gpu):
    import long_context_tree_verify_amd as m
    return m


def _paged(inp, bs, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    S = inp.k.shape[2]
    cap = -(-S // bs) * bs                  # whole blocks: pad the cache with NaN rows
    k, v = inp.k, inp.v
    if cap != S:
        pad = ((0, 0), (0, 0), (0, cap - S), (0, 0))
        fill = synth.gen.BF16_NAN if k.dtype == np.uint16 else np.nan
        k = np.pad(k, pad, constant_values=fill)
        v = np.pad(v, pad, constant_values=fill)
    kp, vp, table = synth.to_paged(k, v, bs, rng)
    return kp, vp, table


def _run(hsv, gpu, inp, kp, vp, table, **kw):
    import torch
    bf = inp.is_bf16
    o, lse = hsv.hsv_verify_attn_paged(
        to_dev(inp.q, bf, gpu), to_dev(kp, bf, gpu), to_dev(vp, bf, gpu),
        torch.from_numpy(table).to(gpu), torch.from_numpy(inp.ctx_lens).to(gpu),
        kw.pop("parent", torch.from_numpy(inp.parent).to(gpu)), kw.pop("anc", None),
        max_ctx=int(inp.ctx_lens.max()), **kw)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


CASES = [
    ("tree32k", (("ctx", (3000, 3000)),), 64),
    ("tree32k", (("ctx", (3000, 3000)),), 1024),
    ("tree32k", (("ctx", (2500, 5000)), ("batch", 2)), 128),
    ("chain_b16", (("ctx", (500, 2100)), ("batch", 4)), 64),
    ("chain_b16", (("ctx", (0, 700)), ("batch", 6), ("n_draft", 3)), 256),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_paged_small_cases(hsv, gpu, case):
    name, over, bs = CASES[case]
    inp = cached_inputs(name, over)
    kp, vp, table = _paged(inp, bs, 90 + case)
    o_ref, l_ref = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent,
                                      bf16=inp.is_bf16)
    for splits in (0, 1, 7):
        o, lse = _run(hsv, gpu, inp, kp, vp, table, num_splits=splits)
        assert_parity(o, lse, o_ref, l_ref, f"{name} {dict(over)} bs={bs} splits={splits}")


def test_paged_explicit_mask(hsv, gpu):
    import torch
    inp = cached_inputs("tree32k", (("ctx", (3000, 3000)),))
    kp, vp, table = _paged(inp, 128, 97)
    N = inp.wl.n_draft
    anc = synth.block_masks(N, 16)[None]
    o, lse = _run(hsv, gpu, inp, kp, vp, table, parent=None,
                  anc=torch.from_numpy(anc.view(np.int64)).to(gpu))
    o_ref, l_ref = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, anc_mask=anc, bf16=True)
    assert_parity(o, lse, o_ref, l_ref, "paged, block masks")


def test_paged_validate_flags_bad_table(hsv, gpu):
    import torch
    inp = cached_inputs("tree32k", (("ctx", (3000, 3000)),))
    kp, vp, table = _paged(inp, 128, 98)
    bad = table.copy()
    bad[0, 3] = kp.shape[0]            # one past the pool, in a block the prefix uses
    with pytest.raises(RuntimeError, match="DEVICE_CHECK"):
        _run(hsv, gpu, inp, kp, vp, bad, flags=hsv.HSV_FLAG_VALIDATE)
    o, lse = _run(hsv, gpu, inp, kp, vp, table, flags=hsv.HSV_FLAG_VALIDATE)
    assert np.isfinite(o).all()


@pytest.mark.parametrize("bs", [64, 256])
def test_paged_full_size_tree32k(hsv, gpu, bs):
    import torch
    inp = cached_inputs("tree32k")
    kp, vp, table = _paged(inp, bs, 99)
    o, lse = _run(hsv, gpu, inp, kp, vp, table)
    o_ref, l_ref = oracle_full("tree32k")
    o_err, l_err = assert_all_rows(o, lse, inp, f"paged tree32k bs={bs}", o_ref, l_ref)
    log(f"paged tree32k bs={bs}: all rows max|dO| = {o_err:.3e}, max rel dLSE = {l_err:.3e}")
    torch.cuda.empty_cache()
