"""GPU parity of verification attention over a paged cache (pool blocks and a
block table; HiSpec page: paged attention with block tables) against the
fp64 oracle on the contiguous view of the same cache.

The pool order is a seeded random permutation and the spare pool blocks hold
NaN, so a kernel that follows a wrong table entry fails parity.  Cases cover
both kernels that take a paged cache (256-row chunks and the small-group
kernel), block sizes 64 to 1024, ragged contexts including c = 0, forced
split counts, explicit masks, and the 32k-context tree at full size.

Sparse index sets over a paged cache (Dustin page: verification over the
selected subset of the cache) are checked against the oracle on the
contiguous view, and bit for bit against the contiguous sparse call, which
runs the same arithmetic; index sets with a -1 tail, a bad table entry under
validation, and the 64k-context sparse workload at full size.
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


def _run_sparse(hsv, gpu, inp, kp, vp, table, kv_idx, **kw):
    import torch
    o, lse = hsv.hsv_verify_attn_sparse_paged(
        to_dev(inp.q, True, gpu), to_dev(kp, True, gpu), to_dev(vp, True, gpu),
        torch.from_numpy(table).to(gpu), torch.from_numpy(inp.ctx_lens).to(gpu),
        torch.from_numpy(inp.parent).to(gpu), None, torch.from_numpy(kv_idx).to(gpu),
        max_ctx=int(inp.ctx_lens.max()), **kw)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def _run_sparse_contiguous(hsv, gpu, inp, kv_idx, **kw):
    import torch
    o, lse = hsv.hsv_verify_attn_sparse(
        to_dev(inp.q, True, gpu), to_dev(inp.k, True, gpu), to_dev(inp.v, True, gpu),
        torch.from_numpy(inp.ctx_lens).to(gpu), torch.from_numpy(inp.parent).to(gpu), None,
        torch.from_numpy(kv_idx).to(gpu), max_ctx=int(inp.ctx_lens.max()), **kw)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def _with_empty_tail(kv_idx, b, n_empty):
    """kv_idx with the last n_empty slots of every head of sequence b set to
    -1 (a shorter selection: the positions before stay strictly increasing)."""
    out = kv_idx.copy()
    out[b, :, out.shape[2] - n_empty:] = -1
    return out


SPARSE_CASES = [  # (workload overrides, block size, empty slots at the end of sequence 0)
    ((("ctx", (3000, 6000)), ("n_sel", 1024), ("n_recent", 128), ("batch", 2)), 64, 0),
    ((("ctx", (2000, 2000)), ("n_sel", 512), ("batch", 3), ("n_recent", 64)), 256, 200),
    ((("ctx", (700, 5000)), ("n_sel", 640), ("batch", 4), ("n_draft", 5), ("n_recent", 32)),
     128, 0),
    ((("ctx", (1500, 1500)), ("n_sel", 1500), ("batch", 1), ("n_q_heads", 8),
      ("n_kv_heads", 2)), 1024, 1),
]


@pytest.mark.parametrize("case", range(len(SPARSE_CASES)))
def test_sparse_paged_small_cases(hsv, gpu, case):
    over, bs, n_empty = SPARSE_CASES[case]
    inp = cached_inputs("sparse64k", over)
    kv_idx = _with_empty_tail(inp.kv_idx, 0, n_empty) if n_empty else inp.kv_idx
    kp, vp, table = _paged(inp, bs, 120 + case)
    kc, vc = oracle.paged_to_contiguous(kp, vp, table)
    o_ref, l_ref = oracle.verify_attn(inp.q, kc, vc, inp.ctx_lens, parent=inp.parent,
                                      kv_idx=kv_idx, bf16=True)
    for splits in (0, 1, 5):
        what = f"sparse paged {dict(over)} bs={bs} empty={n_empty} splits={splits}"
        o, lse = _run_sparse(hsv, gpu, inp, kp, vp, table, kv_idx, num_splits=splits)
        assert_parity(o, lse, o_ref, l_ref, what)
        o_c, l_c = _run_sparse_contiguous(hsv, gpu, inp, kv_idx, num_splits=splits)
        np.testing.assert_array_equal(o, o_c, err_msg=what)
        np.testing.assert_array_equal(lse, l_c, err_msg=what)


def test_sparse_paged_validate(hsv, gpu):
    inp = cached_inputs("sparse64k", SPARSE_CASES[0][0])
    kp, vp, table = _paged(inp, 64, 130)
    bad = table.copy()
    bad[1, 5] = -1                     # a block the prefix of sequence 1 uses
    with pytest.raises(RuntimeError, match="DEVICE_CHECK"):
        _run_sparse(hsv, gpu, inp, kp, vp, bad, inp.kv_idx, flags=hsv.HSV_FLAG_VALIDATE)
    idx = inp.kv_idx.copy()
    idx[0, 1, 7] = idx[0, 1, 6]        # not strictly increasing
    with pytest.raises(RuntimeError, match="DEVICE_CHECK"):
        _run_sparse(hsv, gpu, inp, kp, vp, table, idx, flags=hsv.HSV_FLAG_VALIDATE)
    o, lse = _run_sparse(hsv, gpu, inp, kp, vp, table, _with_empty_tail(inp.kv_idx, 1, 9),
                         flags=hsv.HSV_FLAG_VALIDATE)
    assert np.isfinite(o).all() and np.isfinite(lse).all()


def test_sparse_paged_rejects_other_shapes(hsv, gpu):
    """More than 32 grouped rows run on kernels without a paged form."""
    inp = cached_inputs("sparse64k", (("ctx", (2000, 2000)), ("n_sel", 512), ("batch", 1),
                                      ("n_draft", 16), ("n_recent", 64)))
    kp, vp, table = _paged(inp, 64, 131)
    with pytest.raises(RuntimeError, match="UNSUPPORTED"):
        _run_sparse(hsv, gpu, inp, kp, vp, table, inp.kv_idx)


def test_sparse_paged_full_size_sparse64k(hsv, gpu):
    import torch
    inp = cached_inputs("sparse64k")
    kp, vp, table = _paged(inp, 64, 132)
    o, lse = _run_sparse(hsv, gpu, inp, kp, vp, table, inp.kv_idx)
    o_ref, l_ref = oracle_full("sparse64k")
    o_err, l_err = assert_all_rows(o, lse, inp, "paged sparse64k bs=64", o_ref, l_ref)
    log(f"paged sparse64k bs=64: all rows max|dO| = {o_err:.3e}, max rel dLSE = {l_err:.3e}")
    torch.cuda.empty_cache()


def test_sparse_paged_out_of_range_indices_are_masked(hsv, gpu):
    """Index entries outside [0, c) in a paged sparse call take no part and
    are never turned into a pool address: the result is that of the set
    without them (the pool's spare blocks and unselected rows hold NaN)."""
    from test_gpu_parity import _garbage_indices
    inp = cached_inputs("sparse64k", SPARSE_CASES[0][0], poison=True)
    kp, vp, table = _paged(inp, SPARSE_CASES[0][1], 151)
    bad, clean = _garbage_indices(inp.kv_idx, inp.ctx_lens, inp.k.shape[2], 152)
    o, lse = _run_sparse(hsv, gpu, inp, kp, vp, table, bad)
    o_ref, l_ref = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent,
                                      kv_idx=clean, bf16=True)
    assert_parity(o, lse, o_ref, l_ref, "paged sparse, garbage indices")
