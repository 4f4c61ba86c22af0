"""Caches and pools past the 2 GiB and 4 GiB byte offsets, on the GPU.

A KV cache [B, Hkv, S_cap, D] of a few sequences at long capacities, or a
paged pool of many blocks, passes 2^31 and 2^32 bytes (and, per slice at
16.8M rows of 128 features, 2^31 elements), so every kernel must form its
row addresses in 64 bits.  Each case puts a small seeded problem into such a
buffer -- the rest NaN, so a wrapped address that lands anywhere else fails
-- and compares the result with the fp64 oracle on the small problem:

- one long capacity (1,179,648 rows per (sequence, KV head): 4.8 GB per
  tensor, sequence 1's KV heads from 2.4 GB to 4.5 GB and past), through
  every verification kernel (the 256-row DMA kernel, the small-group kernel
  dense and sparse, the register-staged MFMA kernel, the fp32 VALU kernel),
  the compressed-cache gather and the accepted-path update;
- one (sequence, KV head) of 17,000,000 rows (4.35 GB per tensor): an index
  set whose positions straddle 2^23 and 2^24 rows (2^31 and 2^32 bytes) and
  a draft block past both, against the oracle's dense attention over the
  gathered rows (a gather over a set equals dense attention over it);
- a paged pool of 18,000 blocks (4.7 GB per tensor) whose table names blocks
  on both sides of 2 GiB and 4 GiB, dense and sparse.
"""

import numpy as np
import pytest

import oracle
import synth
from util import assert_parity, log, to_dev

pytestmark = pytest.mark.gpu

BIG_CAP = 1_179_648          # rows per (sequence, KV head): 302 MB slices at D = 128 bf16
DEEP_CAP = 17_000_000        # one slice past 2^24 rows
POOL_BLOCKS = 18_000         # 256 KB pool blocks (8 KV heads x 128 rows x 256 B)


@pytest.fixture(scope="module")
def hsv(gpu):
    import long_context_tree_verify_amd as m
    return m


def _nan_cache(shape, bf16, gpu):
    import torch
    return torch.full(shape, float("nan"), dtype=torch.bfloat16 if bf16 else torch.float32,
                      device=gpu)


def _free():
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# (workload, overrides, kernel the plan takes)
LONG_CASES = [
    ("tree32k", dict(batch=2, ctx=(1500, 3000)), "256-row DMA"),
    ("chain_b16", dict(batch=2, ctx=(1000, 2500)), "small-group dense"),
    ("tree32k", dict(batch=2, n_draft=16, tree="uniform", ctx=(800, 2000)), "MFMA, 64 rows"),
    ("chain_b16", dict(batch=2, ctx=(3000, 4000), n_sel=512, n_sink=4, n_recent=64),
     "small-group sparse"),
    ("tiny_tree", dict(batch=2, n_q_heads=8, n_kv_heads=8, ctx=(300, 600)), "fp32 VALU"),
]


@pytest.mark.parametrize("case", range(len(LONG_CASES)))
def test_long_capacity(hsv, gpu, case):
    import torch
    name, over, kern = LONG_CASES[case]
    inp = synth.make_inputs(name, seed=7100 + case, **over)
    bf = inp.is_bf16
    B, Hkv, S, D = inp.k.shape
    log(f"long capacity case {case} ({kern}): {name} {over}, cache rows {BIG_CAP}")
    k = _nan_cache((B, Hkv, BIG_CAP, D), bf, gpu)
    v = _nan_cache((B, Hkv, BIG_CAP, D), bf, gpu)
    k[:, :, :S].copy_(to_dev(inp.k, bf, gpu))
    v[:, :, :S].copy_(to_dev(inp.v, bf, gpu))
    assert k.numel() * k.element_size() > 4 << 30
    q = to_dev(inp.q, bf, gpu)
    ctx = torch.from_numpy(inp.ctx_lens).to(gpu)
    parent = torch.from_numpy(inp.parent).to(gpu)
    max_ctx = int(inp.ctx_lens.max())
    if inp.kv_idx is not None:
        o, lse = hsv.hsv_verify_attn_sparse(q, k, v, ctx, parent, None,
                                            torch.from_numpy(inp.kv_idx).to(gpu), max_ctx=max_ctx)
    else:
        o, lse = hsv.hsv_verify_attn(q, k, v, ctx, parent, None, max_ctx=max_ctx)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent,
                                      kv_idx=inp.kv_idx, bf16=bf)
    assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"long capacity {kern}")

    if case == 3:
        # the compressed cache from the same slices: a bit-exact copy
        kg, vg = hsv.hsv_gather_kv(k, v, torch.from_numpy(inp.kv_idx).to(gpu))
        rk, rv = oracle.gather_kv(inp.k, inp.v, inp.kv_idx)
        np.testing.assert_array_equal(kg.view(torch.int16).cpu().numpy(), rk.view(np.int16))
        np.testing.assert_array_equal(vg.view(torch.int16).cpu().numpy(), rv.view(np.int16))
        log("  gather over the long slices: identical")
    if case == 0:
        # the accepted-path update in the same slices (deepest node of each tree)
        node = np.array([inp.wl.n_draft - 1] * B, np.int64)
        hsv.hsv_accept_path(k, v, ctx, parent, torch.from_numpy(node.astype(np.int32)).to(gpu))
        torch.cuda.synchronize()
        rk, rv, rc = oracle.accept_path(inp.k, inp.v, inp.ctx_lens, inp.parent, node)
        np.testing.assert_array_equal(ctx.cpu().numpy(), rc)
        np.testing.assert_array_equal(k[:, :, :S].view(torch.int16).cpu().numpy(),
                                      rk.view(np.int16))
        np.testing.assert_array_equal(v[:, :, :S].view(torch.int16).cpu().numpy(),
                                      rv.view(np.int16))
        log(f"  accepted paths in the long slices: caches and lengths identical ({rc.tolist()})")
    del k, v
    _free()


def test_deep_slice_index_set(hsv, gpu):
    import torch
    n_sel, N = 512, 8
    # the small problem: rows [0, n_sel) are the selected rows, [n_sel, n_sel + N) the draft
    inp = synth.make_inputs("chain_b16", seed=7200, batch=1, n_q_heads=4, n_kv_heads=1,
                            ctx=(n_sel, n_sel), n_draft=N)
    c = DEEP_CAP - 64
    rng = np.random.Generator(np.random.PCG64(7201))
    fixed = np.array([0, 1, 2, 3, (1 << 23) - 1, 1 << 23, (1 << 24) - 1, 1 << 24, 1 << 24 | 1,
                      c - 2, c - 1], np.int64)
    rest = np.setdiff1d(np.unique(rng.integers(4, c - 2, size=2 * n_sel)), fixed)
    pos = np.sort(np.concatenate([fixed, rng.choice(rest, n_sel - len(fixed), replace=False)]))
    assert len(np.unique(pos)) == n_sel and pos[-1] < c
    log(f"deep slice: {DEEP_CAP} rows, c = {c}, positions {pos[:6].tolist()} ... "
        f"{pos[-4:].tolist()}")
    D = inp.k.shape[3]
    k = _nan_cache((1, 1, DEEP_CAP, D), True, gpu)
    v = _nan_cache((1, 1, DEEP_CAP, D), True, gpu)
    assert k.numel() * k.element_size() > 4 << 30
    where = torch.from_numpy(pos).to(gpu)
    k[0, 0, where] = to_dev(inp.k[0, 0, :n_sel], True, gpu)
    v[0, 0, where] = to_dev(inp.v[0, 0, :n_sel], True, gpu)
    k[0, 0, c:c + N] = to_dev(inp.k[0, 0, n_sel:n_sel + N], True, gpu)
    v[0, 0, c:c + N] = to_dev(inp.v[0, 0, n_sel:n_sel + N], True, gpu)
    q = to_dev(inp.q, True, gpu)
    ctx = torch.tensor([c], dtype=torch.int32, device=gpu)
    parent = torch.from_numpy(inp.parent).to(gpu)
    idx = torch.from_numpy(pos.astype(np.int32).reshape(1, 1, n_sel)).to(gpu)
    o, lse = hsv.hsv_verify_attn_sparse(q, k, v, ctx, parent, None, idx, max_ctx=c)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent,
                                      bf16=True)
    assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "deep slice, index set")

    # the draft block alone, at rows past 2^24 (the dense call, no prefix)
    o, lse = hsv.hsv_verify_attn(q, k, v, ctx, parent, None, max_ctx=c,
                                 flags=hsv.HSV_FLAG_NO_PREFIX)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent,
                                      bf16=True, parts=oracle.PART_TREE)
    assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "deep slice, draft block")

    # the compressed cache from the deep slice
    kg, vg = hsv.hsv_gather_kv(k, v, idx)
    np.testing.assert_array_equal(kg.view(torch.int16).cpu().numpy()[0, 0],
                                  inp.k[0, 0, :n_sel].view(np.int16))
    np.testing.assert_array_equal(vg.view(torch.int16).cpu().numpy()[0, 0],
                                  inp.v[0, 0, :n_sel].view(np.int16))
    log("  gather from the deep slice: identical")
    del k, v, where
    _free()


@pytest.mark.parametrize("sparse", [False, True])
def test_pool_past_4gib(hsv, gpu, sparse):
    import torch
    bs = 128
    if sparse:
        inp = synth.make_inputs("chain_b16", seed=7300, batch=2, ctx=(3000, 4000), n_sel=512,
                                n_sink=4, n_recent=64)
    else:
        inp = synth.make_inputs("tree32k", seed=7301, batch=2, ctx=(2500, 3800))
    B, Hkv, S, D = inp.k.shape
    cap = -(-S // bs) * bs
    nb = cap // bs
    rng = np.random.Generator(np.random.PCG64(7302 + sparse))
    table = rng.choice(POOL_BLOCKS, size=B * nb, replace=False).astype(np.int32).reshape(B, nb)
    blk_bytes = Hkv * bs * D * 2
    above = int((table.astype(np.int64) * blk_bytes >= 4 << 30).sum())
    log(f"pool of {POOL_BLOCKS} blocks ({POOL_BLOCKS * blk_bytes / 2**30:.2f} GiB per tensor), "
        f"{above} of {table.size} table entries past 4 GiB, sparse={sparse}")
    assert above > 0
    kp = _nan_cache((POOL_BLOCKS, Hkv, bs, D), True, gpu)
    vp = _nan_cache((POOL_BLOCKS, Hkv, bs, D), True, gpu)
    pad = ((0, 0), (0, 0), (0, cap - S), (0, 0))
    for src, pool in ((inp.k, kp), (inp.v, vp)):
        full = np.pad(src, pad, constant_values=synth.gen.BF16_NAN)
        blocks = full.reshape(B, Hkv, nb, bs, D).transpose(0, 2, 1, 3, 4).reshape(B * nb, Hkv,
                                                                                   bs, D)
        pool[torch.from_numpy(table.reshape(-1).astype(np.int64)).to(gpu)] = to_dev(
            np.ascontiguousarray(blocks), True, gpu)
    args = (to_dev(inp.q, True, gpu), kp, vp, torch.from_numpy(table).to(gpu),
            torch.from_numpy(inp.ctx_lens).to(gpu), torch.from_numpy(inp.parent).to(gpu), None)
    if sparse:
        o, lse = hsv.hsv_verify_attn_sparse_paged(*args, torch.from_numpy(inp.kv_idx).to(gpu),
                                                  max_ctx=int(inp.ctx_lens.max()))
    else:
        o, lse = hsv.hsv_verify_attn_paged(*args, max_ctx=int(inp.ctx_lens.max()))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent,
                                      kv_idx=inp.kv_idx, bf16=True)
    assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref,
                  f"pool past 4 GiB, sparse={sparse}")
    del kp, vp
    _free()
