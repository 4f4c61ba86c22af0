"""Pins of the oracle for draft trees of more than 64 nodes (masks of
several 64-bit words; word w holds nodes 64w .. 64w + 63).  Checked against
the Python path walk and depth (a route independent of the C code), between
the oracle's two mask sources (parent walk and explicit words), and a
256-node chain against a direct fp64 softmax."""

import numpy as np
import pytest

import oracle
import synth


def _trees(rng, n):
    return np.stack([
        synth.chain_parents(n),
        np.full(n, -1, np.int32),
        synth.uniform_parents(rng, n),
        synth.random_tree_parents(rng, n, max_depth=12, max_branch=4),
        synth.random_tree_parents(rng, n, max_depth=n, max_branch=2),
    ]).astype(np.int32)


@pytest.mark.parametrize("n", [65, 128, 200, 256])
def test_wide_masks_match_the_path_walk(n):
    rng = np.random.Generator(np.random.PCG64(n))
    par = _trees(rng, n)
    anc = oracle.ancestor_mask(par)
    assert anc.shape == (par.shape[0], n, oracle.mask_words(n))
    depth = oracle.tree_depth(par)
    for b in range(par.shape[0]):
        for i in range(0, n, 7):
            bits = [j for j in range(n) if (int(anc[b, i, j // 64]) >> (j % 64)) & 1]
            np.testing.assert_array_equal(bits, oracle.accepted_path(par[b], i))
            assert len(bits) == depth[b, i]


def test_wide_parent_and_mask_sources_agree():
    rng = np.random.Generator(np.random.PCG64(7))
    inp = synth.make_inputs("tree32k", ctx=(300, 300), n_draft=160, n_q_heads=4, n_kv_heads=2,
                            head_dim=64, max_depth=20)
    rows = [(0, i, h) for i in range(0, 160, 9) for h in range(4)]
    o1, l1 = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent, bf16=True,
                                rows=rows)
    anc = oracle.ancestor_mask(inp.parent)
    o2, l2 = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, anc_mask=anc, bf16=True,
                                rows=rows)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    # and a mask that is not a tree: block-parallel rows see their 40-node block
    blocks = np.arange(160) // 40
    wide = np.zeros((1, 160, 3), np.uint64)
    for i in range(160):
        for j in np.flatnonzero(blocks == blocks[i]):
            wide[0, i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    o3, l3 = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, anc_mask=wide, bf16=True,
                                rows=rows)
    assert not np.array_equal(l3, l1)


def test_chain_of_256_is_causal_attention():
    rng = np.random.Generator(np.random.PCG64(8))
    B, N, H, D, c = 1, 256, 1, 16, 40
    q = rng.standard_normal((B, N, H, D)).astype(np.float32)
    k = rng.standard_normal((B, H, c + N, D)).astype(np.float32)
    v = rng.standard_normal((B, H, c + N, D)).astype(np.float32)
    par = synth.chain_parents(N)[None].astype(np.int32)
    o, lse = oracle.verify_attn(q, k, v, np.array([c], np.int32), parent=par, bf16=False)
    for i in (0, 63, 64, 65, 200, 255):
        s = (k[0, 0, :c + i + 1].astype(np.float64) @ q[0, i, 0].astype(np.float64)) / np.sqrt(D)
        p = np.exp(s - s.max())
        ref_lse = s.max() + np.log(p.sum())
        ref_o = (p / p.sum()) @ v[0, 0, :c + i + 1].astype(np.float64)
        assert abs(lse[0, i, 0] - ref_lse) < 1e-9
        np.testing.assert_allclose(o[0, i, 0], ref_o, atol=1e-9)
