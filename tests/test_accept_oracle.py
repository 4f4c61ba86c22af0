"""Pins of the accepted-path KV update and tree position ids in the oracle
(CPU only): a worked example derived by hand, the ancestor bitmask as an
independent route to depth and path, closed forms for chains and stars, and
the inputs that must leave a sequence untouched."""

import json
import os

import numpy as np

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "accept_path.json")


def _cache(rng, B, H, S, D):
    # each row holds its own index so that moves are visible
    k = np.broadcast_to(np.arange(S, dtype=np.float32)[None, None, :, None], (B, H, S, D)).copy()
    k += rng.standard_normal((B, H, S, D)).astype(np.float32) * 1e-3
    v = -k
    return k, v


def test_worked_example():
    g = json.load(open(GOLDEN))
    par = np.array([g["parent"]], np.int32)
    c = g["ctx"]
    np.testing.assert_array_equal(oracle.tree_depth(par)[0], g["depth"])
    np.testing.assert_array_equal(oracle.tree_position_ids(par, np.array([c]))[0],
                                  g["position_ids"])
    np.testing.assert_array_equal(oracle.accepted_path(par[0], g["accept_node"]), g["path"])
    k = np.arange(20, dtype=np.float32).reshape(1, 1, 20, 1)
    k2, v2, ctx2 = oracle.accept_path(k, -k, np.array([c], np.int32), par,
                                      np.array([g["accept_node"]]))
    for dst, src in g["rows_after"].items():
        assert k2[0, 0, int(dst), 0] == src and v2[0, 0, int(dst), 0] == -src
    assert ctx2[0] == g["ctx_after"]


def test_depth_and_path_agree_with_ancestor_mask():
    rng = np.random.Generator(np.random.PCG64(41))
    trees = [synth.random_tree_parents(rng, 64, max_depth=d, max_branch=br)
             for d, br in ((2, 64), (5, 4), (9, 4), (64, 4))]
    trees += [synth.uniform_parents(rng, 64) for _ in range(4)]
    par = np.stack(trees).astype(np.int32)
    anc = oracle.ancestor_mask(par)
    depth = oracle.tree_depth(par)
    for b in range(par.shape[0]):
        for i in range(64):
            bits = [j for j in range(64) if (int(anc[b, i]) >> j) & 1]
            assert depth[b, i] == len(bits)
            np.testing.assert_array_equal(oracle.accepted_path(par[b], i), bits)


def test_chain_and_star_closed_forms():
    rng = np.random.Generator(np.random.PCG64(42))
    N, c, S = 8, 5, 20
    k, v = _cache(rng, 2, 3, S, 4)
    chain = synth.chain_parents(N)[None].repeat(2, 0)
    star = np.full((2, N), -1, np.int32)
    ctx = np.array([c, c], np.int32)
    np.testing.assert_array_equal(oracle.tree_position_ids(chain, ctx), np.tile(c + np.arange(N), (2, 1)))
    np.testing.assert_array_equal(oracle.tree_position_ids(star, ctx), np.full((2, N), c))
    k2, v2, ctx2 = oracle.accept_path(k, v, ctx, chain, np.array([3, N - 1]))
    np.testing.assert_array_equal(k2, k)          # a chain prefix is already in place
    np.testing.assert_array_equal(ctx2, [c + 4, c + N])
    k2, v2, ctx2 = oracle.accept_path(k, v, ctx, star, np.array([6, 0]))
    np.testing.assert_array_equal(k2[0, :, c], k[0, :, c + 6])
    np.testing.assert_array_equal(np.delete(k2[0], c, axis=1), np.delete(k[0], c, axis=1))
    np.testing.assert_array_equal(k2[1], k[1])
    np.testing.assert_array_equal(ctx2, [c + 1, c + 1])


def test_untouched_sequences():
    rng = np.random.Generator(np.random.PCG64(43))
    N, S = 6, 16
    k, v = _cache(rng, 5, 2, S, 4)
    par = np.array([[-1, 0, 1, 1, 3, 0]] * 5, np.int32)
    par[1, 4] = 4                                # self-parent: invalid
    ctx = np.array([3, 3, 3, 3, S - N + 1], np.int32)   # last: draft rows overflow S
    node = np.array([-1, 4, 6, -2, 4])
    k2, v2, ctx2 = oracle.accept_path(k, v, ctx, par, node)
    np.testing.assert_array_equal(k2, k)
    np.testing.assert_array_equal(v2, v)
    np.testing.assert_array_equal(ctx2, ctx)
    assert (oracle.tree_position_ids(par, ctx)[1] == -1).all()


def test_moved_rows_are_the_path_in_order():
    rng = np.random.Generator(np.random.PCG64(44))
    B, H, N, S, D = 6, 2, 64, 200, 3
    k, v = _cache(rng, B, H, S, D)
    par = np.stack([synth.random_tree_parents(rng, N, max_depth=8, max_branch=3)
                    for _ in range(B)]).astype(np.int32)
    ctx = rng.integers(0, S - N + 1, B).astype(np.int32)
    node = rng.integers(-1, N, B)
    k2, v2, ctx2 = oracle.accept_path(k, v, ctx, par, node)
    anc = oracle.ancestor_mask(par)
    for b in range(B):
        c = ctx[b]
        src = [] if node[b] < 0 else [j for j in range(N) if (int(anc[b, node[b]]) >> j) & 1]
        assert ctx2[b] == c + len(src)
        for t, j in enumerate(src):
            np.testing.assert_array_equal(k2[b, :, c + t], k[b, :, c + j])
            np.testing.assert_array_equal(v2[b, :, c + t], v[b, :, c + j])
        np.testing.assert_array_equal(k2[b, :, c + len(src):], k[b, :, c + len(src):])
        np.testing.assert_array_equal(k2[b, :, :c], k[b, :, :c])
