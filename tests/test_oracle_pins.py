"""Pins for the fp64 oracle against things other than itself.

The pages print no worked example, formula or table for the attention step,
so the oracle is pinned by:
  * brute force at 50 digits (mpmath) on tiny inputs, over every draft tree
    with four nodes;
  * a library routine (torch's scaled_dot_product_attention and logsumexp in
    fp64) with masks built here by transitive closure, not by a parent walk;
  * closed forms (zero query, one allowed key, identical keys);
  * the exactness of the log-sum-exp combination of the cache part and the
    speculative part (LongSpec page, section 2.C), and of any partition of the
    key set into parts;
  * chain-shaped drafts reducing to causal attention (bottom-right tril);
  * the sparse form reducing to the dense one when every index is selected,
    and to dense attention over the gathered (compressed) cache (Dustin page,
    "Verification workflow").
"""

import itertools
import math

import numpy as np
import pytest
import torch

import oracle
import synth

mp = pytest.importorskip("mpmath")


# ----------------------------------------------------------------------------
# independent helpers (closure by boolean matrix powers, not by walking)
# ----------------------------------------------------------------------------

def closure(parent):
    """R[i, j] = node j is node i or an ancestor of i (Warshall-style closure)."""
    parent = np.asarray(parent)
    n = parent.size
    adj = np.zeros((n, n), dtype=bool)
    for i, p in enumerate(parent):
        if p >= 0:
            adj[i, p] = True
    reach = np.eye(n, dtype=bool) | adj
    while True:
        nxt = reach | ((reach.astype(np.int64) @ reach.astype(np.int64)) > 0)
        if (nxt == reach).all():
            return reach
        reach = nxt


def full_mask(parent_b, c, n_draft, prefix_idx=None):
    """Boolean [N, c+N] mask: allowed cache positions for each draft node."""
    m = np.zeros((n_draft, c + n_draft), dtype=bool)
    if prefix_idx is None:
        m[:, :c] = True
    else:
        m[:, prefix_idx] = True
    m[:, c:] = closure(parent_b)
    return m


def to_f64(a, bf16):
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).double()
    return torch.from_numpy(np.ascontiguousarray(a)).double()


def sdpa_reference(q, k, v, ctx, parent, bf16, kv_idx=None, scale=None):
    """torch fp64 SDPA + logsumexp with an explicitly built mask."""
    B, N, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    qt, kt, vt = to_f64(q, bf16), to_f64(k, bf16), to_f64(v, bf16)
    sc = scale if scale is not None else 1.0 / math.sqrt(D)
    o_all = np.zeros((B, N, Hq, D))
    l_all = np.zeros((B, N, Hq))
    for b in range(B):
        c = int(ctx[b])
        for h in range(Hq):
            g = h // G
            mask = full_mask(parent[b], c, N, None if kv_idx is None else kv_idx[b, g])
            mt = torch.from_numpy(mask)
            qq = qt[b, :, h, :]                       # [N, D]
            kk = kt[b, g, :c + N, :]                  # [c+N, D]
            vv = vt[b, g, :c + N, :]
            kk = torch.where(torch.isnan(kk), torch.zeros_like(kk), kk)
            vv = torch.where(torch.isnan(vv), torch.zeros_like(vv), vv)
            o = torch.nn.functional.scaled_dot_product_attention(
                qq[None, None], kk[None, None], vv[None, None], attn_mask=mt[None, None],
                scale=sc)[0, 0]
            s = (qq @ kk.T) * sc
            s = s.masked_fill(~mt, float("-inf"))
            o_all[b, :, h] = o.numpy()
            l_all[b, :, h] = torch.logsumexp(s, dim=-1).numpy()
    return o_all, l_all


def mp_brute(q, k, v, c, parent_b, scale, prefix_idx=None):
    """50-digit brute force: p_t = exp(s_t) / sum exp(s) with no shift."""
    mp.mp.dps = 50
    N, D = q.shape
    mask = full_mask(parent_b, c, N, prefix_idx)
    o = np.zeros((N, D))
    lse = np.zeros(N)
    for i in range(N):
        allowed = [t for t in range(c + N) if mask[i, t]]
        s = {t: mp.mpf(scale) * mp.fsum(mp.mpf(float(q[i, x])) * mp.mpf(float(k[t, x]))
                                        for x in range(D)) for t in allowed}
        z = mp.fsum(mp.exp(s[t]) for t in allowed)
        lse[i] = float(mp.log(z))
        for x in range(D):
            o[i, x] = float(mp.fsum(mp.exp(s[t]) / z * mp.mpf(float(v[t, x])) for t in allowed))
    return o, lse


def all_parent_arrays(n):
    return itertools.product(*[range(-1, i) for i in range(n)])


# ----------------------------------------------------------------------------
# ancestor mask (a1)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_ancestor_mask_all_trees_match_closure(n):
    trees = np.array(list(all_parent_arrays(n)), dtype=np.int32)
    assert trees.shape[0] == math.factorial(n)
    anc = oracle.ancestor_mask(trees)
    for t, row in zip(trees, anc):
        reach = closure(t)
        for i in range(n):
            expect = sum(1 << j for j in range(n) if reach[i, j])
            assert int(row[i]) == expect


def test_ancestor_mask_closed_forms():
    n = 64
    chain = np.arange(-1, n - 1, dtype=np.int32)[None]
    anc = oracle.ancestor_mask(chain)[0]
    for i in range(n):
        assert int(anc[i]) == (1 << (i + 1)) - 1
    star = np.full((1, n), -1, dtype=np.int32)
    anc = oracle.ancestor_mask(star)[0]
    for i in range(n):
        assert int(anc[i]) == 1 << i


def test_ancestor_popcount_is_depth():
    rng = np.random.default_rng(7)
    parent = synth.random_tree_parents(rng, 64, max_depth=8)
    anc = oracle.ancestor_mask(parent[None])[0]
    for i in range(64):
        depth, j = 0, i
        while j >= 0:
            depth += 1
            j = parent[j]
        assert bin(int(anc[i])).count("1") == depth


@pytest.mark.parametrize("bad", [[0], [-2], [-1, 1], [-1, 0, 5]])
def test_ancestor_mask_rejects_bad_parents(bad):
    with pytest.raises(ValueError):
        oracle.ancestor_mask(np.array([bad], dtype=np.int32))


# ----------------------------------------------------------------------------
# masked attention: brute force, library routine, closed forms
# ----------------------------------------------------------------------------

def _tiny_case(rng, c, n, d, hkv=1, g=1, cap_extra=1):
    cap = c + n + cap_extra
    q = rng.standard_normal((1, n, hkv * g, d)).astype(np.float32)
    k = rng.standard_normal((1, hkv, cap, d)).astype(np.float32)
    v = rng.standard_normal((1, hkv, cap, d)).astype(np.float32)
    k[:, :, c + n:] = np.nan
    v[:, :, c + n:] = np.nan
    return q, k, v


def test_brute_force_all_four_node_trees():
    rng = np.random.default_rng(11)
    c, n, d = 3, 4, 3
    q, k, v = _tiny_case(rng, c, n, d)
    scale = 0.7
    for tree in all_parent_arrays(n):
        parent = np.array([tree], dtype=np.int32)
        o, lse = oracle.verify_attn(q, k, v, np.array([c]), parent=parent, bf16=False,
                                    scale=scale)
        ob, lb = mp_brute(q[0, :, 0], k[0, 0], v[0, 0], c, parent[0], scale)
        np.testing.assert_allclose(o[0, :, 0], ob, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[0, :, 0], lb, rtol=0, atol=1e-13)


@pytest.mark.parametrize("c,n,d", [(0, 4, 2), (1, 3, 4), (4, 4, 4), (4, 1, 1)])
def test_brute_force_shapes_and_sparse(c, n, d):
    rng = np.random.default_rng(100 + c * 10 + n)
    q, k, v = _tiny_case(rng, c, n, d)
    parent = np.array([synth.uniform_parents(rng, n)], dtype=np.int32)
    o, lse = oracle.verify_attn(q, k, v, np.array([c]), parent=parent, bf16=False)
    ob, lb = mp_brute(q[0, :, 0], k[0, 0], v[0, 0], c, parent[0], 1 / math.sqrt(d))
    np.testing.assert_allclose(o[0, :, 0], ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, :, 0], lb, rtol=0, atol=1e-13)
    if c >= 2:
        idx = np.array([[[0, c - 1]]], dtype=np.int32)
        o, lse = oracle.verify_attn(q, k, v, np.array([c]), parent=parent, kv_idx=idx,
                                    bf16=False)
        ob, lb = mp_brute(q[0, :, 0], k[0, 0], v[0, 0], c, parent[0], 1 / math.sqrt(d),
                          prefix_idx=[0, c - 1])
        np.testing.assert_allclose(o[0, :, 0], ob, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[0, :, 0], lb, rtol=0, atol=1e-13)


@pytest.mark.parametrize("bf16", [False, True])
def test_matches_torch_sdpa_gqa_ragged(bf16):
    rng = np.random.default_rng(21)
    B, N, Hq, Hkv, D = 3, 9, 6, 2, 16
    ctx = np.array([0, 37, 80], dtype=np.int32)
    cap = 80 + N + 5
    qf = rng.standard_normal((B, N, Hq, D)).astype(np.float32)
    kf = rng.standard_normal((B, Hkv, cap, D)).astype(np.float32) * 0.8
    vf = rng.standard_normal((B, Hkv, cap, D)).astype(np.float32)
    for b in range(B):
        kf[b, :, ctx[b] + N:] = np.nan
        vf[b, :, ctx[b] + N:] = np.nan
    parent = np.stack([synth.uniform_parents(rng, N) for _ in range(B)])
    enc = synth.f32_to_bf16_bits if bf16 else (lambda a: a)
    q, k, v = enc(qf), enc(kf), enc(vf)
    o, lse = oracle.verify_attn(q, k, v, ctx, parent=parent, bf16=bf16)
    o_ref, l_ref = sdpa_reference(q, k, v, ctx, parent, bf16)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, l_ref, rtol=0, atol=1e-12)


def test_explicit_anc_mask_equals_parent_walk_and_general_masks():
    rng = np.random.default_rng(5)
    B, N, Hq, Hkv, D, c = 1, 12, 2, 1, 8, 20
    q, k, v = _tiny_case(rng, c, N, D, hkv=Hkv, g=Hq)
    parent = synth.random_tree_parents(rng, N, max_depth=4)[None]
    anc = oracle.ancestor_mask(parent)
    a = oracle.verify_attn(q, k, v, np.array([c]), parent=parent, bf16=False)
    b = oracle.verify_attn(q, k, v, np.array([c]), anc_mask=anc, bf16=False)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    # a non-tree mask (block-bidirectional draft blocks): compare with SDPA
    blocks = np.arange(N) // 4
    anc2 = np.array([[sum(1 << j for j in range(N) if blocks[j] == blocks[i])
                      for i in range(N)]], dtype=np.uint64)
    o, lse = oracle.verify_attn(q, k, v, np.array([c]), anc_mask=anc2, bf16=False)
    for h in range(Hq):
        mask = np.zeros((N, c + N), dtype=bool)
        mask[:, :c] = True
        mask[:, c:] = blocks[:, None] == blocks[None, :]
        qq = torch.from_numpy(q[0, :, h]).double()
        kk = torch.from_numpy(k[0, 0, :c + N]).double()
        vv = torch.from_numpy(v[0, 0, :c + N]).double()
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq[None], kk[None], vv[None], attn_mask=torch.from_numpy(mask)[None])[0]
        np.testing.assert_allclose(o[0, :, h], ref.numpy(), rtol=0, atol=1e-12)


def test_closed_form_zero_query():
    rng = np.random.default_rng(3)
    c, N, D = 50, 8, 16
    _, k, v = _tiny_case(rng, c, N, D)
    q = np.zeros((1, N, 1, D), dtype=np.float32)
    parent = synth.uniform_parents(rng, N)[None]
    o, lse = oracle.verify_attn(q, k, v, np.array([c]), parent=parent, bf16=False)
    reach = closure(parent[0])
    for i in range(N):
        allowed = list(range(c)) + [c + j for j in range(N) if reach[i, j]]
        np.testing.assert_allclose(lse[0, i, 0], math.log(len(allowed)), rtol=0, atol=1e-13)
        np.testing.assert_allclose(o[0, i, 0], v[0, 0, allowed].astype(np.float64).mean(0),
                                   rtol=0, atol=1e-13)


def test_closed_form_single_key_and_identical_keys():
    rng = np.random.default_rng(4)
    N, D = 5, 8
    q, k, v = _tiny_case(rng, 0, N, D)
    star = np.full((1, N), -1, dtype=np.int32)       # every node sees only itself
    o, lse = oracle.verify_attn(q, k, v, np.array([0]), parent=star, bf16=False, scale=0.3)
    for i in range(N):
        s = 0.3 * float(np.dot(q[0, i, 0].astype(np.float64), k[0, 0, i].astype(np.float64)))
        np.testing.assert_allclose(lse[0, i, 0], s, rtol=0, atol=1e-13)
        np.testing.assert_allclose(o[0, i, 0], v[0, 0, i], rtol=0, atol=1e-15)
    # identical keys: uniform weights
    c = 30
    q, k, v = _tiny_case(rng, c, N, D)
    k[0, 0, :c + N] = k[0, 0, 0]
    chain = synth.chain_parents(N)[None]
    o, lse = oracle.verify_attn(q, k, v, np.array([c]), parent=chain, bf16=False)
    for i in range(N):
        n_allowed = c + i + 1
        s = float(np.dot(q[0, i, 0].astype(np.float64), k[0, 0, 0].astype(np.float64))) / math.sqrt(D)
        np.testing.assert_allclose(lse[0, i, 0], s + math.log(n_allowed), rtol=0, atol=1e-12)
        np.testing.assert_allclose(o[0, i, 0], v[0, 0, :n_allowed].astype(np.float64).mean(0),
                                   rtol=0, atol=1e-12)


def test_empty_row_and_part_selection():
    rng = np.random.default_rng(6)
    N, D = 4, 8
    q, k, v = _tiny_case(rng, 0, N, D)
    parent = synth.chain_parents(N)[None]
    o, lse = oracle.verify_attn(q, k, v, np.array([0]), parent=parent, bf16=False,
                                parts=oracle.PART_PREFIX)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


# ----------------------------------------------------------------------------
# exact merge (a4) and split invariance
# ----------------------------------------------------------------------------

def test_prefix_and_tree_parts_merge_to_whole():
    rng = np.random.default_rng(8)
    B, N, Hq, Hkv, D, c = 1, 16, 4, 2, 32, 300
    q, k, v = _tiny_case(rng, c, N, D, hkv=Hkv, g=Hq // Hkv)
    parent = synth.random_tree_parents(rng, N, max_depth=5)[None]
    args = (q, k, v, np.array([c]))
    whole = oracle.verify_attn(*args, parent=parent, bf16=False)
    pre = oracle.verify_attn(*args, parent=parent, bf16=False, parts=oracle.PART_PREFIX)
    tre = oracle.verify_attn(*args, parent=parent, bf16=False, parts=oracle.PART_TREE)
    for i in range(N):
        for h in range(Hq):
            o, l = oracle.lse_merge([pre[1][0, i, h], tre[1][0, i, h]],
                                    np.stack([pre[0][0, i, h], tre[0][0, i, h]]))
            np.testing.assert_allclose(o, whole[0][0, i, h], rtol=0, atol=1e-12)
            assert abs(l - whole[1][0, i, h]) <= 1e-12


def test_random_partition_of_prefix_merges_to_dense():
    rng = np.random.default_rng(9)
    N, D, c = 6, 16, 200
    q, k, v = _tiny_case(rng, c, N, D)
    parent = synth.uniform_parents(rng, N)[None]
    args = (q, k, v, np.array([c]))
    whole = oracle.verify_attn(*args, parent=parent, bf16=False)
    labels = rng.integers(0, 5, size=c)
    parts_o, parts_l = [], []
    for lab in range(5):
        idx = np.nonzero(labels == lab)[0].astype(np.int32)
        o, l = oracle.verify_attn(*args, parent=parent, kv_idx=idx[None, None], bf16=False,
                                  parts=oracle.PART_PREFIX)
        parts_o.append(o)
        parts_l.append(l)
    o, l = oracle.verify_attn(*args, parent=parent, bf16=False, parts=oracle.PART_TREE)
    parts_o.append(o)
    parts_l.append(l)
    order = rng.permutation(len(parts_o))
    for i in range(N):
        lo = np.array([parts_l[p][0, i, 0] for p in order])
        oo = np.stack([parts_o[p][0, i, 0] for p in order])
        om, lm = oracle.lse_merge(lo, oo)
        np.testing.assert_allclose(om, whole[0][0, i, 0], rtol=0, atol=1e-12)
        assert abs(lm - whole[1][0, i, 0]) <= 1e-12


def test_merge_identity_and_empty():
    o_parts = np.array([[1.0, 2.0], [5.0, 7.0]])
    o, l = oracle.lse_merge(np.array([0.3, -np.inf]), o_parts)
    np.testing.assert_array_equal(o, o_parts[0])
    assert l == 0.3
    o, l = oracle.lse_merge(np.array([-np.inf, -np.inf]), o_parts)
    assert np.all(o == 0) and np.isneginf(l)
    o, l = oracle.lse_merge(np.array([math.log(1.0), math.log(3.0)]), o_parts)
    np.testing.assert_allclose(o, 0.25 * o_parts[0] + 0.75 * o_parts[1], rtol=0, atol=1e-15)
    assert abs(l - math.log(4.0)) < 1e-15


# ----------------------------------------------------------------------------
# chain = causal, GQA, sparse reductions
# ----------------------------------------------------------------------------

def test_chain_is_bottom_right_causal():
    rng = np.random.default_rng(10)
    N, Hq, Hkv, D, c = 8, 4, 2, 32, 120
    q, k, v = _tiny_case(rng, c, N, D, hkv=Hkv, g=Hq // Hkv)
    chain = synth.chain_parents(N)[None]
    o, lse = oracle.verify_attn(q, k, v, np.array([c]), parent=chain, bf16=False)
    causal = torch.ones(N, c + N, dtype=torch.bool).tril(diagonal=c)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        qq = torch.from_numpy(q[0, :, h]).double()
        kk = torch.from_numpy(k[0, g, :c + N]).double()
        vv = torch.from_numpy(v[0, g, :c + N]).double()
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq[None], kk[None], vv[None], attn_mask=causal[None])[0]
        np.testing.assert_allclose(o[0, :, h], ref.numpy(), rtol=0, atol=1e-12)


def test_gqa_equals_mha_on_repeated_kv():
    rng = np.random.default_rng(12)
    N, Hq, Hkv, D, c = 5, 6, 2, 8, 40
    G = Hq // Hkv
    q, k, v = _tiny_case(rng, c, N, D, hkv=Hkv, g=G)
    parent = synth.uniform_parents(rng, N)[None]
    a = oracle.verify_attn(q, k, v, np.array([c]), parent=parent, bf16=False)
    kr = np.repeat(k, G, axis=1)
    vr = np.repeat(v, G, axis=1)
    b = oracle.verify_attn(q, kr, vr, np.array([c]), parent=parent, bf16=False)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-14)


def test_sparse_all_indices_equals_dense():
    inp = synth.make_inputs("sparse64k", ctx=(700, 700), n_sel=700, n_recent=96, batch=2,
                            n_q_heads=4, n_kv_heads=2, head_dim=32)
    assert (inp.kv_idx == np.arange(700)).all()
    dense = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent, bf16=True)
    sparse = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent,
                                kv_idx=inp.kv_idx, bf16=True)
    np.testing.assert_allclose(sparse[0], dense[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(sparse[1], dense[1], rtol=0, atol=1e-12)


def test_sparse_set_with_empty_slots_equals_dense():
    """A set that holds the whole history followed by -1 slots (what the
    selection writes when the history is shorter than the set) attends to
    exactly the dense prefix; a -1 before a position is rejected."""
    inp = synth.make_inputs("sparse64k", ctx=(300, 300), n_sel=300, n_recent=32, batch=2,
                            n_q_heads=4, n_kv_heads=2, head_dim=32)
    c = 300
    assert (inp.kv_idx == np.arange(c)).all()
    padded = np.concatenate([inp.kv_idx, np.full(inp.kv_idx.shape[:2] + (57,), -1, np.int32)],
                            axis=2)
    dense = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent, bf16=True)
    sparse = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent,
                                kv_idx=padded, bf16=True)
    np.testing.assert_allclose(sparse[0], dense[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(sparse[1], dense[1], rtol=0, atol=1e-12)
    bad = padded.copy()
    bad[1, 0, c + 3] = 5                  # a position after a -1 slot
    with pytest.raises(ValueError):
        oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent, kv_idx=bad,
                           bf16=True)
    bad = padded.copy()
    bad[0, 1, 7] = -2
    with pytest.raises(ValueError):
        oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent, kv_idx=bad,
                           bf16=True)


def test_sparse_equals_dense_over_gathered_cache_and_ignores_poison():
    kw = dict(ctx=(1500, 1500), n_sel=300, n_recent=64, batch=2, n_q_heads=4, n_kv_heads=2,
              head_dim=32)
    clean = synth.make_inputs("sparse64k", **kw)
    poisoned = synth.make_inputs("sparse64k", poison_unselected=True, **kw)
    s_clean = oracle.verify_attn(clean.q, clean.k, clean.v, clean.ctx_lens, parent=clean.parent,
                                 kv_idx=clean.kv_idx, bf16=True)
    s_pois = oracle.verify_attn(poisoned.q, poisoned.k, poisoned.v, poisoned.ctx_lens,
                                parent=poisoned.parent, kv_idx=poisoned.kv_idx, bf16=True)
    np.testing.assert_array_equal(s_clean[0], s_pois[0])
    np.testing.assert_array_equal(s_clean[1], s_pois[1])
    assert np.isfinite(s_pois[0]).all()
    # compressed cache: selected rows, then the draft block at its tail
    kg, vg = oracle.gather_kv(clean.k, clean.v, clean.kv_idx)
    B, Hkv, n_sel, D = kg.shape
    N = clean.wl.n_draft
    kc = np.concatenate([kg, clean.k[:, :, 1500:1500 + N]], axis=2)
    vc = np.concatenate([vg, clean.v[:, :, 1500:1500 + N]], axis=2)
    dense = oracle.verify_attn(clean.q, kc, vc, np.full(B, n_sel, dtype=np.int32),
                               parent=clean.parent, bf16=True)
    np.testing.assert_allclose(s_clean[0], dense[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(s_clean[1], dense[1], rtol=0, atol=1e-12)


def test_sparse_matches_sdpa():
    inp = synth.make_inputs("sparse64k", ctx=(900, 900), n_sel=200, n_recent=50, batch=1,
                            n_q_heads=4, n_kv_heads=2, head_dim=16)
    o, lse = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent,
                                kv_idx=inp.kv_idx, bf16=True)
    o_ref, l_ref = sdpa_reference(inp.q, inp.k, inp.v, inp.ctx_lens, inp.parent, True,
                                  kv_idx=inp.kv_idx)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, l_ref, rtol=0, atol=1e-12)


def test_row_subset_matches_full():
    inp = synth.make_inputs("tree32k", ctx=(500, 500), n_q_heads=8, n_kv_heads=2, head_dim=32,
                            n_draft=16)
    full = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent, bf16=True)
    rows = [(0, 3, 5), (0, 15, 0), (0, 0, 7)]
    sub = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent, bf16=True,
                             rows=rows)
    for r, (b, i, h) in enumerate(rows):
        np.testing.assert_array_equal(sub[0][r], full[0][b, i, h])
        assert sub[1][r] == full[1][b, i, h]
