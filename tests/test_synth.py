"""Seeded input generators: determinism and the structure each workload states."""

import numpy as np
import pytest
import torch

import synth


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 3,
        np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 1e-40, 3.3895e38, 65504.0], np.float32),
        # exact ties in the low half: 0x3F808000 rounds to even
        np.array([0x3F808000, 0x3F818000, 0x3F80FFFF, 0x3F807FFF], np.uint32).view(np.float32),
    ])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    nan = synth.f32_to_bf16_bits(np.array([np.nan], np.float32))
    assert np.isnan(synth.bf16_bits_to_f32(nan)).all()


def test_same_seed_same_manifest():
    a = synth.make_inputs("tree32k", ctx=(300, 300))
    b = synth.make_inputs("tree32k", ctx=(300, 300))
    c = synth.make_inputs("tree32k", ctx=(300, 300), seed=99)
    assert a.manifest() == b.manifest()
    assert a.manifest()["q"] != c.manifest()["q"]


@pytest.mark.parametrize("seed,max_depth", [(2, 6), (4, 8), (17, 3)])
def test_tree_depth_and_branching_caps(seed, max_depth):
    rng = np.random.Generator(np.random.PCG64(seed))
    p = synth.random_tree_parents(rng, 64, max_depth=max_depth, max_branch=4)
    assert all(-1 <= p[i] < i for i in range(64))
    depth = np.zeros(64, int)
    for i in range(64):
        depth[i] = 1 if p[i] < 0 else depth[p[i]] + 1
    assert depth.max() <= max_depth
    counts = np.bincount(p + 1, minlength=65)
    assert counts.max() <= 4


def test_workload_shapes_and_poison():
    inp = synth.make_inputs("chain_b16", ctx=(100, 200), batch=3)
    B, N = 3, 8
    assert inp.q.shape == (B, N, 32, 128) and inp.q.dtype == np.uint16
    assert inp.k.shape == (B, 8, 208, 128)
    assert (inp.parent == np.arange(-1, N - 1)).all()
    assert ((inp.ctx_lens >= 100) & (inp.ctx_lens <= 200)).all()
    kf = synth.bf16_bits_to_f32(inp.k)
    for b in range(B):
        c = int(inp.ctx_lens[b])
        assert np.isfinite(kf[b, :, :c + N]).all()
        assert np.isnan(kf[b, :, c + N:]).all()


def test_sink_rows_scaled():
    inp = synth.make_inputs("tree128k", ctx=(2000, 2000))
    kf = synth.bf16_bits_to_f32(inp.k)[0]
    assert np.abs(kf[:, :4]).std() > 6 * np.abs(kf[:, 4:2000]).std()


def test_sparse_index_sets():
    inp = synth.make_inputs("sparse64k", ctx=(20000, 20000), batch=2)
    idx = inp.kv_idx
    assert idx.shape == (2, 8, 4096)
    for b in range(2):
        for g in range(8):
            s = idx[b, g]
            assert (np.diff(s) > 0).all()
            assert s[0] == 0 and (s[:4] == np.arange(4)).all()
            assert (s[-512:] == np.arange(20000 - 512, 20000)).all()
            assert s.max() < 20000
    # ranked fill: earlier-ranked positions are not uniformly spread
    assert not (idx[0, 0] == idx[0, 1]).all()


def test_zipf_fill_prefers_low_ranks():
    rng = np.random.Generator(np.random.PCG64(3))
    m, n = 50000, 2000
    pos, rank = synth.zipf_ranked_draw(rng, m, n, 1.1)
    assert np.unique(pos).size == n and pos.min() >= 0 and pos.max() < m
    # a uniform draw would put the median selected rank near m/2
    assert np.median(rank) < m / 10
    assert (rank <= 10).sum() >= 8
