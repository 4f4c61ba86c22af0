"""Seeded random sweeps of the three small exported operations against the
oracle: the ancestor bitmask (bit-exact; a sequence with a bad parent gets
all-zero masks), the compressed-cache gather (bit-exact; an index outside
[0, S_cap) gives a zero row, as the header states) and the exact LSE merge
of fp32 partials (fp32 or bf16 output; parts with LSE -inf, whose rows hold
NaN, take no part).  Every draw is fixed by its case number.
"""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

N_CASES = 100


@pytest.fixture(scope="module")
def hsv(gpu):
    import long_context_tree_verify_amd as m
    return m


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_ancestor_masks(hsv, gpu, k):
    import torch
    rng = np.random.Generator(np.random.PCG64(5000 + k))
    B = int(rng.integers(1, 9))
    N = int(rng.choice([1, 2, 7, 63, 64, 65, 127, 128, 129, 200, 256]))
    trees = []
    for b in range(B):
        kind = int(rng.integers(4))
        if kind == 0:
            trees.append(synth.chain_parents(N))
        elif kind == 1:
            trees.append(np.full(N, -1, np.int32))
        elif kind == 2:
            trees.append(synth.uniform_parents(rng, N))
        else:
            trees.append(synth.random_tree_parents(rng, N, max_depth=max(4, int(rng.integers(1, N + 1))),
                                                   max_branch=4))
    par = np.stack(trees).astype(np.int32)
    bad = np.zeros(B, bool)
    for b in range(B):
        if N > 1 and rng.random() < 0.2:
            i = int(rng.integers(1, N))
            par[b, i] = int(rng.choice([i, i + 1 if i + 1 < N else i, -2]))
            bad[b] = True
    got = hsv.hsv_tree_ancestor_mask(torch.from_numpy(par).to(gpu)).cpu().numpy().view(np.uint64)
    assert (got[bad] == 0).all(), f"case {k}: a tree with a bad parent has nonzero masks"
    if (~bad).any():
        np.testing.assert_array_equal(got[~bad], oracle.ancestor_mask(par[~bad]),
                                      err_msg=f"case {k}")


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_gather(hsv, gpu, k):
    import torch
    rng = np.random.Generator(np.random.PCG64(6000 + k))
    B, H = int(rng.integers(1, 5)), int(rng.choice([1, 2, 8]))
    cap, D = int(rng.choice([1, 33, 700, 5000])), int(rng.choice([64, 128]))
    n_sel = int(rng.integers(1, 600))
    bf16 = bool(rng.random() < 0.6)
    x = [rng.standard_normal((B, H, cap, D), dtype=np.float32) for _ in range(2)]
    if bf16:
        x = [synth.f32_to_bf16_bits(a) for a in x]
    idx = rng.integers(-2, cap + 3, size=(B, H, n_sel)).astype(np.int32)
    idx[rng.random(idx.shape) < 0.02] = int(rng.choice([-(1 << 31), (1 << 31) - 1]))
    to = (lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)) if bf16 else torch.from_numpy
    kg, vg = hsv.hsv_gather_kv(to(x[0]).to(gpu), to(x[1]).to(gpu), torch.from_numpy(idx).to(gpu))
    torch.cuda.synchronize()
    ok = (idx >= 0) & (idx < cap)
    ref = oracle.gather_kv(x[0], x[1], np.where(ok, idx, 0))
    view = np.uint16 if bf16 else np.float32
    for got, r in zip((kg, vg), ref):
        g = got.cpu().view(torch.int16).numpy().view(np.uint16) if bf16 else got.cpu().numpy()
        want = np.where(ok[..., None], r, np.zeros((), view))
        np.testing.assert_array_equal(g.view(view), want, err_msg=f"case {k}")


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_lse_merge(hsv, gpu, k):
    import torch
    rng = np.random.Generator(np.random.PCG64(7000 + k))
    P = int(rng.choice([1, 2, 31, 64, 65, 200, 1024]))
    R, D = int(rng.integers(1, 300)), int(rng.choice([64, 128]))
    bf16_out = bool(rng.random() < 0.3)
    o_parts = rng.standard_normal((P, R, D)).astype(np.float32)
    lse_parts = (rng.standard_normal((P, R)) * float(rng.uniform(0.1, 20))).astype(np.float32)
    lse_parts[rng.random((P, R)) < float(rng.uniform(0, 0.9))] = -np.inf
    o_parts[np.isneginf(lse_parts)] = np.nan      # never read
    o, lse = hsv.hsv_lse_merge(torch.from_numpy(o_parts).to(gpu), torch.from_numpy(lse_parts).to(gpu),
                               out_dtype=torch.bfloat16 if bf16_out else torch.float32)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    tol = 8e-3 if bf16_out else 1e-5
    for r in range(R):
        ro, rl = oracle.lse_merge(lse_parts[:, r].astype(np.float64),
                                  np.nan_to_num(o_parts[:, r].astype(np.float64)))
        if np.isneginf(rl):
            assert np.isneginf(lse[r]) and (o[r] == 0).all(), f"case {k} row {r}"
            continue
        assert abs(lse[r] - rl) <= 1e-5 * max(1, abs(rl)), f"case {k} row {r}"
        np.testing.assert_allclose(o[r], ro, rtol=0, atol=tol * max(1.0, float(np.abs(ro).max())),
                                   err_msg=f"case {k} row {r}")
