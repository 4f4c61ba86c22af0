"""A seeded random sweep of the cache bookkeeping (HiSpec page: the cache
kept with the rejected tokens' entries removed; Dustin page, verification
workflow step 5), bit-exact against the oracle: hsv_accept_path over whole
caches and context lengths, and hsv_tree_position_ids.

Each case draws the batch, KV heads, draft nodes (1 to 256), cache slots,
head dim, dtype, a mix of chains, flat, uniform and random trees, and per
sequence an accepted node (also -1 and out-of-range ones) and a context
length (also at and past the last one that fits, and negative).  Every draw
is fixed by its case number.
"""

import numpy as np
import pytest

import oracle
from test_gpu_accept import _cache, _check_accept, _trees

pytestmark = pytest.mark.gpu

N_CASES = 200


@pytest.fixture(scope="module")
def hsv(gpu):
    import long_context_tree_verify_amd as m
    return m


def draw_case(k: int):
    rng = np.random.Generator(np.random.PCG64(4000 + k))
    B = int(rng.integers(1, 20))
    H = int(rng.choice([1, 2, 4, 8]))
    N = int(rng.choice([1, 2, 3, 8, 31, 64, 65, 100, 200, 256]))
    S = N + int(rng.choice([0, 1, 7, 100, 1000]))
    D = int(rng.choice([64, 128]))
    bf16 = bool(rng.random() < 0.6)
    par = _trees(rng, B, N)
    ctx = rng.integers(0, S - N + 1, B).astype(np.int32)
    edge = rng.random(B)
    ctx[edge < 0.1] = S - N                 # the last length that fits
    ctx[(edge >= 0.1) & (edge < 0.15)] = S - N + 1   # one past: left unchanged
    ctx[(edge >= 0.15) & (edge < 0.18)] = -1
    node = rng.integers(-1, N, B)
    node[rng.random(B) < 0.05] = N          # out of range: left unchanged
    k_, v_ = _cache(rng, B, H, S, D, bf16)
    return k_, v_, ctx, par, node, bf16, (B, H, N, S, D)


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_accept(hsv, gpu, k):
    import torch
    kc, vc, ctx, par, node, bf16, shape = draw_case(k)
    _check_accept(hsv, gpu, kc, vc, ctx, par, node, bf16, f"accept case {k} {shape} bf16={bf16}")
    got = hsv.hsv_tree_position_ids(torch.from_numpy(par).to(gpu),
                                    torch.from_numpy(ctx).to(gpu)).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.tree_position_ids(par, ctx),
                                  err_msg=f"position ids case {k}")
