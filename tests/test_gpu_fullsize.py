"""Full-size workloads on the GPU, in the launch configuration the benchmark
times (automatic split plan, bf16 inputs, fp32 output): sampled rows against
the fp64 oracle, plus properties that hold at any size for every row."""

import numpy as np
import pytest

import oracle
import synth
from util import assert_parity, device_inputs, errors, log, run_hip

pytestmark = pytest.mark.gpu

FULL = ["tiny_tree", "tree32k", "chain_b16", "tree128k", "sparse64k"]


@pytest.fixture(scope="module")
def hsv(gpu):
    import long_context_tree_verify_amd as m
    return m


def sample_rows(inp, n=48, seed=0):
    """First and last rows of every sequence, the deepest tree node, and a
    seeded spread over the rest."""
    B, N, Hq = inp.wl.batch, inp.wl.n_draft, inp.wl.n_q_heads
    rng = np.random.default_rng(seed)
    rows = {(0, 0, 0), (B - 1, N - 1, Hq - 1)}
    for b in range(B):
        depth = np.zeros(N, int)
        for i in range(N):
            p = inp.parent[b, i]
            depth[i] = 1 if p < 0 else depth[p] + 1
        rows.add((b, int(depth.argmax()), int(rng.integers(Hq))))
    while len(rows) < min(n, B * N * Hq):
        rows.add((int(rng.integers(B)), int(rng.integers(N)), int(rng.integers(Hq))))
    return sorted(rows)


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_rows(hsv, gpu, name):
    import torch
    log(f"full-size {name}: generating")
    inp = synth.make_inputs(name)
    dev = device_inputs(inp, gpu)
    log(f"full-size {name}: running HIP path")
    o, lse = run_hip(hsv, inp, dev)
    o_np, l_np = o.cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(o_np).all() and np.isfinite(l_np).all()
    # property for every row: o is a convex combination of value rows
    vmax = float(torch.nan_to_num(dev["v"].float(), nan=0.0).abs().max())
    assert np.abs(o_np).max() <= vmax * (1 + 1e-3)
    rows = sample_rows(inp)
    log(f"full-size {name}: oracle on {len(rows)} rows")
    o_ref, l_ref = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent,
                                      kv_idx=inp.kv_idx, bf16=inp.is_bf16, rows=rows)
    got_o = np.stack([o_np[b, i, h] for b, i, h in rows])
    got_l = np.array([l_np[b, i, h] for b, i, h in rows])
    o_err, l_err = errors(got_o, got_l, o_ref, l_ref)
    log(f"full-size {name}: max|dO| = {o_err:.3e}, max rel dLSE = {l_err:.3e}")
    assert_parity(got_o, got_l, o_ref, l_ref, name)
    del dev
    torch.cuda.empty_cache()
