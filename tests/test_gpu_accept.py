"""GPU parity of the cache bookkeeping: hsv_tree_position_ids and
hsv_accept_path through the C ABI against the oracle, bit-exact (whole
caches and context lengths compared)."""

import numpy as np
import pytest

import oracle
import synth
from util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hsv(gpu):
    import long_context_tree_verify_amd as m
    return m


def _trees(rng, B, N):
    out = []
    for b in range(B):
        kind = b % 4
        if kind == 0:
            out.append(synth.chain_parents(N))
        elif kind == 1:
            out.append(np.full(N, -1, np.int32))
        elif kind == 2:
            out.append(synth.uniform_parents(rng, N))
        else:
            out.append(synth.random_tree_parents(rng, N, max_depth=min(N, 6),
                                                 max_branch=max(4, N)))
    return np.stack(out).astype(np.int32)


def test_position_ids(hsv, gpu):
    import torch
    rng = np.random.Generator(np.random.PCG64(61))
    for N in (1, 2, 7, 33, 64, 65, 130, 256):
        par = _trees(rng, 12, N)
        if N > 1:
            par[5, N - 1] = N - 1          # self-parent: the sequence is invalid
        ctx = rng.integers(0, 1 << 20, 12).astype(np.int32)
        got = hsv.hsv_tree_position_ids(torch.from_numpy(par).to(gpu),
                                        torch.from_numpy(ctx).to(gpu)).cpu().numpy()
        np.testing.assert_array_equal(got, oracle.tree_position_ids(par, ctx))
    log("  position ids identical for N in 1, 2, 7, 33, 64, 65, 130, 256")


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _run_accept(hsv, gpu, k, v, ctx, par, node, bf16):
    import torch
    if bf16:
        kt = torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).to(gpu)
        vt = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to(gpu)
    else:
        kt, vt = torch.from_numpy(k).to(gpu), torch.from_numpy(v).to(gpu)
    ct = torch.from_numpy(ctx.copy()).to(gpu)
    hsv.hsv_accept_path(kt, vt, ct, torch.from_numpy(par).to(gpu),
                        torch.from_numpy(node.astype(np.int32)).to(gpu))
    torch.cuda.synchronize()
    return _bits(kt).cpu().numpy(), _bits(vt).cpu().numpy(), ct.cpu().numpy()


def _check_accept(hsv, gpu, k, v, ctx, par, node, bf16, what):
    gk, gv, gc = _run_accept(hsv, gpu, k, v, ctx, par, node, bf16)
    rk, rv, rc = oracle.accept_path(k, v, ctx, par, node)
    view = np.int16 if bf16 else np.int32
    np.testing.assert_array_equal(gc, rc, err_msg=what)
    np.testing.assert_array_equal(gk, rk.view(view), err_msg=what)
    np.testing.assert_array_equal(gv, rv.view(view), err_msg=what)
    log(f"  {what}: caches and lengths identical (lengths {rc[:6].tolist()}...)")


def _cache(rng, B, H, S, D, bf16):
    k = rng.standard_normal((B, H, S, D), dtype=np.float32)
    v = rng.standard_normal((B, H, S, D), dtype=np.float32)
    if bf16:
        return synth.f32_to_bf16_bits(k), synth.f32_to_bf16_bits(v)
    return k, v


@pytest.mark.parametrize("bf16,D", [(True, 128), (False, 128), (True, 64), (False, 64)])
def test_accept_random_trees(hsv, gpu, bf16, D):
    rng = np.random.Generator(np.random.PCG64(62 + D + bf16))
    B, H, N, S = 16, 4, 64, 400
    par = _trees(rng, B, N)
    ctx = rng.integers(0, S - N + 1, B).astype(np.int32)
    node = rng.integers(-1, N, B)
    node[0], node[1] = N - 1, 0
    k, v = _cache(rng, B, H, S, D, bf16)
    _check_accept(hsv, gpu, k, v, ctx, par, node, bf16, f"random trees bf16={bf16} D={D}")


def test_accept_left_unchanged(hsv, gpu):
    rng = np.random.Generator(np.random.PCG64(63))
    B, H, N, S, D = 8, 2, 12, 64, 128
    par = _trees(rng, B, N)
    par[2, 5] = 7                       # parent after the node: invalid sequence
    ctx = np.array([10, 10, 10, 10, S - N, S - N + 1, -3, 0], np.int32)
    node = np.array([-1, N, 4, -5, N - 1, 3, 2, N - 1])
    k, v = _cache(rng, B, H, S, D, True)
    _check_accept(hsv, gpu, k, v, ctx, par, node, True, "left-unchanged cases")


@pytest.mark.parametrize("name", ["tree32k", "chain_b16"])
def test_accept_full_size(hsv, gpu, name):
    wl = synth.WORKLOADS[name]
    rng = np.random.Generator(np.random.PCG64(64))
    B, H, N, D = wl.batch, wl.n_kv_heads, wl.n_draft, wl.head_dim
    S = wl.kv_capacity
    if wl.tree == "chain":
        par = np.tile(synth.chain_parents(N), (B, 1)).astype(np.int32)
    else:
        par = np.stack([synth.random_tree_parents(rng, N, wl.max_depth, wl.max_branch)
                        for _ in range(B)]).astype(np.int32)
    lo, hi = wl.ctx
    ctx = rng.integers(lo, hi + 1, B).astype(np.int32)
    depth = oracle.tree_depth(par)
    node = depth.argmax(axis=1)         # the deepest node: the longest path
    # random bf16 bit patterns (NaN patterns included: the update is a copy)
    n = B * H * S * D
    k = rng.integers(0, 1 << 16, n, dtype=np.uint16).reshape(B, H, S, D)
    v = rng.integers(0, 1 << 16, n, dtype=np.uint16).reshape(B, H, S, D)
    _check_accept(hsv, gpu, k, v, ctx, par, node, True, f"{name} shape")


@pytest.mark.parametrize("bf16,D,N", [(True, 128, 256), (False, 128, 200), (True, 64, 97)])
def test_accept_wide_trees(hsv, gpu, bf16, D, N):
    """Trees of more than 64 nodes: chains (the longest paths, moved in
    several staged chunks), deep random trees and the deepest node."""
    rng = np.random.Generator(np.random.PCG64(65 + N))
    B, H, S = 8, 3, N + 500
    par = np.stack([synth.chain_parents(N), np.full(N, -1, np.int32),
                    synth.uniform_parents(rng, N),
                    synth.random_tree_parents(rng, N, max_depth=N, max_branch=2),
                    synth.random_tree_parents(rng, N, max_depth=16, max_branch=4),
                    synth.chain_parents(N), synth.uniform_parents(rng, N),
                    synth.random_tree_parents(rng, N, max_depth=N, max_branch=1)]
                   ).astype(np.int32)
    ctx = rng.integers(0, S - N + 1, B).astype(np.int32)
    depth = oracle.tree_depth(par)
    node = depth.argmax(axis=1)
    node[1], node[6] = -1, rng.integers(0, N)
    k, v = _cache(rng, B, H, S, D, bf16)
    _check_accept(hsv, gpu, k, v, ctx, par, node, bf16, f"N={N} trees bf16={bf16} D={D}")
