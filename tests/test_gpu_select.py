"""GPU parity of the verification index-set selection (Dustin page,
methodology 1): hsv_select_kv_idx through the C ABI against
oracle.select_kv_idx, bit-exact.

Cases: the 65536-position, 8 x 8 (sequence, KV head) shape of the sparse
workload with bf16-precision maps (many equal scores); ragged contexts down
to 0 and below the budget; NaN, +-0 and +-inf scores; a few distinct values
only; the corner budgets (no draft share, draft share beyond the budget, no
sinks or window, budget equal to the context); the largest score row;
full-precision scores and planted ties at the k-th rank.
"""

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


def _select(hsv, gpu, draft, target, ctx, **kw):
    import torch
    out = hsv.hsv_select_kv_idx(torch.from_numpy(np.ascontiguousarray(draft)).to(gpu),
                                torch.from_numpy(np.ascontiguousarray(target)).to(gpu),
                                torch.from_numpy(np.asarray(ctx, np.int32)).to(gpu), **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check(hsv, gpu, draft, target, ctx, what, **kw):
    got = _select(hsv, gpu, draft, target, ctx, **kw)
    ref = oracle.select_kv_idx(draft, target, np.asarray(ctx), **kw)
    bad = np.argwhere((got != ref).any(axis=-1))
    assert bad.size == 0, f"{what}: (b, g) rows differ: {bad[:4].tolist()}"
    log(f"  {what}: {got.shape} identical")


def test_full_size_importance_maps(hsv, gpu):
    rng = np.random.Generator(np.random.PCG64(505))
    ctx = np.full(8, 65536, np.int32)
    draft, target = synth.importance_maps(rng, ctx, 8, 65536)
    _check(hsv, gpu, draft, target, ctx, "B8 Hkv8 L65536 n_sel 4096",
           n_sel=4096, n_sink=4, n_recent=512, n_draft_top=1790)


def test_full_precision_and_planted_ties(hsv, gpu):
    # fp32 scores using every mantissa bit (the low-key-bit pass runs), and
    # rows where 150 (ranked directly by position) or 400 (position passes)
    # candidates share the draft score at the n_draft_top-th rank
    rng = np.random.Generator(np.random.PCG64(515))
    B, H, L = 2, 4, 65536
    n_sink, n_recent, m = 4, 512, 1790
    draft = rng.random((B, H, L), dtype=np.float32)
    target = rng.random((B, H, L), dtype=np.float32)
    cand = np.arange(n_sink, L - n_recent)
    for g, n_tied in ((0, 150), (1, 400), (2, 40)):
        row = draft[0, g]
        v = np.sort(row[cand])[-m]
        row[rng.choice(cand, n_tied, replace=False)] = v
        trow = target[1, g]
        trow[rng.choice(cand, n_tied, replace=False)] = np.sort(trow[cand])[-(4096 - 516 - m)]
    ctx = np.full(B, L, np.int32)
    _check(hsv, gpu, draft, target, ctx, "fp32 scores, planted ties", n_sel=4096,
           n_sink=n_sink, n_recent=n_recent, n_draft_top=m)


def test_ragged_contexts(hsv, gpu):
    rng = np.random.Generator(np.random.PCG64(506))
    ctx = np.array([0, 1, 3, 100, 515, 516, 600, 4095, 4096, 4097, 9000, 20000], np.int32)
    draft, target = synth.importance_maps(rng, ctx, 3, 20000)
    _check(hsv, gpu, draft, target, ctx, "ragged", n_sel=4096, n_sink=4, n_recent=512,
           n_draft_top=1000)
    _check(hsv, gpu, draft, target, ctx, "ragged, small budget", n_sel=37, n_sink=5,
           n_recent=7, n_draft_top=11)


@pytest.mark.parametrize("m", [0, 1, 50, 10 ** 6])
def test_draft_share(hsv, gpu, m):
    rng = np.random.Generator(np.random.PCG64(507 + m % 97))
    ctx = np.array([3000, 2047, 1025], np.int32)
    draft, target = synth.importance_maps(rng, ctx, 2, 3000)
    _check(hsv, gpu, draft, target, ctx, f"n_draft_top {m}", n_sel=300, n_sink=4,
           n_recent=64, n_draft_top=m)


def test_special_values_and_ties(hsv, gpu):
    rng = np.random.Generator(np.random.PCG64(508))
    B, H, L = 4, 4, 5000
    ctx = np.array([5000, 4999, 1234, 77], np.int32)
    vals = np.array([np.nan, -0.0, 0.0, np.inf, -np.inf, 1.0, -1.0, 2.5, 1e-30, -1e-30],
                    np.float32)
    draft = vals[rng.integers(0, vals.size, (B, H, L))]
    target = vals[rng.integers(0, vals.size, (B, H, L))]
    _check(hsv, gpu, draft, target, ctx, "special values", n_sel=700, n_sink=3, n_recent=20,
           n_draft_top=333)
    few = rng.integers(0, 3, (B, H, L)).astype(np.float32)
    _check(hsv, gpu, few, few[:, ::-1].copy(), ctx, "three values", n_sel=1500, n_sink=0,
           n_recent=0, n_draft_top=600)
    allnan = np.full((B, H, L), np.nan, np.float32)
    _check(hsv, gpu, allnan, allnan, ctx, "all NaN", n_sel=100, n_sink=2, n_recent=2,
           n_draft_top=10)


def test_budget_corners(hsv, gpu):
    rng = np.random.Generator(np.random.PCG64(509))
    ctx = np.array([64, 700, 1024], np.int32)
    draft, target = synth.importance_maps(rng, ctx, 2, 1024)
    _check(hsv, gpu, draft, target, ctx, "n_sel = c", n_sel=64, n_sink=4, n_recent=8,
           n_draft_top=20)
    _check(hsv, gpu, draft, target, ctx, "sinks + window = budget", n_sel=40, n_sink=8,
           n_recent=32, n_draft_top=20)
    _check(hsv, gpu, draft, target, ctx, "budget 1", n_sel=1, n_sink=0, n_recent=1,
           n_draft_top=0)
    _check(hsv, gpu, draft, target, ctx, "budget above L", n_sel=2000, n_sink=16, n_recent=16,
           n_draft_top=5)


def test_largest_row(hsv, gpu):
    L = 1 << 19            # the largest score row the ABI accepts
    rng = np.random.Generator(np.random.PCG64(510))
    ctx = np.array([L, L - 12345], np.int32)
    draft, target = synth.importance_maps(rng, ctx, 1, L)
    _check(hsv, gpu, draft, target, ctx, f"L {L}", n_sel=8192, n_sink=4, n_recent=1024,
           n_draft_top=3000)


def test_rows_past_64k(hsv, gpu):
    # score rows of a 64k context plus its 8 draft rows (65544 positions):
    # with a 512-position window the candidates end before 65536 (the list
    # path); without one they reach past it (the streaming fallback there)
    rng = np.random.Generator(np.random.PCG64(516))
    L = 65544
    ctx = np.array([65536, 65544, 65540, 60000], np.int32)
    draft, target = synth.importance_maps(rng, ctx, 2, L)
    _check(hsv, gpu, draft, target, ctx, "L 65544", n_sel=4096, n_sink=4, n_recent=512,
           n_draft_top=1790)
    _check(hsv, gpu, draft, target, ctx, "L 65544, no window", n_sel=4096, n_sink=4,
           n_recent=0, n_draft_top=1790)


def test_candidates_starting_past_the_first_chunk(hsv, gpu):
    # sinks that cover one or more whole 8192-position chunks, so the first
    # candidate (whose chunk publishes the row's floors for the list step)
    # lies in a later chunk, on a chunk boundary or inside one; contexts
    # below the sink count leave rows with no candidates at all
    rng = np.random.Generator(np.random.PCG64(517))
    L = 65536
    ctx = np.array([65536, 40000, 9000, 16384, 20000], np.int32)
    draft, target = synth.importance_maps(rng, ctx, 2, L)
    for n_sink in (9000, 16384, 8191):
        _check(hsv, gpu, draft, target, ctx, f"n_sink {n_sink}", n_sel=n_sink + 4096,
               n_sink=n_sink, n_recent=512, n_draft_top=1790)


def test_rejects_bad_arguments(hsv, gpu):
    import torch
    d = torch.zeros((1, 1, 16), dtype=torch.float32, device=gpu)
    c = torch.tensor([16], dtype=torch.int32, device=gpu)
    with pytest.raises(RuntimeError):
        hsv.hsv_select_kv_idx(d, d, c, n_sel=4, n_sink=3, n_recent=2, n_draft_top=0)
    big = torch.zeros((1, 1, (1 << 19) + 1), dtype=torch.float32, device=gpu)
    with pytest.raises(RuntimeError):
        hsv.hsv_select_kv_idx(big, big, c, n_sel=4, n_sink=0, n_recent=0, n_draft_top=0)


def _sample_positions(lo, hi, L):
    # the floors' sample: 32 segments of 64 consecutive positions spread
    # over the row of L positions (all of them up to 2048), those in [lo, hi)
    if L <= 2048:
        pos = np.arange(L)
    else:
        starts = ((L - 64) * np.arange(32)) // 31
        pos = (starts[:, None] + np.arange(64)[None]).reshape(-1)
    return pos[(pos >= lo) & (pos < hi)]


def test_sample_defeating_maps(hsv, gpu):
    # Row 0: the only large scores sit on 500 sampled positions, so the floor
    # leaves fewer than k candidates: both maps must fall back to the
    # streaming select.  Row 1: 3000 large scores off the sample, packed
    # into one 8192-position chunk: its list (1024 slots) overflows, again a
    # fallback.
    # Row 2: no planted values (the list path).
    L, n_sink, n_recent = 65536, 4, 512
    rng = np.random.Generator(np.random.PCG64(511))
    lo, hi = n_sink, L - n_recent
    sampled = _sample_positions(lo, hi, L)
    off = np.setdiff1d(np.arange(lo, hi), sampled)
    draft = rng.random((3, 1, L), dtype=np.float32)
    target = rng.random((3, 1, L), dtype=np.float32)
    hot0 = rng.choice(sampled, 500, replace=False)
    in_chunk = off[(off >= 16384) & (off < 24576)]
    hot1 = rng.choice(in_chunk, 3000, replace=False)
    for row, hot in ((0, hot0), (1, hot1)):
        draft[row, 0, hot] += 1000.0
        target[row, 0, hot] += 1000.0
    ctx = np.full(3, L, np.int32)
    _check(hsv, gpu, draft, target, ctx, "sample-defeating", n_sel=4096, n_sink=n_sink,
           n_recent=n_recent, n_draft_top=1790)


def test_tiny_rows(hsv, gpu):
    # rows with fewer than 4 candidates take the single-load staging path
    rng = np.random.Generator(np.random.PCG64(512))
    ctx = np.array([3, 2, 1, 7], np.int32)
    draft = rng.random((4, 2, 7), dtype=np.float32)
    target = rng.random((4, 2, 7), dtype=np.float32)
    _check(hsv, gpu, draft, target, ctx, "tiny rows", n_sel=2, n_sink=0, n_recent=0,
           n_draft_top=1)
    _check(hsv, gpu, draft, target, ctx, "tiny rows, window", n_sel=3, n_sink=0, n_recent=1,
           n_draft_top=1)


def test_recall_rate_parity(hsv, gpu):
    # Attention recall rate of a selected set, exp(lse_set - lse_full) over
    # the prefix, from the GPU's LSEs against the oracle's.  Bound: each LSE
    # is within 1e-3 * max(|lse|, 1) of the oracle's, so the rate is within
    # a factor exp(+-2e-3 * max|lse|) of the oracle's rate.  On a workload
    # with planted heavy-hitter keys the selected set must also keep more
    # mass than the random set of the same size.
    import torch
    inp = synth.make_inputs("sparse64k_hh", batch=2, n_kv_heads=2, n_q_heads=8,
                            ctx=(8192, 8192), n_heavy=64, n_sel=1024, n_recent=128)
    L = inp.k.shape[2]
    rng = np.random.Generator(np.random.PCG64(513))
    draft, target = synth.heavy_importance_maps(rng, inp, L)
    kw = dict(n_sel=1024, n_sink=4, n_recent=128, n_draft_top=400)
    ctx = inp.ctx_lens
    kv = _select(hsv, gpu, draft, target, ctx, **kw)
    np.testing.assert_array_equal(kv, oracle.select_kv_idx(draft, target, ctx, **kw))

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(gpu)

    q, k, v = up(inp.q), up(inp.k), up(inp.v)
    c = torch.from_numpy(ctx).to(gpu)
    flags = hsv.HSV_FLAG_NO_TREE
    _, l_full = hsv.hsv_verify_attn(q, k, v, c, None, max_ctx=int(ctx.max()), flags=flags)
    _, l_sel = hsv.hsv_verify_attn_sparse(q, k, v, c, None, None, torch.from_numpy(kv).to(gpu),
                                          max_ctx=int(ctx.max()), flags=flags)
    _, l_rand = hsv.hsv_verify_attn_sparse(q, k, v, c, None, None,
                                           torch.from_numpy(inp.kv_idx).to(gpu),
                                           max_ctx=int(ctx.max()), flags=flags)
    torch.cuda.synchronize()
    l_full, l_sel, l_rand = (x.cpu().numpy().astype(np.float64) for x in (l_full, l_sel, l_rand))
    _, r_full = oracle.verify_attn(inp.q, inp.k, inp.v, ctx, parent=inp.parent, bf16=True,
                                   parts=oracle.PART_PREFIX)
    _, r_sel = oracle.verify_attn(inp.q, inp.k, inp.v, ctx, parent=inp.parent, kv_idx=kv,
                                  bf16=True, parts=oracle.PART_PREFIX)
    arr_gpu = np.exp(l_sel - l_full)
    arr_ref = oracle.recall_rate(r_sel, r_full)
    bound = np.exp(2e-3 * np.maximum(np.abs(r_full), 1.0)) - 1.0
    rel = np.abs(arr_gpu / arr_ref - 1.0)
    log(f"  recall rate: mean {arr_gpu.mean():.4f} (oracle {arr_ref.mean():.4f}), "
        f"max rel diff {rel.max():.2e}, random set {np.exp(l_rand - l_full).mean():.4f}")
    assert (rel <= bound).all()
    assert arr_gpu.mean() > 2.0 * np.exp(l_rand - l_full).mean()


def test_select_then_sparse_verify_short_histories(hsv, gpu):
    """The selection's -1 tail (histories shorter than the set) is a valid
    sparse index set: the sparse call accepts it under HSV_FLAG_VALIDATE and
    matches the oracle on the same set (which, for those sequences, is the
    whole history: dense attention)."""
    import torch
    inp = synth.make_inputs("chain_b16", ctx=(200, 1500), batch=6)
    B, Hkv, cap = inp.k.shape[:3]
    ctx = inp.ctx_lens
    assert (ctx < 512).any() and (ctx > 512).any()
    rng = np.random.Generator(np.random.PCG64(509))
    draft, target = synth.importance_maps(rng, ctx, Hkv, int(ctx.max()))
    kw = dict(n_sel=512, n_sink=4, n_recent=64, n_draft_top=200)
    idx = _select(hsv, gpu, draft, target, ctx, **kw)
    np.testing.assert_array_equal(idx, oracle.select_kv_idx(draft, target, ctx, **kw))
    assert (idx == -1).any()
    up = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(gpu)
    o, lse = hsv.hsv_verify_attn_sparse(
        up(inp.q), up(inp.k), up(inp.v), torch.from_numpy(ctx).to(gpu),
        torch.from_numpy(inp.parent).to(gpu), None, torch.from_numpy(idx).to(gpu),
        max_ctx=int(ctx.max()), flags=hsv.HSV_FLAG_VALIDATE)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.verify_attn(inp.q, inp.k, inp.v, ctx, parent=inp.parent, kv_idx=idx,
                                      bf16=True)
    from util import assert_parity
    assert_parity(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "select -> sparse verify")
    short = ctx < 512
    dense_ref = oracle.verify_attn(inp.q[short], inp.k[short], inp.v[short], ctx[short],
                                   parent=inp.parent[short], bf16=True)
    np.testing.assert_allclose(o_ref[short], dense_ref[0], rtol=0, atol=1e-12)
