"""Seeded generators for verification-attention workloads.

Nothing here computes attention.  The generators only draw numbers with a
``numpy.random.Generator(PCG64(seed))`` in a fixed order and lay them out in
the layouts the C ABI takes:

* ``q``        ``[B, N, Hq, D]``
* ``k``, ``v`` ``[B, Hkv, S_cap, D]``; the draft block's K/V sit at cache
  positions ``[ctx_b, ctx_b + N)``; slots at ``ctx_b + N`` and beyond are NaN.
* ``ctx_lens`` ``int32 [B]``
* ``parent``   ``int32 [B, N]`` with ``parent[i]`` in ``[-1, i-1]``; -1 is the
  cached prefix (the tree root).
* ``kv_idx``   ``int32 [B, Hkv, n_sel]`` sorted and unique (sparse workloads).

Floating values are drawn in fp32 and, for bf16 workloads, rounded to bf16
with round-to-nearest-even; bf16 tensors are carried as their ``uint16`` bit
patterns so that the oracle and the GPU see exactly the same numbers.

Draw order (fixed): ctx_lens -> parents -> index sets -> Q -> K -> V.
"""

from __future__ import annotations

import dataclasses
import hashlib
from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


# ----------------------------------------------------------------------------
# bf16 bit handling (input preparation, not method arithmetic)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    out = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to the fp32 values they denote (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# draft-tree shapes
# ----------------------------------------------------------------------------

def uniform_parents(rng: np.random.Generator, n: int) -> np.ndarray:
    """parent[i] uniform in [-1, i-1] (the tiny tree workload's recipe)."""
    return np.array([rng.integers(-1, i) for i in range(n)], dtype=np.int32)


def chain_parents(n: int) -> np.ndarray:
    """A linear draft block: node i's parent is i-1 (causal inside the block)."""
    return np.arange(-1, n - 1, dtype=np.int32)


def random_tree_parents(rng: np.random.Generator, n: int, max_depth: int,
                        max_branch: int = 4) -> np.ndarray:
    """Seeded draft tree with bounded depth and branching.

    Node i picks its parent uniformly among the prefix root (-1) and the earlier
    nodes j < i whose depth is below ``max_depth`` and that have fewer than
    ``max_branch`` children.  The prefix root counts for branching too; its
    children have depth 1.
    """
    parent = np.empty(n, dtype=np.int32)
    depth = np.zeros(n, dtype=np.int64)
    children = np.zeros(n, dtype=np.int64)
    root_children = 0
    for i in range(n):
        eligible = []
        if root_children < max_branch:
            eligible.append(-1)
        for j in range(i):
            if depth[j] < max_depth and children[j] < max_branch:
                eligible.append(j)
        if not eligible:
            raise ValueError("tree capacity exhausted: raise max_depth or max_branch")
        p = eligible[int(rng.integers(0, len(eligible)))]
        parent[i] = p
        if p < 0:
            root_children += 1
            depth[i] = 1
        else:
            children[p] += 1
            depth[i] = depth[p] + 1
    return parent


def block_masks(n: int, block: int) -> np.ndarray:
    """Visibility masks of block-parallel drafting (FlexDraft page, attention
    tuning): the n draft tokens form consecutive blocks of `block` tokens;
    a token sees every token of its own block, earlier and later ones alike,
    and none of the other blocks.  uint64 [n] for n <= 64 (bit j = token j
    visible), else [n, ceil(n/64)] (word w holds tokens 64w .. 64w+63)."""
    if not 1 <= n <= 256:
        raise ValueError("1 to 256 draft tokens")
    W = (n + 63) // 64
    blk = np.arange(n) // block
    out = np.zeros((n, W), dtype=np.uint64)
    for i in range(n):
        for j in np.flatnonzero(blk == blk[i]):
            out[i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return out[:, 0] if W == 1 else out


def random_masks(rng: np.random.Generator, batch: int, n: int, density: float = 0.5):
    """Arbitrary visibility masks: each bit j < n set with probability
    `density`.  uint64 [batch, n]."""
    bits = rng.random((batch, n, n)) < density
    weights = np.uint64(1) << np.arange(n, dtype=np.uint64)
    return (bits.astype(np.uint64) * weights).sum(axis=2, dtype=np.uint64)


def zipf_ranked_draw(rng: np.random.Generator, m: int, n_draw: int, zipf_a: float):
    """Draw ``n_draw`` of ``m`` positions without replacement, P ~ rank**-a.

    Each position gets a random rank (a permutation of 1..m); the draw is a
    Gumbel-top-k over log-weights.  Returns (positions, their ranks).
    """
    rank = rng.permutation(m).astype(np.float64) + 1.0
    u = rng.random(m)
    key = -zipf_a * np.log(rank) - np.log(-np.log(np.maximum(u, 1e-300)))
    if n_draw:
        pick = np.argpartition(-key, n_draw - 1)[:n_draw]
    else:
        pick = np.empty(0, dtype=np.int64)
    return pick, rank[pick]


def zipf_index_set(rng: np.random.Generator, ctx: int, n_sel: int, n_sink: int,
                   n_recent: int, zipf_a: float) -> np.ndarray:
    """Sorted unique index set: sinks + recent window + Zipf-ranked fill.

    The middle positions ``[n_sink, ctx - n_recent)`` get a seeded random rank
    r (a permutation of 1..M); ``n_sel - n_sink - n_recent`` of them are drawn
    without replacement with probability proportional to ``r ** -zipf_a``
    (Gumbel-top-k).  The set mimics the Dustin page's fixed-size verification
    set (sink prefix, recent window, ranked fill).
    """
    n_fill = n_sel - n_sink - n_recent
    mid_lo, mid_hi = n_sink, ctx - n_recent
    m = mid_hi - mid_lo
    if n_fill < 0 or n_fill > m:
        raise ValueError("index-set budget does not fit the context")
    pick, _ = zipf_ranked_draw(rng, m, n_fill, zipf_a)
    idx = np.concatenate([np.arange(0, n_sink), pick + mid_lo, np.arange(mid_hi, ctx)])
    idx = np.sort(idx).astype(np.int32)
    assert idx.size == n_sel and np.unique(idx).size == n_sel
    return idx


def importance_maps(rng: np.random.Generator, ctx_lens: np.ndarray, n_kv_heads: int,
                    score_len: int, zipf_a: float = 1.1, noise: float = 0.5):
    """Synthetic draft-lookahead and target-historical importance maps.

    For each (sequence b, KV head g) the positions [0, ctx_b) get a random rank
    r (a permutation of 1..ctx_b) and a base weight r ** -zipf_a.  The target
    map is base * exp(noise * z1), the draft map base ** 0.8 * exp(noise * z2)
    (z1, z2 independent standard normals), each normalised to sum 1 over the
    row like an attention-mass map and rounded to bf16 precision (equal values
    occur, as they do in maps kept at that precision).  Positions at or past
    ctx_b are NaN: a reader of them is wrong.  Returns (draft, target), float32
    [B, Hkv, score_len].  Draw order: per (b, g): rank, z1, z2.
    """
    B = int(ctx_lens.shape[0])
    draft = np.full((B, n_kv_heads, score_len), np.nan, dtype=np.float32)
    target = np.full((B, n_kv_heads, score_len), np.nan, dtype=np.float32)
    for b in range(B):
        c = int(min(max(int(ctx_lens[b]), 0), score_len))
        for g in range(n_kv_heads):
            rank = rng.permutation(c).astype(np.float64) + 1.0
            base = rank ** -zipf_a
            z1 = rng.standard_normal(c)
            z2 = rng.standard_normal(c)
            for out, w in ((target, base * np.exp(noise * z1)),
                           (draft, base ** 0.8 * np.exp(noise * z2))):
                if c:
                    w = (w / w.sum()).astype(np.float32)
                    out[b, g, :c] = bf16_bits_to_f32(f32_to_bf16_bits(w))
    return draft, target


def to_paged(k: np.ndarray, v: np.ndarray, block_size: int, rng: np.random.Generator,
             spare_blocks: int = 3):
    """Lay a contiguous cache [B, Hkv, S_cap, D] out as a paged pool
    [n_blocks, Hkv, block_size, D] with a block table [B, S_cap / block_size]
    (HiSpec page: paged attention with block tables).  Logical block j of
    sequence b goes to pool block table[b, j]; the pool order is a seeded
    random permutation, and `spare_blocks` extra pool blocks that no table
    entry names are filled with NaN (a kernel reading them fails parity).
    Returns (k_pool, v_pool, table)."""
    B, H, S, D = k.shape
    if S % block_size:
        raise ValueError("capacity must be a whole number of blocks")
    nb = S // block_size
    n_pool = B * nb + spare_blocks
    perm = rng.permutation(n_pool)
    table = perm[:B * nb].reshape(B, nb).astype(np.int32)
    pools = []
    for src in (k, v):
        pool = np.empty((n_pool, H, block_size, D), dtype=src.dtype)
        if src.dtype == np.uint16:
            pool[...] = BF16_NAN
        else:
            pool[...] = np.nan
        blocks = src.reshape(B, H, nb, block_size, D).transpose(0, 2, 1, 3, 4)
        pool[table.reshape(-1)] = blocks.reshape(B * nb, H, block_size, D)
        pools.append(pool)
    return pools[0], pools[1], table


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_draft: int
    ctx: Tuple[int, int]          # ctx_b drawn uniformly in [lo, hi]; lo == hi: fixed
    dtype: str                    # "f32" or "bf16"
    tree: str                     # "uniform", "tree" or "chain"
    max_depth: int = 0
    max_branch: int = 4
    q_scale: float = 1.0
    kv_scale: float = 1.0
    sink_rows: int = 0            # first rows of K and V scaled by sink_scale
    sink_scale: float = 1.0
    n_sel: int = 0                # > 0: sparse workload with an index set per (b, kv head)
    n_sink: int = 4
    n_recent: int = 512
    zipf_a: float = 1.1
    n_heavy: int = 0              # > 0: keys planted per (b, kv head) that draw most attention
    heavy_logit: float = 6.0      # their score against the head's mean query direction
    description: str = ""

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def kv_capacity(self) -> int:
        return self.ctx[1] + self.n_draft

    @property
    def sparse(self) -> bool:
        return self.n_sel > 0

    def scaled(self, **kw) -> "Workload":
        """Same recipe with some fields replaced (smaller parity cases)."""
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "tiny_tree": Workload(
        name="tiny_tree", seed=1, batch=1, n_q_heads=1, n_kv_heads=1, head_dim=64,
        n_draft=8, ctx=(256, 256), dtype="f32", tree="uniform",
        description="batch 1, 1/1 heads, D64, fp32, 256-token prefix, 8-node uniform tree"),
    "tree32k": Workload(
        name="tree32k", seed=2, batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
        n_draft=64, ctx=(32768, 32768), dtype="bf16", tree="tree", max_depth=6,
        q_scale=1.0, kv_scale=0.5,
        description="batch 1, 32/8 heads, D128, bf16, 32768-token context, 64-node tree"),
    "chain_b16": Workload(
        name="chain_b16", seed=3, batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128,
        n_draft=8, ctx=(16384, 32768), dtype="bf16", tree="chain",
        q_scale=0.5, kv_scale=0.5,
        description="batch 16, 32/8 heads, D128, bf16, contexts in [16384, 32768], 8-token chain"),
    "tree128k": Workload(
        name="tree128k", seed=4, batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
        n_draft=64, ctx=(131072, 131072), dtype="bf16", tree="tree", max_depth=8,
        q_scale=1.0, kv_scale=0.5, sink_rows=4, sink_scale=8.0,
        description="batch 1, 32/8 heads, D128, bf16, 131072-token context, 64-node tree, x8 sinks"),
    "sparse64k": Workload(
        name="sparse64k", seed=5, batch=8, n_q_heads=32, n_kv_heads=8, head_dim=128,
        n_draft=8, ctx=(65536, 65536), dtype="bf16", tree="chain",
        q_scale=0.5, kv_scale=0.5, n_sel=4096, n_sink=4, n_recent=512, zipf_a=1.1,
        description="batch 8, 32/8 heads, D128, bf16, 65536-token context, 4096-entry index sets"),
    "sparse64k_hh": Workload(
        name="sparse64k_hh", seed=6, batch=8, n_q_heads=32, n_kv_heads=8, head_dim=128,
        n_draft=8, ctx=(65536, 65536), dtype="bf16", tree="chain",
        q_scale=0.5, kv_scale=0.5, n_sel=4096, n_sink=4, n_recent=512, zipf_a=1.1,
        n_heavy=256, heavy_logit=8.0,
        description="sparse64k with 256 planted heavy-hitter keys per (sequence, KV head)"),
}


@dataclass
class VerifyInputs:
    wl: Workload
    q: np.ndarray                  # f32, or uint16 bf16 bits
    k: np.ndarray
    v: np.ndarray
    ctx_lens: np.ndarray           # int32 [B]
    parent: np.ndarray             # int32 [B, N]
    kv_idx: Optional[np.ndarray] = None   # int32 [B, Hkv, n_sel]
    meta: Dict[str, str] = field(default_factory=dict)
    heavy: Optional[np.ndarray] = None    # int32 [B, Hkv, n_heavy] planted positions

    @property
    def is_bf16(self) -> bool:
        return self.wl.dtype == "bf16"

    def manifest(self) -> Dict[str, str]:
        """SHA-256 of every tensor (reproducibility check across machines)."""
        out = {}
        for name in ("q", "k", "v", "ctx_lens", "parent", "kv_idx"):
            a = getattr(self, name)
            if a is not None:
                out[name] = hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
        return out


def _normal(rng: np.random.Generator, shape, scale: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def _encode(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def make_inputs(wl, seed: Optional[int] = None, poison_unselected: bool = False,
                **overrides) -> VerifyInputs:
    """Draw one workload.  ``wl`` is a Workload or a key of ``WORKLOADS``.

    ``overrides`` replace Workload fields (e.g. ``ctx=(1000, 1000)`` for a
    smaller parity case with the same recipe).  ``poison_unselected`` writes
    NaN into every prefix row a sparse index set leaves out, so that a kernel
    that reads an unselected row cannot pass a parity test.
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    if overrides:
        wl = wl.scaled(**overrides)
    if seed is None:
        seed = wl.seed
    rng = np.random.Generator(np.random.PCG64(seed))
    B, N, Hq, Hkv, D = wl.batch, wl.n_draft, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    if Hq % Hkv:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    s_cap = wl.kv_capacity

    # 1. context lengths
    lo, hi = wl.ctx
    if lo == hi:
        ctx = np.full(B, lo, dtype=np.int32)
    else:
        ctx = rng.integers(lo, hi + 1, size=B).astype(np.int32)

    # 2. parents
    parent = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        if wl.tree == "chain":
            parent[b] = chain_parents(N)
        elif wl.tree == "uniform":
            parent[b] = uniform_parents(rng, N)
        elif wl.tree == "tree":
            parent[b] = random_tree_parents(rng, N, wl.max_depth, wl.max_branch)
        else:
            raise ValueError(f"unknown tree shape {wl.tree!r}")

    # 3. index sets
    kv_idx = None
    if wl.sparse:
        kv_idx = np.empty((B, Hkv, wl.n_sel), dtype=np.int32)
        for b in range(B):
            for g in range(Hkv):
                kv_idx[b, g] = zipf_index_set(rng, int(ctx[b]), wl.n_sel, wl.n_sink,
                                              wl.n_recent, wl.zipf_a)

    # 4. Q
    q = _encode(_normal(rng, (B, N, Hq, D), wl.q_scale), wl.dtype)

    # 5./6. K then V, one batch entry at a time to bound host memory
    caches = []
    for _ in range(2):
        dt = np.uint16 if wl.dtype == "bf16" else np.float32
        cache = np.empty((B, Hkv, s_cap, D), dtype=dt)
        for b in range(B):
            x = _normal(rng, (Hkv, s_cap, D), wl.kv_scale)
            if wl.sink_rows:
                x[:, :wl.sink_rows, :] *= np.float32(wl.sink_scale)
            x[:, int(ctx[b]) + N:, :] = np.nan
            if poison_unselected and kv_idx is not None:
                keep = np.zeros((Hkv, s_cap), dtype=bool)
                for g in range(Hkv):
                    keep[g, kv_idx[b, g]] = True
                keep[:, int(ctx[b]):] = True
                x[~keep] = np.nan
            cache[b] = _encode(x, wl.dtype)
        caches.append(cache)
    k, v = caches

    # 7. planted heavy hitters: each (b, g) gets a random unit direction u;
    # its queries gain u (unit length) and n_heavy of its prefix positions
    # (not sinks, not the recent window) gain heavy_logit * sqrt(D) * u, so
    # those keys score about heavy_logit against every query of the group and
    # draw most of the softmax mass
    heavy = None
    if wl.n_heavy:
        heavy = np.empty((B, Hkv, wl.n_heavy), dtype=np.int32)
        G = Hq // Hkv
        qf = bf16_bits_to_f32(q) if wl.dtype == "bf16" else q.copy()
        for b in range(B):
            c = int(ctx[b])
            lo, hi = min(wl.n_sink, c), max(c - wl.n_recent, min(wl.n_sink, c))
            for g in range(Hkv):
                pos = np.sort(rng.choice(np.arange(lo, hi), wl.n_heavy, replace=False))
                heavy[b, g] = pos
                u = rng.standard_normal(D)
                u = (u / np.linalg.norm(u)).astype(np.float32)
                qf[b, :, g * G:(g + 1) * G, :] += u
                kf = bf16_bits_to_f32(k[b, g, pos]) if wl.dtype == "bf16" else k[b, g, pos]
                kf = kf + np.float32(wl.heavy_logit * np.sqrt(D)) * u[None]
                k[b, g, pos] = _encode(kf.astype(np.float32), wl.dtype)
        q = _encode(qf, wl.dtype)
    out = VerifyInputs(wl=wl, q=q, k=k, v=v, ctx_lens=ctx, parent=parent, kv_idx=kv_idx,
                       meta={"seed": str(seed), "workload": wl.name})
    out.heavy = heavy
    return out


def heavy_importance_maps(rng: np.random.Generator, inp: "VerifyInputs", score_len: int,
                          recall_target: float = 0.8, recall_draft: float = 0.7,
                          lift: float = 50.0):
    """Importance maps for a workload with planted heavy hitters: the
    background of `importance_maps`, with a `recall_target` share (target
    map) and a separately drawn `recall_draft` share (draft map) of each
    (b, g)'s heavy positions raised `lift` times -- signals that point at
    most, not all, of the keys that matter.  Returns (draft, target)."""
    draft, target = importance_maps(rng, inp.ctx_lens, inp.wl.n_kv_heads, score_len)
    B, H = inp.heavy.shape[:2]
    for b in range(B):
        for g in range(H):
            pos = inp.heavy[b, g]
            for m, share in ((target, recall_target), (draft, recall_draft)):
                pick = pos[rng.random(pos.size) < share]
                m[b, g, pick] = (m[b, g, pick] * lift).astype(np.float32)
    return draft, target
