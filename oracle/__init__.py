"""fp64 CPU oracle for verification attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the package smoke check and the benchmark's CPU-baseline leg
may import this module.  The product path (the HIP library and its binding)
never does, and the oracle imports nothing from the product.

The arithmetic lives in ``oracle.c`` (plain C, fp64, explicit mask rows);
this file only builds it with gcc and marshals numpy arrays through ctypes.
The sparse-cache gather (Dustin page, "Verification workflow": a compressed
cache formed from the selected tokens) is a pure copy and is written here
with numpy indexing.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional, Sequence, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

F32, BF16 = 0, 1
PART_PREFIX, PART_TREE = 1, 2
PART_BOTH = PART_PREFIX | PART_TREE

_lock = threading.Lock()
_lib = None


class _Desc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_draft", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("kv_capacity", ctypes.c_int32),
        ("n_sel", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32),
        ("parts", ctypes.c_int32),
        ("scale", ctypes.c_double),
    ]


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < max(
            os.path.getmtime(SRC), os.path.getmtime(os.path.join(HERE, "oracle.h"))):
        tmp = LIB + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-o", tmp, SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(LIB)
            P = ctypes.c_void_p
            lib.oracle_ancestor_mask.argtypes = [P, ctypes.c_int32, ctypes.c_int32, P]
            lib.oracle_ancestor_mask.restype = ctypes.c_int
            lib.oracle_verify_attn.argtypes = [ctypes.POINTER(_Desc), P, P, P, P, P, P, P, P,
                                               ctypes.c_int64, P, P]
            lib.oracle_verify_attn.restype = ctypes.c_int
            lib.oracle_lse_merge.argtypes = [ctypes.c_int32, ctypes.c_int32, P, P, P, P]
            lib.oracle_lse_merge.restype = None
            lib.oracle_num_threads.argtypes = []
            lib.oracle_num_threads.restype = ctypes.c_int
            lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
            lib.oracle_set_num_threads.restype = None
            _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of later oracle calls (timing only; results do not depend on it)."""
    _load().oracle_set_num_threads(int(n))


def mask_words(n: int) -> int:
    """64-bit words of one node's mask: word w holds nodes 64w .. 64w + 63."""
    return (n + 63) // 64


def ancestor_mask(parent: np.ndarray) -> np.ndarray:
    """Ancestor-or-self bitmask by walking parent pointers: uint64 [B, N] for
    N <= 64, else [B, N, W] with W = ceil(N / 64) words per node."""
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    if parent.ndim == 1:
        parent = parent[None]
    B, N = parent.shape
    W = mask_words(N)
    out = np.zeros((B, N, W), dtype=np.uint64)
    rc = _load().oracle_ancestor_mask(_ptr(parent), B, N, _ptr(out))
    if rc != 0:
        raise ValueError("invalid parent array")
    return out.reshape(B, N) if W == 1 else out


def verify_attn(q: np.ndarray, k: np.ndarray, v: np.ndarray, ctx_lens: np.ndarray,
                parent: Optional[np.ndarray] = None, anc_mask: Optional[np.ndarray] = None,
                kv_idx: Optional[np.ndarray] = None, *, bf16: bool,
                scale: Optional[float] = None, parts: int = PART_BOTH,
                rows: Optional[Sequence[Tuple[int, int, int]]] = None
                ) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 verification attention.

    q ``[B, N, Hq, D]``; k, v ``[B, Hkv, S_cap, D]`` (float32, or uint16 bf16
    bits when ``bf16``); ctx_lens ``[B]``; one of parent / anc_mask ``[B, N]``;
    kv_idx ``[B, Hkv, n_sel]`` for the sparse prefix.  Returns (o, lse):
    ``[B, N, Hq, D]`` / ``[B, N, Hq]`` for all rows, or ``[R, D]`` / ``[R]``
    for the (b, i, h) triples in ``rows``.
    """
    B, N, Hq, D = q.shape
    Bk, Hkv, cap, Dk = k.shape
    if (Bk, Dk) != (B, D) or v.shape != k.shape:
        raise ValueError("shape mismatch")
    want = np.uint16 if bf16 else np.float32
    q = np.ascontiguousarray(q, dtype=want)
    k = np.ascontiguousarray(k, dtype=want)
    v = np.ascontiguousarray(v, dtype=want)
    ctx_lens = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    if parent is not None:
        parent = np.ascontiguousarray(parent, dtype=np.int32).reshape(B, N)
    if anc_mask is not None:
        anc_mask = np.ascontiguousarray(anc_mask, dtype=np.uint64).reshape(B, N, mask_words(N))
    n_sel = 0
    if kv_idx is not None:
        kv_idx = np.ascontiguousarray(kv_idx, dtype=np.int32)
        n_sel = kv_idx.shape[-1]
        if kv_idx.shape != (B, Hkv, n_sel) or n_sel == 0:
            raise ValueError("kv_idx must be [B, Hkv, n_sel] with n_sel > 0")
    d = _Desc(B, N, Hq, Hkv, D, cap, n_sel, BF16 if bf16 else F32, parts,
              float(scale) if scale is not None else 1.0 / float(np.sqrt(D)))
    if rows is None:
        rows_arr = None
        o = np.zeros((B, N, Hq, D), dtype=np.float64)
        lse = np.zeros((B, N, Hq), dtype=np.float64)
        n_rows = 0
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
        n_rows = rows_arr.shape[0]
        o = np.zeros((n_rows, D), dtype=np.float64)
        lse = np.zeros((n_rows,), dtype=np.float64)
    rc = _load().oracle_verify_attn(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(ctx_lens),
                                    _ptr(parent), _ptr(anc_mask), _ptr(kv_idx), _ptr(rows_arr),
                                    n_rows, _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_verify_attn rejected its arguments")
    return o, lse


def lse_merge(lse_parts: np.ndarray, o_parts: np.ndarray) -> Tuple[np.ndarray, float]:
    """Merge P partial (o, lse) results of one row: lse_parts [P], o_parts [P, D]."""
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64).reshape(-1)
    o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
    P, D = o_parts.shape
    assert lse_parts.shape == (P,)
    o = np.zeros(D, dtype=np.float64)
    lse = np.zeros(1, dtype=np.float64)
    _load().oracle_lse_merge(P, D, _ptr(lse_parts), _ptr(o_parts), _ptr(o), _ptr(lse))
    return o, float(lse[0])


def gather_kv(k: np.ndarray, v: np.ndarray, kv_idx: np.ndarray):
    """Compressed cache: K_sel[b, g, s] = K[b, g, kv_idx[b, g, s]] (and V)."""
    B, Hkv, n_sel = kv_idx.shape
    bi = np.arange(B)[:, None, None]
    gi = np.arange(Hkv)[None, :, None]
    return k[bi, gi, kv_idx], v[bi, gi, kv_idx]


def paged_to_contiguous(k_pool: np.ndarray, v_pool: np.ndarray, table: np.ndarray):
    """Contiguous cache of a paged one (HiSpec page: paged attention with
    block tables): row t of sequence b, head g is row t % bs of pool block
    table[b, t // bs].  k_pool, v_pool [n_blocks, Hkv, bs, D]; table
    [B, nb] -> k, v [B, Hkv, nb * bs, D].  Attention over a paged cache is
    attention over this one."""
    n_pool, H, bs, D = k_pool.shape
    B, nb = table.shape
    out = []
    for pool in (k_pool, v_pool):
        x = np.empty((B, H, nb * bs, D), dtype=pool.dtype)
        for b in range(B):
            for j in range(nb):
                x[b, :, j * bs:(j + 1) * bs] = pool[table[b, j]]
        out.append(x)
    return out[0], out[1]


def _top_positions(scores: np.ndarray, pos: np.ndarray, k: int) -> np.ndarray:
    """The k best positions: higher score first, NaN below every number,
    -0 equal to +0, ties to the lower position."""
    if k <= 0 or pos.size == 0:
        return np.zeros(0, dtype=np.int64)
    s = np.asarray(scores, dtype=np.float64)
    nan = np.isnan(s)
    neg = np.where(nan, 0.0, -s)            # -0 and +0 compare equal
    order = np.lexsort((pos, neg, nan))     # last key is the primary one
    return pos[order[:k]]


def select_kv_idx(draft_score: np.ndarray, target_score: np.ndarray, ctx_lens: np.ndarray,
                  n_sel: int, n_sink: int, n_recent: int, n_draft_top: int) -> np.ndarray:
    """Fixed-size verification index set per (sequence b, KV head g)
    (Dustin page, methodology 1, hybrid attention aggregation; verification
    workflow step 3: the compressed cache is formed from these positions).

    Of the positions [0, c) with c = ctx_lens[b] (clipped to the score rows'
    length): the first n_sink and the last n_recent are always kept; of the
    positions between them, the n_draft_top best by the draft-lookahead score,
    then the best by the target-historical score until n_sel positions are
    chosen.  "Best" is `_top_positions`.  Output: int32 [B, Hkv, n_sel],
    ascending; if fewer than n_sel positions exist the tail is -1.
    Requires n_sink + n_recent <= n_sel.
    """
    draft_score = np.asarray(draft_score)
    target_score = np.asarray(target_score)
    B, Hkv, S = draft_score.shape
    assert target_score.shape == (B, Hkv, S)
    assert 0 <= n_sink and 0 <= n_recent and n_sink + n_recent <= n_sel and n_draft_top >= 0
    out = np.full((B, Hkv, n_sel), -1, dtype=np.int32)
    for b in range(B):
        c = int(min(max(int(ctx_lens[b]), 0), S))
        lo = min(n_sink, c)
        hi = max(c - n_recent, lo)
        protected = np.concatenate([np.arange(0, lo), np.arange(hi, c)]).astype(np.int64)
        fill = n_sel - protected.size
        cand = np.arange(lo, hi, dtype=np.int64)
        for g in range(Hkv):
            m = min(n_draft_top, fill, cand.size)
            top_d = _top_positions(draft_score[b, g, cand], cand, m)
            rest_pos = np.setdiff1d(cand, top_d, assume_unique=True)
            rest = min(fill - m, rest_pos.size)
            top_t = _top_positions(target_score[b, g, rest_pos], rest_pos, rest)
            sel = np.sort(np.concatenate([protected, top_d, top_t]))
            out[b, g, :sel.size] = sel
    return out


def recall_rate(lse_subset: np.ndarray, lse_full: np.ndarray) -> np.ndarray:
    """Attention recall rate of a key subset for each query row: the share of
    the full prefix's softmax mass that falls on the subset,
    sum_{t in I} exp(s_t) / sum_{t < c} exp(s_t) = exp(lse_I - lse_full)
    (the pages name the rate without defining it; this is the plain
    reading)."""
    return np.exp(np.asarray(lse_subset, dtype=np.float64) - np.asarray(lse_full, np.float64))


def tree_depth(parent: np.ndarray) -> np.ndarray:
    """Depth of each draft node, counting the node itself: a child of the
    cached prefix (parent -1) has depth 1, its children depth 2, and so on
    (LongSpec section 2.C: draft tokens form a tree rooted at the prefix).
    Sequences whose parent array is invalid (an entry outside [-1, i-1])
    get -1 everywhere."""
    parent = np.atleast_2d(np.asarray(parent, dtype=np.int64))
    B, N = parent.shape
    depth = np.full((B, N), -1, dtype=np.int64)
    for b in range(B):
        if any(not (-1 <= parent[b, i] <= i - 1) for i in range(N)):
            continue
        for i in range(N):
            p = parent[b, i]
            depth[b, i] = 1 if p < 0 else depth[b, p] + 1
    return depth


def tree_position_ids(parent: np.ndarray, ctx_lens: np.ndarray) -> np.ndarray:
    """Sequence position of each draft node, ctx_b + depth(i) - 1: the node
    takes the place it would have in the sequence if its branch were
    accepted (the position a rotary embedding uses).  -1 for every node of
    a sequence with an invalid parent array.  int32 [B, N]."""
    depth = tree_depth(parent)
    ctx = np.asarray(ctx_lens, dtype=np.int64)[:, None]
    return np.where(depth < 0, -1, ctx + depth - 1).astype(np.int32)


def accepted_path(parent: np.ndarray, node: int) -> np.ndarray:
    """Nodes from the root's child down to `node`, in that order (empty for
    node -1).  Parents precede children, so this is the ancestor-or-self set
    of `node` in increasing index order."""
    path = []
    while node >= 0:
        path.append(int(node))
        node = int(parent[node])
    return np.array(path[::-1], dtype=np.int64)


def accept_path(k: np.ndarray, v: np.ndarray, ctx_lens: np.ndarray, parent: np.ndarray,
                accept_node: np.ndarray):
    """KV-cache update after verification: the accepted draft tokens join the
    cache and the rejected ones are dropped (HiSpec page, KV and hidden-state
    reuse; Dustin page, verification workflow step 5).

    k, v [B, Hkv, S_cap, D] hold the draft tree's rows at [c_b, c_b + N).
    For each sequence b with accept_node[b] = a >= 0, the path
    p_0 < p_1 < ... < p_{L-1} = a (root side first) is moved so that row
    c_b + t receives what row c_b + p_t held, for t < L; c_b becomes
    c_b + L.  Rows at c_b + L and beyond keep whatever they held.  A
    sequence with accept_node -1 (nothing accepted), an invalid parent array,
    accept_node outside [-1, N) or c_b + N > S_cap is left unchanged.
    Returns new (k, v, ctx_lens) arrays; the inputs are not modified."""
    k2, v2 = np.array(k, copy=True), np.array(v, copy=True)
    ctx2 = np.array(ctx_lens, dtype=np.int32, copy=True)
    parent = np.atleast_2d(np.asarray(parent, dtype=np.int64))
    B, N = parent.shape
    S = k.shape[2]
    depth = tree_depth(parent)
    for b in range(B):
        a = int(accept_node[b])
        c = int(ctx_lens[b])
        if a < 0 or a >= N or depth[b, 0] < 0 or c < 0 or c + N > S:
            continue
        path = accepted_path(parent[b], a)
        k2[b, :, c:c + path.size] = k[b][:, c + path]
        v2[b, :, c:c + path.size] = v[b][:, c + path]
        ctx2[b] = c + path.size
    return k2, v2, ctx2
