"""Verification attention for speculative decoding on MI355X (gfx950).

Thin Python binding over the C ABI in ``include/hsv.h`` (``libhsv.so``).
Functions carry the C names; they only check and marshal torch tensors
(PyTorch supplies device memory and streams) and call the library, where
every step of the computation runs in hand-written HIP kernels.  There is no
CPU fallback: if ``libhsv.so`` is missing, importing this package fails.
"""

from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import (  # noqa: F401
    EXPORTS,
    HSV_BF16,
    HSV_ERR_DEVICE_CHECK,
    HSV_ERR_HIP,
    HSV_ERR_NULL,
    HSV_ERR_SHAPE,
    HSV_ERR_UNSUPPORTED,
    HSV_ERR_WORKSPACE,
    HSV_F32,
    HSV_FLAG_F32_PARTIALS,
    HSV_FLAG_NO_PREFIX,
    HSV_FLAG_NO_TREE,
    HSV_FLAG_PHASE_MERGE,
    HSV_FLAG_PHASE_PARTIALS,
    HSV_FLAG_VALIDATE,
    HSV_NOALLOC_SCRATCH_BYTES,
    HSV_OK,
    HsvError,
    HsvVerifyDesc,
)

lib = _lib.load()

_DT = {torch.float32: HSV_F32, torch.bfloat16: HSV_BF16}


def _dtype_code(t: torch.Tensor, what: str) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"{what}: dtype {t.dtype} not supported (float32 or bfloat16)")
    return _DT[t.dtype]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("all tensors must be on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


def mask_words(n: int) -> int:
    """64-bit words of one draft node's mask (word w: nodes 64w .. 64w+63)."""
    return (n + 63) // 64


def _check_mask(anc_mask, B, N):
    shapes = {(B, N)} if N <= 64 else {(B, N, mask_words(N))}
    if anc_mask is not None and (anc_mask.dtype not in (torch.int64, torch.uint64)
                                 or tuple(anc_mask.shape) not in shapes):
        raise ValueError("anc_mask must be 64-bit [B, N] (N <= 64) or [B, N, ceil(N/64)]")


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(code: int, where: str):
    if code != HSV_OK:
        raise HsvError(code, where)


def make_desc(*, batch, n_draft, n_q_heads, n_kv_heads, head_dim, kv_capacity, max_ctx,
              n_sel=0, in_dtype=HSV_BF16, out_dtype=HSV_F32, scale=0.0, num_splits=0,
              flags=0, block_size=0) -> HsvVerifyDesc:
    return HsvVerifyDesc(batch, n_draft, n_q_heads, n_kv_heads, head_dim, kv_capacity, max_ctx,
                         n_sel, in_dtype, out_dtype, float(scale), num_splits, flags,
                         block_size)


def hsv_verify_workspace_bytes(desc: HsvVerifyDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.hsv_verify_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)),
           "hsv_verify_workspace_bytes")
    return int(n.value)


def _verify(sparse: bool, q, k_cache, v_cache, ctx_lens, parent, anc_mask, kv_idx, *, max_ctx,
            out_dtype, scale, num_splits, flags, o, lse, workspace, stream):
    B, N, Hq, D = q.shape
    Bk, Hkv, cap, Dk = k_cache.shape
    if (Bk, Dk) != (B, D) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q / k_cache / v_cache shapes disagree")
    in_dt = _dtype_code(q, "q")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache and v_cache must share a dtype")
    if ctx_lens.dtype != torch.int32 or tuple(ctx_lens.shape) != (B,):
        raise ValueError("ctx_lens must be int32 [B]")
    if parent is not None and (parent.dtype != torch.int32 or tuple(parent.shape) != (B, N)):
        raise ValueError("parent must be int32 [B, N]")
    _check_mask(anc_mask, B, N)
    n_sel = 0
    if sparse:
        if kv_idx is None or kv_idx.dtype != torch.int32 or kv_idx.dim() != 3 or \
                tuple(kv_idx.shape[:2]) != (B, Hkv):
            raise ValueError("kv_idx must be int32 [B, Hkv, n_sel]")
        n_sel = kv_idx.shape[2]
    if o is None:
        o = torch.empty((B, N, Hq, D), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, N, Hq), dtype=torch.float32, device=q.device)
    out_dt = _dtype_code(o, "o")
    if tuple(o.shape) != (B, N, Hq, D) or lse.dtype != torch.float32 or \
            tuple(lse.shape) != (B, N, Hq):
        raise ValueError("o must be [B, N, Hq, D] and lse float32 [B, N, Hq]")
    desc = make_desc(batch=B, n_draft=N, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D,
                     kv_capacity=cap, max_ctx=int(max_ctx), n_sel=n_sel, in_dtype=in_dt,
                     out_dtype=out_dt, scale=scale, num_splits=num_splits, flags=flags)
    need = hsv_verify_workspace_bytes(desc)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check_dev(q, k_cache, v_cache, ctx_lens, parent, anc_mask, kv_idx, o, lse, workspace)
    s = _stream(stream, q.device)
    common = (ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(ctx_lens),
              _ptr(parent), _ptr(anc_mask))
    tail = (_ptr(o), _ptr(lse), _ptr(workspace), ctypes.c_size_t(workspace.numel()), s)
    if sparse:
        code = lib.hsv_verify_attn_sparse(*common, _ptr(kv_idx), *tail)
        _check(code, "hsv_verify_attn_sparse")
    else:
        code = lib.hsv_verify_attn(*common, *tail)
        _check(code, "hsv_verify_attn")
    return o, lse


def hsv_verify_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    ctx_lens: torch.Tensor, parent: Optional[torch.Tensor] = None,
                    anc_mask: Optional[torch.Tensor] = None, *, max_ctx: int,
                    out_dtype=torch.float32, scale: float = 0.0, num_splits: int = 0,
                    flags: int = 0, o=None, lse=None, workspace=None, stream=None
                    ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Dense verification attention (see include/hsv.h).  Returns (o, lse)."""
    return _verify(False, q, k_cache, v_cache, ctx_lens, parent, anc_mask, None,
                   max_ctx=max_ctx, out_dtype=out_dtype, scale=scale, num_splits=num_splits,
                   flags=flags, o=o, lse=lse, workspace=workspace, stream=stream)


def hsv_verify_attn_sparse(q, k_cache, v_cache, ctx_lens, parent=None, anc_mask=None,
                           kv_idx=None, *, max_ctx: int, out_dtype=torch.float32,
                           scale: float = 0.0, num_splits: int = 0, flags: int = 0, o=None,
                           lse=None, workspace=None, stream=None):
    """Sparse verification attention over kv_idx (see include/hsv.h)."""
    return _verify(True, q, k_cache, v_cache, ctx_lens, parent, anc_mask, kv_idx,
                   max_ctx=max_ctx, out_dtype=out_dtype, scale=scale, num_splits=num_splits,
                   flags=flags, o=o, lse=lse, workspace=workspace, stream=stream)


def hsv_verify_attn_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            ctx_lens: torch.Tensor, parent: Optional[torch.Tensor] = None,
                            anc_mask: Optional[torch.Tensor] = None, *, max_ctx: int,
                            o: torch.Tensor, lse: torch.Tensor, scale: float = 0.0,
                            num_splits: int = 0, flags: int = 0, stream=None) -> None:
    """hsv_verify_attn with the library's own per-GPU scratch instead of a
    workspace (see include/hsv.h).  Allocates nothing: the caller passes o
    [B, N, Hq, D] (float32 or bfloat16) and lse float32 [B, N, Hq]."""
    B, N, Hq, D = q.shape
    Bk, Hkv, cap, Dk = k_cache.shape
    if (Bk, Dk) != (B, D) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q / k_cache / v_cache shapes disagree")
    in_dt = _dtype_code(q, "q")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache and v_cache must share a dtype")
    if ctx_lens.dtype != torch.int32 or tuple(ctx_lens.shape) != (B,):
        raise ValueError("ctx_lens must be int32 [B]")
    if parent is not None and (parent.dtype != torch.int32 or tuple(parent.shape) != (B, N)):
        raise ValueError("parent must be int32 [B, N]")
    _check_mask(anc_mask, B, N)
    out_dt = _dtype_code(o, "o")
    if tuple(o.shape) != (B, N, Hq, D) or lse.dtype != torch.float32 or \
            tuple(lse.shape) != (B, N, Hq):
        raise ValueError("o must be [B, N, Hq, D] and lse float32 [B, N, Hq]")
    desc = make_desc(batch=B, n_draft=N, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D,
                     kv_capacity=cap, max_ctx=int(max_ctx), in_dtype=in_dt, out_dtype=out_dt,
                     scale=scale, num_splits=num_splits, flags=flags)
    _check_dev(q, k_cache, v_cache, ctx_lens, parent, anc_mask, o, lse)
    _check(lib.hsv_verify_attn_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_cache),
                                       _ptr(v_cache), _ptr(ctx_lens), _ptr(parent),
                                       _ptr(anc_mask), _ptr(o), _ptr(lse),
                                       _stream(stream, q.device)), "hsv_verify_attn_noalloc")


def _verify_paged(sparse: bool, q, k_pool, v_pool, block_table, ctx_lens, parent, anc_mask,
                  kv_idx, *, max_ctx, out_dtype, scale, num_splits, flags, o, lse, workspace,
                  stream):
    B, N, Hq, D = q.shape
    n_pool, Hkv, bs, Dk = k_pool.shape
    if Dk != D or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("q / k_pool / v_pool shapes disagree")
    in_dt = _dtype_code(q, "q")
    if k_pool.dtype != q.dtype or v_pool.dtype != q.dtype:
        raise TypeError("q, k_pool and v_pool must share a dtype")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_blocks]")
    if ctx_lens.dtype != torch.int32 or tuple(ctx_lens.shape) != (B,):
        raise ValueError("ctx_lens must be int32 [B]")
    if parent is not None and (parent.dtype != torch.int32 or tuple(parent.shape) != (B, N)):
        raise ValueError("parent must be int32 [B, N]")
    _check_mask(anc_mask, B, N)
    n_sel = 0
    if sparse:
        if kv_idx is None or kv_idx.dtype != torch.int32 or kv_idx.dim() != 3 or \
                tuple(kv_idx.shape[:2]) != (B, Hkv):
            raise ValueError("kv_idx must be int32 [B, Hkv, n_sel]")
        n_sel = kv_idx.shape[2]
    if o is None:
        o = torch.empty((B, N, Hq, D), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, N, Hq), dtype=torch.float32, device=q.device)
    out_dt = _dtype_code(o, "o")
    if tuple(o.shape) != (B, N, Hq, D) or lse.dtype != torch.float32 or \
            tuple(lse.shape) != (B, N, Hq):
        raise ValueError("o must be [B, N, Hq, D] and lse float32 [B, N, Hq]")
    desc = make_desc(batch=B, n_draft=N, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D,
                     kv_capacity=block_table.shape[1] * bs, max_ctx=int(max_ctx), n_sel=n_sel,
                     in_dtype=in_dt, out_dtype=out_dt, scale=scale, num_splits=num_splits,
                     flags=flags, block_size=bs)
    need = hsv_verify_workspace_bytes(desc)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check_dev(q, k_pool, v_pool, block_table, ctx_lens, parent, anc_mask, kv_idx, o, lse,
               workspace)
    head = (ctypes.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), n_pool,
            _ptr(ctx_lens), _ptr(parent), _ptr(anc_mask))
    tail = (_ptr(o), _ptr(lse), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
            _stream(stream, q.device))
    if sparse:
        _check(lib.hsv_verify_attn_sparse_paged(*head, _ptr(kv_idx), *tail),
               "hsv_verify_attn_sparse_paged")
    else:
        _check(lib.hsv_verify_attn_paged(*head, *tail), "hsv_verify_attn_paged")
    return o, lse


def hsv_verify_attn_paged(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                          block_table: torch.Tensor, ctx_lens: torch.Tensor,
                          parent: Optional[torch.Tensor] = None,
                          anc_mask: Optional[torch.Tensor] = None, *, max_ctx: int,
                          out_dtype=torch.float32, scale: float = 0.0, num_splits: int = 0,
                          flags: int = 0, o=None, lse=None, workspace=None, stream=None
                          ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Dense verification attention over a paged cache (see include/hsv.h):
    k_pool, v_pool [n_blocks, Hkv, block_size, D]; block_table int32
    [B, max_blocks].  Returns (o, lse)."""
    return _verify_paged(False, q, k_pool, v_pool, block_table, ctx_lens, parent, anc_mask,
                         None, max_ctx=max_ctx, out_dtype=out_dtype, scale=scale,
                         num_splits=num_splits, flags=flags, o=o, lse=lse,
                         workspace=workspace, stream=stream)


def hsv_verify_attn_sparse_paged(q, k_pool, v_pool, block_table, ctx_lens, parent=None,
                                 anc_mask=None, kv_idx=None, *, max_ctx: int,
                                 out_dtype=torch.float32, scale: float = 0.0,
                                 num_splits: int = 0, flags: int = 0, o=None, lse=None,
                                 workspace=None, stream=None):
    """Sparse verification attention over a paged cache (see include/hsv.h):
    the pool and table as in hsv_verify_attn_paged, kv_idx int32
    [B, Hkv, n_sel] of logical positions.  Returns (o, lse)."""
    return _verify_paged(True, q, k_pool, v_pool, block_table, ctx_lens, parent, anc_mask,
                         kv_idx, max_ctx=max_ctx, out_dtype=out_dtype, scale=scale,
                         num_splits=num_splits, flags=flags, o=o, lse=lse,
                         workspace=workspace, stream=stream)


def hsv_tree_ancestor_mask(parent: torch.Tensor, anc_mask: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """Ancestor bitmask of the draft trees in ``parent``: 64-bit [B, N] for
    N <= 64, else [B, N, ceil(N/64)] (word w: nodes 64w .. 64w+63)."""
    if parent.dtype != torch.int32 or parent.dim() != 2:
        raise ValueError("parent must be int32 [B, N]")
    B, N = parent.shape
    if anc_mask is None:
        shape = (B, N) if N <= 64 else (B, N, mask_words(N))
        anc_mask = torch.empty(shape, dtype=torch.int64, device=parent.device)
    _check_mask(anc_mask, B, N)
    _check_dev(parent, anc_mask)
    _check(lib.hsv_tree_ancestor_mask(_ptr(parent), _ptr(anc_mask), B, N,
                                      _stream(stream, parent.device)), "hsv_tree_ancestor_mask")
    return anc_mask


def hsv_gather_kv(k_cache, v_cache, kv_idx, k_out=None, v_out=None, stream=None):
    """Compressed cache: rows kv_idx[b, g, :] of k_cache / v_cache."""
    B, Hkv, cap, D = k_cache.shape
    n_sel = kv_idx.shape[2]
    dt = _dtype_code(k_cache, "k_cache")
    if k_out is None:
        k_out = torch.empty((B, Hkv, n_sel, D), dtype=k_cache.dtype, device=k_cache.device)
    if v_out is None:
        v_out = torch.empty((B, Hkv, n_sel, D), dtype=v_cache.dtype, device=v_cache.device)
    if kv_idx.dtype != torch.int32 or tuple(kv_idx.shape[:2]) != (B, Hkv):
        raise ValueError("kv_idx must be int32 [B, Hkv, n_sel]")
    _check_dev(k_cache, v_cache, kv_idx, k_out, v_out)
    _check(lib.hsv_gather_kv(_ptr(k_cache), _ptr(v_cache), _ptr(kv_idx), _ptr(k_out),
                             _ptr(v_out), B, Hkv, cap, D, n_sel, dt,
                             _stream(stream, k_cache.device)), "hsv_gather_kv")
    return k_out, v_out


def hsv_lse_merge(o_parts: torch.Tensor, lse_parts: torch.Tensor, out_dtype=torch.float32,
                  o=None, lse=None, stream=None):
    """Exact merge of partials: o_parts [P, R, D], lse_parts [P, R] -> (o [R, D], lse [R])."""
    P, R, D = o_parts.shape
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32 or \
            tuple(lse_parts.shape) != (P, R):
        raise ValueError("o_parts float32 [P, R, D] and lse_parts float32 [P, R] expected")
    if o is None:
        o = torch.empty((R, D), dtype=out_dtype, device=o_parts.device)
    if lse is None:
        lse = torch.empty((R,), dtype=torch.float32, device=o_parts.device)
    _check_dev(o_parts, lse_parts, o, lse)
    _check(lib.hsv_lse_merge(_ptr(o_parts), _ptr(lse_parts), P, R, D, _ptr(o), _ptr(lse),
                             _dtype_code(o, "o"), _stream(stream, o_parts.device)),
           "hsv_lse_merge")
    return o, lse


def hsv_select_workspace_bytes(batch: int, n_kv_heads: int, score_len: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.hsv_select_workspace_bytes(batch, n_kv_heads, score_len, ctypes.byref(n)),
           "hsv_select_workspace_bytes")
    return int(n.value)


def hsv_select_kv_idx(draft_score: torch.Tensor, target_score: torch.Tensor,
                      ctx_lens: torch.Tensor, *, n_sel: int, n_sink: int, n_recent: int,
                      n_draft_top: int, kv_idx=None, workspace=None, stream=None
                      ) -> torch.Tensor:
    """Verification index set (see include/hsv.h): draft_score, target_score
    float32 [B, Hkv, L]; returns kv_idx int32 [B, Hkv, n_sel]."""
    if draft_score.dtype != torch.float32 or target_score.dtype != torch.float32 or \
            draft_score.dim() != 3 or tuple(target_score.shape) != tuple(draft_score.shape):
        raise ValueError("draft_score and target_score must be float32 [B, Hkv, L]")
    B, Hkv, L = draft_score.shape
    if ctx_lens.dtype != torch.int32 or tuple(ctx_lens.shape) != (B,):
        raise ValueError("ctx_lens must be int32 [B]")
    if kv_idx is None:
        kv_idx = torch.empty((B, Hkv, n_sel), dtype=torch.int32, device=draft_score.device)
    if kv_idx.dtype != torch.int32 or tuple(kv_idx.shape) != (B, Hkv, n_sel):
        raise ValueError("kv_idx must be int32 [B, Hkv, n_sel]")
    if workspace is None:
        workspace = torch.empty(max(hsv_select_workspace_bytes(B, Hkv, L), 256),
                                dtype=torch.uint8, device=draft_score.device)
    _check_dev(draft_score, target_score, ctx_lens, kv_idx, workspace)
    _check(lib.hsv_select_kv_idx(_ptr(draft_score), _ptr(target_score), L, _ptr(ctx_lens), B, Hkv,
                                 n_sel, n_sink, n_recent, n_draft_top, _ptr(kv_idx),
                                 _ptr(workspace), ctypes.c_size_t(workspace.numel()),
                                 _stream(stream, draft_score.device)), "hsv_select_kv_idx")
    return kv_idx


def hsv_tree_position_ids(parent: torch.Tensor, ctx_lens: torch.Tensor,
                          pos_ids: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Sequence position c_b + depth(i) - 1 of each draft node (int32 [B, N])."""
    if parent.dtype != torch.int32 or parent.dim() != 2:
        raise ValueError("parent must be int32 [B, N]")
    B, N = parent.shape
    if ctx_lens.dtype != torch.int32 or tuple(ctx_lens.shape) != (B,):
        raise ValueError("ctx_lens must be int32 [B]")
    if pos_ids is None:
        pos_ids = torch.empty((B, N), dtype=torch.int32, device=parent.device)
    if pos_ids.dtype != torch.int32 or tuple(pos_ids.shape) != (B, N):
        raise ValueError("pos_ids must be int32 [B, N]")
    _check_dev(parent, ctx_lens, pos_ids)
    _check(lib.hsv_tree_position_ids(_ptr(parent), _ptr(ctx_lens), _ptr(pos_ids), B, N,
                                     _stream(stream, parent.device)), "hsv_tree_position_ids")
    return pos_ids


def hsv_accept_path(k_cache: torch.Tensor, v_cache: torch.Tensor, ctx_lens: torch.Tensor,
                    parent: torch.Tensor, accept_node: torch.Tensor, stream=None) -> None:
    """In-place cache update: the accepted node's path moves to [c_b, c_b + L)
    and ctx_lens grows by L (see include/hsv.h)."""
    B, Hkv, cap, D = k_cache.shape
    dt = _dtype_code(k_cache, "k_cache")
    if v_cache.dtype != k_cache.dtype or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("v_cache must match k_cache")
    if parent.dtype != torch.int32 or parent.dim() != 2 or parent.shape[0] != B:
        raise ValueError("parent must be int32 [B, N]")
    N = parent.shape[1]
    for name, t in (("ctx_lens", ctx_lens), ("accept_node", accept_node)):
        if t.dtype != torch.int32 or tuple(t.shape) != (B,):
            raise ValueError(f"{name} must be int32 [B]")
    _check_dev(k_cache, v_cache, ctx_lens, parent, accept_node)
    _check(lib.hsv_accept_path(_ptr(k_cache), _ptr(v_cache), _ptr(ctx_lens), _ptr(parent),
                               _ptr(accept_node), B, Hkv, cap, D, N, dt,
                               _stream(stream, k_cache.device)), "hsv_accept_path")


def hsv_status_string(code: int) -> str:
    return _lib.status_string(code)


def hsv_version() -> int:
    return int(lib.hsv_version())
