// C ABI of the verification-attention library: argument checks, the split
// plan, workspace carving and kernel launches.  No device memory is
// allocated here; nothing is printed.
#include <hip/hip_runtime_api.h>

#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <cstring>

#include "hsv.h"
#include "launch.h"
#include "plan.h"

namespace hsv {

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxSplits = 256;
constexpr int kTile = 64;
constexpr int kMaxDraft = 256;  // draft nodes per sequence (masks of up to 4 words)

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

hsv_status check_desc(const hsv_verify_desc *d, bool sparse) {
  if (!d) return HSV_ERR_NULL;
  if (d->block_size != 0) {
    const int bs = d->block_size;
    if (bs < 64 || bs > (1 << 20) || (bs & (bs - 1)) || d->kv_capacity % bs) return HSV_ERR_SHAPE;
    if (d->flags & HSV_FLAG_NO_PREFIX) return HSV_ERR_UNSUPPORTED;
  }
  if (d->batch < 1 || d->n_draft < 1 || d->n_draft > kMaxDraft) return HSV_ERR_SHAPE;
  if (d->n_kv_heads < 1 || d->n_q_heads < 1 || d->n_q_heads % d->n_kv_heads) return HSV_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return HSV_ERR_UNSUPPORTED;
  if (d->max_ctx < 0 || d->kv_capacity < 1) return HSV_ERR_SHAPE;
  if (static_cast<int64_t>(d->max_ctx) + d->n_draft > d->kv_capacity) return HSV_ERR_SHAPE;
  if (d->in_dtype != HSV_F32 && d->in_dtype != HSV_BF16) return HSV_ERR_UNSUPPORTED;
  if (d->out_dtype != HSV_F32 && d->out_dtype != HSV_BF16) return HSV_ERR_UNSUPPORTED;
  if (d->num_splits < 0 || d->num_splits > kMaxSplits) return HSV_ERR_SHAPE;
  if (!(d->scale >= 0.f) || isinf(d->scale)) return HSV_ERR_SHAPE;
  const uint32_t known = HSV_FLAG_VALIDATE | HSV_FLAG_NO_PREFIX | HSV_FLAG_NO_TREE |
                         HSV_FLAG_PHASE_PARTIALS | HSV_FLAG_PHASE_MERGE |
                         HSV_FLAG_F32_PARTIALS;
  if (d->flags & ~known) return HSV_ERR_UNSUPPORTED;
  if ((d->flags & HSV_FLAG_NO_PREFIX) && (d->flags & HSV_FLAG_NO_TREE)) return HSV_ERR_SHAPE;
  if (sparse) {
    if (d->n_sel < 1 || d->n_sel > d->max_ctx) return HSV_ERR_SHAPE;
  } else if (d->n_sel != 0) {
    return HSV_ERR_SHAPE;
  }
  const int64_t rows = static_cast<int64_t>(d->n_q_heads / d->n_kv_heads) * d->n_draft;
  if (rows > 4096) return HSV_ERR_UNSUPPORTED;
  // all flat indices below must fit comfortably in int64; cache slots in int32
  const int64_t cache_elems =
      static_cast<int64_t>(d->batch) * d->n_kv_heads * d->kv_capacity * d->head_dim;
  if (cache_elems / d->head_dim / d->n_kv_heads / d->batch != d->kv_capacity) return HSV_ERR_SHAPE;
  return HSV_OK;
}

// Workspace of a plan: the partial rows (fp32, or fp16 plus a per-row scale),
// their LSEs, and the validation error word; each region 256-byte aligned.
size_t workspace_bytes(const Plan &p) {
  const size_t rows = static_cast<size_t>(p.n_parts) * p.B * p.Hkv * p.R;
  size_t off = 0;
  off += align_up(rows * p.D * (p.part_f16 ? 2 : sizeof(float)));  // o_part
  off += align_up(rows * sizeof(float));                           // lse_part
  if (p.part_f16) off += align_up(rows * sizeof(float));            // o_scale
  off += kAlign;                                                   // error word
  if (p.anc_words > 1)                                             // wide masks
    off += align_up(static_cast<size_t>(p.B) * p.N * p.anc_words * sizeof(uint64_t));
  return off;
}

// Resolve the descriptor into a launch plan (no pointers yet) and the bytes
// of workspace it needs.
hsv_status make_plan(const hsv_verify_desc *d, bool sparse, Plan *p, size_t *ws_bytes) {
  hsv_status st = check_desc(d, sparse);
  if (st != HSV_OK) return st;
  *p = Plan{};
  p->B = d->batch;
  p->N = d->n_draft;
  p->Hq = d->n_q_heads;
  p->Hkv = d->n_kv_heads;
  p->G = d->n_q_heads / d->n_kv_heads;
  p->D = d->head_dim;
  p->R = p->G * p->N;
  p->anc_words = (p->N + 63) / 64;
  p->cap = d->kv_capacity;
  p->n_sel = sparse ? d->n_sel : 0;
  p->max_ctx = d->max_ctx;
  p->in_dtype = d->in_dtype;
  p->out_dtype = d->out_dtype;
  p->scale = d->scale > 0.f ? d->scale : 1.0f / sqrtf(static_cast<float>(d->head_dim));
  p->scale_log2 = p->scale * 1.4426950408889634f;

  const bool with_prefix = !(d->flags & HSV_FLAG_NO_PREFIX);
  const bool with_tree = !(d->flags & HSV_FLAG_NO_TREE);

  // Kernel variant: bf16 inputs run on the matrix cores, fp32 on the VALU.
  int tile = kTile;
  if (p->in_dtype == kBF16) {
    p->kernel = p->R <= 32 ? kKernMfma32
              : p->R <= 64 ? kKernMfma64
              : p->R <= 128 ? kKernMfma128
                            : kKernMfma256;
    const MfmaShape sh = mfma_shape(p->kernel, p->D);
    p->kgroups = sh.kgroups;
    p->row_chunks = static_cast<int32_t>(ceil_div(p->R, sh.rows_per_wg));
    tile = sh.tile_keys;
    if (dma_supports(*p)) {
      p->kernel = kKernDma256;
      p->kgroups = 1;
      p->row_chunks = static_cast<int32_t>(ceil_div(p->R, dma_rows_per_wg()));
      tile = dma_tile_keys();
    } else if (dma_small_supports(*p)) {
      p->kernel = kKernDmaSmall;
      p->kgroups = 1;
      p->row_chunks = 1;
      tile = dma_small_tile_keys();
    }
  } else {
    p->kernel = kKernValu;
    p->kgroups = 1;
    p->row_chunks = 1;
  }

  p->has_prefix = with_prefix;
  p->has_tree = with_tree;
  p->unified = p->kernel == kKernDma256 || p->kernel == kKernDmaSmall;
  const bool paged = d->block_size > 0;
  if (paged && !p->unified) return HSV_ERR_UNSUPPORTED;
  // paged sparse: the small-group kernel, with the block table in LDS
  if (paged && sparse &&
      (p->kernel != kKernDmaSmall || d->kv_capacity / d->block_size > dma_small_table_entries()))
    return HSV_ERR_UNSUPPORTED;
  if (p->unified) {
    // One key range per (b, kv head): prefix (or index set) then draft rows.  As many
    // splits as fit in one round of the CUs (one workgroup per CU, two for
    // dense calls on the small-group kernel; splits of a multiple of 32 keys), more only
    // when the batch is ragged and a split would exceed 64 tiles.
    const int64_t keys = (with_prefix ? (sparse ? d->n_sel : d->max_ctx) : 0) +
                         (with_tree ? d->n_draft : 0);
    const int64_t units = static_cast<int64_t>(p->B) * p->Hkv * p->row_chunks;
    int64_t target;
    if (d->num_splits > 0) {
      target = d->num_splits;
    } else {
      // the small-group kernel runs several workgroups per CU
      const int64_t slots =
          p->kernel == kKernDmaSmall ? kPlanCUs * dma_small_wgs_per_cu(sparse) : kPlanCUs;
      target = std::max<int64_t>(1, slots / units);
      // A dense batch there takes two rounds of workgroups: its slots are
      // shared out by key range (see below), and the second round evens out
      // what the rounding of that share leaves unequal.
      if (p->kernel == kKernDmaSmall && !sparse && p->B > 1) target *= 2;
      if (p->B > 1)
        while (ceil_div(keys, target * tile) > 64 && target * 2 <= kMaxSplits) target *= 2;
    }
    // Paged dense: splits of whole 64-key tiles (a tile then lies in one
    // pool block) spanning at most 33 pool blocks (one table entry per
    // lane).  Paged sparse rows are translated one by one: no constraint.
    int64_t quantum = 32;
    target = std::max<int64_t>(1, std::min<int64_t>(target, kMaxSplits));
    if (paged && !sparse) {
      quantum = 64;
      const int64_t need = ceil_div(keys, 32 * static_cast<int64_t>(d->block_size));
      if (need > kMaxSplits) return HSV_ERR_UNSUPPORTED;
      target = std::max<int64_t>(target, need);
    }
    const int64_t kps =
        std::max<int64_t>(quantum, ceil_div(ceil_div(keys, target), quantum) * quantum);
    p->keys_per_split = static_cast<int32_t>(kps);
    p->n_splits = keys > 0 ? static_cast<int32_t>(ceil_div(keys, kps)) : 0;
    p->tree_slot = -1;
    p->n_slots = p->n_splits;
    // A dense batch of several sequences on the small-group kernel: the
    // kernel shares n_splits * B slots among the sequences in proportion to
    // their key ranges, so one sequence may take more than n_splits; the
    // workspace holds 2 * n_splits slots per (sequence, KV head), and a
    // longer share is capped there.
    if (p->kernel == kKernDmaSmall && !sparse && p->B > 1 && p->B <= 64 && p->n_splits > 0)
      p->n_slots = 2 * p->n_splits;
    p->n_parts = p->n_slots * p->kgroups;
    p->part_f16 = (d->flags & HSV_FLAG_F32_PARTIALS) ? 0 : 1;
    *ws_bytes = workspace_bytes(*p);
    return HSV_OK;
  }

  const int64_t keys = sparse ? d->n_sel : d->max_ctx;
  if (with_prefix && keys > 0) {
    int64_t target;
    if (d->num_splits > 0) {
      target = d->num_splits;
    } else if (p->kernel == kKernValu) {
      const int64_t units = static_cast<int64_t>(p->B) * p->Hkv;
      target = std::min<int64_t>(ceil_div(2 * kPlanCUs, units), ceil_div(keys, tile));
    } else {
      // One workgroup per CU (each holds the CU's LDS); split the prefix so
      // the (split, b, kv head, row chunk) workgroups cover the CUs, and
      // split further while a split is longer than 64 tiles so that ragged
      // contexts still balance.
      const int64_t units = static_cast<int64_t>(p->B) * p->Hkv * p->row_chunks;
      target = ceil_div(kPlanCUs, units);
      while (ceil_div(keys, target * tile) > 64 && target * 2 <= kMaxSplits) target *= 2;
      target = std::min<int64_t>(target, ceil_div(keys, tile));
    }
    target = std::max<int64_t>(1, std::min<int64_t>(target, kMaxSplits));
    p->keys_per_split = static_cast<int32_t>(ceil_div(ceil_div(keys, target), tile) * tile);
    p->n_splits = static_cast<int32_t>(target);
  } else {
    p->n_splits = 0;
    p->keys_per_split = tile;
  }
  p->tree_slot = with_tree ? p->n_splits : -1;
  p->n_slots = p->n_splits + (with_tree ? 1 : 0);
  p->n_parts = p->n_slots * p->kgroups;
  p->part_f16 = 0;
  *ws_bytes = workspace_bytes(*p);
  return HSV_OK;
}

void carve_workspace(Plan *p, void *ws) {
  char *base = static_cast<char *>(ws);
  const size_t rows = static_cast<size_t>(p->n_parts) * p->B * p->Hkv * p->R;
  p->o_part = reinterpret_cast<float *>(base);
  base += align_up(rows * p->D * (p->part_f16 ? 2 : sizeof(float)));
  p->lse_part = reinterpret_cast<float *>(base);
  base += align_up(rows * sizeof(float));
  p->o_scale = nullptr;
  if (p->part_f16) {
    p->o_scale = reinterpret_cast<float *>(base);
    base += align_up(rows * sizeof(float));
  }
  p->err = reinterpret_cast<int32_t *>(base);
  base += kAlign;
  p->anc_ws = p->anc_words > 1 ? reinterpret_cast<uint64_t *>(base) : nullptr;
}

hsv_status run_verify(const hsv_verify_desc *d, bool sparse, const void *q, const void *k,
                      const void *v, const int32_t *ctx_lens, const int32_t *parent,
                      const uint64_t *anc, const int32_t *kv_idx, void *o, float *lse, void *ws,
                      size_t ws_bytes, hipStream_t stream, const int32_t *block_table = nullptr,
                      int32_t n_pool_blocks = 0) {
  if (!d) return HSV_ERR_NULL;
  // a contiguous call must not carry a block size (the paged entry point
  // passes the table)
  if (!block_table && d->block_size != 0) return HSV_ERR_SHAPE;
  if (block_table && n_pool_blocks < 1) return HSV_ERR_SHAPE;
  Plan p;
  size_t need = 0;
  hsv_status st = make_plan(d, sparse, &p, &need);
  if (st != HSV_OK) return st;
  const bool with_tree = p.has_tree;
  if (!q || !k || !v || !ctx_lens || !o || !lse) return HSV_ERR_NULL;
  if (sparse && !kv_idx) return HSV_ERR_NULL;
  if (with_tree && ((parent == nullptr) == (anc == nullptr))) return HSV_ERR_NULL;
  if (!ws) return HSV_ERR_WORKSPACE;
  if (ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) % kAlign)) return HSV_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
       reinterpret_cast<uintptr_t>(v)) % 16)
    return HSV_ERR_SHAPE;  // 16-byte vector loads

  p.q = q;
  p.k = k;
  p.v = v;
  p.ctx_lens = ctx_lens;
  p.parent = with_tree ? parent : nullptr;
  p.anc = with_tree ? anc : nullptr;
  p.kv_idx = sparse ? kv_idx : nullptr;
  if (block_table) {
    p.block_table = block_table;
    p.block_shift = __builtin_ctz(static_cast<unsigned>(d->block_size));
    p.max_blocks = d->kv_capacity / d->block_size;
    p.n_pool_blocks = n_pool_blocks;
  }
  p.o = o;
  p.lse = lse;
  carve_workspace(&p, ws);

  if (d->flags & HSV_FLAG_VALIDATE) {
    if (hipMemsetAsync(p.err, 0, sizeof(int32_t), stream) != hipSuccess) return HSV_ERR_HIP;
    if (launch_validate(p, stream) != hipSuccess) return HSV_ERR_HIP;
    int32_t host_err = 0;
    if (hipMemcpyAsync(&host_err, p.err, sizeof host_err, hipMemcpyDeviceToHost, stream) !=
        hipSuccess)
      return HSV_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return HSV_ERR_HIP;
    if (host_err) return HSV_ERR_DEVICE_CHECK;
  }
  // trees of more than 64 nodes given as parents: their multi-word masks
  // first, into the workspace
  if (p.has_tree && p.anc_words > 1 && p.parent) {
    if (launch_tree_mask(p.parent, p.anc_ws, p.B, p.N, stream) != hipSuccess) return HSV_ERR_HIP;
    p.anc = p.anc_ws;
    p.parent = nullptr;
  }
  const uint32_t phase = d->flags & (HSV_FLAG_PHASE_PARTIALS | HSV_FLAG_PHASE_MERGE);
  const bool run_partials = phase != HSV_FLAG_PHASE_MERGE;
  const bool run_merge = phase != HSV_FLAG_PHASE_PARTIALS;
  if (run_partials && p.n_parts > 0 && launch_attn_partials(p, stream) != hipSuccess)
    return HSV_ERR_HIP;
  if (run_merge && launch_merge_verify(p, stream) != hipSuccess) return HSV_ERR_HIP;
  return HSV_OK;
}

}  // namespace

hipError_t launch_attn_partials(const Plan &p, hipStream_t s) {
  switch (p.kernel) {
    case kKernValu: return launch_attn_partials_valu(p, s);
    case kKernDma256: return launch_attn_partials_dma(p, s);
    case kKernDmaSmall: return launch_attn_partials_dma_small(p, s);
    default: return launch_attn_partials_mfma(p, s);
  }
}

}  // namespace hsv

using namespace hsv;

extern "C" {

hsv_status hsv_verify_workspace_bytes(const hsv_verify_desc *d, size_t *bytes) {
  if (!d || !bytes) return HSV_ERR_NULL;
  Plan p;
  return make_plan(d, d->n_sel > 0, &p, bytes);
}

hsv_status hsv_verify_attn(const hsv_verify_desc *d, const void *q, const void *k_cache,
                           const void *v_cache, const int32_t *ctx_lens, const int32_t *parent,
                           const uint64_t *anc_mask, void *o, float *lse, void *workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  return run_verify(d, false, q, k_cache, v_cache, ctx_lens, parent, anc_mask, nullptr, o, lse,
                    workspace, workspace_bytes, stream);
}

hsv_status hsv_verify_attn_sparse(const hsv_verify_desc *d, const void *q, const void *k_cache,
                                  const void *v_cache, const int32_t *ctx_lens,
                                  const int32_t *parent, const uint64_t *anc_mask,
                                  const int32_t *kv_idx, void *o, float *lse, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  return run_verify(d, true, q, k_cache, v_cache, ctx_lens, parent, anc_mask, kv_idx, o, lse,
                    workspace, workspace_bytes, stream);
}

hsv_status hsv_verify_attn_paged(const hsv_verify_desc *d, const void *q, const void *k_pool,
                                 const void *v_pool, const int32_t *block_table,
                                 int32_t n_pool_blocks, const int32_t *ctx_lens,
                                 const int32_t *parent, const uint64_t *anc_mask, void *o,
                                 float *lse, void *workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  if (!d) return HSV_ERR_NULL;
  if (d->block_size == 0) return HSV_ERR_SHAPE;
  if (!block_table) return HSV_ERR_NULL;
  return run_verify(d, false, q, k_pool, v_pool, ctx_lens, parent, anc_mask, nullptr, o, lse,
                    workspace, workspace_bytes, stream, block_table, n_pool_blocks);
}

hsv_status hsv_verify_attn_sparse_paged(const hsv_verify_desc *d, const void *q,
                                        const void *k_pool, const void *v_pool,
                                        const int32_t *block_table, int32_t n_pool_blocks,
                                        const int32_t *ctx_lens, const int32_t *parent,
                                        const uint64_t *anc_mask, const int32_t *kv_idx, void *o,
                                        float *lse, void *workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
  if (!d) return HSV_ERR_NULL;
  if (d->block_size == 0) return HSV_ERR_SHAPE;
  if (!block_table) return HSV_ERR_NULL;
  return run_verify(d, true, q, k_pool, v_pool, ctx_lens, parent, anc_mask, kv_idx, o, lse,
                    workspace, workspace_bytes, stream, block_table, n_pool_blocks);
}

hsv_status hsv_tree_ancestor_mask(const int32_t *parent, uint64_t *anc_mask, int32_t batch,
                                  int32_t n_draft, hipStream_t stream) {
  if (!parent || !anc_mask) return HSV_ERR_NULL;
  if (batch < 1 || n_draft < 1 || n_draft > kMaxDraft) return HSV_ERR_SHAPE;
  return launch_tree_mask(parent, anc_mask, batch, n_draft, stream) == hipSuccess ? HSV_OK
                                                                                  : HSV_ERR_HIP;
}

hsv_status hsv_gather_kv(const void *k_cache, const void *v_cache, const int32_t *kv_idx,
                         void *k_out, void *v_out, int32_t batch, int32_t n_kv_heads,
                         int32_t kv_capacity, int32_t head_dim, int32_t n_sel, int32_t dtype,
                         hipStream_t stream) {
  if (!k_cache || !v_cache || !kv_idx || !k_out || !v_out) return HSV_ERR_NULL;
  if (dtype != HSV_F32 && dtype != HSV_BF16) return HSV_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return HSV_ERR_UNSUPPORTED;
  if (batch < 1 || n_kv_heads < 1 || kv_capacity < 1 || n_sel < 1) return HSV_ERR_SHAPE;
  if (static_cast<int64_t>(batch) * n_kv_heads > 65535) return HSV_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache) |
       reinterpret_cast<uintptr_t>(k_out) | reinterpret_cast<uintptr_t>(v_out)) % 16)
    return HSV_ERR_SHAPE;
  const int elem = dtype == HSV_F32 ? 4 : 2;
  return launch_gather_kv(k_cache, v_cache, kv_idx, k_out, v_out, batch, n_kv_heads, kv_capacity,
                          head_dim, n_sel, elem, stream) == hipSuccess
             ? HSV_OK
             : HSV_ERR_HIP;
}

hsv_status hsv_select_workspace_bytes(int32_t batch, int32_t n_kv_heads, int32_t score_len,
                                      size_t *bytes) {
  if (!bytes) return HSV_ERR_NULL;
  if (batch < 1 || n_kv_heads < 1 || score_len < 1) return HSV_ERR_SHAPE;
  if (score_len > select_max_positions()) return HSV_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(batch) * n_kv_heads > (int64_t{1} << 24)) return HSV_ERR_SHAPE;
  *bytes = select_workspace_bytes(batch, n_kv_heads, score_len);
  return HSV_OK;
}

hsv_status hsv_select_kv_idx(const float *draft_score, const float *target_score,
                             int32_t score_len, const int32_t *ctx_lens, int32_t batch,
                             int32_t n_kv_heads, int32_t n_sel, int32_t n_sink, int32_t n_recent,
                             int32_t n_draft_top, int32_t *kv_idx, void *workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  if (!draft_score || !target_score || !ctx_lens || !kv_idx) return HSV_ERR_NULL;
  size_t need = 0;
  const hsv_status st = hsv_select_workspace_bytes(batch, n_kv_heads, score_len, &need);
  if (st != HSV_OK) return st;
  if (n_sel < 1) return HSV_ERR_SHAPE;
  if (n_sink < 0 || n_recent < 0 || n_draft_top < 0 ||
      static_cast<int64_t>(n_sink) + n_recent > n_sel)
    return HSV_ERR_SHAPE;
  if (!workspace) return HSV_ERR_WORKSPACE;
  if (workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) % kAlign))
    return HSV_ERR_WORKSPACE;
  return launch_select_kv_idx(draft_score, target_score, score_len, ctx_lens, batch, n_kv_heads,
                              n_sel, n_sink, n_recent, n_draft_top, kv_idx, workspace,
                              stream) == hipSuccess
             ? HSV_OK
             : HSV_ERR_HIP;
}

hsv_status hsv_tree_position_ids(const int32_t *parent, const int32_t *ctx_lens,
                                 int32_t *pos_ids, int32_t batch, int32_t n_draft,
                                 hipStream_t stream) {
  if (!parent || !ctx_lens || !pos_ids) return HSV_ERR_NULL;
  if (batch < 1 || n_draft < 1 || n_draft > kMaxDraft) return HSV_ERR_SHAPE;
  return launch_tree_position_ids(parent, ctx_lens, pos_ids, batch, n_draft, stream) == hipSuccess
             ? HSV_OK
             : HSV_ERR_HIP;
}

hsv_status hsv_accept_path(void *k_cache, void *v_cache, int32_t *ctx_lens, const int32_t *parent,
                           const int32_t *accept_node, int32_t batch, int32_t n_kv_heads,
                           int32_t kv_capacity, int32_t head_dim, int32_t n_draft, int32_t dtype,
                           hipStream_t stream) {
  if (!k_cache || !v_cache || !ctx_lens || !parent || !accept_node) return HSV_ERR_NULL;
  if (dtype != HSV_F32 && dtype != HSV_BF16) return HSV_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return HSV_ERR_UNSUPPORTED;
  if (batch < 1 || n_kv_heads < 1 || n_draft < 1 || n_draft > kMaxDraft || kv_capacity < n_draft)
    return HSV_ERR_SHAPE;
  if (static_cast<int64_t>(batch) * n_kv_heads > (int64_t{1} << 31) - 1) return HSV_ERR_SHAPE;
  const int row_bytes = head_dim * (dtype == HSV_F32 ? 4 : 2);
  return launch_accept_path(k_cache, v_cache, ctx_lens, parent, accept_node, batch, n_kv_heads,
                            kv_capacity, row_bytes, n_draft, stream) == hipSuccess
             ? HSV_OK
             : HSV_ERR_HIP;
}

hsv_status hsv_lse_merge(const float *o_parts, const float *lse_parts, int32_t n_parts,
                         int64_t n_rows, int32_t head_dim, void *o, float *lse, int32_t out_dtype,
                         hipStream_t stream) {
  if (!o_parts || !lse_parts || !o || !lse) return HSV_ERR_NULL;
  if (n_parts < 1 || n_parts > 1024 || n_rows < 1) return HSV_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return HSV_ERR_UNSUPPORTED;
  if (out_dtype != HSV_F32 && out_dtype != HSV_BF16) return HSV_ERR_UNSUPPORTED;
  if (n_rows > (int64_t{1} << 40)) return HSV_ERR_SHAPE;
  return launch_merge_rows(o_parts, lse_parts, n_parts, n_rows, head_dim, o, lse, out_dtype,
                           stream) == hipSuccess
             ? HSV_OK
             : HSV_ERR_HIP;
}

const char *hsv_status_string(hsv_status s) {
  // A C caller may pass any int: read its bits instead of loading the enum
  // (a value outside the enumeration's range is not a valid hsv_status).
  static_assert(sizeof(hsv_status) == sizeof(int), "hsv_status is passed as an int");
  int code;
  std::memcpy(&code, &s, sizeof code);
  switch (code) {
    case HSV_OK: return "HSV_OK: success";
    case HSV_ERR_NULL: return "HSV_ERR_NULL: a required pointer is NULL";
    case HSV_ERR_SHAPE: return "HSV_ERR_SHAPE: sizes out of range or inconsistent";
    case HSV_ERR_UNSUPPORTED: return "HSV_ERR_UNSUPPORTED: a valid request the library does not implement";
    case HSV_ERR_WORKSPACE: return "HSV_ERR_WORKSPACE: workspace missing, too small or misaligned";
    case HSV_ERR_DEVICE_CHECK: return "HSV_ERR_DEVICE_CHECK: device-side input check failed";
    case HSV_ERR_HIP: return "HSV_ERR_HIP: HIP runtime or launch failure";
  }
  return "unknown hsv_status";
}

int32_t hsv_version(void) { return HSV_VERSION; }

}  // extern "C"
