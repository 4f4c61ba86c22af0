// Host-side launchers for the gfx950 kernels (one per kernel family).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "plan.h"

namespace hsv {

// Number of compute units the split heuristic plans for (MI355X: 8 XCDs x 32).
constexpr int kPlanCUs = 256;

// Geometry of an MFMA partial-attention variant, for the planner.
struct MfmaShape {
  int kgroups;      // partial results per workgroup (waves along keys)
  int tile_keys;    // keys per LDS tile; split lengths are multiples of it
  int rows_per_wg;  // grouped query rows per workgroup
};
MfmaShape mfma_shape(int kernel, int head_dim);

hipError_t launch_attn_partials_valu(const Plan &p, hipStream_t s);
hipError_t launch_attn_partials_mfma(const Plan &p, hipStream_t s);
hipError_t launch_attn_partials_dma(const Plan &p, hipStream_t s);
// The DMA-pipelined variant: dense bf16 prefix, head_dim 128, > 128 rows.
bool dma_supports(const Plan &p);
int dma_rows_per_wg();
int dma_tile_keys();
hipError_t launch_attn_partials_dma_small(const Plan &p, hipStream_t s);
// The per-wave DMA variant for small groups: dense bf16, head_dim 128, <= 32 rows.
bool dma_small_supports(const Plan &p);
int dma_small_tile_keys();
int dma_small_wgs_per_cu(bool sparse);
int dma_small_table_entries();  // block-table columns a paged sparse call may have

// Prefix splits and the tree part -> o_part / lse_part.
hipError_t launch_attn_partials(const Plan &p, hipStream_t s);
// Partials -> o [B, N, Hq, D], lse [B, N, Hq].
hipError_t launch_merge_verify(const Plan &p, hipStream_t s);
// Generic merge: o_parts [P, R, D], lse_parts [P, R] -> o [R, D], lse [R].
hipError_t launch_merge_rows(const float *o_parts, const float *lse_parts, int n_parts,
                             int64_t n_rows, int head_dim, void *o, float *lse, int out_dtype,
                             hipStream_t s);
hipError_t launch_tree_mask(const int32_t *parent, uint64_t *anc, int batch, int n_draft,
                            hipStream_t s);
hipError_t launch_gather_kv(const void *k, const void *v, const int32_t *idx, void *k_out,
                            void *v_out, int batch, int hkv, int cap, int head_dim, int n_sel,
                            int elem_bytes, hipStream_t s);
// Verification index-set selection (one workgroup per (b, kv head)).
hipError_t launch_select_kv_idx(const float *draft, const float *target, int score_len,
                                const int32_t *ctx_lens, int batch, int hkv, int n_sel,
                                int n_sink, int n_recent, int n_draft_top, int32_t *kv_idx,
                                void *workspace, hipStream_t s);
int select_max_positions();
size_t select_workspace_bytes(int batch, int hkv, int score_len);
// Tree position ids and the accepted-path cache update.
hipError_t launch_tree_position_ids(const int32_t *parent, const int32_t *ctx_lens,
                                    int32_t *pos_ids, int batch, int n_draft, hipStream_t s);
hipError_t launch_accept_path(void *k_cache, void *v_cache, int32_t *ctx_lens,
                              const int32_t *parent, const int32_t *accept_node, int batch,
                              int hkv, int s_cap, int row_bytes, int n_draft, hipStream_t s);
// Device-side precondition check; ORs HSV-internal error bits into p.err.
hipError_t launch_validate(const Plan &p, hipStream_t s);

// Error bits written by the validation kernel.
enum : int32_t {
  kErrCtx = 1,     // ctx_lens[b] < 0, > max_ctx, or ctx + N > S_cap
  kErrParent = 2,  // parent[b, i] outside [-1, i-1]
  kErrIndex = 4,   // kv_idx not strictly increasing or outside [0, ctx_b)
};

}  // namespace hsv
