// Launch plan shared by the host library and the kernels (plain data only).
#pragma once

#include <stdint.h>

namespace hsv {

enum : int { kF32 = 0, kBF16 = 1 };

// Partial-attention kernel variants.
enum : int {
  kKernValu = 0,   // vector ALU, any dtype
  kKernMfma32 = 1, // bf16 MFMA, <= 32 grouped rows, 4 key-waves
  kKernMfma64 = 2, // bf16 MFMA, <= 64 grouped rows, 4 key-waves
  kKernMfma128 = 3,// bf16 MFMA, <= 128 grouped rows, 2 row-waves x 2 key-waves
  kKernMfma256 = 4,// bf16 MFMA, 256-row chunks, register-staged tiles
  kKernDma256 = 5, // bf16 MFMA, 256-row chunks, HBM->LDS DMA pipeline (dense, D=128)
  kKernDmaSmall = 6 // bf16 MFMA, <= 32 rows, per-wave HBM->LDS DMA streams (dense, D=128)
};

// One verify call, resolved on the host.  Grouped row r of KV head g is
// (node i, query head g*G + hh) with r = i*G + hh; a KV head owns R = G*N
// query rows.  Keys are cut into "slots".  Separate layout (unified == 0):
// slots [0, n_splits) are contiguous ranges of the prefix (keys_per_split
// each), slot tree_slot (if >= 0) is the draft block under the ancestor mask.
// Unified layout (unified == 1): the prefix rows [0, c) and the draft rows
// [c, c+N) that follow them in the cache form one key range, cut into
// n_splits slots of keys_per_split keys; keys at or past c are masked by the
// ancestor bits.  A workgroup of slot s writes kgroups partial results, parts
// s*kgroups .. s*kgroups + kgroups-1.
struct Plan {
  // inputs
  const void *q;
  const void *k;
  const void *v;
  const int32_t *ctx_lens;
  const int32_t *parent;    // NULL when anc is given (or no tree part)
  const uint64_t *anc;      // NULL when parent is given; [B][N][anc_words]
  uint64_t *anc_ws;         // workspace for the masks of trees of more than 64 nodes
  const int32_t *kv_idx;    // sparse prefix, else NULL
  const int32_t *block_table; // paged cache: [B][max_blocks] pool block of each
                              // logical block of block_size rows; else NULL
  // outputs
  void *o;
  float *lse;
  // workspace partials: o_part [n_parts][B][Hkv][R][D], lse_part [n_parts][B][Hkv][R].
  // With part_f16, o_part holds fp16 rows and o_scale [n_parts][B][Hkv][R] the
  // power of two each row was divided by (row = o_scale * fp16 row).
  float *o_part;
  float *lse_part;
  float *o_scale;
  int32_t *err;             // validation error word (workspace)

  int32_t B, N, Hq, Hkv, G, D, R, cap;
  int32_t n_sel;            // > 0: sparse prefix
  int32_t max_ctx;
  int32_t in_dtype, out_dtype;
  int32_t kernel;           // kKern*
  int32_t n_splits;         // prefix slots (0 when the prefix is left out)
  int32_t keys_per_split;   // multiple of the kernel's key tile
  int32_t has_prefix;       // the prefix part is included
  int32_t has_tree;         // the draft (tree) part is included
  int32_t unified;          // slot layout (see above)
  int32_t part_f16;         // partial rows stored as scaled fp16
  int32_t tree_slot;        // slot index of the tree part (separate layout), or -1
  int32_t n_slots;          // n_splits + (tree_slot >= 0)
  int32_t kgroups;          // partial results per slot workgroup
  int32_t n_parts;          // n_slots * kgroups
  int32_t row_chunks;       // workgroups per (slot, b, kv head) along rows
  int32_t anc_words;        // 64-bit words per node's mask: ceil(N / 64)
  int32_t block_shift;      // paged: log2(block_size)
  int32_t max_blocks;       // paged: cap / block_size (columns of block_table)
  int32_t n_pool_blocks;    // paged: pool blocks in k and v
  float scale;              // score scale
  float scale_log2;         // scale * log2(e)
};

}  // namespace hsv
