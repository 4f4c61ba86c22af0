// Launch plan shared by the host library and the kernels (plain data only).
#pragma once

#include <stdint.h>

namespace hsv {

enum : int { kF32 = 0, kBF16 = 1 };

// One verify call, resolved on the host.  Grouped row r of KV head g is
// (node i, query head g*G + hh) with r = i*G + hh; a KV head owns R = G*N
// query rows.  Partial results are indexed by "part": parts [0, n_splits)
// are contiguous key ranges of the prefix, part tree_part (if >= 0) is the
// draft block under the tree mask.
struct Plan {
  // inputs
  const void *q;
  const void *k;
  const void *v;
  const int32_t *ctx_lens;
  const int32_t *parent;    // NULL when anc is given (or no tree part)
  const uint64_t *anc;      // NULL when parent is given
  const int32_t *kv_idx;    // sparse prefix, else NULL
  // outputs
  void *o;
  float *lse;
  // workspace partials: o_part [n_parts][B][Hkv][R][D], lse_part [n_parts][B][Hkv][R]
  float *o_part;
  float *lse_part;
  int32_t *err;             // validation error word (workspace)

  int32_t B, N, Hq, Hkv, G, D, R, cap;
  int32_t n_sel;            // > 0: sparse prefix
  int32_t max_ctx;
  int32_t in_dtype, out_dtype;
  int32_t n_splits;         // prefix parts (0 when the prefix is left out)
  int32_t keys_per_split;   // multiple of 64
  int32_t tree_part;        // index of the tree part, or -1
  int32_t n_parts;
  float scale;              // score scale
  float scale_log2;         // scale * log2(e)
};

}  // namespace hsv
