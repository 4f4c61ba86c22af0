/*
 * hsv — verification attention for speculative decoding on MI355X (gfx950).
 *
 * C ABI.  Every pointer argument is a device pointer unless stated
 * otherwise; every buffer belongs to the caller.  The library allocates and
 * frees no device memory: scratch lives in the caller's workspace, sized by
 * hsv_verify_workspace_bytes() (hsv_verify_attn_noalloc: a static array the
 * library's code object holds on each GPU).  Work is enqueued on `stream` and the calls
 * return without synchronising the host (except under HSV_FLAG_VALIDATE).
 * The library keeps no mutable global state, so concurrent calls on different
 * streams with different workspaces are safe -- except hsv_verify_attn_noalloc,
 * whose scratch is one library-owned array per GPU (see there).
 * Except under HSV_FLAG_VALIDATE, a call enqueues kernel launches only (no
 * memset, copy or synchronisation), so it may be captured into a HIP graph
 * and replayed; a validating call synchronises `stream` and cannot be
 * captured.
 *
 * What is computed.  LongSpec ("Long-Context Lossless Speculative Decoding
 * with Efficient Drafting and Verification"), section 2.C "Hybrid Tree
 * Attention": the target model verifies a tree of draft tokens; attention is
 * divided into a cache part (the long history, no mask) and a speculative
 * part (the draft tokens, under a mask that follows the branches of the
 * tree), and the two parts' outputs are combined exactly through their
 * log-sum-exp.  The combined result is therefore plain masked softmax
 * attention:
 *
 *   for sequence b, draft node i, query head h, KV head g = h / (Hq / Hkv):
 *     A(b,i,g) = P(b,g)  u  { c_b + j : node j is node i or an ancestor of i }
 *     P(b,g)   = [0, c_b)                       (hsv_verify_attn)
 *              = { kv_idx[b,g,s] : s < n_sel }  (hsv_verify_attn_sparse)
 *     s_t  = scale * <q[b,i,h,:], k[b,g,t,:]>
 *     lse  = log sum_{t in A} exp(s_t)          (natural log)
 *     o    = sum_{t in A} exp(s_t - lse) * v[b,g,t,:]
 *
 * The sparse form follows the Dustin page ("Verification workflow" and
 * "Limitations"): the target verifies against a compressed cache made of a
 * selected token subset while the full history stays in place and indexed.
 *
 * Conventions (fixed here; the pages leave them open):
 *   - the draft block's K and V sit in the same cache at positions
 *     [c_b, c_b + N), node j at c_b + j;
 *   - node i sees itself and its ancestors (parent chain), never siblings or
 *     descendants; parent[i] in [-1, i-1], -1 meaning the cached prefix;
 *   - query head h uses KV head h / (Hq / Hkv) (contiguous groups);
 *   - an empty key set gives o = 0, lse = -inf (cannot happen when the tree
 *     part is on: a node always sees itself).
 *
 * Layouts (row-major, innermost last, no padding):
 *   q        [B, N, Hq, D]       in_dtype
 *   k, v     [B, Hkv, S_cap, D]  in_dtype
 *   ctx_lens [B]                 int32
 *   parent   [B, N]              int32
 *   anc_mask [B, N, W]           uint64, W = ceil(N / 64) words per node;
 *                                bit j % 64 of word j / 64 = node j visible
 *                                from node i ([B, N] when N <= 64)
 *   kv_idx   [B, Hkv, n_sel]     int32: strictly increasing positions < c_b,
 *                                optionally followed by -1 entries (empty
 *                                slots of a set larger than the history)
 *   o        [B, N, Hq, D]       out_dtype
 *   lse      [B, N, Hq]          float
 *
 * Errors.  Calls return a status and never print.  Argument checks that need
 * no device data run first and return before anything is enqueued.  Data
 * preconditions held in device memory (parent range, ctx_lens bounds, index
 * order and range) are the caller's contract; with HSV_FLAG_VALIDATE a check
 * kernel runs first and the call synchronises `stream` to report
 * HSV_ERR_DEVICE_CHECK.  HIP launch failures return HSV_ERR_HIP.
 */
#ifndef HSV_H
#define HSV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HSV_VERSION 1

typedef enum hsv_status {
  HSV_OK = 0,
  HSV_ERR_NULL = 1,         /* a required pointer is NULL                        */
  HSV_ERR_SHAPE = 2,        /* sizes out of range or inconsistent                */
  HSV_ERR_UNSUPPORTED = 3,  /* valid request the library does not implement     */
  HSV_ERR_WORKSPACE = 4,    /* workspace missing, too small or misaligned        */
  HSV_ERR_DEVICE_CHECK = 5, /* HSV_FLAG_VALIDATE found bad device-side data      */
  HSV_ERR_HIP = 6           /* a HIP runtime call or kernel launch failed        */
} hsv_status;

typedef enum hsv_dtype { HSV_F32 = 0, HSV_BF16 = 1 } hsv_dtype;

/* Run a device-side check of parent, ctx_lens and kv_idx first; synchronises. */
#define HSV_FLAG_VALIDATE 1u
/* Leave out the cache part (prefix) or the speculative part (draft tree).
 * Each alone is one of the two partial attentions of LongSpec section 2.C. */
#define HSV_FLAG_NO_PREFIX 2u
#define HSV_FLAG_NO_TREE 4u
/* Run one phase only.  A verify call is two phases: PARTIALS (partial
 * attentions over splits of the key set, written to the workspace) and MERGE
 * (the exact log-sum-exp combination into o and lse).  A MERGE-only call must follow a
 * PARTIALS-only call with the same descriptor and workspace on the same
 * stream (or be otherwise ordered after it).  Neither or both bits: both
 * phases.  Lets a caller time the phases apart or place work between them. */
#define HSV_FLAG_PHASE_PARTIALS 8u
#define HSV_FLAG_PHASE_MERGE 16u
/* Keep the split partials in fp32.  By default the bf16, D = 128 kernels
 * with more than 128 or at most 32 grouped rows store each normalised
 * partial row as fp16 times a power of two (the row's largest |value| in
 * [0.5, 1), 11 significant bits per value, half the workspace and traffic
 * of fp32); the other kernels always use fp32.  The flag doubles the
 * partials' bytes; it serves to measure what the fp16 storage costs in
 * accuracy, which stays within 2^-11 of the largest |o| of a row per split. */
#define HSV_FLAG_F32_PARTIALS 32u

typedef struct hsv_verify_desc {
  int32_t batch;       /* B >= 1                                                */
  int32_t n_draft;     /* N in [1, 256] (above 64, masks of ceil(N/64) words)   */
  int32_t n_q_heads;   /* Hq >= 1, a multiple of n_kv_heads                     */
  int32_t n_kv_heads;  /* Hkv >= 1                                              */
  int32_t head_dim;    /* D: 64 or 128                                          */
  int32_t kv_capacity; /* S_cap: token slots per (b, kv head) in k and v        */
  int32_t max_ctx;     /* host-known upper bound on ctx_lens[]; sizes the grid; */
                       /* max_ctx + N <= S_cap                                  */
  int32_t n_sel;       /* sparse call: indices per (b, kv head), 1..max_ctx;    */
                       /* dense call: must be 0                                 */
  int32_t in_dtype;    /* hsv_dtype of q, k, v                                  */
  int32_t out_dtype;   /* hsv_dtype of o                                        */
  float scale;         /* score scale; 0 means 1/sqrt(head_dim)                 */
  int32_t num_splits;  /* key splits; 0 = automatic, else 1..256.  bf16 calls  */
                       /* with D = 128 and more than 128 grouped rows (G*N,    */
                       /* dense) or at most 32 (dense or sparse) treat the     */
                       /* prefix (or index set) and the draft rows as one key  */
                       /* range cut into that many slots (with at most 32      */
                       /* rows, each sequence's range into equal slots); other */
                       /* calls split the prefix (or index set) and add one    */
                       /* part for the draft tree.  Results do not depend on   */
                       /* the split count beyond rounding.                     */
  uint32_t flags;      /* HSV_FLAG_* bits                                       */
  int32_t block_size;  /* paged calls: tokens per pool block, a power         */
                       /* of two >= 64 dividing kv_capacity; 0 for the other    */
                       /* calls                                                 */
} hsv_verify_desc;

/* Bytes of workspace hsv_verify_attn / hsv_verify_attn_sparse need for `d`.
 * Writes *bytes; returns HSV_ERR_SHAPE / HSV_ERR_UNSUPPORTED for a
 * descriptor the verify calls would reject. */
hsv_status hsv_verify_workspace_bytes(const hsv_verify_desc *d, size_t *bytes);

/* Dense verification attention: prefix [0, c_b) plus the draft tree.
 * Give exactly one of `parent` / `anc_mask` (the other NULL); with
 * HSV_FLAG_NO_TREE both may be NULL.  Writes every element of o and lse.
 * `workspace` must be 256-byte aligned and at least the reported size;
 * its contents on entry do not matter. */
hsv_status hsv_verify_attn(const hsv_verify_desc *d, const void *q,
                           const void *k_cache, const void *v_cache,
                           const int32_t *ctx_lens, const int32_t *parent,
                           const uint64_t *anc_mask, void *o, float *lse,
                           void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Sparse verification attention: prefix = the cache positions in
 * kv_idx[b, g, :] (strictly increasing, each < c_b; a tail of -1 entries
 * marks empty slots, as hsv_select_kv_idx writes when c_b < n_sel), plus the
 * draft tree.
 * Same arguments and rules as hsv_verify_attn otherwise. */
hsv_status hsv_verify_attn_sparse(const hsv_verify_desc *d, const void *q,
                                  const void *k_cache, const void *v_cache,
                                  const int32_t *ctx_lens,
                                  const int32_t *parent,
                                  const uint64_t *anc_mask,
                                  const int32_t *kv_idx, void *o, float *lse,
                                  void *workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* Dense verification attention over a paged cache (HiSpec page: paged
 * attention with block tables, so that sequences of a batch can accept
 * different numbers of tokens without padding).  Same computation as
 * hsv_verify_attn on the cache whose row t of sequence b, KV head g is row
 * t % bs of pool block block_table[b, t / bs], bs = d->block_size:
 *   k_pool, v_pool [n_pool_blocks, Hkv, bs, D]  (bf16, D = 128)
 *   block_table    [B, kv_capacity / bs] int32 in [0, n_pool_blocks)
 * Logical rows [0, c_b) are the prefix and [c_b, c_b + N) the draft tree,
 * as in the contiguous cache; every table entry those rows fall in must name
 * a pool block (an entry outside the pool is clamped into it, which gives
 * wrong values but reads no memory outside the pool; HSV_FLAG_VALIDATE
 * reports it as HSV_ERR_DEVICE_CHECK).  Runs where the contiguous call
 * would use the 16-byte DMA kernels (bf16, D = 128, at most 32 or more than
 * 128 grouped rows); other shapes, HSV_FLAG_NO_PREFIX and more than
 * 256 * 32 * bs keys return HSV_ERR_UNSUPPORTED.  The workspace size comes
 * from hsv_verify_workspace_bytes with the same descriptor. */
hsv_status hsv_verify_attn_paged(const hsv_verify_desc *d, const void *q,
                                 const void *k_pool, const void *v_pool,
                                 const int32_t *block_table, int32_t n_pool_blocks,
                                 const int32_t *ctx_lens, const int32_t *parent,
                                 const uint64_t *anc_mask, void *o, float *lse,
                                 void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Sparse verification attention over a paged cache (Dustin page: the
 * verification attends to a selected subset of a fully indexed cache;
 * HiSpec page: that cache paged with block tables).  Same computation as
 * hsv_verify_attn_sparse on the cache that the pool and table describe as in
 * hsv_verify_attn_paged: kv_idx[b, g, :] holds logical positions (strictly
 * increasing, each < c_b, then an optional tail of -1 slots) and each
 * selected row, like each draft row c_b + j, is read from the pool block its
 * table entry names.  Runs where the contiguous sparse call uses the
 * small-group DMA kernel (bf16, D = 128, at most 32 grouped rows) and the
 * table has at most 6144 columns (kv_capacity / block_size); other shapes
 * and HSV_FLAG_NO_PREFIX return HSV_ERR_UNSUPPORTED.  Table entries outside
 * the pool are clamped into it (wrong values, no read outside the pool;
 * HSV_FLAG_VALIDATE reports them).  The pool may exceed 4 GiB.  Workspace
 * size from hsv_verify_workspace_bytes with the same descriptor. */
hsv_status hsv_verify_attn_sparse_paged(const hsv_verify_desc *d, const void *q,
                                        const void *k_pool, const void *v_pool,
                                        const int32_t *block_table, int32_t n_pool_blocks,
                                        const int32_t *ctx_lens, const int32_t *parent,
                                        const uint64_t *anc_mask, const int32_t *kv_idx, void *o,
                                        float *lse, void *workspace, size_t workspace_bytes,
                                        hipStream_t stream);

/* Ancestor bitmask of each draft tree (LongSpec section 2.C: the mask of the
 * speculative part follows the branches of the tree).
 * parent [B, N] int32 in [-1, i-1]; anc_mask [B, N, W] uint64 out
 * (W = ceil(N / 64)), bit j % 64 of word j / 64 set iff node j is node i or
 * an ancestor of i.  N in [1, 256].  Entries of a sequence with an
 * out-of-range parent are written as 0. */
hsv_status hsv_tree_ancestor_mask(const int32_t *parent, uint64_t *anc_mask,
                                  int32_t batch, int32_t n_draft,
                                  hipStream_t stream);

/* Compressed cache of the sparse form (Dustin page, "Verification workflow",
 * step 3): k_out[b,g,s,:] = k_cache[b,g,kv_idx[b,g,s],:], same for v.
 * k_cache, v_cache [B, Hkv, S_cap, D]; kv_idx [B, Hkv, n_sel] with entries in
 * [0, S_cap) (an out-of-range entry yields a zero row); k_out, v_out
 * [B, Hkv, n_sel, D].  A bit-exact copy; dtype is the element type. */
hsv_status hsv_gather_kv(const void *k_cache, const void *v_cache,
                         const int32_t *kv_idx, void *k_out, void *v_out,
                         int32_t batch, int32_t n_kv_heads, int32_t kv_capacity,
                         int32_t head_dim, int32_t n_sel, int32_t dtype,
                         hipStream_t stream);

/* Sequence position of each draft node (LongSpec section 2.C: the draft
 * tokens form a tree rooted at the cached prefix): pos_ids[b, i] =
 * ctx_lens[b] + depth(i) - 1, where a child of the prefix (parent -1) has
 * depth 1 -- the position node i would take if its branch were accepted, as
 * a rotary embedding needs it.  parent [B, N] int32 in [-1, i-1]; ctx_lens
 * [B] int32; pos_ids [B, N] int32 out.  N in [1, 256].  Every entry of a
 * sequence with an out-of-range parent is written as -1. */
hsv_status hsv_tree_position_ids(const int32_t *parent, const int32_t *ctx_lens,
                                 int32_t *pos_ids, int32_t batch, int32_t n_draft,
                                 hipStream_t stream);

/* Cache update after verification (HiSpec page, reuse of the KV cache with
 * the entries of rejected tokens removed; Dustin page, verification
 * workflow step 5: accepted tokens join the cache, rejected ones are
 * dropped).  k_cache, v_cache [B, Hkv, S_cap, D] (dtype HSV_F32 or
 * HSV_BF16, D 64 or 128) hold the draft tree's rows at [c_b, c_b + N),
 * c_b = ctx_lens[b].  For accept_node[b] = a in [0, N), the path
 * p_0 < ... < p_{L-1} = a from the prefix down to a is moved in place so
 * that row c_b + t holds what row c_b + p_t held, and ctx_lens[b] becomes
 * c_b + L; rows at c_b + L and beyond are not written.  accept_node -1
 * accepts nothing.  A sequence with accept_node outside [-1, N), an
 * out-of-range parent, c_b < 0 or c_b + N > S_cap is left unchanged.
 * ctx_lens is read and updated on the device (stream-ordered: two
 * launches); parent [B, N] and accept_node [B] are int32.  N in [1, 256]. */
hsv_status hsv_accept_path(void *k_cache, void *v_cache, int32_t *ctx_lens,
                           const int32_t *parent, const int32_t *accept_node,
                           int32_t batch, int32_t n_kv_heads, int32_t kv_capacity,
                           int32_t head_dim, int32_t n_draft, int32_t dtype,
                           hipStream_t stream);

/* Fixed-size verification index set (Dustin page, methodology 1: hybrid
 * attention aggregation of a draft-lookahead and a target-historical signal;
 * the sparse verification attention then reads only these positions).
 * For each (sequence b, KV head g), of the positions [0, c) with
 * c = min(ctx_lens[b], score_len): the first n_sink and the last n_recent
 * are kept; of the positions between them, the n_draft_top best by
 * draft_score, then the best remaining ones by target_score, until n_sel
 * positions are chosen.  Best = higher score; NaN ranks below every number;
 * -0 equals +0; ties go to the lower position.
 * draft_score, target_score [B, Hkv, score_len] float (entries at or past
 * c_b do not affect the result; the whole rows may be read);
 * ctx_lens [B] int32 (device); kv_idx [B, Hkv, n_sel]
 * int32 out, strictly increasing -- if c_b < n_sel the tail is -1.
 * Requires n_sink + n_recent <= n_sel, n_draft_top >= 0 and
 * score_len <= 524288; the chosen set is unique (no randomness).
 * `workspace` (device, 256-byte aligned, at least
 * hsv_select_workspace_bytes) holds the per-row floors and the candidate
 * lists between the call's three launches; its contents on entry do not
 * matter. */
hsv_status hsv_select_kv_idx(const float *draft_score, const float *target_score,
                             int32_t score_len, const int32_t *ctx_lens, int32_t batch,
                             int32_t n_kv_heads, int32_t n_sel, int32_t n_sink,
                             int32_t n_recent, int32_t n_draft_top, int32_t *kv_idx,
                             void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Bytes of workspace hsv_select_kv_idx needs for these sizes (per (b, KV
 * head) four words of floors, and per 8192-position chunk of its score rows
 * two candidate lists of 1024 (key, position) slots and their counts).  HSV_ERR_SHAPE /
 * HSV_ERR_UNSUPPORTED for sizes the call would reject. */
hsv_status hsv_select_workspace_bytes(int32_t batch, int32_t n_kv_heads, int32_t score_len,
                                      size_t *bytes);

/* Exact log-sum-exp merge of partial attention results (LongSpec section
 * 2.C: the parts' outputs are combined exactly), e.g. partials over disjoint
 * key ranges computed on several devices.
 * o_parts [P, R, D] float, each part normalised within itself;
 * lse_parts [P, R] float; o [R, D] out_dtype; lse [R] float.
 *   lse = log sum_p exp(lse_p),  o = sum_p exp(lse_p - lse) * o_p
 * Parts with lse_p = -inf are skipped (their o_p is never read); a row whose
 * parts are all -inf gets o = 0, lse = -inf.  P in [1, 1024], D in {64, 128}. */
hsv_status hsv_lse_merge(const float *o_parts, const float *lse_parts,
                         int32_t n_parts, int64_t n_rows, int32_t head_dim,
                         void *o, float *lse, int32_t out_dtype,
                         hipStream_t stream);

/* Size of the scratch array hsv_verify_attn_noalloc uses on each GPU. */
#define HSV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* hsv_verify_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same computation, arguments, kernels
 * and results as hsv_verify_attn; the scratch those kernels use is a
 * library-owned device array of HSV_NOALLOC_SCRATCH_BYTES on each GPU, held
 * from the first call on that GPU until the process ends.  No device memory
 * is allocated or freed by the call.  A descriptor whose workspace
 * (hsv_verify_workspace_bytes) exceeds HSV_NOALLOC_SCRATCH_BYTES returns
 * HSV_ERR_WORKSPACE; a paged (block_size != 0) or sparse (n_sel != 0)
 * descriptor returns HSV_ERR_SHAPE.  Every call on one GPU shares that GPU's
 * array and it keeps the last call's contents (nothing in it needs to start
 * at zero): calls that overlap on one GPU (different streams, or
 * different host threads without ordering) race and give wrong results.
 * The GPU is the device of `stream` (the current device for the null
 * stream). */
hsv_status hsv_verify_attn_noalloc(const hsv_verify_desc *d, const void *q,
                                   const void *k_cache, const void *v_cache,
                                   const int32_t *ctx_lens, const int32_t *parent,
                                   const uint64_t *anc_mask, void *o, float *lse,
                                   hipStream_t stream);

/* Static description of a status code (never NULL). */
const char *hsv_status_string(hsv_status s);

/* HSV_VERSION of the built library. */
int32_t hsv_version(void);

#ifdef __cplusplus
}
#endif
#endif /* HSV_H */
