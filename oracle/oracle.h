/*
 * Verification-attention oracle: plain fp64 CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this library; only the tests, the package smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code with the HIP path.
 *
 * What it computes (LongSpec page, section 2.C "Hybrid Tree Attention": the
 * verification attention of the draft tokens, whose cache part and
 * speculative part are combined exactly, so the result is one masked softmax
 * attention over the union of both parts; Dustin page, "Verification
 * workflow" and "Limitations": the sparse form attends to a selected subset of
 * a fully indexed cache):
 *
 *   for each sequence b, draft node i, query head h, with g = h / (Hq/Hkv):
 *     A = P(b,g) u { c_b + j : j in T(b,i) }        (explicit 0/1 mask row)
 *       P(b,g) = [0, c_b)                 dense
 *              = { kv_idx[b,g,k] : kv_idx[b,g,k] >= 0 }   sparse (-1: empty slot,
 *                                                  only in a tail of -1 entries)
 *       T(b,i) = { i, parent[i], parent[parent[i]], ... }   (walk until -1)
 *                or the set bits of anc_mask[b,i,:] when given instead
 *     s_t = scale * sum_d q[b,i,h,d] * k[b,g,t,d]          (fp64)
 *     lse = log sum_{t in A} exp(s_t)                      (max-shifted)
 *     o   = sum_{t in A} exp(s_t - lse) * v[b,g,t,:]
 *   An empty A gives o = 0, lse = -inf.
 */
#ifndef ORACLE_H
#define ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };
enum { ORACLE_PART_PREFIX = 1, ORACLE_PART_TREE = 2 };
enum { ORACLE_MAX_DRAFT = 256 }; /* draft nodes per sequence */

typedef struct {
  int32_t batch, n_draft, n_q_heads, n_kv_heads, head_dim;
  int32_t kv_capacity; /* token slots per (b, kv head) */
  int32_t n_sel;       /* 0: dense prefix; >0: sparse prefix from kv_idx */
  int32_t in_dtype;    /* ORACLE_F32 or ORACLE_BF16 (uint16 bit patterns) */
  int32_t parts;       /* ORACLE_PART_PREFIX | ORACLE_PART_TREE */
  double scale;
} oracle_desc;

/* Ancestor sets by walking parent pointers one by one.
 * parent: [B, N], parent[i] in [-1, i-1], N <= ORACLE_MAX_DRAFT.
 * anc: [B, N, W], W = ceil(N / 64); bit j % 64 of word j / 64 set iff node j
 * is node i or one of its ancestors.  Returns 0, or -1 for a parent out of
 * range (anc left unspecified). */
int oracle_ancestor_mask(const int32_t *parent, int32_t batch, int32_t n_draft,
                         uint64_t *anc);

/* Verification attention for a list of rows.
 * q: [B, N, Hq, D]; k, v: [B, Hkv, S_cap, D]; ctx_lens: [B];
 * exactly one of parent [B, N] / anc_mask [B, N, ceil(N/64)] non-NULL;
 * kv_idx: [B, Hkv, n_sel] when n_sel > 0, else ignored.
 * rows: n_rows (b, i, h) triples, or NULL for every row (n_rows ignored).
 * o: [n_rows, D] (or [B, N, Hq, D] when rows is NULL), lse: [n_rows].
 * Returns 0, or -1 on a malformed argument. */
int oracle_verify_attn(const oracle_desc *d, const void *q, const void *k,
                       const void *v, const int32_t *ctx_lens,
                       const int32_t *parent, const uint64_t *anc_mask,
                       const int32_t *kv_idx, const int32_t *rows,
                       int64_t n_rows, double *o, double *lse);

/* Exact log-sum-exp merge of n_parts partial results of one row.
 * lse_parts: [P]; o_parts: [P, D] (each normalised within its part).
 * lse = log sum_p exp(lse_p); o = sum_p exp(lse_p - lse) * o_p.
 * Parts with lse_p = -inf contribute nothing; all -inf gives o = 0, -inf. */
void oracle_lse_merge(int32_t n_parts, int32_t head_dim, const double *lse_parts,
                      const double *o_parts, double *o, double *lse);

/* Number of OpenMP threads the oracle uses. */
int oracle_num_threads(void);

/* Set the number of OpenMP threads of later calls (n > 0); used to time the
   oracle on one thread as well as on every core. */
void oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
