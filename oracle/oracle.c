/*
 * Verification-attention oracle: plain fp64 CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY: called by the tests, the package smoke check and
 * the CPU-baseline leg of the benchmark; never by the product path.  It
 * shares no code with the HIP path.  Every step follows the definition in
 * oracle.h, written as plainly as possible: the mask row is materialised in
 * full, scores are fp64 dot products, the softmax is a max-shifted sum.
 * Parallelism is over independent rows only (OpenMP); the arithmetic of one
 * row is in definition order.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double load_value(const void *base, int32_t dtype, int64_t idx) {
  if (dtype == ORACLE_F32) return (double)((const float *)base)[idx];
  /* bf16: the 16 stored bits are the high half of an fp32 word */
  uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

int oracle_ancestor_mask(const int32_t *parent, int32_t batch, int32_t n_draft,
                         uint64_t *anc) {
  /* LongSpec page, section 1 (tree attention) and 2.C (masks specific to the
   * branches of the speculation tree): node i sees itself and the nodes on its
   * path to the prefix root.  Walk the path one parent at a time.  A node's
   * mask takes W = ceil(N / 64) words; word w holds nodes 64w .. 64w + 63. */
  if (n_draft < 0 || n_draft > ORACLE_MAX_DRAFT) return -1;
  const int32_t W = (n_draft + 63) / 64;
  for (int32_t b = 0; b < batch; ++b) {
    for (int32_t i = 0; i < n_draft; ++i) {
      int32_t p = parent[(int64_t)b * n_draft + i];
      if (p < -1 || p >= i) return -1;
    }
    for (int32_t i = 0; i < n_draft; ++i) {
      uint64_t *row = anc + ((int64_t)b * n_draft + i) * W;
      for (int32_t w = 0; w < W; ++w) row[w] = 0;
      int32_t j = i;
      while (j >= 0) {
        row[j / 64] |= (uint64_t)1 << (j % 64);
        j = parent[(int64_t)b * n_draft + j];
      }
    }
  }
  return 0;
}

void oracle_lse_merge(int32_t n_parts, int32_t head_dim, const double *lse_parts,
                      const double *o_parts, double *o, double *lse) {
  /* LongSpec page, section 2.C: the two parts' outputs are combined exactly
   * through their log-sum-exp. */
  double m = -INFINITY;
  for (int32_t p = 0; p < n_parts; ++p)
    if (lse_parts[p] > m) m = lse_parts[p];
  for (int32_t d = 0; d < head_dim; ++d) o[d] = 0.0;
  if (m == -INFINITY) {
    *lse = -INFINITY;
    return;
  }
  double sum = 0.0;
  for (int32_t p = 0; p < n_parts; ++p)
    if (lse_parts[p] != -INFINITY) sum += exp(lse_parts[p] - m);
  double total = m + log(sum);
  for (int32_t p = 0; p < n_parts; ++p) {
    if (lse_parts[p] == -INFINITY) continue;
    double w = exp(lse_parts[p] - total);
    for (int32_t d = 0; d < head_dim; ++d) o[d] += w * o_parts[(int64_t)p * head_dim + d];
  }
  *lse = total;
}

/* One output row: explicit mask, fp64 scores, max-shifted softmax. */
static void attend_row(const oracle_desc *d, const void *q, const void *k,
                       const void *v, const int32_t *ctx_lens,
                       const int32_t *parent, const uint64_t *anc_mask,
                       const int32_t *kv_idx, int32_t b, int32_t i, int32_t h,
                       unsigned char *mask, double *score, double *o_row,
                       double *lse_out) {
  const int32_t N = d->n_draft, Hq = d->n_q_heads, Hkv = d->n_kv_heads;
  const int32_t D = d->head_dim, G = Hq / Hkv, g = h / G;
  const int64_t cap = d->kv_capacity;
  const int32_t c = ctx_lens[b];
  const int64_t span = (int64_t)c + N; /* mask covers cache positions [0, c+N) */

  /* 1. the mask row */
  memset(mask, 0, (size_t)span);
  if (d->parts & ORACLE_PART_PREFIX) {
    if (d->n_sel > 0) {
      /* Dustin page, methodology 1: a fixed-size verification set; when the
       * history is shorter than the set, the set is all of it and the slots
       * left over hold -1 (no position). */
      const int32_t *idx = kv_idx + ((int64_t)b * Hkv + g) * d->n_sel;
      for (int32_t s = 0; s < d->n_sel; ++s)
        if (idx[s] >= 0) mask[idx[s]] = 1;
    } else {
      for (int64_t t = 0; t < c; ++t) mask[t] = 1;
    }
  }
  if (d->parts & ORACLE_PART_TREE) {
    if (anc_mask) {
      const int32_t W = (N + 63) / 64;
      const uint64_t *row = anc_mask + ((int64_t)b * N + i) * W;
      for (int32_t j = 0; j < N; ++j)
        if ((row[j / 64] >> (j % 64)) & 1u) mask[c + j] = 1;
    } else {
      int32_t j = i;
      while (j >= 0) {
        mask[c + j] = 1;
        j = parent[(int64_t)b * N + j];
      }
    }
  }

  /* 2. scores over allowed positions */
  const int64_t qoff = (((int64_t)b * N + i) * Hq + h) * D;
  const int64_t kvbase = ((int64_t)b * Hkv + g) * cap;
  double m = -INFINITY;
  for (int64_t t = 0; t < span; ++t) {
    if (!mask[t]) continue;
    double s = 0.0;
    for (int32_t x = 0; x < D; ++x)
      s += load_value(q, d->in_dtype, qoff + x) *
           load_value(k, d->in_dtype, (kvbase + t) * D + x);
    s *= d->scale;
    score[t] = s;
    if (s > m) m = s;
  }

  /* 3. softmax and weighted sum of values */
  for (int32_t x = 0; x < D; ++x) o_row[x] = 0.0;
  if (m == -INFINITY) {
    *lse_out = -INFINITY;
    return;
  }
  double sum = 0.0;
  for (int64_t t = 0; t < span; ++t)
    if (mask[t]) sum += exp(score[t] - m);
  const double lse = m + log(sum);
  for (int64_t t = 0; t < span; ++t) {
    if (!mask[t]) continue;
    const double p = exp(score[t] - lse);
    for (int32_t x = 0; x < D; ++x)
      o_row[x] += p * load_value(v, d->in_dtype, (kvbase + t) * D + x);
  }
  *lse_out = lse;
}

int oracle_verify_attn(const oracle_desc *d, const void *q, const void *k,
                       const void *v, const int32_t *ctx_lens,
                       const int32_t *parent, const uint64_t *anc_mask,
                       const int32_t *kv_idx, const int32_t *rows,
                       int64_t n_rows, double *o, double *lse) {
  if (!d || !q || !k || !v || !ctx_lens || !o || !lse) return -1;
  if ((parent == NULL) == (anc_mask == NULL)) return -1;
  if (d->n_draft < 1 || d->n_draft > ORACLE_MAX_DRAFT || d->head_dim < 1) return -1;
  if (d->n_kv_heads < 1 || d->n_q_heads % d->n_kv_heads) return -1;
  if (d->n_sel > 0 && !kv_idx) return -1;
  for (int32_t b = 0; b < d->batch; ++b) {
    if (ctx_lens[b] < 0 || (int64_t)ctx_lens[b] + d->n_draft > d->kv_capacity) return -1;
    if (parent)
      for (int32_t i = 0; i < d->n_draft; ++i) {
        int32_t p = parent[(int64_t)b * d->n_draft + i];
        if (p < -1 || p >= i) return -1;
      }
    if (d->n_sel > 0)
      for (int64_t s = 0; s < (int64_t)d->n_kv_heads * d->n_sel; ++s) {
        const int32_t *row = kv_idx + (int64_t)b * d->n_kv_heads * d->n_sel;
        int32_t t = row[s];
        /* a position in [0, c_b), or -1 in a tail of -1 entries */
        if (t < -1 || t >= ctx_lens[b]) return -1;
        if (s % d->n_sel > 0 && row[s - 1] == -1 && t != -1) return -1;
      }
  }
  const int64_t total = rows ? n_rows : (int64_t)d->batch * d->n_draft * d->n_q_heads;
  if (rows)
    for (int64_t r = 0; r < n_rows; ++r) {
      const int32_t *t = rows + 3 * r;
      if (t[0] < 0 || t[0] >= d->batch || t[1] < 0 || t[1] >= d->n_draft || t[2] < 0 ||
          t[2] >= d->n_q_heads)
        return -1;
    }
  int32_t max_ctx = 0;
  for (int32_t b = 0; b < d->batch; ++b)
    if (ctx_lens[b] > max_ctx) max_ctx = ctx_lens[b];
  const int64_t span = (int64_t)max_ctx + d->n_draft;
  int failed = 0;

#pragma omp parallel
  {
    unsigned char *mask = (unsigned char *)malloc((size_t)span);
    double *score = (double *)malloc(sizeof(double) * (size_t)span);
    if (!mask || !score) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < total; ++r) {
        int32_t b, i, h;
        if (rows) {
          b = rows[3 * r];
          i = rows[3 * r + 1];
          h = rows[3 * r + 2];
        } else {
          h = (int32_t)(r % d->n_q_heads);
          i = (int32_t)((r / d->n_q_heads) % d->n_draft);
          b = (int32_t)(r / ((int64_t)d->n_q_heads * d->n_draft));
        }
        attend_row(d, q, k, v, ctx_lens, parent, anc_mask, kv_idx, b, i, h, mask, score,
                   o + r * d->head_dim, lse + r);
      }
    }
    free(mask);
    free(score);
  }
  return failed ? -1 : 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
