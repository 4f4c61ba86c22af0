/*
 * Drives every entry point of the fp64 oracle on small seeded inputs, for a
 * build under AddressSanitizer and UndefinedBehaviorSanitizer: each buffer is
 * allocated at exactly the size the oracle's header states, so a read or
 * write past it is reported.  Cases cover dense and sparse prefixes (with -1
 * tails), fp32 and bf16 inputs, parent arrays and explicit masks of one to
 * four words per node, each part alone, empty contexts, row subsets, bad
 * parents and merges with empty parts.  Exit status 0 when every call
 * returned what its contract says and every result row is sane.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t g_state = 0x243F6A8885A308D3ull;

static uint64_t next_u64(void) {  /* splitmix64 */
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static int rand_int(int lo, int hi) { /* inclusive */
  return lo + (int)(next_u64() % (uint64_t)(hi - lo + 1));
}

static float rand_f(void) { return (float)((double)(next_u64() >> 11) / 9007199254740992.0 - 0.5); }

static uint16_t to_bf16(float f) {  /* round to nearest even */
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static void *xmalloc(size_t n) {
  void *p = malloc(n ? n : 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}

static void fill(void *buf, int dtype, size_t n) {
  if (dtype == ORACLE_F32) {
    float *f = (float *)buf;
    for (size_t i = 0; i < n; ++i) f[i] = rand_f();
  } else {
    uint16_t *h = (uint16_t *)buf;
    for (size_t i = 0; i < n; ++i) h[i] = to_bf16(rand_f());
  }
}

static int failures = 0;
#define CHECK(cond, ...)                  \
  do {                                    \
    if (!(cond)) {                        \
      fprintf(stderr, __VA_ARGS__);       \
      fputc('\n', stderr);                \
      ++failures;                         \
    }                                     \
  } while (0)

static void run_case(int B, int N, int Hq, int Hkv, int D, int max_ctx, int n_sel, int dtype,
                     int parts, int use_anc, int n_rows) {
  const int G = Hq / Hkv;
  const int cap = max_ctx + N;
  const int W = (N + 63) / 64;
  const size_t es = dtype == ORACLE_F32 ? 4 : 2;
  void *q = xmalloc((size_t)B * N * Hq * D * es);
  void *k = xmalloc((size_t)B * Hkv * cap * D * es);
  void *v = xmalloc((size_t)B * Hkv * cap * D * es);
  fill(q, dtype, (size_t)B * N * Hq * D);
  fill(k, dtype, (size_t)B * Hkv * cap * D);
  fill(v, dtype, (size_t)B * Hkv * cap * D);
  int32_t *ctx = (int32_t *)xmalloc((size_t)B * 4);
  for (int b = 0; b < B; ++b) ctx[b] = rand_int(0, max_ctx);
  int32_t *parent = (int32_t *)xmalloc((size_t)B * N * 4);
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < N; ++i) parent[b * N + i] = rand_int(-1, i - 1);
  uint64_t *anc = (uint64_t *)xmalloc((size_t)B * N * W * 8);
  CHECK(oracle_ancestor_mask(parent, B, N, anc) == 0, "ancestor mask failed (N=%d)", N);
  int32_t *kv_idx = NULL;
  if (n_sel > 0) {
    kv_idx = (int32_t *)xmalloc((size_t)B * Hkv * n_sel * 4);
    for (int b = 0; b < B; ++b)
      for (int g = 0; g < Hkv; ++g) {
        int32_t *row = kv_idx + ((size_t)b * Hkv + g) * n_sel;
        int s = 0;
        /* strictly increasing positions below ctx, then a -1 tail */
        for (int t = 0; t < ctx[b] && s < n_sel; ++t)
          if (rand_int(0, 2) == 0) row[s++] = t;
        for (; s < n_sel; ++s) row[s] = -1;
      }
  }
  int32_t *rows = NULL;
  int64_t nr = (int64_t)B * N * Hq;
  if (n_rows > 0) {
    rows = (int32_t *)xmalloc((size_t)n_rows * 3 * 4);
    for (int r = 0; r < n_rows; ++r) {
      rows[3 * r] = rand_int(0, B - 1);
      rows[3 * r + 1] = rand_int(0, N - 1);
      rows[3 * r + 2] = rand_int(0, Hq - 1);
    }
    nr = n_rows;
  }
  double *o = (double *)xmalloc((size_t)nr * D * 8);
  double *lse = (double *)xmalloc((size_t)nr * 8);
  oracle_desc d = {B, N, Hq, Hkv, D, cap, n_sel, dtype, parts, 1.0 / sqrt((double)D)};
  const int rc = oracle_verify_attn(&d, q, k, v, ctx, use_anc ? NULL : parent,
                                    use_anc ? anc : NULL, kv_idx, rows, nr, o, lse);
  CHECK(rc == 0, "verify returned %d (B=%d N=%d sel=%d parts=%d)", rc, B, N, n_sel, parts);
  for (int64_t r = 0; r < nr && rc == 0; ++r) {
    const int has_tree_part = (parts & ORACLE_PART_TREE) != 0;
    CHECK(!isnan(lse[r]) && lse[r] < INFINITY, "row %lld: lse %g", (long long)r, lse[r]);
    if (has_tree_part) CHECK(isfinite(lse[r]), "row %lld: tree part gives no keys", (long long)r);
    for (int e = 0; e < D; ++e) {
      const double x = o[r * D + e];
      CHECK(isfinite(x), "row %lld: o not finite", (long long)r);
      if (isinf(lse[r])) CHECK(x == 0.0, "row %lld: empty row with o != 0", (long long)r);
    }
  }
  (void)G;
  free(q); free(k); free(v); free(ctx); free(parent); free(anc); free(kv_idx); free(rows);
  free(o); free(lse);
}

static void merge_cases(void) {
  for (int P = 0; P <= 6; ++P)
    for (int D = 1; D <= 128; D *= 4) {
      double *lp = (double *)xmalloc((size_t)P * 8);
      double *op = (double *)xmalloc((size_t)P * D * 8);
      double *o = (double *)xmalloc((size_t)D * 8);
      double lse;
      int live = 0;
      for (int p = 0; p < P; ++p) {
        lp[p] = rand_int(0, 2) == 0 ? -INFINITY : 4.0 * rand_f();
        live += isfinite(lp[p]);
        for (int e = 0; e < D; ++e) op[p * D + e] = rand_f();
      }
      oracle_lse_merge(P, D, lp, op, o, &lse);
      CHECK(live ? isfinite(lse) : (isinf(lse) && lse < 0), "merge P=%d: lse %g", P, lse);
      for (int e = 0; e < D; ++e)
        CHECK(isfinite(o[e]) && (live || o[e] == 0.0), "merge P=%d: o[%d] %g", P, e, o[e]);
      free(lp); free(op); free(o);
    }
}

static void bad_parent_cases(void) {
  const int ns[] = {1, 2, 63, 64, 65, 128, 256};
  for (size_t t = 0; t < sizeof ns / sizeof ns[0]; ++t) {
    const int N = ns[t], W = (N + 63) / 64;
    int32_t *parent = (int32_t *)xmalloc((size_t)N * 4);
    uint64_t *anc = (uint64_t *)xmalloc((size_t)N * W * 8);
    for (int i = 0; i < N; ++i) parent[i] = rand_int(-1, i - 1);
    const int i = rand_int(0, N - 1);
    parent[i] = rand_int(0, 1) ? i : -2;  /* itself or below -1 */
    CHECK(oracle_ancestor_mask(parent, 1, N, anc) == -1, "bad parent accepted (N=%d)", N);
    free(parent); free(anc);
  }
}

int main(void) {
  oracle_set_num_threads(4);
  const int Ns[] = {1, 8, 64, 65, 130, 256};
  for (int rep = 0; rep < 3; ++rep)
    for (size_t t = 0; t < sizeof Ns / sizeof Ns[0]; ++t) {
      const int N = Ns[t];
      for (int dtype = 0; dtype <= 1; ++dtype)
        for (int parts = 1; parts <= 3; ++parts) {
          run_case(2, N, 4, 2, 64, rand_int(0, 200), 0, dtype, parts, rep & 1, 0);
          run_case(3, N, 2, 1, 32, rand_int(1, 150), rand_int(1, 40), dtype, parts, 1, 0);
          run_case(2, N, 8, 8, 128, rand_int(0, 90), 0, dtype, parts, 0, 17);
        }
    }
  run_case(1, 8, 1, 1, 16, 0, 0, ORACLE_F32, 3, 0, 0);          /* empty prefix */
  run_case(2, 4, 2, 2, 8, 10, 12, ORACLE_BF16, 1, 0, 0);        /* index sets all -1 past c */
  merge_cases();
  bad_parent_cases();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle driver: all cases passed\n");
  return 0;
}
