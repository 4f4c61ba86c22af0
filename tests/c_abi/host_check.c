/*
 * A C caller of libhsv.so: the header compiles as C11 (and as C++), the
 * library links, and the host side of the C ABI answers as include/hsv.h
 * states -- version, status strings, workspace sizes, and every entry point
 * rejecting a missing pointer with HSV_ERR_NULL before any device work (so
 * no GPU is needed).  Prints "all checks passed" and exits 0, or names the
 * first failed check and exits 1.
 */
#include <stdio.h>
#include <string.h>

#include "hsv.h"

static int failed = 0;
#define CHECK(cond)                                   \
  do {                                                \
    if (!(cond) && !failed) {                         \
      fprintf(stderr, "check failed: %s\n", #cond);   \
      failed = 1;                                     \
    }                                                 \
  } while (0)

int main(void) {
  CHECK(hsv_version() >= 1);
  for (int c = 0; c <= 6; ++c)
    CHECK(strncmp(hsv_status_string((hsv_status)c), "HSV_", 4) == 0);

  hsv_verify_desc d;
  memset(&d, 0, sizeof d);
  d.batch = 1; d.n_draft = 64; d.n_q_heads = 32; d.n_kv_heads = 8; d.head_dim = 128;
  d.kv_capacity = 32832; d.max_ctx = 32768; d.in_dtype = HSV_BF16; d.out_dtype = HSV_BF16;
  size_t n = 0;
  CHECK(hsv_verify_workspace_bytes(&d, &n) == HSV_OK && n > 0);
  CHECK(hsv_verify_workspace_bytes(NULL, &n) == HSV_ERR_NULL);
  hsv_verify_desc bad = d;
  bad.n_draft = 0;
  CHECK(hsv_verify_workspace_bytes(&bad, &n) == HSV_ERR_SHAPE);
  bad = d;
  bad.head_dim = 96;
  CHECK(hsv_verify_workspace_bytes(&bad, &n) == HSV_ERR_UNSUPPORTED);
  size_t sn = 0;
  CHECK(hsv_select_workspace_bytes(8, 8, 65536, &sn) == HSV_OK && sn > 0);

  /* Never dereferenced: every call below fails its argument checks first. */
  void *p = (void *)(size_t)0x10000;
  int32_t *ip = (int32_t *)p;
  float *fp = (float *)p;
  uint64_t *up = (uint64_t *)p;
  hipStream_t s = NULL;
  CHECK(hsv_verify_attn(&d, NULL, p, p, ip, ip, NULL, p, fp, p, n, s) == HSV_ERR_NULL);
  /* the tree part takes exactly one of parent and anc_mask */
  CHECK(hsv_verify_attn(&d, p, p, p, ip, ip, up, p, fp, p, n, s) == HSV_ERR_NULL);
  CHECK(hsv_verify_attn(&d, p, p, p, ip, NULL, NULL, p, fp, p, n, s) == HSV_ERR_NULL);
  hsv_verify_desc ds = d;
  ds.n_sel = 64;
  CHECK(hsv_verify_attn_sparse(&ds, p, p, p, ip, ip, NULL, NULL, p, fp, p, 1u << 30, s) ==
        HSV_ERR_NULL);
  hsv_verify_desc dp = d;
  dp.block_size = 64;
  CHECK(hsv_verify_attn_paged(&dp, p, p, p, NULL, 10, ip, ip, NULL, p, fp, p, 1u << 30, s) ==
        HSV_ERR_NULL);
  hsv_verify_desc dsp = ds;
  dsp.block_size = 64;
  dsp.n_draft = 8; /* 32 grouped rows: a shape the sparse paged call runs */
  CHECK(hsv_verify_attn_sparse_paged(&dsp, p, p, p, ip, 10, ip, ip, NULL, NULL, p, fp, p,
                                     1u << 30, s) == HSV_ERR_NULL);
  CHECK(hsv_verify_attn_noalloc(&d, NULL, p, p, ip, ip, NULL, p, fp, s) == HSV_ERR_NULL);
  CHECK(hsv_verify_attn_noalloc(&d, p, p, p, ip, NULL, NULL, p, fp, s) == HSV_ERR_NULL);
  CHECK(hsv_tree_ancestor_mask(NULL, up, 1, 8, s) == HSV_ERR_NULL);
  CHECK(hsv_gather_kv(NULL, p, ip, p, p, 1, 1, 64, 128, 8, HSV_BF16, s) == HSV_ERR_NULL);
  CHECK(hsv_lse_merge(NULL, fp, 2, 8, 128, p, fp, HSV_F32, s) == HSV_ERR_NULL);
  CHECK(hsv_select_kv_idx(fp, fp, 1024, ip, 1, 1, 64, 4, 8, 16, NULL, p, sn, s) ==
        HSV_ERR_NULL);
  CHECK(hsv_tree_position_ids(NULL, ip, ip, 1, 8, s) == HSV_ERR_NULL);
  CHECK(hsv_accept_path(NULL, p, ip, ip, ip, 1, 8, 64, 128, 8, HSV_BF16, s) == HSV_ERR_NULL);

  if (failed) return 1;
  printf("all checks passed\n");
  return 0;
}
