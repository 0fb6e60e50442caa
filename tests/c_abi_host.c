/*
 * A plain C consumer of the library's host-only entry points (no GPU
 * needed): the bucket layout, the fused layout, the group ranks and the
 * argument errors, checked against values derived by hand from the
 * fixed-size dim-0 chunk rule (FSDP dim-0 non-uniform sharding RFC, 6.4),
 * the 512-byte fused alignment (Hyper communication-overlap PR #758
 * write-up, 2.1) and the two-group rank model (FullyShard multi-dimensional
 * RFC, 2.2.1 and 2.2.5).  Prints "ok" and exits 0 on success.
 */
#include <stdio.h>
#include <string.h>

#include "fsdp_flat.h"

static int failures = 0;

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static int eq64(const int64_t* a, const int64_t* b, int n) {
  for (int k = 0; k < n; ++k)
    if (a[k] != b[k]) return 0;
  return 1;
}

int main(void) {
  /* (7,8), (5,3), (16,) over 4 ranks: chunks of 2, 2 and 4 rows */
  const int32_t ndim[3] = {2, 2, 1};
  const int64_t shape[5] = {7, 8, 5, 3, 16};
  fsdp_bucket_t b = {3, ndim, shape, 0, NULL};
  int64_t I = -1, padded[3], in_off[3], row_off[12], row_len[12];
  CHECK(fsdp_bucket_layout(&b, 4, &I, padded, in_off, row_off, row_len) == FSDP_OK);
  const int64_t want_padded[3] = {16, 6, 4}, want_in_off[3] = {0, 16, 22};
  const int64_t want_off[12] = {0, 2, 4, 6, 0, 2, 4, 5, 0, 4, 8, 12};
  const int64_t want_len[12] = {2, 2, 2, 1, 2, 2, 1, 0, 4, 4, 4, 4};
  CHECK(I == 26);
  CHECK(eq64(padded, want_padded, 3) && eq64(in_off, want_in_off, 3));
  CHECK(eq64(row_off, want_off, 12) && eq64(row_len, want_len, 12));

  /* per-parameter dims: (6,8) on dim 1 over 2 ranks = 6 runs of 4 */
  const int32_t nd2[1] = {2}, dims2[1] = {1};
  const int64_t sh2[2] = {6, 8};
  fsdp_bucket_t b2 = {1, nd2, sh2, 0, dims2};
  CHECK(fsdp_bucket_layout(&b2, 2, &I, padded, in_off, row_off, row_len) == FSDP_OK);
  CHECK(I == 24 && padded[0] == 24 && row_off[1] == 4 && row_len[1] == 4);
  /* an uneven non-zero dim is not implemented; a dim out of range is invalid */
  const int64_t sh3[2] = {6, 7};
  fsdp_bucket_t b3 = {1, nd2, sh3, 0, dims2};
  CHECK(fsdp_bucket_layout(&b3, 2, &I, NULL, NULL, NULL, NULL) == FSDP_ENOTIMPL);
  CHECK(strlen(fsdp_last_error()) > 0);
  fsdp_bucket_t b4 = {1, nd2, sh2, 2, NULL};
  CHECK(fsdp_bucket_layout(&b4, 2, &I, NULL, NULL, NULL, NULL) == FSDP_EINVAL);

  /* fused layout: 100 fp32 (400 B), then 3 at byte 512 -> element 128;
     end 524 B rounds up to 1024 B -> 256 elements */
  const int64_t segs[2] = {100, 3};
  int64_t off[2] = {-1, -1}, F = -1;
  CHECK(fsdp_fused_layout(2, segs, 4, off, &F) == FSDP_OK);
  CHECK(off[0] == 0 && off[1] == 128 && F == 256);
  CHECK(fsdp_fused_layout(2, segs, 2, off, &F) == FSDP_OK);
  CHECK(off[0] == 0 && off[1] == 256 && F == 512);
  CHECK(fsdp_fused_layout(2, segs, 8, off, &F) == FSDP_EINVAL);

  /* HSDP 8 = 2 x 4: RS groups {0..3}, {4..7}; AR groups {s, 4+s} */
  int32_t n_rs = -1, n_ar = -1, rs[8], ar[8];
  CHECK(fsdp_group_ranks(8, 4, &n_rs, rs, &n_ar, ar) == FSDP_OK);
  CHECK(n_rs == 2 && n_ar == 4);
  for (int k = 0; k < 8; ++k) CHECK(rs[k] == k);
  for (int s = 0; s < 4; ++s) CHECK(ar[2 * s] == s && ar[2 * s + 1] == 4 + s);
  /* pure-TP compatible: shard 1, dp 8 -> no RS, one AR group of all 8 */
  CHECK(fsdp_group_ranks(8, 1, &n_rs, rs, &n_ar, ar) == FSDP_OK);
  CHECK(n_rs == 0 && n_ar == 1);
  CHECK(fsdp_group_ranks(8, 3, &n_rs, rs, &n_ar, ar) == FSDP_EINVAL);

  /* device entry points reject bad arguments before any HIP call */
  CHECK(fsdp_ag_copy_in(&b, 4, 7, NULL, NULL, NULL) == FSDP_ENOTIMPL);
  CHECK(fsdp_rs_reduce(&b, 8, 4, 3, FSDP_SUM, FSDP_F32, NULL, NULL, NULL) == FSDP_EINVAL);
  CHECK(fsdp_rs_copy_reduce_noalloc(&b, 8, 4, 3, FSDP_SUM, FSDP_F32, NULL, NULL, NULL) == FSDP_EINVAL);

  if (failures) return 1;
  printf("ok\n");
  return 0;
}
