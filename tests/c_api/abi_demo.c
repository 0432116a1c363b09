/* A plain C99 caller of the LVSA C ABI (include/lvsa.h): builds, sizes and
 * validates masks on the host and checks argument errors that return before
 * any device work.  Prints "ok" and exits 0 on success; exits 1 with a
 * message on the first mismatch.  Used by tests/test_c_api.py. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lvsa.h"

#define CHECK(cond, ...)                      \
  do {                                        \
    if (!(cond)) {                            \
      fprintf(stderr, __VA_ARGS__);           \
      fprintf(stderr, " (line %d)\n", __LINE__); \
      return 1;                               \
    }                                         \
  } while (0)

int main(void) {
  CHECK(lvsa_version() == LVSA_ABI_VERSION, "version %d", lvsa_version());

  /* The 121-frame, C = 21, W = 9 schedule: Tper = 11, 11 anchors, 21 frames per row. */
  const int32_t T = 121, C = 21, W = 9;
  int32_t nnz = 0;
  CHECK(lvsa_mask_nnz(T, C, W, &nnz) == LVSA_OK && nnz == T * C, "nnz %d", nnz);
  int32_t *row_ptr = malloc(sizeof(int32_t) * (T + 1));
  int32_t *col_idx = malloc(sizeof(int32_t) * nnz);
  lvsa_mask_info info;
  memset(&info, 0, sizeof info);
  CHECK(lvsa_build_mask(T, C, W, 3, LVSA_ROT_MOD_TPER, row_ptr, col_idx, nnz, &info) == LVSA_OK, "%s",
        lvsa_last_error());
  CHECK(info.c_eff == 21 && info.t_per == 11 && info.n_anchor == 11 && info.offset == 3 && info.nnz == nnz,
        "info %d %d %d %d %d", info.c_eff, info.t_per, info.n_anchor, info.offset, info.nnz);
  CHECK(lvsa_validate_mask(T, row_ptr, col_idx, nnz) == LVSA_OK, "%s", lvsa_last_error());
  /* every row holds its own frame and the anchors 3, 14, ..., 113 */
  for (int32_t t = 0; t < T; ++t) {
    int self = 0, anchors = 0;
    for (int32_t e = row_ptr[t]; e < row_ptr[t + 1]; ++e) {
      self |= col_idx[e] == t;
      anchors += (col_idx[e] % 11) == 3;
    }
    CHECK(self && anchors == 11, "row %d: self %d anchors %d", t, self, anchors);
  }

  /* A run of 50 steps in one buffer: step 3 of it equals the single build. */
  int32_t *steps = malloc(sizeof(int32_t) * (size_t)nnz * 50);
  int32_t rp2[122];
  CHECK(lvsa_build_mask_steps(T, C, W, 0, 50, LVSA_ROT_MOD_TPER, rp2, steps, (int64_t)nnz * 50, NULL) == LVSA_OK,
        "%s", lvsa_last_error());
  CHECK(memcmp(steps + 3 * nnz, col_idx, sizeof(int32_t) * nnz) == 0, "step 3 differs");
  CHECK(memcmp(rp2, row_ptr, sizeof rp2) == 0, "row_ptr differs");

  /* Errors come back as status codes with a message; nothing is written. */
  col_idx[0] = -7;
  CHECK(lvsa_build_mask(T, C, W, 0, 0, row_ptr, col_idx, nnz - 1, NULL) == LVSA_ERR_CAPACITY, "capacity");
  CHECK(col_idx[0] == -7 && strlen(lvsa_last_error()) > 0, "wrote on error");
  CHECK(lvsa_build_mask(T, C, C, 0, 0, row_ptr, col_idx, nnz, NULL) == LVSA_ERR_ARG, "W == C accepted");
  col_idx[5] = col_idx[4];
  CHECK(lvsa_validate_mask(T, row_ptr, col_idx, nnz) == LVSA_ERR_MASK, "repeated frame accepted");

  /* lvsa_attention argument errors are reported before any device work. */
  lvsa_tensor q = {(void *)(uintptr_t)0x100000000ull, 1, 2, 512, 64, 2 * 512 * 64, 512 * 64, 64, 0};
  lvsa_tensor k = q, v = q, out = q;
  k.data = (void *)(uintptr_t)0x100100000ull;
  v.data = (void *)(uintptr_t)0x100200000ull;
  out.data = (void *)(uintptr_t)0x100300000ull;
  CHECK(lvsa_attention(&q, &k, &v, row_ptr, col_idx, 8, 32, &out, 0.f, NULL) == LVSA_ERR_DTYPE, "dtype");
  q.dtype = k.dtype = v.dtype = out.dtype = LVSA_DTYPE_BF16;
  CHECK(lvsa_attention(&q, &k, &v, row_ptr, col_idx, 7, 32, &out, 0.f, NULL) == LVSA_ERR_SHAPE, "N %% T");
  out.data = q.data;
  CHECK(lvsa_attention(&q, &k, &v, row_ptr, col_idx, 8, 32, &out, 0.f, NULL) == LVSA_ERR_SHAPE, "out aliases q");

  free(row_ptr);
  free(col_idx);
  free(steps);
  printf("ok\n");
  return 0;
}
