/* A plain C99 caller that runs the attention through the LVSA C ABI on device
 * memory it allocates itself (HIP runtime C API), on the NULL stream:
 *
 *   attn_demo B H T P D C W step qkv.bin out_plain.bin out_ws.bin
 *
 * qkv.bin holds q, then k, then v, each [B, H, T*P, D] bf16, contiguous.  The
 * program builds the step's mask on the host, copies it to the device, runs
 * lvsa_attention and lvsa_attention_ws (workspace sized by
 * lvsa_attention_workspace_bytes) and writes both outputs as raw bf16.  Exits
 * 0 on success, 1 with a message on the first failure.  Used by
 * tests/test_gpu_c_api.py. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "lvsa.h"

#define CHECK(cond, ...)                         \
  do {                                           \
    if (!(cond)) {                               \
      fprintf(stderr, __VA_ARGS__);              \
      fprintf(stderr, " (line %d)\n", __LINE__); \
      return 1;                                  \
    }                                            \
  } while (0)
#define HIP(call) CHECK((call) == hipSuccess, "%s failed", #call)

static lvsa_tensor record(void *data, int64_t B, int64_t H, int64_t N, int64_t D) {
  lvsa_tensor t;
  memset(&t, 0, sizeof t);
  t.data = data;
  t.B = B;
  t.H = H;
  t.N = N;
  t.D = D;
  t.stride_n = D;
  t.stride_h = N * D;
  t.stride_b = H * N * D;
  t.dtype = LVSA_DTYPE_BF16;
  return t;
}

int main(int argc, char **argv) {
  CHECK(argc == 12, "usage: attn_demo B H T P D C W step qkv.bin out_plain.bin out_ws.bin");
  const int64_t B = atoll(argv[1]), H = atoll(argv[2]);
  const int32_t T = atoi(argv[3]), P = atoi(argv[4]);
  const int64_t D = atoll(argv[5]);
  const int32_t C = atoi(argv[6]), W = atoi(argv[7]), step = atoi(argv[8]);
  const int64_t N = (int64_t)T * P;
  const size_t elems = (size_t)(B * H * N * D), bytes = elems * 2;

  /* inputs */
  uint16_t *host = malloc(3 * bytes);
  CHECK(host != NULL, "out of host memory");
  FILE *f = fopen(argv[9], "rb");
  CHECK(f != NULL, "cannot open %s", argv[9]);
  CHECK(fread(host, 1, 3 * bytes, f) == 3 * bytes, "short read from %s", argv[9]);
  fclose(f);
  void *q, *k, *v, *o_plain, *o_ws;
  HIP(hipMalloc(&q, bytes));
  HIP(hipMalloc(&k, bytes));
  HIP(hipMalloc(&v, bytes));
  HIP(hipMalloc(&o_plain, bytes));
  HIP(hipMalloc(&o_ws, bytes));
  HIP(hipMemcpy(q, host, bytes, hipMemcpyHostToDevice));
  HIP(hipMemcpy(k, host + elems, bytes, hipMemcpyHostToDevice));
  HIP(hipMemcpy(v, host + 2 * elems, bytes, hipMemcpyHostToDevice));

  /* the step's mask: built on the host, copied to the device */
  int32_t nnz = 0;
  CHECK(lvsa_mask_nnz(T, C, W, &nnz) == LVSA_OK, "%s", lvsa_last_error());
  int32_t *row_ptr = malloc(sizeof(int32_t) * (size_t)(T + 1));
  int32_t *col_idx = malloc(sizeof(int32_t) * (size_t)nnz);
  CHECK(row_ptr != NULL && col_idx != NULL, "out of host memory");
  CHECK(lvsa_build_mask(T, C, W, step, LVSA_ROT_MOD_TPER, row_ptr, col_idx, nnz, NULL) == LVSA_OK, "%s",
        lvsa_last_error());
  void *d_rp, *d_ci;
  HIP(hipMalloc(&d_rp, sizeof(int32_t) * (size_t)(T + 1)));
  HIP(hipMalloc(&d_ci, sizeof(int32_t) * (size_t)nnz));
  HIP(hipMemcpy(d_rp, row_ptr, sizeof(int32_t) * (size_t)(T + 1), hipMemcpyHostToDevice));
  HIP(hipMemcpy(d_ci, col_idx, sizeof(int32_t) * (size_t)nnz, hipMemcpyHostToDevice));

  /* both entry points, default scale, NULL stream */
  lvsa_tensor tq = record(q, B, H, N, D), tk = record(k, B, H, N, D), tv = record(v, B, H, N, D);
  lvsa_tensor to_plain = record(o_plain, B, H, N, D), to_ws = record(o_ws, B, H, N, D);
  CHECK(lvsa_attention(&tq, &tk, &tv, d_rp, d_ci, T, nnz, &to_plain, 0.0f, NULL) == LVSA_OK, "%s",
        lvsa_last_error());
  int64_t ws_bytes = 0;
  CHECK(lvsa_attention_workspace_bytes(B, H, N, D, T, &ws_bytes) == LVSA_OK, "%s", lvsa_last_error());
  void *ws;
  HIP(hipMalloc(&ws, (size_t)ws_bytes));
  CHECK(lvsa_attention_ws(&tq, &tk, &tv, d_rp, d_ci, T, nnz, &to_ws, 0.0f, ws, ws_bytes, NULL) == LVSA_OK, "%s",
        lvsa_last_error());
  HIP(hipDeviceSynchronize());

  /* outputs */
  const char *names[2] = {argv[10], argv[11]};
  void *outs[2] = {o_plain, o_ws};
  for (int i = 0; i < 2; ++i) {
    HIP(hipMemcpy(host, outs[i], bytes, hipMemcpyDeviceToHost));
    FILE *g = fopen(names[i], "wb");
    CHECK(g != NULL, "cannot open %s", names[i]);
    CHECK(fwrite(host, 1, bytes, g) == bytes, "short write to %s", names[i]);
    fclose(g);
  }

  HIP(hipFree(ws));
  HIP(hipFree(d_ci));
  HIP(hipFree(d_rp));
  HIP(hipFree(o_ws));
  HIP(hipFree(o_plain));
  HIP(hipFree(v));
  HIP(hipFree(k));
  HIP(hipFree(q));
  free(col_idx);
  free(row_ptr);
  free(host);
  printf("ok\n");
  return 0;
}
