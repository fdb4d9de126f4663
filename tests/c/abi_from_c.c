/* A C99 caller of libbtq: compiles against include/btq.h with a C compiler,
 * links the shared library, and calls the entry points that need no GPU
 * (size helpers, status strings, argument checks that return before any
 * HIP call). Prints one line per check; exits non-zero on the first
 * failure. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "btq.h"

#define CHECK(cond)                                             \
  do {                                                          \
    if (!(cond)) {                                              \
      printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);    \
      return 1;                                                 \
    }                                                           \
    printf("ok %s\n", #cond);                                   \
  } while (0)

int main(void) {
  /* fake, never dereferenced device addresses: every call below fails its
     host-side checks before it reaches the HIP runtime */
  void *A = (void *)(uintptr_t)0x10000;
  CHECK(btq_packed_row_bytes(4096, 64) == 2016);
  CHECK(btq_packed_row_bytes(9, 2) == 4);
  CHECK(btq_packed_row_bytes(8, 9) == -1);
  CHECK(btq_packed_pitch(4096, 64) == 2048);
  CHECK(btq_select_workspace_bytes(8, 4096, 64) == (size_t)8 * 4096 * 4);
  CHECK(btq_calib_workspace_bytes(0, 1, 1) == 0);
  CHECK(strcmp(btq_status_str(BTQ_OK), "ok") == 0);
  CHECK(btq_status_str(12345) != NULL);
  CHECK(btq_version() != NULL && strlen(btq_version()) >= 5);
  CHECK(btq_compress_pack(A, 2, 4, 16, 17, A, A, A, A, A, A, NULL) == BTQ_ERR_SHAPE);
  CHECK(btq_compress_pack(A, 2, 4, 16, 4, NULL, A, A, A, A, A, NULL) == BTQ_ERR_ARG);
  CHECK(btq_decompress_reduce(A, A, 2, 4, 16, 4, A, A, NULL, A, NULL) == BTQ_ERR_ARG);
  CHECK(btq_decompress_reduce(A, A, 0, 4, 16, 4, A, A, A, A, NULL) == BTQ_ERR_SHAPE);
  CHECK(btq_decompress_reduce_bf16(A, A, 2, 4, 16, 4, A, A, A, NULL, NULL) == BTQ_ERR_ARG);
  CHECK(btq_calib_update(A, 2, 4, 16, 1.0f, 1, A, A, A, 1u << 20, NULL) == BTQ_ERR_ARG);
  CHECK(btq_select_outliers(A, A, 2, 16, 4, A, A, A, A, A, A, A, 4, NULL) == BTQ_ERR_WORKSPACE);
  CHECK(btq_select_outliers_rule(A, A, 2, 16, 4, 7, A, A, A, A, A, A, A, 1u << 20, NULL) ==
        BTQ_ERR_ARG);
  {
    const int32_t unsorted[2] = {5, 3};
    CHECK(btq_select_features(A, A, 2, 16, 2, unsorted, A, A, A, A, A, A, NULL) == BTQ_ERR_ARG);
  }
  CHECK(btq_compress_pack_per_shard(A, 2, 4, 16, 4, A, A, NULL, A, A, A, NULL) == BTQ_ERR_ARG);
  CHECK(btq_decompress_reduce_per_shard(A, A, 2, 4, 16, 4, A, A, NULL, A, NULL) == BTQ_ERR_ARG);
  CHECK(btq_select_outliers_per_shard(A, A, 2, 16, 4, A, A, A, A, A, A, A, 4, NULL) ==
        BTQ_ERR_WORKSPACE);
  CHECK(btq_compress_pack_ex(A, 2, 4, 16, 4, A, A, A, A, BTQ_SETS_SHARED, A, 5, A, NULL) ==
        BTQ_ERR_SHAPE);
  CHECK(btq_decompress_reduce_ex(A, 128, A, 2, 4, 16, 4, A, A, A, BTQ_SETS_PER_SHARD, A, 9,
                                 NULL) == BTQ_ERR_ARG);
  printf("all ok\n");
  return 0;
}
