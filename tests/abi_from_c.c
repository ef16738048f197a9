/* A C99 caller of the decode library: the header compiles as C, every declared entry
 * point links, and the host-side checks reject bad arguments with the documented codes.
 * Only calls that never reach the GPU are made (sizing, status strings, and arguments
 * rejected before any HIP call: null pointers, bad sizes, strides, scale, dtype). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mla_decode.h"

static int failures = 0;
#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      printf("FAIL line %d: %s\n", __LINE__, #cond);                    \
      ++failures;                                                       \
    }                                                                   \
  } while (0)

int main(void) {
  /* every declared entry point resolves at link time */
  const void* fns[] = {
      (const void*)mla_device_workgroups, (const void*)mla_plan_size,
      (const void*)mla_get_split_metadata, (const void*)mla_decode_fwd,
      (const void*)mla_decode_fwd_strided, (const void*)mla_decode_main,
      (const void*)mla_decode_combine, (const void*)mla_sparse_plan_size,
      (const void*)mla_decode_sparse_fwd, (const void*)mla_fp8_plan_size,
      (const void*)mla_decode_fp8_fwd, (const void*)mla_kv_append,
      (const void*)mla_decode_fwd_noalloc, (const void*)mla_read_status,
      (const void*)mla_status_string};
  for (size_t i = 0; i < sizeof fns / sizeof fns[0]; ++i) CHECK(fns[i] != NULL);

  /* sizing is host-only */
  size_t meta = 0, ws = 0, meta2 = 0, ws2 = 0;
  CHECK(mla_plan_size(64, 1, 128, 256, &meta, &ws) == MLA_OK);
  CHECK(meta > 0 && ws > 0);
  CHECK(mla_plan_size(128, 2, 128, 256, &meta2, &ws2) == MLA_OK);
  CHECK(meta2 > meta && ws2 > ws);
  CHECK(mla_plan_size(1, 0, 16, 256, &meta, &ws) == MLA_ERR_INVALID_ARG);
  CHECK(mla_plan_size(1, 2, 8193, 256, &meta, &ws) == MLA_ERR_UNSUPPORTED);
  CHECK(mla_sparse_plan_size(64, 128, 2048, 256, &meta, &ws) == MLA_OK);
  CHECK(mla_sparse_plan_size(64, 128, 100, 256, &meta, &ws) == MLA_ERR_INVALID_ARG);
  CHECK(mla_fp8_plan_size(64, 1, 128, 128, 256, &meta, &ws) == MLA_OK);

  /* status strings */
  CHECK(strcmp(mla_status_string(MLA_OK), "ok") == 0);
  CHECK(strcmp(mla_status_string(MLA_ERR_PLAN), "ok") != 0);
  CHECK(strcmp(mla_status_string(12345), "unknown status code") == 0);
  CHECK(mla_read_status(NULL, NULL, NULL) == MLA_ERR_INVALID_ARG);

  /* decode: rejected on the host, nothing enqueued */
  CHECK(mla_decode_fwd(7, NULL, NULL, 4, NULL, 4, NULL, 1, 1, 16, 0, 0.1f, NULL, NULL, NULL, 0,
                       8, NULL, 0, NULL) == MLA_ERR_UNSUPPORTED);
  CHECK(mla_decode_fwd(MLA_DTYPE_BF16, NULL, NULL, 4, NULL, 4, NULL, 1, 1, 16, 0, 0.1f, NULL,
                       NULL, NULL, 0, 8, NULL, 0, NULL) == MLA_ERR_INVALID_ARG);
  CHECK(mla_decode_fwd(MLA_DTYPE_BF16, NULL, NULL, 4, NULL, 4, NULL, 1, 1, 0, 0, 0.1f, NULL,
                       NULL, NULL, 0, 8, NULL, 0, NULL) == MLA_ERR_INVALID_ARG);
  CHECK(mla_decode_fwd(MLA_DTYPE_BF16, NULL, NULL, 4, NULL, 4, NULL, 1, 1, 16, 0, NAN, NULL,
                       NULL, NULL, 0, 8, NULL, 0, NULL) == MLA_ERR_INVALID_ARG);
  CHECK(mla_decode_fwd(MLA_DTYPE_F32, NULL, NULL, 4, NULL, 4, NULL, 1, 1, 16, 2, 0.1f, NULL,
                       NULL, NULL, 0, 8, NULL, 0, NULL) == MLA_ERR_INVALID_ARG);
  CHECK(mla_decode_main(MLA_DTYPE_BF16, NULL, NULL, 4, NULL, 4, NULL, 1, 1, 16, 0, 0.1f, NULL,
                        NULL, NULL, 0, 8, NULL, 0, NULL) == MLA_ERR_INVALID_ARG);
  CHECK(mla_decode_combine(MLA_DTYPE_BF16, NULL, NULL, 4, NULL, 4, NULL, 1, 1, 16, 0, -1.0f,
                           NULL, NULL, NULL, 0, 8, NULL, 0, NULL) == MLA_ERR_INVALID_ARG);
  /* strided rows: a row stride below the row width or off the 16-byte grid */
  CHECK(mla_decode_fwd_strided(MLA_DTYPE_BF16, NULL, 500, NULL, 4, NULL, 4, NULL, 1, 1, 16, 0,
                               0.1f, NULL, 512, NULL, NULL, 0, 8, NULL, 0, NULL) ==
        MLA_ERR_INVALID_ARG);
  CHECK(mla_decode_fwd_strided(MLA_DTYPE_BF16, NULL, 580, NULL, 4, NULL, 4, NULL, 1, 1, 16, 0,
                               0.1f, NULL, 512, NULL, NULL, 0, 8, NULL, 0, NULL) ==
        MLA_ERR_INVALID_ARG);
  CHECK(mla_decode_fwd_strided(MLA_DTYPE_F32, NULL, 576, NULL, 4, NULL, 4, NULL, 1, 1, 16, 0,
                               0.1f, NULL, 514, NULL, NULL, 0, 8, NULL, 0, NULL) ==
        MLA_ERR_INVALID_ARG);
  CHECK(mla_decode_fwd_noalloc(MLA_DTYPE_BF16, NULL, NULL, 4, NULL, 4, NULL, 1, 1, 16, 0, 0.1f,
                               NULL, NULL, 8, NULL) == MLA_ERR_INVALID_ARG);
  CHECK(mla_get_split_metadata(NULL, 2, 1, 16, 0, 4, 8, 0, NULL, 0, NULL) ==
        MLA_ERR_INVALID_ARG);
  CHECK(mla_kv_append(MLA_DTYPE_BF16, NULL, NULL, 4, NULL, 4, NULL, 2, 1, NULL, NULL) ==
        MLA_ERR_INVALID_ARG);
  CHECK(mla_kv_append(9, NULL, NULL, 4, NULL, 4, NULL, 2, 1, NULL, NULL) == MLA_ERR_UNSUPPORTED);

  printf("%d failures\n", failures);
  return failures ? 1 : 0;
}
