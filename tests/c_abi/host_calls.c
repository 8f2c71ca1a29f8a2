/* A C11 program against include/tf_exl3.h and libtf_exl3.so: host-only calls (the
 * planner, stream sizes, status strings and refusals decided before any launch), so
 * it runs without a GPU. Exit status 0 means every check held. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tf_exl3.h"

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

int main(void) {
  tf_exl3_plan p;
  CHECK(tf_exl3_linear_plan(4, 16, 5120, 129280, 0, &p) == TF_OK);
  CHECK(p.waves == 8 && p.grid_x == 1010 && p.passes == 1 && p.rows_kernel == 16 && p.column_split == 0);
  CHECK(tf_exl3_linear_plan(4, 1, 512, 128, 0, &p) == TF_OK && p.waves == 4 && p.column_split == 1);
  CHECK(tf_exl3_linear_plan(7, 1, 512, 128, 0, &p) == TF_E_BITS);
  CHECK(tf_exl3_linear_plan(4, 1, 500, 128, 0, &p) == TF_E_SHAPE);
  CHECK(tf_exl3_linear_plan(4, -1, 512, 128, 0, &p) == TF_E_ROWS);
  CHECK(tf_exl3_linear_plan(4, 1, 512, 128, 6, &p) == TF_E_WAVES);
  CHECK(tf_exl3_linear_plan(4, 1, 512, 128, 0, NULL) == TF_E_NULL);
  CHECK(tf_exl3_trellis_bytes(4, 5120, 129280) == (size_t)330956800);
  CHECK(tf_exl3_trellis_bytes(3, 100, 128) == 0);
  CHECK(strcmp(tf_exl3_status_string(TF_OK), "ok") == 0);
  CHECK(tf_exl3_status_string(-1234) != NULL);
  /* Refusals with pointers that are never dereferenced. */
  void* fake = (void*)(uintptr_t)0x7F0000000000ull;
  char* f = (char*)fake;
  CHECK(tf_exl3_linear(9, 1, 256, 256, (const uint16_t*)f, (const uint32_t*)(f + 0x100000),
                       (const uint16_t*)(f + 0x200000), f + 0x300000, TF_DT_F32, 0, NULL) == TF_E_BITS);
  CHECK(tf_exl3_linear(4, 1, 256, 256, NULL, (const uint32_t*)(f + 0x100000), (const uint16_t*)(f + 0x200000),
                       f + 0x300000, TF_DT_F32, 0, NULL) == TF_E_NULL);
  CHECK(tf_exl3_rot_in(f, TF_DT_F16, (const uint16_t*)(f + 0x10000), (uint16_t*)(f + 0x80), 1, 128, NULL) ==
        TF_E_ALIAS);
  CHECK(tf_exl3_project_pass_rows(16, 5120, 129280, 0) == 2);
  CHECK(tf_exl3_repack_strips(4, 256, 256, (const uint32_t*)f, (uint32_t*)f, NULL) == TF_E_ALIAS);
  if (failures == 0) printf("c abi ok\n");
  return failures == 0 ? 0 : 1;
}
