/* A plain C99 consumer of include/mla.h, linked against libmla.so: the header compiles as
 * C, the entry points link with C names, and the host-only calls (planner, validation,
 * status strings) behave as documented.  Nothing here touches a GPU.  Prints "ok" and
 * returns 0 on success; prints the failing check and returns 1 otherwise. */
#include <stdio.h>
#include <string.h>

#include "mla.h"

#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      printf("check failed at line %d: %s\n", __LINE__, #c);  \
      return 1;                                               \
    }                                                         \
  } while (0)

int main(void) {
  CHECK(mla_abi_version() == MLA_ABI_VERSION);
  CHECK(strcmp(mla_status_string(MLA_OK), "") != 0);
  CHECK(mla_status_string(MLA_ERR_WORKSPACE_TOO_SMALL) != NULL);

  /* the long-context shape: 16 sequences of 65,536 tokens, 16 heads, 64-token pages */
  mla_problem_t p;
  memset(&p, 0, sizeof p);
  p.batch = 16;
  p.q_len = 1;
  p.num_heads = 16;
  p.head_dim_qk = 576;
  p.head_dim_v = 512;
  p.page_size = 64;
  p.num_pages = 16 * 1024;
  p.max_pages_per_seq = 1024;
  p.out_dtype = MLA_DTYPE_BF16;
  p.causal = 0;
  p.kv_dtype = MLA_KV_BF16;
  int32_t lens[16];
  for (int b = 0; b < 16; ++b) lens[b] = 65536;

  mla_plan_options_t opt;
  memset(&opt, 0, sizeof opt);
  opt.num_cus = 256;   /* plan without asking a device */
  mla_plan_t plan = NULL;
  CHECK(mla_plan(&p, lens, &opt, &plan) == MLA_OK && plan != NULL);
  mla_plan_info_t info;
  CHECK(mla_plan_get_info(plan, &info) == MLA_OK);
  CHECK(info.num_workers == 256 && info.rows_per_group == 16 && info.num_combine == 16);
  CHECK(info.workspace_bytes > 0 && (size_t)info.workspace_bytes == mla_plan_workspace_bytes(plan));
  {
    int32_t seg[4 * 256], off[257];
    CHECK(mla_plan_get_segments(plan, seg, 4 * 256, off, 257) == MLA_OK);
    int64_t tokens = 0;
    for (int i = 0; i < info.num_segments; ++i) tokens += seg[4 * i + 2] - seg[4 * i + 1];
    CHECK(tokens == 16 * 65536 && off[0] == 0 && off[info.num_workers] == info.num_segments);
  }
  /* bad arguments come back as status codes, with a message, before any launch */
  CHECK(mla_plan_upload(plan, NULL, (size_t)info.workspace_bytes, NULL) == MLA_ERR_INVALID_ARGUMENT);
  CHECK(strlen(mla_last_error()) > 0);
  mla_plan_destroy(plan);
  mla_plan_destroy(NULL);

  p.num_heads = 8;   /* R = 8 is not a multiple of 16 */
  plan = NULL;
  CHECK(mla_plan(&p, lens, &opt, &plan) == MLA_ERR_UNSUPPORTED && plan == NULL);
  p.num_heads = 128;
  p.kv_dtype = MLA_KV_FP8_E4M3;
  opt.rows_per_group = 32;   /* the 32-row kernel reads bf16 rows only */
  CHECK(mla_plan(&p, lens, &opt, &plan) == MLA_ERR_UNSUPPORTED);
  opt.rows_per_group = 64;   /* FP8 rows, 64 per work-group: the wide kernel, two row groups */
  CHECK(mla_plan(&p, lens, &opt, &plan) == MLA_OK);
  CHECK(mla_plan_get_info(plan, &info) == MLA_OK && info.rows_per_group == 64 && info.row_groups == 2);
  mla_plan_destroy(plan);
  opt.rows_per_group = 0;   /* FP8 rows at R = 128: the wide kernel, one row group */
  CHECK(mla_plan(&p, lens, &opt, &plan) == MLA_OK);
  CHECK(mla_plan_get_info(plan, &info) == MLA_OK && info.rows_per_group == 128 && info.row_groups == 1);
  mla_plan_destroy(plan);
  opt.rows_per_group = 16;
  CHECK(mla_plan(&p, lens, &opt, &plan) == MLA_OK);
  CHECK(mla_plan_get_info(plan, &info) == MLA_OK && info.rows_per_group == 16 && info.row_groups == 8);
  mla_plan_destroy(plan);

  CHECK(mla_devplan_workspace_bytes(&p, 256) > 0);
  printf("ok\n");
  return 0;
}
