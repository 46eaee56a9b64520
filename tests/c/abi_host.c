/* A C99 program against the public headers and the shared library, with
 * no GPU: planning, workspace sizes, status strings and argument checks.
 * Built and run by tests/test_c_abi.py; prints one line per check. */
#include <stdio.h>
#include <string.h>

#include "gqa_append.h"
#include "gqa_decode.h"

static int failures = 0;

#define CHECK(cond, what)                                                  \
  do {                                                                     \
    if (cond) {                                                            \
      printf("ok %s\n", what);                                             \
    } else {                                                               \
      printf("FAIL %s (last error: %s)\n", what, gqa_last_error());        \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

int main(void) {
  CHECK(gqa_abi_version() == GQA_DECODE_ABI_VERSION, "abi version");
  CHECK(strcmp(gqa_status_string(GQA_OK), "GQA_OK") == 0, "status string");

  gqa_decode_params p;
  memset(&p, 0, sizeof p);
  p.batch = 1;
  p.s_q = 2;
  p.h_q = 64;
  p.h_kv = 8;
  p.head_dim = 128;
  p.layout = GQA_LAYOUT_CONTIGUOUS;
  p.kv_dtype = GQA_KV_BF16;
  p.causal = 1;
  p.max_seqlen_kv = 131072;
  p.seq_capacity = 131072;
  p.kv_rows = 131072;
  p.num_cus = 256;
  gqa_decode_plan plan;
  CHECK(gqa_decode_make_plan(&p, &plan) == GQA_OK, "plan 64/8 d128 S_q 2 128K");
  CHECK(plan.rows == 16 && plan.math == GQA_MATH_MFMA && plan.combine == 1, "plan fields");
  CHECK((long long)plan.num_splits * plan.kv_chunk >= 131072, "splits cover the list");
  size_t ws = 0;
  CHECK(gqa_decode_workspace_size(&p, &ws) == GQA_OK && ws == plan.workspace_bytes, "workspace size");

  p.kv_dtype = GQA_KV_INT8;
  CHECK(gqa_decode_make_plan(&p, &plan) == GQA_OK, "int8 plan");
  p.s_q = 64;
  CHECK(gqa_decode_make_plan(&p, &plan) == GQA_OK && plan.rows == 512, "S_q 64 plan (512 rows)");
  p.s_q = 65;
  CHECK(gqa_decode_make_plan(&p, &plan) == GQA_ERR_UNSUPPORTED, "S_q 65 rejected");
  CHECK(strlen(gqa_last_error()) > 0, "last error set");
  p.s_q = 2;
  p.head_dim = 96;
  CHECK(gqa_decode_make_plan(&p, &plan) == GQA_ERR_UNSUPPORTED, "head_dim 96 rejected");
  p.head_dim = 128;

  /* a run with a NULL q fails on the host before anything is enqueued */
  CHECK(gqa_decode_run(&p, NULL, (void*)0x10000, (void*)0x10000, (const int32_t*)0x10000, NULL, NULL, NULL,
                       (const float*)0x10000, (const float*)0x10000, NULL, (void*)0x10000, (float*)0x10000, NULL,
                       0, NULL) == GQA_ERR_INVALID_ARG,
        "run without q rejected");

  /* the no-allocation entry point refuses a plan whose split partials
   * exceed its scratch array before it touches a device (64 query tokens of
   * 64/8 heads over 128K tokens: 512 rows per KV head) */
  p.s_q = 64;
  CHECK(gqa_decode_make_plan(&p, &plan) == GQA_OK && plan.workspace_bytes > GQA_NOALLOC_SCRATCH_BYTES,
        "a plan beyond the scratch array");
  CHECK(gqa_decode_run_noalloc(&p, (void*)0x10000, (void*)0x10000, (void*)0x10000, (const int32_t*)0x10000, NULL,
                               NULL, NULL, NULL, NULL, NULL, (void*)0x10000, (float*)0x10000, NULL) == GQA_ERR_WORKSPACE,
        "no-allocation call beyond the scratch array refused");
  p.s_q = 2;

  gqa_append_params ap;
  memset(&ap, 0, sizeof ap);
  ap.batch = 32;
  ap.s_new = 8192;
  ap.h_kv = 8;
  ap.head_dim = 128;
  ap.layout = GQA_LAYOUT_PAGED;
  ap.kv_dtype = GQA_KV_FP8_E4M3FN;
  ap.scale_policy = GQA_SCALE_FIRST_BLOCK;
  ap.kv_rows = 32 * 8192;
  ap.page_size = 16;
  ap.max_pages_per_seq = 512;
  CHECK(gqa_kv_append_workspace_size(&ap, &ws) == GQA_OK && ws == (size_t)32 * 128 * 2 * 8 * 4,
        "append workspace (32 requests x 128 workgroups x K, V x 8 heads)");
  ap.scale_policy = GQA_SCALE_GIVEN;
  CHECK(gqa_kv_append_workspace_size(&ap, &ws) == GQA_OK && ws == 0, "append workspace, given scales");
  ap.layout = GQA_LAYOUT_RAGGED;
  CHECK(gqa_kv_append_workspace_size(&ap, &ws) == GQA_ERR_UNSUPPORTED, "append to a ragged cache rejected");

  printf("%d failures\n", failures);
  return failures == 0 ? 0 : 1;
}
