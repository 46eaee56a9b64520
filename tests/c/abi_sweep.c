/* A seeded sweep of the C ABI's host side: decode and append parameters
 * drawn from edge values (zero, one, the documented limits and just past
 * them, negative, INT32_MAX), through planning, workspace sizing, runs with
 * placeholder pointers and resolve calls.  Linked against a build with
 * stand-in launchers (tests/c/launch_stubs.cpp) that check each launch
 * the planner asks for, and run under AddressSanitizer and
 * UndefinedBehaviorSanitizer: no call may read or write out of bounds,
 * overflow a signed integer, or hand a kernel a launch it cannot take.
 * Usage: abi_sweep [iterations] [seed].  Prints a summary line. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gqa_append.h"
#include "gqa_decode.h"

extern long long gqa_stub_launches;

static uint64_t state;
static uint64_t next_u64(void) { /* xorshift64* */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return state * 2685821657736338717ull;
}
#define PICK(arr) ((arr)[next_u64() % (sizeof(arr) / sizeof((arr)[0]))])

static int failures = 0;
#define EXPECT(cond, ...)             \
  do {                                \
    if (!(cond)) {                    \
      printf("FAIL: " __VA_ARGS__);   \
      printf("\n");                   \
      ++failures;                     \
    }                                 \
  } while (0)

static void* const FAKE = (void*)(uintptr_t)0x100000; /* 16-byte aligned, never dereferenced on the host */

static void decode_case(const gqa_decode_params* p, long* ok_plans) {
  gqa_decode_plan plan;
  memset(&plan, 0xA5, sizeof plan);
  gqa_status st = gqa_decode_make_plan(p, &plan);
  size_t ws = 12345;
  gqa_status st2 = gqa_decode_workspace_size(p, &ws);
  EXPECT(st == st2, "plan and workspace_size disagree: %d vs %d", st, st2);
  if (st != GQA_OK) {
    EXPECT(strlen(gqa_last_error()) > 0, "status %d without a message", st);
    return;
  }
  ++*ok_plans;
  EXPECT(ws == plan.workspace_bytes, "workspace size %zu vs plan %zu", ws, plan.workspace_bytes);
  EXPECT(plan.rows == (p->h_q / p->h_kv) * p->s_q, "rows");
  EXPECT(plan.kv_chunk >= 32 && plan.kv_chunk % 32 == 0, "chunk %d", plan.kv_chunk);
  EXPECT(plan.num_splits >= 1, "splits %d", plan.num_splits);
  if (p->layout != GQA_LAYOUT_RAGGED || p->topk > 0) {
    const long long L = p->topk > 0 ? p->topk : p->max_seqlen_kv;
    EXPECT((long long)plan.num_splits * plan.kv_chunk >= L, "splits x chunk %lld < list %lld",
           (long long)plan.num_splits * plan.kv_chunk, L);
  } else {
    EXPECT((long long)plan.num_splits * plan.kv_chunk >= p->kv_rows, "packed chunks do not cover kv_rows");
  }
  EXPECT(plan.combine == 0 || plan.workspace_bytes > 0 || p->batch == 0, "combine without workspace");
  if (plan.combine) {
    /* the partials' own size, in floating point (no wrap): the plan's byte
     * count must cover it and stay under the 2^40 limit */
    const int packed = p->layout == GQA_LAYOUT_RAGGED && p->topk == 0;
    const long double slots = packed ? ((long double)p->batch + plan.num_splits - 1) * p->h_kv
                                     : (long double)p->batch * p->h_kv * plan.num_splits;
    const long double need = slots * plan.rows * (p->head_dim + 1) * 4.0L;
    EXPECT((long double)plan.workspace_bytes >= need, "workspace %zu < partials %.6Lg", plan.workspace_bytes, need);
    EXPECT(plan.workspace_bytes <= ((size_t)1 << 40), "workspace %zu over the limit", plan.workspace_bytes);
  }
  if (plan.workspace_bytes > ((size_t)1 << 40)) return; /* not worth a fake buffer */
  const int32_t* i32 = (const int32_t*)FAKE;
  const float* f32 = (const float*)FAKE;
  const long long before = gqa_stub_launches;
  st = gqa_decode_run(p, FAKE, FAKE, FAKE, i32, i32, i32, i32, f32, f32, FAKE, FAKE, (float*)FAKE, FAKE,
                      plan.workspace_bytes, NULL);
  EXPECT(st == GQA_OK, "run failed after a good plan: %s", gqa_last_error());
  if (st == GQA_OK && p->batch > 0)
    EXPECT(gqa_stub_launches - before == 1 + plan.combine, "launch count %lld", gqa_stub_launches - before);
  if (plan.workspace_bytes > 0) {
    st = gqa_decode_run(p, FAKE, FAKE, FAKE, i32, i32, i32, i32, f32, f32, FAKE, FAKE, (float*)FAKE, FAKE,
                        plan.workspace_bytes - 1, NULL);
    EXPECT(st == GQA_ERR_WORKSPACE, "a short workspace was accepted");
  }
  st = gqa_resolve_rows(p, i32, i32, i32, i32, (int64_t*)FAKE, NULL);
  EXPECT(st == GQA_OK, "resolve failed after a good plan: %s", gqa_last_error());
  /* the no-allocation entry point: the same plan, or a clear refusal when
   * the partials exceed its scratch array */
  const long long launches = gqa_stub_launches;
  st = gqa_decode_run_noalloc(p, FAKE, FAKE, FAKE, i32, i32, i32, i32, f32, f32, FAKE, FAKE, (float*)FAKE, NULL);
  if (plan.workspace_bytes > GQA_NOALLOC_SCRATCH_BYTES) {
    EXPECT(st == GQA_ERR_WORKSPACE, "no-allocation call with %zu bytes of partials: status %d", plan.workspace_bytes, st);
    EXPECT(gqa_stub_launches == launches, "a refused no-allocation call launched");
  } else {
    EXPECT(st == GQA_OK, "no-allocation call failed after a good plan: %s", gqa_last_error());
  }
}

static void append_case(const gqa_append_params* p, long* ok_plans) {
  size_t ws = 777;
  gqa_status st = gqa_kv_append_workspace_size(p, &ws);
  if (st != GQA_OK) {
    EXPECT(strlen(gqa_last_error()) > 0, "append status %d without a message", st);
    return;
  }
  ++*ok_plans;
  const int32_t* i32 = (const int32_t*)FAKE;
  float* f32 = (float*)FAKE;
  st = gqa_kv_append(p, FAKE, FAKE, i32, (int32_t*)((char*)FAKE + 4096), i32, FAKE, FAKE, f32, f32,
                     ws ? FAKE : NULL, ws, NULL);
  EXPECT(st == GQA_OK, "append failed after a good size: %s", gqa_last_error());
}

int main(int argc, char** argv) {
  const long iters = argc > 1 ? atol(argv[1]) : 200000;
  state = argc > 2 ? strtoull(argv[2], NULL, 10) : 0x9E3779B97F4A7C15ull;
  if (state == 0) state = 1;
  static const int32_t batches[] = {0, 1, 2, 7, 64, 256, 65535, 65536, -1};
  static const int32_t sqs[] = {0, 1, 2, 8, 16, 33, 64, 65};
  static const int32_t hqs[] = {1, 2, 8, 32, 64, 128, 512, 4096, 0, -8, 65535 * 4};
  static const int32_t hkvs[] = {1, 2, 3, 8, 16, 65535, 65536, 0, -1};
  static const int32_t dims[] = {64, 128, 256, 96, 0, 512};
  static const int32_t lens[] = {0, 1, 31, 1024, 131072, 1 << 24, INT32_MAX, -1};
  static const int32_t caps[] = {0, 1, 1024, 131072, INT32_MAX};
  static const int64_t rowss[] = {0, 1, 1024, 1 << 20, INT32_MAX, (int64_t)INT32_MAX + 1, (int64_t)1 << 40, -5};
  static const int32_t pages[] = {1, 16, 17, 1024, 2048, 0};
  static const int32_t mpps[] = {0, 1, 32, 2048, 1 << 20, INT32_MAX};
  static const int32_t topks[] = {0, 1, 512, 4096, 1 << 20, INT32_MAX, -1};
  static const float scales[] = {0.f, 0.1f, -1.f, INFINITY, NAN};
  static const int32_t chunks[] = {0, 0, 0, 32, 64, 100, 4096, 4128, 1 << 24, (1 << 24) + 32, INT32_MAX};
  static const int32_t cus[] = {256, 256, 1, 304, 1 << 20};
  static const int32_t small[] = {0, 1, 2, 3, -1};
  long ok_decode = 0, ok_append = 0;
  {
    /* every size field at its limit at once: the planner's products of
     * requests x heads x list length x row groups must not overflow */
    gqa_decode_params p;
    memset(&p, 0, sizeof p);
    p.batch = 65535;
    p.h_kv = 65535;
    p.h_q = 65535 * 4;
    p.s_q = 4;
    p.head_dim = 128;
    p.layout = GQA_LAYOUT_PAGED;
    p.max_seqlen_kv = INT32_MAX;
    p.page_size = 1024;
    p.max_pages_per_seq = INT32_MAX / 1024 + 1;
    p.kv_rows = (int64_t)INT32_MAX / 1024 * 1024;
    p.topk = INT32_MAX;
    p.num_cus = 256;
    for (int k = 0; k < 2; ++k) {
      decode_case(&p, &ok_decode);
      p.layout = GQA_LAYOUT_CONTIGUOUS;
      p.seq_capacity = INT32_MAX;
      p.kv_rows = INT32_MAX;
      p.topk = 0;
      p.batch = 1;
    }
  }
  for (long it = 0; it < iters; ++it) {
    /* a valid decode call (one of the layouts, types and row counts the
     * library builds), then up to three fields set to edge values */
    gqa_decode_params p;
    memset(&p, 0, sizeof p);
    static const int32_t groups[] = {1, 2, 4, 8, 16, 32, 64};
    static const int32_t good_hkv[] = {1, 2, 3, 4, 8};
    p.h_kv = PICK(good_hkv);
    p.s_q = 1 + (int32_t)(next_u64() % 8) * (next_u64() % 4 == 0 ? 8 : 1);
    p.h_q = p.h_kv * PICK(groups);
    while ((p.h_q / p.h_kv) * p.s_q > 512) p.s_q /= 2;
    if (p.s_q < 1) p.s_q = 1;
    p.head_dim = 64 << (next_u64() % 3);
    p.layout = (int32_t)(next_u64() % 3);
    p.kv_dtype = (int32_t)(next_u64() % 3);
    p.causal = (int32_t)(next_u64() % 2);
    p.batch = 1 + (int32_t)(next_u64() % 300);
    p.max_seqlen_kv = (int32_t)(next_u64() % 200000);
    p.page_size = 1 << (next_u64() % 11);
    p.max_pages_per_seq = (p.max_seqlen_kv + p.page_size - 1) / p.page_size + (int32_t)(next_u64() % 3);
    if (p.max_pages_per_seq < 1) p.max_pages_per_seq = 1;
    if (p.layout == GQA_LAYOUT_CONTIGUOUS) {
      p.seq_capacity = p.max_seqlen_kv + (int32_t)(next_u64() % 5) + 1;
      p.kv_rows = (int64_t)p.batch * p.seq_capacity;
    } else if (p.layout == GQA_LAYOUT_RAGGED) {
      p.kv_rows = 1 + (int64_t)(next_u64() % ((uint64_t)p.batch * (p.max_seqlen_kv + 1)));
    } else {
      p.kv_rows = ((int64_t)p.batch * p.max_pages_per_seq + (int64_t)(next_u64() % 7)) * p.page_size;
    }
    if (p.kv_rows > INT32_MAX) p.kv_rows = INT32_MAX / p.page_size * p.page_size;
    p.topk = (next_u64() % 3 == 0) ? (int32_t)(1 + next_u64() % 4096) : 0;
    p.gate_mode = (int32_t)(next_u64() % 3);
    p.softmax_scale = (next_u64() & 1) ? 0.f : -0.3f;
    p.kv_chunk = (next_u64() % 3 == 0) ? 32 * (int32_t)(1 + next_u64() % 128) : 0;
    p.num_cus = PICK(cus);
    p.math = (int32_t)(next_u64() % 3);
    const int nmut = (int)(next_u64() % 4);
    for (int m = 0; m < nmut; ++m) {
      switch (next_u64() % 17) {
        case 0: p.batch = PICK(batches); break;
        case 1: p.s_q = PICK(sqs); break;
        case 2: p.h_q = PICK(hqs); break;
        case 3: p.h_kv = PICK(hkvs); break;
        case 4: p.head_dim = PICK(dims); break;
        case 5: p.layout = PICK(small); break;
        case 6: p.kv_dtype = PICK(small); break;
        case 7: p.causal = PICK(small); break;
        case 8: p.max_seqlen_kv = PICK(lens); break;
        case 9: p.seq_capacity = PICK(caps); break;
        case 10: p.kv_rows = PICK(rowss); break;
        case 11: p.page_size = PICK(pages); break;
        case 12: p.max_pages_per_seq = PICK(mpps); break;
        case 13: p.topk = PICK(topks); break;
        case 14: p.softmax_scale = PICK(scales); break;
        case 15: p.kv_chunk = PICK(chunks); break;
        default: p.math = PICK(small); p.gate_mode = PICK(small); p.num_cus = PICK(cus); break;
      }
    }
    decode_case(&p, &ok_decode);

    gqa_append_params a;
    memset(&a, 0, sizeof a);
    a.batch = 1 + (int32_t)(next_u64() % 300);
    a.s_new = 1 + (int32_t)(next_u64() % 20000);
    a.h_kv = PICK(good_hkv);
    a.head_dim = 64 << (next_u64() % 3);
    a.layout = (next_u64() & 1) ? GQA_LAYOUT_PAGED : GQA_LAYOUT_CONTIGUOUS;
    a.kv_dtype = (int32_t)(next_u64() % 3);
    a.scale_policy = (int32_t)(next_u64() % 2);
    a.seq_capacity = a.s_new + (int32_t)(next_u64() % 100);
    a.page_size = 1 << (next_u64() % 11);
    a.max_pages_per_seq = (a.seq_capacity + a.page_size - 1) / a.page_size;
    a.kv_rows = a.layout == GQA_LAYOUT_PAGED ? (int64_t)a.batch * a.max_pages_per_seq * a.page_size
                                             : (int64_t)a.batch * a.seq_capacity;
    const int amut = (int)(next_u64() % 4);
    for (int m = 0; m < amut; ++m) {
      switch (next_u64() % 10) {
        case 0: a.batch = PICK(batches); break;
        case 1: a.s_new = PICK(lens); break;
        case 2: a.h_kv = PICK(hkvs); break;
        case 3: a.head_dim = PICK(dims); break;
        case 4: a.layout = PICK(small); break;
        case 5: a.kv_dtype = PICK(small); break;
        case 6: a.scale_policy = PICK(small); break;
        case 7: a.seq_capacity = PICK(caps); break;
        case 8: a.kv_rows = PICK(rowss); break;
        default: a.page_size = PICK(pages); a.max_pages_per_seq = PICK(mpps); break;
      }
    }
    append_case(&a, &ok_append);
  }
  printf("%ld iterations, %ld decode plans and %ld appends accepted, %lld stub launches, %d failures\n", iters,
         ok_decode, ok_append, gqa_stub_launches, failures);
  return failures == 0 ? 0 : 1;
}
