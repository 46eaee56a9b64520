/*
 * libgqa_decode — appending new K/V rows to a KV cache, with FP8 E4M3FN or
 * int8 quantisation on write, for AMD Instinct MI355X (gfx950).
 *
 * The decode path reads a cache of FP8 E4M3FN codes with one fp32 scale per
 * (request, KV head), a code meaning value(code) * scale ("Sparse paged GQA
 * decode attention with FP8 KV cache on SM89", sections "Workload" and
 * "Implementations").  This call is the step that writes such a cache: it
 * stores the S_new K and V rows a model step produces for each request at
 * logical positions n_b .. n_b + S_new - 1, converting bf16 to FP8 as it
 * writes.  Only the appended rows are touched; stored codes are never read
 * back or re-scaled (re-materialising a whole quantised cache per step is
 * what "Profiling down to the register, then an extension that broke my
 * assumptions twice" reports against, in its int8 KV-cache section).
 *
 * Quantisation of a value x (bf16, exact in fp32) under scale s:
 *     y = fp32(x / s)            IEEE fp32 division, round to nearest even
 *   FP8 E4M3FN (GQA_KV_FP8_E4M3FN), Q = 448:
 *     y = clamp(y, -448, 448)    the E4M3FN range (no infinity)
 *     code = E4M3FN(y)           round to nearest, ties to even mantissa;
 *                                the sign is kept (-0 -> 0x80)
 *   int8 (GQA_KV_INT8), Q = 127 (a reading: the int8 KV-cache section of
 *   the page above gives no encoding):
 *     code = clamp(round(y), -127, 127), round to the nearest integer with
 *     ties to even, stored as a two's-complement byte (-128 is never
 *     written; the decode path reads any code as code * s)
 * Scale policies (FP8 and int8):
 *     GQA_SCALE_GIVEN        k_scale / v_scale [B, H_kv] are read as given.
 *     GQA_SCALE_FIRST_BLOCK  a request with n_b == 0 before the call takes,
 *                            per KV head, s = fp32(absmax / Q) over the
 *                            S_new rows it appends (s = 1 when they are all
 *                            zero), written to k_scale / v_scale; a request
 *                            with n_b > 0 reads its scales as given, so
 *                            later appends reuse the first block's scale and
 *                            saturate what lies beyond +-Q * s.
 * A bf16 cache stores the rows as they are (k_scale / v_scale unused).
 *
 * The conventions of gqa_decode.h hold: the caller owns every buffer, the
 * call only enqueues work on `stream`, arguments are checked on the host
 * before anything is enqueued, and device-side data is not checked there.
 * Positions past a request's capacity (contiguous: t >= seq_capacity;
 * paged: t / page_size >= max_pages_per_seq, or a block-table entry that
 * puts the row outside [0, kv_rows)) are not written.
 */
#ifndef GQA_APPEND_H
#define GQA_APPEND_H

#include "gqa_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

enum { GQA_SCALE_GIVEN = 0, GQA_SCALE_FIRST_BLOCK = 1 };

typedef struct gqa_append_params {
  int32_t batch;             /* 0 <= B <= 65535                                         */
  int32_t s_new;             /* rows appended per request, >= 1                         */
  int32_t h_kv;              /* KV heads, 1..256                                        */
  int32_t head_dim;          /* 64, 128 or 256                                          */
  int32_t layout;            /* GQA_LAYOUT_CONTIGUOUS or GQA_LAYOUT_PAGED               */
  int32_t kv_dtype;          /* GQA_KV_BF16, GQA_KV_FP8_E4M3FN or GQA_KV_INT8           */
  int32_t scale_policy;      /* GQA_SCALE_* (FP8 and int8)                              */
  int32_t seq_capacity;      /* contiguous: token stride between requests               */
  int64_t kv_rows;           /* token rows in k_cache / v_cache (>= 1)                  */
  int32_t page_size;         /* paged: a power of two, 1..1024                          */
  int32_t max_pages_per_seq; /* paged: block_table row length                           */
  int32_t reserved[4];       /* must be 0                                               */
} gqa_append_params;

/* Workspace bytes gqa_kv_append needs for *p: per-block absolute maxima
 * when GQA_SCALE_FIRST_BLOCK spans several workgroups per request, else 0. */
gqa_status gqa_kv_append_workspace_size(const gqa_append_params* p, size_t* bytes);

/* Append.
 *   k_new, v_new  bf16 [B, S_new, H_kv, d]
 *   seqlens       int32 [B]: n_b before the call
 *   seqlens_out   int32 [B] or NULL: receives n_b + S_new; must not alias
 *                 seqlens (every workgroup of a request reads n_b)
 *   block_table   int32 [B, max_pages_per_seq] (paged); else NULL
 *   k_cache,      the cache, layout p->layout, dtype p->kv_dtype, written in
 *   v_cache       place at the appended rows only
 *   k_scale,      fp32 [B, H_kv] (FP8, int8): read (GQA_SCALE_GIVEN, or n_b > 0)
 *   v_scale       or written (GQA_SCALE_FIRST_BLOCK with n_b == 0); else NULL
 *   workspace     >= gqa_kv_append_workspace_size bytes, or NULL when that is 0
 * Base pointers of k_new, v_new, k_cache and v_cache must be 16-byte aligned. */
gqa_status gqa_kv_append(const gqa_append_params* p, const void* k_new, const void* v_new,
                         const int32_t* seqlens, int32_t* seqlens_out, const int32_t* block_table,
                         void* k_cache, void* v_cache, float* k_scale, float* v_scale, void* workspace,
                         size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_APPEND_H */
