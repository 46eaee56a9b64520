/*
 * libgqa_decode — grouped-query attention at decode over a KV cache, for
 * AMD Instinct MI355X (gfx950).
 *
 * One call computes, for every request b, query position i < S_q and query
 * head h < H_q,
 *
 *     O[b,i,h,:]  = sum_j softmax_j(scale * q[b,i,h,:] . K[j, g(h), :]) V[j, g(h), :]
 *     LSE[b,h,i]  = log sum_j exp(scale * q[b,i,h,:] . K[j, g(h), :])
 *
 * over the tokens j visible to (b, i), with the KV head g(h) = h / (H_q / H_kv)
 * shared by a group of H_q / H_kv consecutive query heads.  The head map is
 * the one the kernels compute in "When the K/V copy costs more than the
 * attention" (section "What I was looking at"; head-mapping table in "Why it
 * closed, and the tests that merged").  K and V are read from the cache as
 * stored, once per KV head, and never expanded to H_q heads.
 *
 * The cache can be contiguous, ragged (packed with offsets) or paged
 * through a block table; a per-request top-K list can restrict attention to
 * selected tokens; K/V can be FP8 E4M3FN (or int8) with one fp32 scale per
 * (request, KV head); and the output can be multiplied by sigmoid(gate).
 * These follow "Sparse paged GQA decode attention with FP8 KV cache on
 * SM89" (sections "Workload" and "Implementations").
 *
 * Conventions (all entry points):
 *   - The caller owns every buffer.  The library allocates no device memory
 *     and keeps no pointer after a call returns.
 *   - Device work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) and runs asynchronously: buffers must stay valid until the
 *     stream has passed the call.  No call synchronises with the device.
 *   - Arguments are validated on the host before any device work.  On a
 *     non-zero status nothing has been enqueued and nothing written.
 *   - Device-side data (lengths, offsets, block-table entries, top-K
 *     entries) is not checked on the host.  Top-K entries outside [0, n_b)
 *     are masked by definition.  Lengths above max_seqlen_kv are clamped to
 *     it, and every physical row is clamped into [0, kv_rows) so that bad
 *     offsets or block-table entries cannot make the kernels read outside
 *     the cache (the result for such inputs is unspecified).
 *   - Calls are thread-safe; the last error message is kept per host thread.
 */
#ifndef GQA_DECODE_H
#define GQA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GQA_DECODE_ABI_VERSION 1

typedef enum gqa_status {
  GQA_OK = 0,
  GQA_ERR_INVALID_ARG = 1,  /* a null required pointer, a bad size or enum  */
  GQA_ERR_UNSUPPORTED = 2,  /* valid but not built: head_dim, S_q, group    */
  GQA_ERR_ALIGNMENT = 3,    /* a tensor base pointer is not 16-byte aligned */
  GQA_ERR_WORKSPACE = 4,    /* workspace missing or smaller than required   */
  GQA_ERR_HIP = 5           /* a HIP runtime call or kernel launch failed   */
} gqa_status;

/* Cache layouts.  A "token row" is H_kv * head_dim elements (all KV heads of
 * one token); the cache is an array of token rows.                          */
enum {
  GQA_LAYOUT_CONTIGUOUS = 0, /* [B, seq_capacity, H_kv, d]; token t of b is row b*seq_capacity + t */
  GQA_LAYOUT_RAGGED = 1,     /* [sum n_b, H_kv, d];   token t of b is row cu_seqlens[b] + t        */
  GQA_LAYOUT_PAGED = 2       /* [pages, page_size, H_kv, d]; token t of b is row
                                block_table[b, t / page_size] * page_size + t % page_size           */
};

/* Stored K/V element types.  FP8 E4M3FN and int8 (two's complement) are
 * codes with one fp32 scale per (request, KV head): the stored value is
 * code * k_scale[b, g] (K) or code * v_scale[b, g] (V).  The kernels convert
 * codes to bf16 tile by tile in registers, never the whole cache (the int8
 * KV-cache section of "Profiling down to the register, then an extension
 * that broke my assumptions twice" reports what a whole-cache conversion
 * costs).                                                                    */
enum { GQA_KV_BF16 = 0, GQA_KV_FP8_E4M3FN = 1, GQA_KV_INT8 = 2 };

/* GQA_GATE_ELEMENTWISE: gate bf16 [B, S_q, H_q, d], O *= sigmoid(gate).
 * GQA_GATE_HEADWISE:    gate bf16 [B, S_q, H_q],    one value per head.     */
enum { GQA_GATE_NONE = 0, GQA_GATE_ELEMENTWISE = 1, GQA_GATE_HEADWISE = 2 };

/* Arithmetic of the two products (scores and P.V).  Both run on the same K/V
 * loads and LDS staging; they differ only in the units that multiply:
 *   GQA_MATH_MFMA  v_mfma_f32_16x16x32_bf16 on 16-row blocks of query rows
 *                  (the rows of a KV head's group padded to a multiple of 16);
 *   GQA_MATH_VALU  v_dot2_f32_bf16 and fp32 FMAs on exactly the group's rows,
 *                  for at most 8 query rows per KV head;
 *   GQA_MATH_AUTO  the faster one for the row count, as measured on MI355X:
 *                  MFMA at every row count (VALU is at best level with it
 *                  at 1 row and slower from 2 rows up).
 * At decode the products are skinny (rows = (H_q / H_kv) * S_q by d); a
 * tile sized for prefill leaves almost every row of a matrix-unit tile idle
 * ("When the K/V copy costs more than the attention", "What I was looking
 * at").  Whether the matrix unit still pays is a question of row count,
 * settled by measurement.                                                   */
enum { GQA_MATH_AUTO = 0, GQA_MATH_MFMA = 1, GQA_MATH_VALU = 2 };

typedef struct gqa_decode_params {
  int32_t batch;             /* 0 <= B <= 65535                                         */
  int32_t s_q;               /* query tokens per request, 1..64                         */
  int32_t h_q;               /* query heads                                             */
  int32_t h_kv;              /* KV heads; h_q % h_kv == 0, (h_q/h_kv)*s_q <= 512        */
  int32_t head_dim;          /* 64, 128 or 256 (the VALU path: 64 or 128)              */
  int32_t layout;            /* GQA_LAYOUT_*                                            */
  int32_t kv_dtype;          /* GQA_KV_*                                                */
  int32_t causal;            /* 1: query i of an S_q block sits at position n_b - S_q + i
                                and sees tokens t <= n_b - S_q + i; 0: sees all tokens   */
  int32_t max_seqlen_kv;     /* upper bound on every n_b (sizes the grid)               */
  int32_t seq_capacity;      /* contiguous: token stride between requests (>= max_seqlen_kv) */
  int64_t kv_rows;           /* number of token rows in k_cache / v_cache (>= 1)        */
  int32_t page_size;         /* paged: a power of two, 1..1024                          */
  int32_t max_pages_per_seq; /* paged: block_table row length;
                                max_pages_per_seq * page_size >= max_seqlen_kv          */
  int32_t topk;              /* 0: dense; > 0: each request attends to the K = topk
                                logical positions listed in topk_idx[b, :]               */
  int32_t gate_mode;         /* GQA_GATE_*                                              */
  float softmax_scale;       /* 0: 1/sqrt(head_dim)                                     */
  int32_t kv_chunk;          /* list positions per split-KV workgroup; 0 = automatic;
                                else a multiple of 32 (at most 4096 for paged or top-K) */
  int32_t num_cus;           /* compute units to plan for; 0 = ask the current device   */
  int32_t math;              /* GQA_MATH_*; VALU needs (h_q / h_kv) * s_q <= 8          */
  /* Optional timing hooks: hipEvent_t handles that the split-KV partial
   * kernel's dispatch stamps when the kernel starts and when it ends (so
   * their elapsed time is the kernel alone).  NULL = not used.            */
  void* partial_event_begin;
  void* partial_event_end;
} gqa_decode_params;

typedef struct gqa_decode_plan {
  int32_t rows;              /* query rows sharing one KV head: (h_q / h_kv) * s_q      */
  int32_t row_blocks;        /* MFMA: 16-row blocks computed per KV head (the group's
                                rows padded to the tiling); VALU: rows computed (1, 2,
                                4 or 8, at least the group's rows)                      */
  int32_t kv_chunk;          /* list positions per workgroup                            */
  int32_t num_splits;        /* workgroups per (request, KV head) for the longest list  */
  int64_t partial_workgroups;/* grid size of the partial kernel                         */
  int32_t combine;           /* 1 if the LSE-combine kernel runs                        */
  int32_t math;              /* GQA_MATH_MFMA or GQA_MATH_VALU: the path chosen         */
  size_t workspace_bytes;    /* bytes of `workspace` gqa_decode_run needs (0 if none)   */
} gqa_decode_plan;

/* Plan a call: validates the shape fields of *p (pointers are not looked at)
 * and fills *plan.  Needs a device only when p->num_cus == 0.               */
gqa_status gqa_decode_make_plan(const gqa_decode_params* p, gqa_decode_plan* plan);

/* Workspace bytes gqa_decode_run needs for *p: the split partials
 * (num_splits * rows * (head_dim + 1) fp32 per (request, KV head)), 0 when
 * one split covers every list.  The KV walk is split across workgroups
 * (an unsplit walk is one of the causes of slow decode named in "When the
 * K/V copy costs more than the attention", section "What I was looking
 * at"), and each split leaves an output row and its log-sum-exp here for
 * the combine.  The workspace never holds K or V expanded to H_q heads:
 * that expansion is what ran out of memory on the same page ("What it did,
 * and what it didn't").  Shapes whose partials would exceed 2^40 bytes are
 * rejected with GQA_ERR_UNSUPPORTED.                                       */
gqa_status gqa_decode_workspace_size(const gqa_decode_params* p, size_t* bytes);

/* Decode attention.
 *   q           bf16 [B, S_q, H_q, d]
 *   k_cache,    bf16, or FP8 E4M3FN or int8 codes, layout p->layout (see above),
 *   v_cache     same layout, dtype and size as k_cache
 *   seqlens     int32 [B]   n_b (contiguous, paged); NULL for ragged
 *   cu_seqlens  int32 [B+1] ragged offsets (n_b = cu[b+1] - cu[b]); else NULL
 *   block_table int32 [B, max_pages_per_seq] (paged); else NULL
 *   topk_idx    int32 [B, topk] logical token positions (topk > 0); else NULL.
 *               Entries outside [0, n_b) are masked; duplicates count once
 *               per occurrence.
 *   k_scale,    fp32 [B, H_kv] (FP8 and int8, else NULL): stored codes mean
 *   v_scale     code_value * scale
 *   gate        bf16, shape by p->gate_mode; NULL when GQA_GATE_NONE
 *   o           bf16 [B, S_q, H_q, d], written in full
 *   lse         fp32 [B, H_q, S_q], written in full: natural log of the sum
 *               of exp(scaled scores); -inf (with O = 0) when nothing is visible
 *   workspace   device scratch of at least gqa_decode_workspace_size bytes
 *               (may be NULL when that size is 0); contents need no
 *               initialisation and are dead after the call.
 * Pointer alignment: q, k_cache, v_cache, o and an elementwise gate must be
 * 16-byte aligned, every other array 4-byte aligned.                        */
gqa_status gqa_decode_run(const gqa_decode_params* p,
                          const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* seqlens, const int32_t* cu_seqlens,
                          const int32_t* block_table, const int32_t* topk_idx,
                          const float* k_scale, const float* v_scale,
                          const void* gate, void* o, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the scratch array gqa_decode_run_noalloc keeps on each device. */
#define GQA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* Decode attention with no caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments (less the
 * workspace), checks, kernels and results as gqa_decode_run.  The split
 * partials go to a scratch array of GQA_NOALLOC_SCRATCH_BYTES that the
 * library holds on each device it runs on, from the first call on that
 * device until the process ends; no call allocates or frees memory.
 *   - A call whose plan needs more workspace than the array holds (see
 *     gqa_decode_workspace_size) returns GQA_ERR_WORKSPACE and enqueues
 *     nothing.
 *   - Every call on one device uses that device's one array: calls that
 *     may overlap on one device (several streams, several host threads)
 *     race on it, and the caller must order them.
 *   - The scratch needs no initialisation and holds nothing a later call
 *     reads.                                                              */
gqa_status gqa_decode_run_noalloc(const gqa_decode_params* p,
                                  const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* seqlens, const int32_t* cu_seqlens,
                                  const int32_t* block_table, const int32_t* topk_idx,
                                  const float* k_scale, const float* v_scale,
                                  const void* gate, void* o, float* lse, void* stream);

/* Address resolution on the device, with the same code the decode kernels
 * use to turn (request, list slot) into a physical token row: a top-K
 * entry names a token of the request, and a page of page_size tokens found
 * through the request's block-table row holds it ("Sparse paged GQA decode
 * attention with FP8 KV cache on SM89", section "Workload": top-K 512 token
 * indices, pages of 16, 32 pages per request; section "Implementations":
 * the eager version gathers the selected K/V rows before attending).
 * rows_out: int64 [B, S_q, list_len], list_len = topk if topk > 0 else
 * max_seqlen_kv; entry = physical token row of that slot for query i, or -1
 * where the slot is masked (beyond n_b, outside [0, n_b) for a top-K entry,
 * or hidden by the causal rule).  Used to check addressing bit-exactly.     */
gqa_status gqa_resolve_rows(const gqa_decode_params* p, const int32_t* seqlens,
                            const int32_t* cu_seqlens, const int32_t* block_table,
                            const int32_t* topk_idx, int64_t* rows_out, void* stream);

const char* gqa_status_string(gqa_status s);
/* Message describing the last failure on this host thread ("" if none).   */
const char* gqa_last_error(void);
int gqa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_DECODE_H */
