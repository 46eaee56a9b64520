// C ABI of libgqa_decode: host-side validation, the split planner and the
// launch sequence (partial kernel, then the LSE combine when the KV walk is
// split).  No allocation, no device synchronisation.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "gqa_append.h"
#include "gqa_append_args.h"
#include "gqa_decode.h"
#include "gqa_device.h"

namespace gqa {
hipError_t launch_partial(const DecodeArgs& a, int D, int kvt, int mode, int mb, int rv, int share, dim3 grid,
                          hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_combine(const DecodeArgs& a, int D, dim3 grid, hipStream_t st);
hipError_t launch_resolve(const DecodeArgs& a, int64_t* out, int list_cap, hipStream_t st);
hipError_t scratch_address(void** ptr, size_t* bytes);
}  // namespace gqa

namespace {

thread_local std::string g_last_error;

gqa_status fail(gqa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
gqa_status fail(gqa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

constexpr int kMaxChunkIndirect = 4096;
constexpr size_t kMaxLdsPerWorkgroup = 160 * 1024;  // gfx950: 160 KiB of LDS per CU and workgroup
constexpr int kMaxRows = 512;
constexpr int kMaxSq = 64;
constexpr int kMaxValuRows = 8;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int log2_exact(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return (1 << s) == x ? s : -1;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// KV heads per partial workgroup: four when H_kv allows (a workgroup then
// reads 4 heads' contiguous slice of every token row), else two, else one.
int heads_per_wg(int h_kv) { return h_kv % 4 == 0 ? 4 : (h_kv % 2 == 0 ? 2 : 1); }
static_assert(gqa::kPWaves % 4 == 0, "heads per workgroup must divide the waves");
int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

int device_cus() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = cus;
  }
  return cached[dev];
}

// Shape checks shared by every entry point (no pointers looked at).
gqa_status check_shape(const gqa_decode_params* p) {
  if (!p) return fail(GQA_ERR_INVALID_ARG, "params is NULL");
  if (p->batch < 0 || p->batch > 65535) return fail(GQA_ERR_INVALID_ARG, "batch %d outside [0, 65535]", p->batch);
  if (p->h_q <= 0 || p->h_kv <= 0 || p->h_kv > 65535)
    return fail(GQA_ERR_INVALID_ARG, "h_q %d / h_kv %d must be positive (h_kv <= 65535)", p->h_q, p->h_kv);
  if (p->h_q % p->h_kv != 0) return fail(GQA_ERR_INVALID_ARG, "h_q %d is not a multiple of h_kv %d", p->h_q, p->h_kv);
  if (p->s_q < 1 || p->s_q > kMaxSq) return fail(GQA_ERR_UNSUPPORTED, "s_q %d outside [1, %d]", p->s_q, kMaxSq);
  if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 256)
    return fail(GQA_ERR_UNSUPPORTED, "head_dim %d is not 64, 128 or 256", p->head_dim);
  const int64_t rows = (int64_t)(p->h_q / p->h_kv) * p->s_q;
  if (rows > kMaxRows)
    return fail(GQA_ERR_UNSUPPORTED, "(h_q/h_kv)*s_q = %lld query rows per KV head exceeds %d", (long long)rows, kMaxRows);
  if (p->layout < GQA_LAYOUT_CONTIGUOUS || p->layout > GQA_LAYOUT_PAGED)
    return fail(GQA_ERR_INVALID_ARG, "unknown layout %d", p->layout);
  if (p->kv_dtype != GQA_KV_BF16 && p->kv_dtype != GQA_KV_FP8_E4M3FN && p->kv_dtype != GQA_KV_INT8)
    return fail(GQA_ERR_INVALID_ARG, "unknown kv_dtype %d", p->kv_dtype);
  if (p->gate_mode < GQA_GATE_NONE || p->gate_mode > GQA_GATE_HEADWISE)
    return fail(GQA_ERR_INVALID_ARG, "unknown gate_mode %d", p->gate_mode);
  if (p->causal != 0 && p->causal != 1) return fail(GQA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (p->max_seqlen_kv < 0) return fail(GQA_ERR_INVALID_ARG, "max_seqlen_kv %d < 0", p->max_seqlen_kv);
  if (p->kv_rows < 1 || p->kv_rows > INT32_MAX)
    return fail(GQA_ERR_INVALID_ARG, "kv_rows %lld outside [1, 2^31)", (long long)p->kv_rows);
  if (p->layout == GQA_LAYOUT_CONTIGUOUS) {
    if (p->seq_capacity < 1 || p->seq_capacity < p->max_seqlen_kv)
      return fail(GQA_ERR_INVALID_ARG, "seq_capacity %d must be >= max(1, max_seqlen_kv %d)", p->seq_capacity,
                  p->max_seqlen_kv);
    if ((int64_t)p->batch * p->seq_capacity > p->kv_rows)
      return fail(GQA_ERR_INVALID_ARG, "batch * seq_capacity exceeds kv_rows %lld", (long long)p->kv_rows);
  }
  if (p->layout == GQA_LAYOUT_PAGED) {
    if (p->page_size < 1 || p->page_size > 1024 || log2_exact(p->page_size) < 0)
      return fail(GQA_ERR_UNSUPPORTED, "page_size %d is not a power of two in [1, 1024]", p->page_size);
    if (p->max_pages_per_seq < 1 || (int64_t)p->max_pages_per_seq * p->page_size < p->max_seqlen_kv)
      return fail(GQA_ERR_INVALID_ARG, "max_pages_per_seq %d * page_size %d < max_seqlen_kv %d",
                  p->max_pages_per_seq, p->page_size, p->max_seqlen_kv);
    if (p->kv_rows % p->page_size != 0)
      return fail(GQA_ERR_INVALID_ARG, "kv_rows %lld is not a whole number of pages", (long long)p->kv_rows);
  }
  if (p->topk < 0) return fail(GQA_ERR_INVALID_ARG, "topk %d < 0", p->topk);
  if (!std::isfinite(p->softmax_scale)) return fail(GQA_ERR_INVALID_ARG, "softmax_scale is not finite");
  if (p->kv_chunk != 0) {
    const bool indirect = p->layout == GQA_LAYOUT_PAGED || p->topk > 0;
    if (p->kv_chunk < 32 || p->kv_chunk % 32 != 0 || p->kv_chunk > (1 << 24))
      return fail(GQA_ERR_INVALID_ARG, "kv_chunk %d is not a positive multiple of 32", p->kv_chunk);
    if (indirect && p->kv_chunk > kMaxChunkIndirect)
      return fail(GQA_ERR_INVALID_ARG, "kv_chunk %d exceeds %d for paged / top-K lists", p->kv_chunk,
                  kMaxChunkIndirect);
  }
  if (p->num_cus < 0) return fail(GQA_ERR_INVALID_ARG, "num_cus %d < 0", p->num_cus);
  if (p->math < GQA_MATH_AUTO || p->math > GQA_MATH_VALU) return fail(GQA_ERR_INVALID_ARG, "unknown math %d", p->math);
  if (p->math == GQA_MATH_VALU && p->head_dim > 128)
    return fail(GQA_ERR_UNSUPPORTED, "the VALU path is built for head_dim <= 128");
  if (p->math == GQA_MATH_VALU && rows > kMaxValuRows)
    return fail(GQA_ERR_UNSUPPORTED, "the VALU path takes at most %d query rows per KV head, not %lld", kMaxValuRows,
                (long long)rows);
  return GQA_OK;
}

// A ragged cache without a top-K list is split into equal chunks of packed
// rows (each chunk cut at request boundaries inside the kernel) instead of
// per-request chunks: every workgroup then streams the same number of rows
// whatever the mix of lengths.
// K/V stored as one-byte codes (FP8 or int8) with per-(request, head) scales.
bool one_byte(const gqa_decode_params* p) { return p->kv_dtype != GQA_KV_BF16; }
static_assert(GQA_KV_BF16 == gqa::kKvBf16 && GQA_KV_FP8_E4M3FN == gqa::kKvFp8 && GQA_KV_INT8 == gqa::kKvInt8,
              "the public K/V type enum is the kernels' template argument");

bool packed_mode(const gqa_decode_params* p) { return p->layout == GQA_LAYOUT_RAGGED && p->topk == 0; }

// Largest workspace a plan may ask for.  Shapes whose split partials would
// exceed it (no device holds them) are rejected instead of having their
// byte count wrap.
constexpr unsigned __int128 kMaxWorkspaceBytes = (unsigned __int128)1 << 40;

// Bytes of the fp32 partial outputs (the LSE partials follow, rounded up to
// 256 bytes): (request, KV head, split) slots of rows x head_dim each; packed
// chunks use slots (request + chunk, KV head).  Exact in 128 bits: every
// factor is below 2^32.
unsigned __int128 partial_o_bytes(const gqa_decode_params* p, const gqa_decode_plan& plan) {
  const unsigned __int128 slots = packed_mode(p)
                                      ? ((unsigned __int128)p->batch + plan.num_splits - 1) * (unsigned)p->h_kv
                                      : (unsigned __int128)p->batch * (unsigned)p->h_kv * (unsigned)plan.num_splits;
  return slots * (unsigned)plan.rows * (unsigned)p->head_dim * sizeof(float);
}

unsigned __int128 round_up_256(unsigned __int128 x) { return (x + 255) / 256 * 256; }

// The math path GQA_MATH_AUTO takes for a group of `rows` query rows: the
// matrix units at every row count.  Measured on MI355X over 128K-token
// decodes at H_kv = 8 (bf16 d = 128 and 64, FP8 and int8 d = 128; three
// processes each): MFMA is faster from 2 rows up (more than twice as fast
// at 8), its time flat from 1 to 16 rows; at 1 row it is as fast or faster
// too (partial kernel, bf16 d = 128: 81.1-81.8 against 83.1-83.5 us; d = 64:
// 42.2-42.4 against 42.5-43.1; int8: 44.5-46.0 against 49.6-51.1; FP8 equal).
int auto_math(int, int) { return GQA_MATH_MFMA; }

// How a KV head's query rows are laid over waves and workgroups.
struct Tiling {
  int mb = 1;          // 16-row MFMA blocks per wave (VALU: unused)
  int share = 1;       // waves of a head that split the rows (1: they split the tiles)
  int hpw = 1;         // KV heads per workgroup
  int row_groups = 1;  // workgroups along the rows, each share * mb * 16 rows
};
static_assert(gqa::kPWaves == 4, "row sharing is laid out for 4 waves per workgroup");

// Up to 16 rows: one block per wave, the waves of a head taking alternate
// tiles.  17-32 rows: two blocks per wave.  At d = 256 two blocks fit a
// wave's registers only with Q moved to LDS, which the bf16 kernels do
// (contiguous, paged and top-K lists); one-byte codes and packed caches
// with an even H_kv instead have a head's two waves split the rows and
// share the tiles through LDS.  Eight waves per
// head there (two with rows, all eight loading) ran the partial kernel
// faster for bf16 (54.3 against 55.8 us, 32/2 heads at 128K) but the whole
// call slower in back-to-back calls (64.7 against 63.3 us), and FP8 slower
// (54.7 against 45.9 us); they are not used.  33-64 rows: a
// head's four waves split the rows, one block each (FP8 and int8 at d = 64,
// whose tiles are two loads per tensor: two waves per head, two blocks
// each, or one wave of four blocks for odd H_kv).  More rows: a workgroup
// of eight waves per head, one block each up to 128 rows and two beyond
// (d <= 128), and groups of more rows than one workgroup covers take
// several row groups (four-wave row groups of 64 for bf16 d = 64 up to 256
// rows, below).  MI355X, one process, us per call against four
// waves per head (one block each, row groups of 64): 512 rows 653 -> 351
// (bf16 d = 128, 128K) and 638 -> 383 (FP8); 128 rows 47.5 -> 42.6 (bf16
// d = 128, 4 x 32K) and 229 -> 206 (FP8, 8 x 32K).  The exception is bf16
// at d = 64 up to 256 rows: only four of the eight waves load its tiles,
// and four waves per head in two workgroups per CU keep twice the bytes in
// flight.  Measured there: 160 rows (80/1, 128K) 27.9 with four waves
// against 30.3 us, 128 rows 30.8 against 34.2 us (16/2, 4 x 32K) but 160
// against 147 us (64/8, 8 x 32K); at 512 rows (8/1, 128K) eight waves win,
// 55.6 -> 47.3 us.
Tiling plan_tiling(const gqa_decode_params* p, int rows, int math) {
  Tiling t;
  t.hpw = heads_per_wg(p->h_kv);
  // Paged or top-K lists, up to 16 rows, H_kv a multiple of 8, and a wave
  // that fits half the register file: one workgroup of eight waves covers
  // eight KV heads, one each, and resolves the request's row table once for
  // all of them.  MI355X, one process, partial kernel against two
  // workgroups of four heads per CU: paged FP8 (32 x 32K, 64/8) 351 ->
  // 329 us, sparse top-512 FP8 46.3 -> 45.1 us, int8 48.5 -> 48.1 us; dense
  // lists were slower (FP8 64/8 at 128K 46.1 -> 51.0 us, bf16 d = 64 42.7 ->
  // 46.1 us), so they keep four heads.
  const bool indirect = p->layout == GQA_LAYOUT_PAGED || p->topk > 0;
  if (math != GQA_MATH_VALU && rows <= 16 && indirect && p->h_kv % 8 == 0 &&
      gqa::wide_fits(p->head_dim, one_byte(p)))
    t.hpw = 8;
  if (math == GQA_MATH_VALU || rows <= 16) return t;
  if (rows <= 32) {
    if (p->head_dim == 256 && !one_byte(p) && !packed_mode(p)) {
      // bf16 d = 256: two blocks per wave with Q in LDS, one KV head per
      // workgroup (the Q buffer holds one head).  MI355X, 32/2 heads at 128K,
      // against the two waves per head sharing tiles: partial kernel
      // 55.7 -> 54.5 us, call 60.7 -> 58.4 us (half the splits).  FP8 ran
      // slower this way (40.4 against 35.5 us) and keeps the shared tiles.
      t.mb = 2;
      t.hpw = 1;
    } else if (p->head_dim == 256 && p->h_kv % 2 == 0) {
      t.share = 2;
      t.hpw = 2;
    } else {
      t.mb = 2;  // odd H_kv: one head per workgroup (bf16 d = 256 keeps Q in LDS)
    }
    return t;
  }
  const int loads = p->head_dim * (one_byte(p) ? 1 : 2) / 32;  // per tile and tensor
  const bool bf16_d64 = !one_byte(p) && p->head_dim == 64;
  if (rows > 64 && !(bf16_d64 && rows <= 256)) {
    t.share = 8;
    t.hpw = 1;
    t.mb = (rows > 128 && p->head_dim <= 128) ? 2 : 1;
    t.row_groups = (int)cdiv(rows, 128 * t.mb);
  } else if (loads % 4 == 0) {
    t.share = 4;
    t.hpw = 1;
    t.row_groups = (int)cdiv(rows, 64);
  } else if (p->h_kv % 2 == 0) {
    t.share = 2;
    t.hpw = 2;
    t.mb = 2;
    t.row_groups = (int)cdiv(rows, 64);
  } else {
    t.mb = 4;  // rows <= 64 (check_shape)
  }
  return t;
}

gqa_status make_plan(const gqa_decode_params* p, gqa_decode_plan* plan) {
  gqa_status st = check_shape(p);
  if (st != GQA_OK) return st;
  std::memset(plan, 0, sizeof *plan);
  const int rows = (p->h_q / p->h_kv) * p->s_q;
  plan->rows = rows;
  plan->math = p->math == GQA_MATH_AUTO ? auto_math(rows, p->head_dim) : p->math;
  const Tiling tl = plan_tiling(p, rows, plan->math);
  if (plan->math == GQA_MATH_VALU)
    plan->row_blocks = rows <= 2 ? rows : (rows <= 4 ? 4 : 8);
  else
    plan->row_blocks = tl.mb * tl.share * tl.row_groups;
  const bool indirect = p->layout == GQA_LAYOUT_PAGED || p->topk > 0;
  const bool packed = packed_mode(p);
  const int64_t L = p->topk > 0 ? p->topk : p->max_seqlen_kv;
  const int64_t pairs = (int64_t)p->batch * p->h_kv;
  const int hpw = tl.hpw;
  const int lds_waves = hpw == 8 ? 8 : gqa::kPWaves;  // eight heads: a wave each
  const size_t q_bytes = gqa::q_in_lds(p->head_dim, one_byte(p), tl.mb, plan->math == GQA_MATH_VALU ? 1 : 0, tl.share)
                             ? gqa::q_lds_bytes(p->head_dim, tl.mb)
                             : 0;
  // Resident workgroups per CU the grid is sized for.  Measured on MI355X
  // (one process, both plans): the row-sharing variants that fit two per CU
  // run faster with two (32 x 8192 tokens at S_q 16: 229 -> 202 us packed,
  // 192 -> 185 us contiguous); the tile-splitting ones that fit two run
  // faster with one long round (d = 64: 50.2 against 53.0 us; FP8 d = 128:
  // 51.4 against 53.0 us at 128K tokens).
  const int occ = plan->math == GQA_MATH_MFMA && tl.share > 1
                      ? gqa::partial_wgs_per_cu(p->head_dim, one_byte(p), tl.mb, 0, tl.share)
                      : 1;
  const int64_t groups = (int64_t)(p->h_kv / hpw) * tl.row_groups;  // grid.y: head groups x row groups
  if (groups > 65535) return fail(GQA_ERR_UNSUPPORTED, "h_kv %d with %d row groups exceeds the grid", p->h_kv, tl.row_groups);
  int64_t chunk = p->kv_chunk;
  if (chunk == 0) {
    int cus = p->num_cus ? p->num_cus : device_cus();
    if (cus <= 0) return fail(GQA_ERR_HIP, "cannot query the device's compute-unit count");
    if (packed) {
      // One round of resident workgroups over the packed rows, each the same size.
      const int64_t per = cdiv(p->kv_rows * groups, (int64_t)cus * occ);
      chunk = std::min<int64_t>(round_up(std::max<int64_t>(per, 64), 32), 1 << 24);
    } else {
      // A workgroup covers hpw heads x chunk list positions (x one row
      // group).  Aim for one resident round of workgroups over the whole
      // grid -- occ per CU (MI355X measurements: one resident round of long
      // workgroups streams best and writes the fewest partials), with
      // 128..4096 positions per workgroup and never more than the list.
      const int64_t per = cdiv(std::max<int64_t>(pairs * L * tl.row_groups, 1), (int64_t)cus * occ * hpw);
      chunk = round_up(std::max<int64_t>(per, 128), 128);
      chunk = std::min<int64_t>(chunk, 4096);
      chunk = std::min<int64_t>(chunk, round_up(std::max<int64_t>(L, 1), 32));
      if (indirect) {
        // the row table (8 bytes per position) must fit beside the tiles
        const size_t tiles = gqa::partial_lds_bytes(p->head_dim, one_byte(p), false, 0, lds_waves, q_bytes);
        chunk = std::min<int64_t>(chunk, (int64_t)((kMaxLdsPerWorkgroup - tiles - gqa::table_bytes(true, 0)) / 8 /
                                                   128 * 128));
      }
    }
  }
  // Shared memory of one partial workgroup (per-wave K/V tiles plus the
  // row table of paged / top-K chunks) must fit a workgroup's LDS.
  const size_t lds = gqa::partial_lds_bytes(p->head_dim, one_byte(p), indirect, (int)chunk, lds_waves, q_bytes);
  if (lds > kMaxLdsPerWorkgroup)
    return fail(GQA_ERR_UNSUPPORTED, "kv_chunk %lld needs %zu bytes of LDS per workgroup (limit %zu)",
                (long long)chunk, lds, kMaxLdsPerWorkgroup);
  const int64_t splits = packed ? cdiv(p->kv_rows, chunk) : std::max<int64_t>(1, cdiv(L, chunk));
  if (splits > INT32_MAX) return fail(GQA_ERR_UNSUPPORTED, "too many splits");
  plan->kv_chunk = (int32_t)chunk;
  plan->num_splits = (int32_t)splits;
  plan->partial_workgroups = groups * splits * (packed ? 1 : p->batch);
  // Packed: requests that span chunks are merged by the combine, which
  // also writes the empty requests; partial slots are (request + chunk).
  plan->combine = (packed || splits > 1) ? 1 : 0;
  if (plan->combine) {
    const unsigned __int128 opart = partial_o_bytes(p, *plan);
    const unsigned __int128 ws = round_up_256(opart) + round_up_256(opart / p->head_dim);
    if (ws > kMaxWorkspaceBytes)
      return fail(GQA_ERR_UNSUPPORTED, "the split partials would need %.3g bytes of workspace (limit 2^40)",
                  (double)ws);
    plan->workspace_bytes = (size_t)ws;
  }
  return GQA_OK;
}

gqa_status hip_fail(hipError_t e, const char* what) {
  return fail(GQA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Combine workgroup shape: enough split lanes that each thread merges at
// most 16 splits of the longest list (two rounds of 8 loads); with few
// splits, several rows per workgroup, with many, a slice of the columns
// (at least 8 quads, so that a row's split lanes stay at lane strides of
// 8 or more).  cols * rows * quads and the split lanes fill 256 threads.
// MI355X timings of the combine alone (128K tokens, 128 or 256 splits; 32
// requests of 8192 tokens at S_q 8, 4-5 splits): a target of 16 splits
// per thread beat 8 and 4, whose extra workgroups cost more than the
// second round of loads saves, and beat one workgroup per row (many
// idle split lanes when splits are few).
void combine_shape(const gqa_decode_params* p, const gqa_decode_plan& plan, int32_t* cols, int32_t* rows) {
  const int q4 = p->head_dim / 4;
  int64_t nsp = plan.num_splits;
  if (packed_mode(p)) nsp = std::min<int64_t>(nsp, cdiv(std::max(p->max_seqlen_kv, 1), plan.kv_chunk) + 1);
  int need = 1;
  while (need * 16 < nsp && need * 8 < gqa::kThreads) need *= 2;
  int cb = 1, rb = 1;
  if (need * q4 <= gqa::kThreads) {
    while (rb < plan.rows && rb * 2 * need * q4 <= gqa::kThreads) rb *= 2;
  } else {
    cb = std::min(q4 / 8, need * q4 / gqa::kThreads);
  }
  *cols = cb;
  *rows = rb;
}

void fill_args(gqa::DecodeArgs& a, const gqa_decode_params* p, const gqa_decode_plan& plan) {
  std::memset(&a, 0, sizeof a);
  a.kv_rows = p->kv_rows;
  a.batch = p->batch;
  a.s_q = p->s_q;
  a.h_q = p->h_q;
  a.h_kv = p->h_kv;
  a.group = p->h_q / p->h_kv;
  a.rows = plan.rows;
  a.layout = p->layout;
  a.causal = p->causal;
  a.max_seqlen = p->max_seqlen_kv;
  a.seq_cap = p->seq_capacity;
  a.page_shift = p->layout == GQA_LAYOUT_PAGED ? log2_exact(p->page_size) : 0;
  a.max_pages = p->max_pages_per_seq;
  a.topk_len = p->topk;
  a.gate_mode = p->gate_mode;
  a.chunk = plan.kv_chunk;
  a.num_splits = plan.num_splits;
  a.heads_per_wg = plan_tiling(p, plan.rows, plan.math).hpw;
  a.packed = packed_mode(p) ? 1 : 0;
  if (a.packed) {
    a.part_sb = (int64_t)p->h_kv * plan.rows;
    a.part_sg = plan.rows;
    a.part_ss = (int64_t)p->h_kv * plan.rows;
  } else {
    a.part_sb = (int64_t)p->h_kv * plan.num_splits * plan.rows;
    a.part_sg = (int64_t)plan.num_splits * plan.rows;
    a.part_ss = plan.rows;
  }
  combine_shape(p, plan, &a.comb_cols, &a.comb_rows);
  // Row groups of a chunk on one XCD (see the partial kernel): only when
  // the grid is a whole number of rounds of 8 x row groups.
  {
    const Tiling tl = plan_tiling(p, plan.rows, plan.math);
    const int64_t wgs = plan.partial_workgroups;
    a.xcd_rows = (tl.row_groups > 1 && wgs % ((int64_t)gqa::kXcds * tl.row_groups) == 0) ? tl.row_groups : 1;
  }
  const float scale = p->softmax_scale != 0.f ? p->softmax_scale : 1.0f / std::sqrt((float)p->head_dim);
  a.scale_log2 = (float)((double)scale * 1.4426950408889634074);
}

// ---- K/V append --------------------------------------------------------

gqa_status check_append(const gqa_append_params* p) {
  if (!p) return fail(GQA_ERR_INVALID_ARG, "params is NULL");
  if (p->batch < 0 || p->batch > 65535 || p->s_new < 1)
    return fail(GQA_ERR_INVALID_ARG, "batch must be in [0, 65535] and s_new >= 1");  // batch is grid.y
  if (p->h_kv < 1 || p->h_kv > gqa::kAppendMaxHeads)
    return fail(GQA_ERR_UNSUPPORTED, "h_kv must be 1..%d", gqa::kAppendMaxHeads);
  if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 256)
    return fail(GQA_ERR_UNSUPPORTED, "head_dim %d not built (64, 128, 256)", p->head_dim);
  if (p->kv_dtype != GQA_KV_BF16 && p->kv_dtype != GQA_KV_FP8_E4M3FN && p->kv_dtype != GQA_KV_INT8)
    return fail(GQA_ERR_INVALID_ARG, "bad kv_dtype");
  if (p->scale_policy != GQA_SCALE_GIVEN && p->scale_policy != GQA_SCALE_FIRST_BLOCK)
    return fail(GQA_ERR_INVALID_ARG, "bad scale_policy");
  if (p->kv_rows < 1) return fail(GQA_ERR_INVALID_ARG, "kv_rows must be >= 1");
  for (int r : p->reserved)
    if (r != 0) return fail(GQA_ERR_INVALID_ARG, "reserved fields must be 0");
  if (p->layout == GQA_LAYOUT_CONTIGUOUS) {
    if (p->seq_capacity < 1) return fail(GQA_ERR_INVALID_ARG, "contiguous layout needs seq_capacity >= 1");
    if ((int64_t)p->batch * p->seq_capacity > p->kv_rows)
      return fail(GQA_ERR_INVALID_ARG, "batch * seq_capacity exceeds kv_rows");
  } else if (p->layout == GQA_LAYOUT_PAGED) {
    if (p->page_size < 1 || p->page_size > 1024 || log2_exact(p->page_size) < 0)
      return fail(GQA_ERR_INVALID_ARG, "page_size must be a power of two in 1..1024");
    if (p->max_pages_per_seq < 1) return fail(GQA_ERR_INVALID_ARG, "paged layout needs max_pages_per_seq >= 1");
  } else {
    return fail(GQA_ERR_UNSUPPORTED, "append writes contiguous or paged caches (a packed ragged cache has no room)");
  }
  return GQA_OK;
}

// New tokens per append workgroup: as many as fit kAppendElemsPerWorkgroup
// elements (all KV heads of a token together), at least one.
int append_chunk_tokens(const gqa_append_params* p) {
  const int fit = std::max(1, gqa::kAppendElemsPerWorkgroup / (p->h_kv * p->head_dim));
  return std::min(fit, p->s_new);
}

size_t append_workspace(const gqa_append_params* p) {
  const int chunks = (int)cdiv(p->s_new, append_chunk_tokens(p));
  if (p->kv_dtype == GQA_KV_BF16 || p->scale_policy != GQA_SCALE_FIRST_BLOCK || chunks == 1) return 0;
  return (size_t)p->batch * chunks * 2 * p->h_kv * sizeof(uint32_t);
}

}  // namespace

extern "C" {

int gqa_abi_version(void) { return GQA_DECODE_ABI_VERSION; }

const char* gqa_last_error(void) { return g_last_error.c_str(); }

const char* gqa_status_string(gqa_status s) {
  switch (s) {
    case GQA_OK: return "GQA_OK";
    case GQA_ERR_INVALID_ARG: return "GQA_ERR_INVALID_ARG";
    case GQA_ERR_UNSUPPORTED: return "GQA_ERR_UNSUPPORTED";
    case GQA_ERR_ALIGNMENT: return "GQA_ERR_ALIGNMENT";
    case GQA_ERR_WORKSPACE: return "GQA_ERR_WORKSPACE";
    case GQA_ERR_HIP: return "GQA_ERR_HIP";
  }
  return "GQA_ERR_UNKNOWN";
}

gqa_status gqa_decode_make_plan(const gqa_decode_params* p, gqa_decode_plan* plan) {
  g_last_error.clear();
  if (!plan) return fail(GQA_ERR_INVALID_ARG, "plan is NULL");
  return make_plan(p, plan);
}

gqa_status gqa_decode_workspace_size(const gqa_decode_params* p, size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(GQA_ERR_INVALID_ARG, "bytes is NULL");
  gqa_decode_plan plan;
  gqa_status st = make_plan(p, &plan);
  if (st != GQA_OK) return st;
  *bytes = plan.workspace_bytes;
  return GQA_OK;
}

gqa_status gqa_decode_run(const gqa_decode_params* p, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* seqlens, const int32_t* cu_seqlens,
                          const int32_t* block_table, const int32_t* topk_idx, const float* k_scale,
                          const float* v_scale, const void* gate, void* o, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  gqa_decode_plan plan;
  gqa_status st = make_plan(p, &plan);
  if (st != GQA_OK) return st;
  if (!q || !k_cache || !v_cache || !o || !lse) return fail(GQA_ERR_INVALID_ARG, "q, k_cache, v_cache, o and lse are required");
  if (p->layout == GQA_LAYOUT_RAGGED) {
    if (!cu_seqlens) return fail(GQA_ERR_INVALID_ARG, "ragged layout needs cu_seqlens");
  } else if (!seqlens) {
    return fail(GQA_ERR_INVALID_ARG, "seqlens is required for contiguous and paged layouts");
  }
  if (p->layout == GQA_LAYOUT_PAGED && !block_table) return fail(GQA_ERR_INVALID_ARG, "paged layout needs block_table");
  if (p->topk > 0 && !topk_idx) return fail(GQA_ERR_INVALID_ARG, "topk > 0 needs topk_idx");
  if (one_byte(p) && (!k_scale || !v_scale))
    return fail(GQA_ERR_INVALID_ARG, "FP8 K/V need k_scale and v_scale");
  if (p->gate_mode != GQA_GATE_NONE && !gate) return fail(GQA_ERR_INVALID_ARG, "gate_mode set but gate is NULL");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
      (p->gate_mode == GQA_GATE_ELEMENTWISE && !aligned(gate, 16)))
    return fail(GQA_ERR_ALIGNMENT, "q, k_cache, v_cache, o and an elementwise gate must be 16-byte aligned");
  const void* small[] = {seqlens, cu_seqlens, block_table, topk_idx, k_scale, v_scale, lse, gate};
  for (const void* ptr : small)
    if (ptr && !aligned(ptr, 4)) return fail(GQA_ERR_ALIGNMENT, "index, scale, gate and lse arrays must be 4-byte aligned");
  if (plan.workspace_bytes > 0) {
    if (!workspace || workspace_bytes < plan.workspace_bytes)
      return fail(GQA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", plan.workspace_bytes,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 16)) return fail(GQA_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
  }
  if (p->batch == 0) return GQA_OK;

  gqa::DecodeArgs a;
  fill_args(a, p, plan);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint8_t*>(k_cache);
  a.v = static_cast<const uint8_t*>(v_cache);
  a.seqlens = seqlens;
  a.cu_seqlens = cu_seqlens;
  a.block_table = block_table;
  a.topk = topk_idx;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.gate = static_cast<const uint16_t*>(gate);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  if (plan.workspace_bytes > 0) {
    a.o_part = static_cast<float*>(workspace);
    a.lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + (size_t)round_up_256(partial_o_bytes(p, plan)));
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool indirect = p->layout == GQA_LAYOUT_PAGED || p->topk > 0;
  const int mode = a.packed ? 2 : (indirect ? 1 : 0);
  // Packed chunks span requests: one grid row covers the whole batch.
  const Tiling tl = plan_tiling(p, plan.rows, plan.math);
  const dim3 grid(plan.num_splits, (p->h_kv / tl.hpw) * tl.row_groups, a.packed ? 1 : p->batch);
  const bool valu = plan.math == GQA_MATH_VALU;
  hipError_t e = gqa::launch_partial(a, p->head_dim, p->kv_dtype, mode, valu ? 1 : tl.mb,
                                     valu ? plan.row_blocks : 0, tl.share, grid, s,
                                     static_cast<hipEvent_t>(p->partial_event_begin),
                                     static_cast<hipEvent_t>(p->partial_event_end));
  if (e != hipSuccess) return hip_fail(e, "partial kernel launch");
  if (plan.combine) {
    const int64_t xblocks = cdiv(plan.rows, a.comb_rows) * a.comb_cols;
    e = gqa::launch_combine(a, p->head_dim, dim3((unsigned)xblocks, p->h_kv, p->batch), s);
    if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
  }
  return GQA_OK;
}

gqa_status gqa_decode_run_noalloc(const gqa_decode_params* p, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* seqlens, const int32_t* cu_seqlens,
                                  const int32_t* block_table, const int32_t* topk_idx, const float* k_scale,
                                  const float* v_scale, const void* gate, void* o, float* lse, void* stream) {
  g_last_error.clear();
  gqa_decode_plan plan;
  gqa_status st = make_plan(p, &plan);
  if (st != GQA_OK) return st;
  if (plan.workspace_bytes > GQA_NOALLOC_SCRATCH_BYTES)
    return fail(GQA_ERR_WORKSPACE, "this call needs %zu bytes of split partials; the no-allocation entry point "
                "holds %zu (use gqa_decode_run with a workspace)", plan.workspace_bytes,
                (size_t)GQA_NOALLOC_SCRATCH_BYTES);
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  if (plan.workspace_bytes > 0) {
    const hipError_t e = gqa::scratch_address(&scratch, &scratch_bytes);
    if (e != hipSuccess) return hip_fail(e, "scratch array address");
  }
  // The same checks and launches as a call with a caller workspace.
  return gqa_decode_run(p, q, k_cache, v_cache, seqlens, cu_seqlens, block_table, topk_idx, k_scale, v_scale, gate,
                        o, lse, scratch, scratch_bytes, stream);
}

gqa_status gqa_resolve_rows(const gqa_decode_params* p, const int32_t* seqlens, const int32_t* cu_seqlens,
                            const int32_t* block_table, const int32_t* topk_idx, int64_t* rows_out,
                            void* stream) {
  g_last_error.clear();
  gqa_status st = check_shape(p);
  if (st != GQA_OK) return st;
  if (!rows_out) return fail(GQA_ERR_INVALID_ARG, "rows_out is NULL");
  if (p->layout == GQA_LAYOUT_RAGGED ? !cu_seqlens : !seqlens)
    return fail(GQA_ERR_INVALID_ARG, "lengths are required (seqlens, or cu_seqlens for ragged)");
  if (p->layout == GQA_LAYOUT_PAGED && !block_table) return fail(GQA_ERR_INVALID_ARG, "paged layout needs block_table");
  if (p->topk > 0 && !topk_idx) return fail(GQA_ERR_INVALID_ARG, "topk > 0 needs topk_idx");
  if (!aligned(rows_out, 8)) return fail(GQA_ERR_ALIGNMENT, "rows_out must be 8-byte aligned");
  const int list_cap = p->topk > 0 ? p->topk : p->max_seqlen_kv;
  if (p->batch == 0 || list_cap == 0) return GQA_OK;
  gqa_decode_plan plan;
  st = make_plan(p, &plan);
  if (st != GQA_OK) return st;
  gqa::DecodeArgs a;
  fill_args(a, p, plan);
  a.seqlens = seqlens;
  a.cu_seqlens = cu_seqlens;
  a.block_table = block_table;
  a.topk = topk_idx;
  hipError_t e = gqa::launch_resolve(a, rows_out, list_cap, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "resolve kernel launch");
  return GQA_OK;
}

gqa_status gqa_kv_append_workspace_size(const gqa_append_params* p, size_t* bytes) {
  g_last_error.clear();
  gqa_status st = check_append(p);
  if (st != GQA_OK) return st;
  if (!bytes) return fail(GQA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = append_workspace(p);
  return GQA_OK;
}

gqa_status gqa_kv_append(const gqa_append_params* p, const void* k_new, const void* v_new,
                         const int32_t* seqlens, int32_t* seqlens_out, const int32_t* block_table,
                         void* k_cache, void* v_cache, float* k_scale, float* v_scale, void* workspace,
                         size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  gqa_status st = check_append(p);
  if (st != GQA_OK) return st;
  if (!k_new || !v_new || !seqlens || !k_cache || !v_cache)
    return fail(GQA_ERR_INVALID_ARG, "k_new, v_new, seqlens, k_cache and v_cache are required");
  if (seqlens_out && seqlens_out == seqlens)
    return fail(GQA_ERR_INVALID_ARG, "seqlens_out must not alias seqlens");
  if (p->layout == GQA_LAYOUT_PAGED && !block_table) return fail(GQA_ERR_INVALID_ARG, "paged layout needs block_table");
  const bool fp8 = p->kv_dtype != GQA_KV_BF16;  // one-byte codes with scales
  if (fp8 && (!k_scale || !v_scale)) return fail(GQA_ERR_INVALID_ARG, "FP8 and int8 caches need k_scale and v_scale");
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(GQA_ERR_ALIGNMENT, "k_new, v_new, k_cache and v_cache must be 16-byte aligned");
  const void* small[] = {seqlens, seqlens_out, block_table, k_scale, v_scale};
  for (const void* ptr : small)
    if (ptr && !aligned(ptr, 4)) return fail(GQA_ERR_ALIGNMENT, "length, block-table and scale arrays must be 4-byte aligned");
  const size_t need = append_workspace(p);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(GQA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 4)) return fail(GQA_ERR_ALIGNMENT, "workspace must be 4-byte aligned");
  }
  if (p->batch == 0) return GQA_OK;

  gqa::AppendArgs a;
  std::memset(&a, 0, sizeof a);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.seqlens = seqlens;
  a.seqlens_out = seqlens_out;
  a.block_table = block_table;
  a.k_cache = static_cast<uint8_t*>(k_cache);
  a.v_cache = static_cast<uint8_t*>(v_cache);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.amax = static_cast<uint32_t*>(workspace);
  a.kv_rows = p->kv_rows;
  a.batch = p->batch;
  a.s_new = p->s_new;
  a.h_kv = p->h_kv;
  a.head_dim = p->head_dim;
  a.paged = p->layout == GQA_LAYOUT_PAGED;
  a.fp8 = fp8;
  a.int8 = p->kv_dtype == GQA_KV_INT8;
  a.first_block = p->scale_policy == GQA_SCALE_FIRST_BLOCK;
  a.seq_cap = p->seq_capacity;
  a.page_shift = a.paged ? log2_exact(p->page_size) : 0;
  a.max_pages = p->max_pages_per_seq;
  a.chunk_tokens = append_chunk_tokens(p);
  a.chunks = (int32_t)cdiv(p->s_new, a.chunk_tokens);
  hipError_t e = gqa::launch_append(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append kernel launch");
  return GQA_OK;
}

}  // extern "C"
