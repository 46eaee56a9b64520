// Device-side building blocks shared by the decode kernels: argument block,
// address policies (contiguous / ragged / paged / top-K), wave64 reductions,
// bf16 and FP8 E4M3FN unpacking, and the MFMA wrapper.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kLayoutContiguous = 0;
constexpr int kLayoutRagged = 1;
constexpr int kLayoutPaged = 2;
constexpr int kGateNone = 0;
constexpr int kGateElementwise = 1;
constexpr int kGateHeadwise = 2;

constexpr int kThreads = 256;   // 4 wave64s per workgroup (combine, resolve)
constexpr int kWaves = 4;
constexpr int kTile = 32;       // list positions per wave iteration

// Waves per split-KV partial workgroup (a build-time tuning constant).
#ifndef GQA_PARTIAL_WAVES
#define GQA_PARTIAL_WAVES 4
#endif
constexpr int kPWaves = GQA_PARTIAL_WAVES;

// Resident partial workgroups per CU that a kernel variant's register
// budget is built for (its launch bounds), and that the planner sizes the
// grid for.  Two for one 16-row block of one-byte tiles at d <= 128 or of
// d = 64 tiles (one-byte d = 256 tiles do not fit half the file), for the
// four-wave row-sharing variants with one block per wave at d <= 128, and
// for the eight-wave ones with one block per wave at d = 64 (four waves per
// SIMD in 128 VGPRs each; at d = 128 and 256 those spill); one (the whole
// register file, or half of it for eight waves) otherwise: for bf16
// d = 128 with the waves splitting the tiles, whose
// two register buffers of whole-row loads alone take 128 VGPRs -- squeezed
// into half the file it spills, and every spill reload waits for all loads
// in flight.  The VALU variant keeps RV x (8 or 16) fp32 accumulators and
// every score of a tile per lane, and also takes the whole file.
__host__ __device__ constexpr int partial_wgs_per_cu(int D, bool fp8, int mb, int rv, int share) {
  return (rv == 0 && mb == 1 &&
          ((share == 1 && ((fp8 && D <= 128) || D == 64)) || (share == 4 && D <= 128) || (share == 8 && D == 64)))
             ? 2
             : 1;
}
constexpr int kPThreads = 64 * kPWaves;
// The eight-wave, eight-head variant (one 16-row block per wave, the waves
// splitting the tiles) exists where such a wave fits half the register
// file: one-byte tiles at d <= 128 and bf16 tiles at d = 64.
__host__ __device__ constexpr bool wide_fits(int D, bool fp8) { return (fp8 && D <= 128) || D == 64; }
// Two 16-row MFMA blocks of bf16 d = 256 per wave (the waves splitting the
// tiles) keep Q's operands in LDS, 16 KiB for the workgroup's one KV head.
__host__ __device__ constexpr bool q_in_lds(int D, bool fp8, int mb, int rv, int share) {
  return D == 256 && !fp8 && mb == 2 && rv == 0 && share == 1;
}
__host__ __device__ constexpr size_t q_lds_bytes(int D, int mb) { return (size_t)mb * (D / 32) * 64 * 16; }

// Shared memory of the partial kernel: per wave a K tile (raw 16-byte
// chunks) and a V tile (bf16), statically allocated; after the tile loop
// the same space holds the waves' fp32 accumulators.  The dynamic part
// holds the resolved row table of paged / top-K chunks.
__host__ __device__ constexpr int ktile_chunks(int D, bool fp8) { return kTile * D * (fp8 ? 1 : 2) / 16; }
__host__ __device__ constexpr int vtile_elems(int D) { return kTile * D; }
__host__ __device__ constexpr int wave_tile_bytes(int D, bool fp8) { return ktile_chunks(D, fp8) * 16 + vtile_elems(D) * 2; }
// Paged top-K lists also copy the request's block-table row, when it has at
// most kBtCache pages, to LDS beside the row table (4 KiB).
constexpr int kBtCache = 1024;
__host__ __device__ constexpr size_t table_bytes(bool indirect, int chunk) {
  return indirect ? (size_t)chunk * 8 + (size_t)kBtCache * 4 : 0;
}
// LDS bytes of one partial workgroup of `waves` waves: the tiles, the merge
// statistics, Q (when it is kept in LDS, `q_bytes`) and the row table.
__host__ __device__ constexpr size_t partial_lds_bytes(int D, bool fp8, bool indirect, int chunk, int waves = kPWaves,
                                                       size_t q_bytes = 0) {
  return (size_t)waves * wave_tile_bytes(D, fp8) + 2 * waves * 16 * 4 + q_bytes + table_bytes(indirect, chunk);
}

// Everything a kernel needs, passed by value (kernarg segment).
struct DecodeArgs {
  const uint16_t* q;          // bf16 [B, S_q, H_q, D]
  const uint8_t* k;           // cache bytes (bf16 or fp8)
  const uint8_t* v;
  const int32_t* seqlens;     // [B]
  const int32_t* cu_seqlens;  // [B+1]
  const int32_t* block_table; // [B, max_pages]
  const int32_t* topk;        // [B, topk_len]
  const float* k_scale;       // [B, H_kv]
  const float* v_scale;
  const uint16_t* gate;       // bf16
  uint16_t* o;                // bf16 [B, S_q, H_q, D]
  float* lse;                 // fp32 [B, H_q, S_q]
  float* o_part;              // fp32 partial rows x D (row index below)
  float* lse_part;            // fp32 partial rows, base-2
  // Partial row of (request b, KV head g, split s, query row r):
  // b * part_sb + g * part_sg + s * part_ss + r.
  int64_t part_sb, part_sg, part_ss;
  int64_t kv_rows;
  int32_t batch, s_q, h_q, h_kv, group, rows;
  int32_t layout, causal, max_seqlen, seq_cap;
  int32_t page_shift, max_pages, topk_len, gate_mode;
  int32_t chunk, num_splits;
  int32_t heads_per_wg;       // KV heads one partial workgroup covers (1, 2, 4 or 8)
  int32_t packed;             // 1: ragged cache split into equal row chunks (split s = chunk s)
  int32_t comb_cols, comb_rows;  // combine: column slices per row, rows per workgroup
  int32_t xcd_rows;           // row groups whose workgroups share a chunk on one XCD (1: none)
  float scale_log2;           // softmax scale * log2(e)
};

// XCDs of MI355X; the dispatcher deals a grid's workgroups to them in turn
// (workgroup i to XCD i mod 8).
constexpr int kXcds = 8;

// ---------------------------------------------------------------------------
// Address policy.  A request's list has L entries: its n tokens (dense) or
// its top-K positions.  Slot p names logical token t; t names a physical
// token row of the cache.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int seq_len(const DecodeArgs& a, int b) {
  int n = (a.layout == kLayoutRagged) ? (a.cu_seqlens[b + 1] - a.cu_seqlens[b]) : a.seqlens[b];
  return max(0, min(n, a.max_seqlen));
}

__device__ __forceinline__ int list_len(const DecodeArgs& a, int n) {
  return a.topk_len > 0 ? a.topk_len : n;
}

// First token row of request b for the non-paged layouts.
__device__ __forceinline__ int64_t row_base(const DecodeArgs& a, int b) {
  if (a.layout == kLayoutContiguous) return (int64_t)b * a.seq_cap;
  if (a.layout == kLayoutRagged) return (int64_t)a.cu_seqlens[b];
  return 0;
}

// Logical token of list slot p (p < L), or -1 if the slot is masked.
__device__ __forceinline__ int slot_token(const DecodeArgs& a, int b, int n, int p) {
  int t = (a.topk_len > 0) ? a.topk[(int64_t)b * a.topk_len + p] : p;
  return (t >= 0 && t < n) ? t : -1;
}

// Packed ragged cache: the request whose rows hold packed row x, i.e. the
// largest b < batch with cu_seqlens[b] <= x (0 if there is none), found by a
// 64-way search with one wave's lanes (one ballot per round, at most three
// rounds for 65535 requests).  Every lane gets the same result.  With
// offsets that decrease the result is some b in [0, batch).
__device__ __forceinline__ int packed_request(const DecodeArgs& a, int64_t x, int lane) {
  int lo = 0, hi = a.batch;
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) / 64;
    const int idx = lo + lane * step;
    const bool le = idx < hi && (int64_t)a.cu_seqlens[idx] <= x;
    const int cnt = __popcll(__ballot(le));
    lo += max(cnt - 1, 0) * step;
    hi = min(lo + step, hi);
  }
  return lo;
}

// Contiguous / ragged layouts: the same row as token_row, without the
// paged branch (a dependent load there would make the compiler drain all
// outstanding memory operations at every join).
__device__ __forceinline__ int64_t dense_row(const DecodeArgs& a, int t, int64_t base) {
  return min(max(base + t, (int64_t)0), a.kv_rows - 1);
}

// Physical token row of logical token t (0 <= t < n) of request b, clamped
// into the cache so that no offset can address memory outside it.
__device__ __forceinline__ int64_t token_row(const DecodeArgs& a, int b, int t, int64_t base) {
  int64_t row;
  if (a.layout == kLayoutPaged) {
    const int page = a.block_table[(int64_t)b * a.max_pages + (t >> a.page_shift)];
    row = ((int64_t)page << a.page_shift) + (t & ((1 << a.page_shift) - 1));
    return min(max(row, (int64_t)0), a.kv_rows - 1);
  }
  return dense_row(a, t, base);
}

// ---------------------------------------------------------------------------
// Wave64 helpers
// ---------------------------------------------------------------------------

// Cross-lane exchanges without LDS.  gfx950's row swaps: permlane16_swap
// of a value with itself returns {x[l], x[l ^ 16]} (in some order) in every
// lane, permlane32_swap {x[l], x[l ^ 32]}; combining the pair with a
// commutative op gives the same result in both partner lanes.
__device__ __forceinline__ float max_xor16(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Workgroup barrier that orders LDS only: the release/acquire fences are
// scoped to local memory, so the waves' HBM loads in flight stay in flight
// (a full __syncthreads waits for them too).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// DPP lane patterns within a row of 16 lanes: xor 1, xor 2 (quad perms),
// reverse within 8 (half mirror), reverse within 16 (mirror), rotate by 4
// and by 8.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
constexpr int kDppRor4 = 0x124, kDppRor8 = 0x128;
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_amdgcn_update_dpp(0.0f, x, CTRL, 0xF, 0xF, false);
}

// Max / sum with lane l ^ st, st = 8, 16 or 32 (row_ror:8 is l ^ 8 inside
// a row of 16 lanes).
__device__ __forceinline__ float max_lanes_xor(float x, int st) {
  if (st == 8) return fmaxf(x, dpp<0x128>(x));
  return st == 16 ? max_xor16(x) : max_xor32(x);
}
__device__ __forceinline__ float sum_lanes_xor(float x, int st) {
  if (st == 8) return x + dpp<0x128>(x);
  return st == 16 ? sum_xor16(x) : sum_xor32(x);
}

// Sum over the CPR lanes l ^ m (m < CPR; CPR = 4, 8 or 16 consecutive
// lanes), result in all of them.  Pairs are added in an order that
// commutativity makes identical in every lane.
template <int CPR>
__device__ __forceinline__ float sum_low_lanes(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  if constexpr (CPR >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (CPR >= 16) x += dpp<kDppMirror>(x);
  return x;
}

// Max / sum over the lanes that share l % CPR (the 64 / CPR lanes l + k CPR),
// result in all of them.
template <int CPR>
__device__ __forceinline__ float max_high_lanes(float x) {
  if constexpr (CPR <= 4) x = fmaxf(x, dpp<kDppRor4>(x));
  if constexpr (CPR <= 8) x = fmaxf(x, dpp<kDppRor8>(x));
  return max_xor32(max_xor16(x));
}
template <int CPR>
__device__ __forceinline__ float sum_high_lanes(float x) {
  if constexpr (CPR <= 4) x += dpp<kDppRor4>(x);
  if constexpr (CPR <= 8) x += dpp<kDppRor8>(x);
  return sum_xor32(sum_xor16(x));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xFFFF0000u); }

// Two floats -> packed bf16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Four FP8 E4M3FN codes (one dword, lowest byte first) -> four bf16 in two
// dwords.  Every E4M3FN value is exactly representable in bf16.
__device__ __forceinline__ void fp8x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

// Four int8 codes (one dword, lowest byte first) -> four bf16 in two dwords.
// Every int8 value is exactly representable in bf16: convert each
// sign-extended byte to fp32 (one v_cvt_f32_i32 with an SDWA byte select
// each) and keep the upper halves of the results (exact: at most 8
// significant bits, so the lower halves are zero).
__device__ __forceinline__ void int8x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const float f0 = (float)(int8_t)(w & 0xffu);
  const float f1 = (float)(int8_t)((w >> 8) & 0xffu);
  const float f2 = (float)(int8_t)((w >> 16) & 0xffu);
  const float f3 = (float)(int8_t)(w >> 24);
  // v_perm_b32: bytes 2,3 of the second operand, then bytes 2,3 of the first
  lo = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f1), __builtin_bit_cast(uint32_t, f0), 0x07060302u);
  hi = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f3), __builtin_bit_cast(uint32_t, f2), 0x07060302u);
}

// Stored K/V element types; one-byte codes carry a scale per (request, KV head).
constexpr int kKvBf16 = 0, kKvFp8 = 1, kKvInt8 = 2;

template <int KVT>
__device__ __forceinline__ void codes4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  static_assert(KVT == kKvFp8 || KVT == kKvInt8, "one-byte codes");
  if constexpr (KVT == kKvFp8)
    fp8x4_to_bf16x4(w, lo, hi);
  else
    int8x4_to_bf16x4(w, lo, hi);
}

// Two bf16 products plus c, accumulated in fp32 (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// D(16x16 fp32) += A(16x32 bf16) * B(32x16 bf16).  Lane l holds A row l%16,
// B column l%16, each for k = 8*(l/16) .. 8*(l/16)+7, and D rows
// 4*(l/16) .. 4*(l/16)+3 of column l%16.
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of
// 16 lanes, lane r's address names a row M[r] of four consecutive bf16; lane
// i receives M[4k + i/4][i%4] for k = 0..3 (packed two per dword).
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(const_cast<uint16_t*>(p)));
  return __builtin_bit_cast(uint2, v);
}

// sigmoid(x) = 1 / (1 + e^-x), with the hardware reciprocal (about 1 ulp
// of fp32): every use rounds the gated output to bf16 (8 significant bits).
__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

}  // namespace gqa
