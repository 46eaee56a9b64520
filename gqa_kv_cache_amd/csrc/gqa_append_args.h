// Arguments of the K/V append kernels (host and device).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace gqa {

constexpr int kAppendThreads = 256;
constexpr int kAppendMaxHeads = 256;
// Elements (tokens x H_kv x d) one append workgroup covers at most, and the
// most tokens that can be (H_kv x d >= 64).
constexpr int kAppendElemsPerWorkgroup = 65536;
constexpr int kAppendMaxChunkTokens = kAppendElemsPerWorkgroup / 64;

struct AppendArgs {
  const uint16_t* k_new;  // bf16 [B, S_new, H_kv, d]
  const uint16_t* v_new;
  const int32_t* seqlens;  // [B] n_b before the call
  int32_t* seqlens_out;    // [B] or null
  const int32_t* block_table;
  uint8_t* k_cache;  // token rows [kv_rows, H_kv, d] of 1 (FP8, int8) or 2 (bf16) bytes
  uint8_t* v_cache;
  float* k_scale;  // [B, H_kv]
  float* v_scale;
  uint32_t* amax;  // workspace [B, chunks, H_kv, 2]: fp32 bits of per-workgroup maxima
  int64_t kv_rows;
  int32_t batch, s_new, h_kv, head_dim;
  int32_t paged, fp8, first_block;  // fp8: one-byte codes with scales (FP8 E4M3FN, or int8 when int8)
  int32_t int8;
  int32_t seq_cap, page_shift, max_pages;
  int32_t chunk_tokens, chunks;
  // Set by the launcher: 1 = this launch takes the maxima (else it
  // writes); 1 = requests in reverse order.
  int32_t maxima, reverse;
};

hipError_t launch_append(const AppendArgs& a, hipStream_t st);

}  // namespace gqa
