// Host-only stand-ins for the kernel launchers of libgqa_decode, for a
// build of the C ABI (validation, planning, argument set-up) that links no
// GPU code, so that the host side can run under AddressSanitizer and
// UndefinedBehaviorSanitizer on a machine without a GPU.  Each stub checks
// on the host what the real kernel and its launch assume -- grid limits,
// LDS, chunk sizes, pointer presence -- and counts the launch; it enqueues
// nothing.  A violated assumption aborts with a message.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#include "gqa_append_args.h"
#include "gqa_device.h"

extern "C" long long gqa_stub_launches = 0;

namespace {
void need(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "launch stub: %s\n", what);
    std::abort();
  }
}
void grid_ok(dim3 g) {
  if (g.x >= 1 && g.y >= 1 && g.z >= 1 && g.x <= 0x7fffffffu && g.y <= 65535u && g.z <= 65535u) return;
  std::fprintf(stderr, "launch stub: grid (%u, %u, %u)\n", g.x, g.y, g.z);
  need(false, "empty grid, or one beyond the dispatch limits");
}
}  // namespace

namespace gqa {

hipError_t launch_partial(const DecodeArgs& a, int D, int kvt, int mode, int mb, int rv, int share, dim3 grid,
                          hipStream_t, hipEvent_t, hipEvent_t) {
  grid_ok(grid);
  need(D == 64 || D == 128 || D == 256, "head dim");
  need(kvt >= kKvBf16 && kvt <= kKvInt8 && mode >= 0 && mode <= 2, "variant");
  need(a.chunk >= 32 && a.chunk % 32 == 0, "chunk is a positive multiple of the 32-position tile");
  need(a.num_splits >= 1 && a.heads_per_wg >= 1 && a.h_kv % a.heads_per_wg == 0, "splits and head groups");
  need(rv == 0 || (D <= 128 && a.rows <= rv && share == 1), "VALU rows");
  need(share == 1 || share == 2 || share == 4 || share == 8, "row sharing width");
  need(mb >= 1 && mb <= 4, "row blocks per wave");
  need(rv > 0 || (long long)grid.y / (a.h_kv / a.heads_per_wg) * share * mb * 16 >= a.rows, "row groups cover the rows");
  need(a.heads_per_wg != 8 || (share == 1 && mb == 1 && rv == 0 && wide_fits(D, kvt != kKvBf16)),
       "eight heads per workgroup only for the one-block variants that fit two waves per SIMD");
  const int waves = a.heads_per_wg == 8 ? 8 : kPWaves;
  const bool qlds = q_in_lds(D, kvt != kKvBf16, mb, rv, share);
  need(!qlds || a.heads_per_wg == 1, "Q kept in LDS holds one KV head");
  need(partial_lds_bytes(D, kvt != kKvBf16, mode == 1, a.chunk, waves, qlds ? q_lds_bytes(D, mb) : 0) <= 160 * 1024,
       "LDS per workgroup");
  need(a.q && a.k && a.v && a.o && a.lse, "required pointers");
  need(mode != 1 || a.block_table || a.topk, "indirect mode without a table");
  need(a.num_splits == 1 && !a.packed ? true : (a.o_part && a.lse_part), "partials without a workspace");
  ++gqa_stub_launches;
  return hipSuccess;
}

hipError_t launch_combine(const DecodeArgs& a, int D, dim3 grid, hipStream_t) {
  grid_ok(grid);
  need(D == 64 || D == 128 || D == 256, "head dim");
  need(a.comb_cols >= 1 && a.comb_rows >= 1 && (D / 4 / a.comb_cols) * a.comb_rows <= kThreads, "combine shape");
  need(a.o_part && a.lse_part, "combine without partials");
  ++gqa_stub_launches;
  return hipSuccess;
}

hipError_t launch_resolve(const DecodeArgs&, int64_t* out, int list_cap, hipStream_t) {
  need(out != nullptr && list_cap >= 1, "resolve output");
  ++gqa_stub_launches;
  return hipSuccess;
}

// The no-allocation entry point's scratch array: a placeholder address
// (16-byte aligned, never dereferenced on the host).
hipError_t scratch_address(void** ptr, size_t* bytes) {
  *ptr = reinterpret_cast<void*>(static_cast<uintptr_t>(0x7f0000000000ull));
  *bytes = (size_t)32 << 20;
  return hipSuccess;
}

hipError_t launch_append(const AppendArgs& a, hipStream_t) {
  need(a.chunk_tokens >= 1 && a.chunk_tokens <= kAppendMaxChunkTokens, "append chunk tokens");
  need((long long)a.chunk_tokens * a.h_kv * a.head_dim <= kAppendElemsPerWorkgroup || a.chunk_tokens == 1,
       "append workgroup size");
  need(a.chunks >= 1 && (long long)a.chunks * a.chunk_tokens >= a.s_new, "append chunks cover the new rows");
  grid_ok(dim3((unsigned)a.chunks, (unsigned)a.batch, 1));
  need(!a.first_block || !a.fp8 || a.chunks == 1 || a.amax, "first-block maxima without a workspace");
  ++gqa_stub_launches;
  return hipSuccess;
}

}  // namespace gqa
