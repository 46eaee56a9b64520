// K/V append with FP8 E4M3FN or int8 quantisation on write (gfx950).
//
// Writes the S_new bf16 K and V rows of each request at logical positions
// n_b .. n_b + S_new - 1 of a contiguous or paged cache, as bf16 or as FP8
// E4M3FN or int8 codes under one scale per (request, KV head) -- the
// storage the decode kernels read ("Sparse paged GQA decode attention with
// FP8 KV cache on SM89", "Workload" and "Implementations"; the int8
// KV-cache section of "Profiling down to the register, then an extension
// that broke my assumptions twice").  Only the appended rows are touched.
//
// Work split: a workgroup takes `chunk_tokens` consecutive new tokens of one
// request, all KV heads (a token's H_kv * d elements are contiguous in both
// the input and the cache row).  A thread handles 8 elements at a time: one
// 16-byte bf16 load, and an 8-byte (FP8) or 16-byte (bf16) store, with 8
// such loads of K and of V in flight per round.  HBM-bound: 2 bytes read and
// 1 (FP8) or 2 (bf16) written per element.  The quantiser's VALU work
// (quotient, clamp, convert) was measured to matter: with a full IEEE
// division per element the prefill-sized append ran at 3.8 TB/s, with the
// corrected reciprocal and the hardware convert at 4.8 TB/s, against 5.2
// TB/s for a plain device-to-device copy of the same bytes.
//
// First-block scales: a request with n_b == 0 takes scale = absmax / 448
// (FP8) or absmax / 127 (int8) per KV head over its appended rows.  One
// workgroup per request reduces its rows in LDS; requests whose rows span
// several workgroups take a maxima launch first (see the kernel below).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gqa_append_args.h"

namespace gqa {

namespace {

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __builtin_bit_cast(float, bits16 << 16); }

__device__ __forceinline__ float absmax8(const uint4 x) {
  float m = 0.f;
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    m = fmaxf(m, __builtin_fabsf(bf16_to_f32(w[c] & 0xffffu)));
    m = fmaxf(m, __builtin_fabsf(bf16_to_f32(w[c] >> 16)));
  }
  return m;
}

// The IEEE fp32 quotient x / s, from y = the correctly rounded 1/s: with
// q0 = RN(x y) and the exact residual e = x - s q0 (one FMA), RN(q0 + e y)
// is the correctly rounded x / s (Markstein's theorem; it needs no
// overflow or underflow on the way).  A q0 beyond +-448 saturates below
// whatever the exact quotient is (it lies within an ulp of q0), and a
// tiny q0 encodes as a signed zero either way, so only those two ends
// skip the correction.  Heads whose 1/s overflows (a subnormal scale)
// take the full division.
__device__ __forceinline__ float quotient(float x, float s, float y, bool exact) {
  if (exact) return x / s;
  const float q0 = x * y;
  if (!(__builtin_fabsf(q0) <= 448.f) || __builtin_fabsf(q0) < 1e-30f) return q0;
  return __builtin_fmaf(__builtin_fmaf(-q0, s, x), y, q0);
}

// gfx950's v_cvt_pk_fp8_f32 rounds two fp32 values to OCP E4M3FN codes
// (nearest even, the mode register's default; the sign of a value that
// rounds to zero is kept) and packs them into one half of a dword; the
// values are clamped to +-448 first.  Checked against the format's
// definition for every finite bf16 value under 8192 scales.
__device__ __forceinline__ uint2 quantize8(const uint4 x, float s, float y, bool exact) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  float q[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    q[2 * i] = fminf(fmaxf(quotient(bf16_to_f32(w[i] & 0xffffu), s, y, exact), -448.f), 448.f);
    q[2 * i + 1] = fminf(fmaxf(quotient(bf16_to_f32(w[i] >> 16), s, y, exact), -448.f), 448.f);
  }
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], hi, true);
  return uint2{(uint32_t)lo, (uint32_t)hi};
}

// Int8 codes of eight bf16 values: the same fp32 quotient, rounded to the
// nearest integer with ties to even (v_rndne_f32), clamped to +-127, packed
// as two's-complement bytes (lowest element in the lowest byte).  Clamping
// before rounding gives the same code: +-127 are integers.
__device__ __forceinline__ uint2 quantize_i8(const uint4 x, float s, float y, bool exact) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t b[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float q0 = fminf(fmaxf(quotient(bf16_to_f32(w[i] & 0xffffu), s, y, exact), -127.f), 127.f);
    const float q1 = fminf(fmaxf(quotient(bf16_to_f32(w[i] >> 16), s, y, exact), -127.f), 127.f);
    b[2 * i] = (uint32_t)(int)__builtin_rintf(q0) & 0xffu;
    b[2 * i + 1] = (uint32_t)(int)__builtin_rintf(q1) & 0xffu;
  }
  return uint2{b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24), b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24)};
}

// Absolute maxima of this workgroup's T new tokens, per KV head, into smax
// (fp32 bits; zeroed by the caller, then a barrier).
//
// When a token row's 8-element items (H_kv * d / 8 of them) divide the
// workgroup's threads, the workgroup reads whole rows, contiguously: thread
// t always meets item t % (items per row), so it always sees the same head
// and keeps one maximum per tensor.  Lanes of one head then reduce with
// cross-lane swaps (within the head's items, and across the rows a wave
// covers), and one lane per head and wave does an LDS atomic.  Otherwise one
// head at a time: each thread keeps its own maximum over its items, then a
// wave reduction and one LDS atomic per wave.  U loads of K and of V are in
// flight per thread either way.
template <int U>
__device__ __forceinline__ void block_absmax(const AppendArgs& a, int64_t in_base, int T, uint32_t* smax) {
  const int d8 = a.head_dim / 8;
  const int rc = a.h_kv * d8;  // items per token row
  if (kAppendThreads % rc == 0) {
    const int total = T * rc;
    float mk = 0.f, mv = 0.f;
    for (int base = 0; base < total; base += U * kAppendThreads) {
      uint4 kx[U], vx[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        int it = base + u * kAppendThreads + (int)threadIdx.x;
        if (it >= total) it = it % rc;  // the same item of row 0: the same head, harmless for a maximum
        kx[u] = *reinterpret_cast<const uint4*>(a.k_new + in_base + (int64_t)it * 8);
        vx[u] = *reinterpret_cast<const uint4*>(a.v_new + in_base + (int64_t)it * 8);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        mk = fmaxf(mk, absmax8(kx[u]));
        mv = fmaxf(mv, absmax8(vx[u]));
      }
    }
    const int lane = threadIdx.x & 63;
    for (int off = 1; off < d8; off <<= 1) {  // the head's items in a row
      mk = fmaxf(mk, __shfl_xor(mk, off));
      mv = fmaxf(mv, __shfl_xor(mv, off));
    }
    for (int off = rc; off < 64; off <<= 1) {  // the rows one wave covers
      mk = fmaxf(mk, __shfl_xor(mk, off));
      mv = fmaxf(mv, __shfl_xor(mv, off));
    }
    if (lane % d8 == 0 && lane < rc) {
      const int g = ((int)threadIdx.x % rc) / d8;
      atomicMax(&smax[2 * g], __builtin_bit_cast(uint32_t, mk));  // |x| >= 0: integer order = float order
      atomicMax(&smax[2 * g + 1], __builtin_bit_cast(uint32_t, mv));
    }
    return;
  }
  const int per_head = T * d8;
  for (int g = 0; g < a.h_kv; ++g) {
    float mk = 0.f, mv = 0.f;
    for (int base = 0; base < per_head; base += U * kAppendThreads) {
      uint4 kx[U], vx[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int it = min(base + u * kAppendThreads + (int)threadIdx.x, per_head - 1);
        const int j = it / d8;
        const int64_t off = in_base + ((int64_t)j * a.h_kv + g) * a.head_dim + (it - j * d8) * 8;
        kx[u] = *reinterpret_cast<const uint4*>(a.k_new + off);
        vx[u] = *reinterpret_cast<const uint4*>(a.v_new + off);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        mk = fmaxf(mk, absmax8(kx[u]));  // a clamped index repeats a valid item: harmless for a maximum
        mv = fmaxf(mv, absmax8(vx[u]));
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      mk = fmaxf(mk, __shfl_xor(mk, off));
      mv = fmaxf(mv, __shfl_xor(mv, off));
    }
    if ((threadIdx.x & 63) == 0) {
      atomicMax(&smax[2 * g], __builtin_bit_cast(uint32_t, mk));  // |x| >= 0: integer order = float order
      atomicMax(&smax[2 * g + 1], __builtin_bit_cast(uint32_t, mv));
    }
  }
}

// Physical token row of logical token t of request b, or -1 (not written).
__device__ __forceinline__ int64_t append_row(const AppendArgs& a, int b, int64_t t) {
  if (t < 0) return -1;
  int64_t row;
  if (a.paged) {
    const int64_t page = t >> a.page_shift;
    if (page >= a.max_pages) return -1;
    row = (int64_t)a.block_table[(int64_t)b * a.max_pages + page] * (1 << a.page_shift) +
          (t & ((1 << a.page_shift) - 1));
  } else {
    if (t >= a.seq_cap) return -1;
    row = (int64_t)b * a.seq_cap + t;
  }
  return (row >= 0 && row < a.kv_rows) ? row : -1;
}

}  // namespace

// Maxima of one workgroup's rows (c-th chunk of request b) into the
// workspace: fp32 bits of |x|, K and V per head.
__device__ __forceinline__ void chunk_maxima(const AppendArgs& a, int b, int c, uint32_t* smax) {
  constexpr int U = 8;
  const int t0 = c * a.chunk_tokens;
  const int T = min(a.chunk_tokens, a.s_new - t0);
  const int64_t in_base = ((int64_t)b * a.s_new + t0) * a.h_kv * a.head_dim;
  for (int i = threadIdx.x; i < 2 * a.h_kv; i += kAppendThreads) smax[i] = 0u;
  __syncthreads();
  block_absmax<U>(a, in_base, T, smax);
  __syncthreads();
  for (int i = threadIdx.x; i < 2 * a.h_kv; i += kAppendThreads)
    a.amax[((int64_t)b * a.chunks + c) * 2 * a.h_kv + i] = smax[i];
}

// The c-th chunk's writes of request b.  scales: 0 = the given ones (or none
// for bf16), 1 = this workgroup's own maxima (the request fits one
// workgroup), 2 = the request's per-workgroup maxima in the workspace.
__device__ __forceinline__ void chunk_writes(const AppendArgs& a, int b, int c, int n, int scales, uint32_t* smax,
                                             float* sscale, float* sinv, int64_t* srow) {
  constexpr int U = 8;  // 8-element items per thread in flight per round (K and V each)
  const int d8 = a.head_dim / 8;
  const int per_tok = a.h_kv * d8;  // 8-element items per token row
  const float qmax = a.int8 ? 127.f : 448.f;  // largest code magnitude
  const int t0 = c * a.chunk_tokens;
  const int T = min(a.chunk_tokens, a.s_new - t0);
  const int items = T * per_tok;
  const int64_t in_base = ((int64_t)b * a.s_new + t0) * a.h_kv * a.head_dim;

  if (scales == 1) {
    for (int i = threadIdx.x; i < 2 * a.h_kv; i += kAppendThreads) smax[i] = 0u;
    __syncthreads();
    block_absmax<U>(a, in_base, T, smax);
  } else if (scales == 2) {
    // The request's per-workgroup maxima: each thread takes the running
    // maximum of one (tensor, head) slot over every L-th workgroup in
    // registers, then one LDS atomic (an atomic per value made all 256
    // threads queue on the 2 H_kv slots).
    for (int i = threadIdx.x; i < 2 * a.h_kv; i += kAppendThreads) smax[i] = 0u;
    __syncthreads();
    const int S2 = 2 * a.h_kv;
    const int L = max(1, kAppendThreads / S2);
    const uint32_t* am = a.amax + (int64_t)b * a.chunks * S2;
    for (int idx = threadIdx.x; idx < S2 * L; idx += kAppendThreads) {
      const int slot = idx % S2;
      uint32_t m = 0u;
      for (int cc = idx / S2; cc < a.chunks; cc += L) m = max(m, am[(int64_t)cc * S2 + slot]);
      atomicMax(&smax[slot], m);
    }
  }
  __syncthreads();
  if (scales != 0) {
    for (int i = threadIdx.x; i < 2 * a.h_kv; i += kAppendThreads) {
      const float amax = __builtin_bit_cast(float, smax[i]);
      const float s = amax > 0.f ? amax / qmax : 1.f;
      sscale[i] = s;
      if (c == 0) ((i & 1) ? a.v_scale : a.k_scale)[(int64_t)b * a.h_kv + (i >> 1)] = s;
    }
  } else if (a.fp8) {
    for (int i = threadIdx.x; i < 2 * a.h_kv; i += kAppendThreads)
      sscale[i] = ((i & 1) ? a.v_scale : a.k_scale)[(int64_t)b * a.h_kv + (i >> 1)];
  }
  __syncthreads();
  if (a.fp8)
    for (int i = threadIdx.x; i < 2 * a.h_kv; i += kAppendThreads) sinv[i] = 1.0f / sscale[i];
  for (int j = threadIdx.x; j < T; j += kAppendThreads) srow[j] = append_row(a, b, (int64_t)n + t0 + j);
  __syncthreads();

  // Writes: each round issues U loads of K and of V per thread before any
  // conversion, so that 16 loads per thread are in flight.
  const int64_t esz = a.fp8 ? 1 : 2;
  for (int base = 0; base < items; base += U * kAppendThreads) {
    uint4 kx[U], vx[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = base + u * kAppendThreads + threadIdx.x;
      const int64_t src = in_base + (int64_t)min(it, items - 1) * 8;
      kx[u] = *reinterpret_cast<const uint4*>(a.k_new + src);
      vx[u] = *reinterpret_cast<const uint4*>(a.v_new + src);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = base + u * kAppendThreads + threadIdx.x;
      if (it >= items) break;
      const int j = it / per_tok;
      const int r = it - j * per_tok;  // item within the token row: head r / d8, elements 8 (r % d8) ..
      const int64_t row = srow[j];
      if (row < 0) continue;
      const int64_t dst = (row * a.h_kv * a.head_dim + (int64_t)r * 8) * esz;
      if (a.fp8) {
        const int g = r / d8;
        const float sk = sscale[2 * g], sv = sscale[2 * g + 1];
        const float yk = sinv[2 * g], yv = sinv[2 * g + 1];
        if (a.int8) {
          *reinterpret_cast<uint2*>(a.k_cache + dst) = quantize_i8(kx[u], sk, yk, !(yk < INFINITY));
          *reinterpret_cast<uint2*>(a.v_cache + dst) = quantize_i8(vx[u], sv, yv, !(yv < INFINITY));
        } else {
          *reinterpret_cast<uint2*>(a.k_cache + dst) = quantize8(kx[u], sk, yk, !(yk < INFINITY));
          *reinterpret_cast<uint2*>(a.v_cache + dst) = quantize8(vx[u], sv, yv, !(yv < INFINITY));
        }
      } else {
        *reinterpret_cast<uint4*>(a.k_cache + dst) = kx[u];
        *reinterpret_cast<uint4*>(a.v_cache + dst) = vx[u];
      }
    }
  }
  if (c == 0 && threadIdx.x == 0 && a.seqlens_out) a.seqlens_out[b] = n + a.s_new;
}

// One kernel for every append, in one of two roles: the maxima of a chunk
// of a first-block request (into the workspace), or a chunk's writes.
// Workgroup (c, y) takes chunk c of request y (maxima, or writes in request
// order) or of request batch - 1 - y (writes after a maxima launch).
// Without first-block requests spread over several workgroups one launch
// writes everything.  With them, a first launch takes the maxima and a
// second writes; each writing workgroup of such a request reduces the
// request's per-workgroup maxima itself (no separate reduction launch), and
// the writes take the requests last to first, so that the first re-read
// rows are the ones the maxima launch read last, when the on-package cache
// may still hold them.  No atomics in HBM, no zero-initialised memory.
__global__ void __launch_bounds__(kAppendThreads) gqa_append_kernel(AppendArgs a) {
  __shared__ uint32_t smax[2 * kAppendMaxHeads];  // fp32 bits of |x| maxima (K, V per head)
  __shared__ float sscale[2 * kAppendMaxHeads];
  __shared__ float sinv[2 * kAppendMaxHeads];      // correctly rounded 1 / scale
  __shared__ int64_t srow[kAppendMaxChunkTokens];  // physical row of each new token (-1: not written)
  const int c = blockIdx.x;
  const int b = a.reverse ? a.batch - 1 - (int)blockIdx.y : (int)blockIdx.y;
  const int n = a.seqlens[b];
  const bool calib = a.fp8 && a.first_block && n == 0;
  if (a.maxima) {
    if (calib) chunk_maxima(a, b, c, smax);
    return;
  }
  chunk_writes(a, b, c, n, calib ? (a.chunks == 1 ? 1 : 2) : 0, smax, sscale, sinv, srow);
}

hipError_t launch_append(const AppendArgs& a0, hipStream_t st) {
  AppendArgs a = a0;
  const dim3 grid(a.chunks, a.batch);
  a.maxima = 0;
  a.reverse = 0;
  if (a.fp8 && a.first_block && a.chunks > 1) {
    a.maxima = 1;
    hipLaunchKernelGGL(gqa_append_kernel, grid, dim3(kAppendThreads), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.maxima = 0;
    a.reverse = 1;
  }
  hipLaunchKernelGGL(gqa_append_kernel, grid, dim3(kAppendThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace gqa
