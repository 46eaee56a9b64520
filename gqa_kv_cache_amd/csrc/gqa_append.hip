// K/V append with FP8 E4M3FN quantisation on write (gfx950).
//
// Writes the S_new bf16 K and V rows of each request at logical positions
// n_b .. n_b + S_new - 1 of a contiguous or paged cache, as bf16 or as FP8
// E4M3FN codes under one scale per (request, KV head) -- the storage the
// decode kernels read ("Sparse paged GQA decode attention with FP8 KV cache
// on SM89", "Workload" and "Implementations").  Only the appended rows are
// touched.
//
// Work split: a workgroup takes `chunk_tokens` consecutive new tokens of one
// request, all KV heads (a token's H_kv * d elements are contiguous in both
// the input and the cache row).  A thread handles 8 elements at a time: one
// 16-byte bf16 load, and an 8-byte (FP8) or 16-byte (bf16) store.  HBM-bound:
// 2 bytes read and 1 (FP8) or 2 (bf16) written per element.
//
// First-block scales: a request with n_b == 0 takes scale = absmax / 448 per
// KV head over its appended rows.  One workgroup per request reduces its
// rows in LDS; when a request's rows span several workgroups, a first pass
// writes each workgroup's per-head maxima to the workspace and a
// per-request pass reduces them to the scales (no atomics in HBM, no
// zero-initialised memory).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gqa_append_args.h"

namespace gqa {

namespace {

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __builtin_bit_cast(float, bits16 << 16); }

// E4M3FN code of y, |y| <= 448: round to nearest, ties to even mantissa,
// sign kept.  Normal range [2^-6, 448]: drop 20 of the 23 fp32 mantissa
// bits with round-to-nearest-even on the bit pattern (a carry moves into
// the exponent, which is what rounding up to the next binade means), then
// rebias the exponent (127 -> 7).  Below 2^-6 the code is the subnormal
// count of 2^-9 steps, y * 512 rounded to nearest even (exact product).
__device__ __forceinline__ uint32_t e4m3fn_code(float y) {
  const uint32_t bits = __builtin_bit_cast(uint32_t, y);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = __builtin_fabsf(y);
  uint32_t mag;
  if (a < 0.015625f) {
    mag = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    const uint32_t u = bits & 0x7fffffffu;
    const uint32_t r = (u + 0x7ffffu + ((u >> 20) & 1u)) >> 20;  // exponent:8 | mantissa:3
    mag = r - (120u << 3);
  }
  return sign | mag;
}

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

__device__ __forceinline__ uint2 quantize8(const uint4 x, float s) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = fminf(fmaxf(bf16_to_f32(w[i] & 0xffffu) / s, -448.f), 448.f);
    const float hi = fminf(fmaxf(bf16_to_f32(w[i] >> 16) / s, -448.f), 448.f);
    c[2 * i] = e4m3fn_code(lo);
    c[2 * i + 1] = e4m3fn_code(hi);
  }
  return uint2{c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24), c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
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

// Three kernels, by PASS:
//   0  per-workgroup absolute maxima of first-block requests whose rows span
//      several workgroups, into the workspace;
//   2  one workgroup per request: the maxima of all its workgroups -> its
//      scales (written to k_scale / v_scale);
//   1  the writes.  A first-block request covered by one workgroup takes its
//      maxima in LDS here; every other request reads its scales.
// Passes 0 and 2 run only when some first-block request spans several
// workgroups.
template <int PASS>
__global__ void __launch_bounds__(kAppendThreads) gqa_append_kernel(AppendArgs a) {
  constexpr int U = 8;  // 8-element items per thread in flight per round (K and V each)
  __shared__ uint32_t smax[2 * kAppendMaxHeads];  // fp32 bits of |x| maxima (K, V per head)
  __shared__ float sscale[2 * kAppendMaxHeads];
  __shared__ int64_t srow[kAppendMaxChunkTokens];  // physical row of each new token (-1: not written)
  const int c = blockIdx.x, b = blockIdx.y;
  const int n = a.seqlens[b];
  const bool calib = a.fp8 && a.first_block && n == 0;
  if (PASS != 1 && !calib) return;
  const int d8 = a.head_dim / 8;
  const int per_tok = a.h_kv * d8;  // 8-element items per token row

  if (PASS == 2) {
    // per-request reduction of the per-workgroup maxima
    for (int i = threadIdx.x; i < 2 * a.h_kv; i += kAppendThreads) smax[i] = 0u;
    __syncthreads();
    const int total = a.chunks * 2 * a.h_kv;
    for (int k = threadIdx.x; k < total; k += kAppendThreads)
      atomicMax(&smax[k % (2 * a.h_kv)], a.amax[(int64_t)b * total + k]);
    __syncthreads();
    for (int i = threadIdx.x; i < 2 * a.h_kv; i += kAppendThreads) {
      const float amax = __builtin_bit_cast(float, smax[i]);
      ((i & 1) ? a.v_scale : a.k_scale)[(int64_t)b * a.h_kv + (i >> 1)] = amax > 0.f ? amax / 448.f : 1.f;
    }
    return;
  }

  const int t0 = c * a.chunk_tokens;
  const int T = min(a.chunk_tokens, a.s_new - t0);
  const int items = T * per_tok;
  const int64_t in_base = ((int64_t)b * a.s_new + t0) * a.h_kv * a.head_dim;

  if (calib && (PASS == 0 || a.chunks == 1)) {
    for (int i = threadIdx.x; i < 2 * a.h_kv; i += kAppendThreads) smax[i] = 0u;
    __syncthreads();
    for (int it = threadIdx.x; it < items; it += kAppendThreads) {
      const int g = (it % per_tok) / d8;
      const int64_t off = in_base + (int64_t)it * 8;
      const float mk = absmax8(*reinterpret_cast<const uint4*>(a.k_new + off));
      const float mv = absmax8(*reinterpret_cast<const uint4*>(a.v_new + off));
      atomicMax(&smax[2 * g], __builtin_bit_cast(uint32_t, mk));  // |x| >= 0: integer order = float order
      atomicMax(&smax[2 * g + 1], __builtin_bit_cast(uint32_t, mv));
    }
    __syncthreads();
    if (PASS == 0) {
      for (int i = threadIdx.x; i < 2 * a.h_kv; i += kAppendThreads)
        a.amax[((int64_t)b * a.chunks + c) * 2 * a.h_kv + i] = smax[i];
      return;
    }
    for (int i = threadIdx.x; i < 2 * a.h_kv; i += kAppendThreads) {
      const float amax = __builtin_bit_cast(float, smax[i]);
      const float s = amax > 0.f ? amax / 448.f : 1.f;
      sscale[i] = s;
      ((i & 1) ? a.v_scale : a.k_scale)[(int64_t)b * a.h_kv + (i >> 1)] = s;
    }
  } else if (a.fp8) {
    for (int i = threadIdx.x; i < 2 * a.h_kv; i += kAppendThreads)
      sscale[i] = ((i & 1) ? a.v_scale : a.k_scale)[(int64_t)b * a.h_kv + (i >> 1)];
  }
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
        *reinterpret_cast<uint2*>(a.k_cache + dst) = quantize8(kx[u], sscale[2 * g]);
        *reinterpret_cast<uint2*>(a.v_cache + dst) = quantize8(vx[u], sscale[2 * g + 1]);
      } else {
        *reinterpret_cast<uint4*>(a.k_cache + dst) = kx[u];
        *reinterpret_cast<uint4*>(a.v_cache + dst) = vx[u];
      }
    }
  }
  if (c == 0 && threadIdx.x == 0 && a.seqlens_out) a.seqlens_out[b] = n + a.s_new;
}

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
  const dim3 grid(a.chunks, a.batch);
  if (a.fp8 && a.first_block && a.chunks > 1) {
    hipLaunchKernelGGL(gqa_append_kernel<0>, grid, dim3(kAppendThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gqa_append_kernel<2>, dim3(1, a.batch), dim3(kAppendThreads), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(gqa_append_kernel<1>, grid, dim3(kAppendThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace gqa
