// GQA decode kernels for gfx950 (MI355X).
//
// Split-KV partial kernel: one workgroup per (list chunk, KV head, request).
// Its 4 waves walk the chunk in 32-position tiles (wave w takes tiles w,
// w+4, ...).  Each K/V tile of the KV head is loaded from HBM once, with
// 16-byte loads, and serves every query row of the group: the G query heads
// times S_q query tokens, padded to 16-row MFMA blocks.  This is the
// load-sharing the grouped kernels of "Sparse paged GQA decode attention
// with FP8 KV cache on SM89" leave open ("Open problem"); the kernel never
// expands K/V to H_q heads ("When the K/V copy costs more than the
// attention").
//
//   S^T (tokens x rows) = K (tokens x d) . Q^T (d x rows)     MFMA, K from registers
//   online softmax in base 2, scale folded into one multiplier
//   O^T (d x rows)     += V^T (d x tokens) . P^T (tokens x rows)  MFMA, V^T from LDS
//
// K is loaded straight into the MFMA A-operand layout (lane = token, 8
// consecutive d).  The contraction index of the QK product may be permuted
// freely as long as Q uses the same permutation, which lets each lane issue
// full 16-byte loads for both bf16 and FP8.  V must be contracted over
// tokens, so each wave stages its V tile in LDS (XOR-swizzled rows) and
// reads it back transposed.  The QK result already sits in the layout the PV
// B operand needs (lane = query row, 4+4 tokens), so P never leaves
// registers.
//
// FP8 E4M3FN K/V are unpacked tile by tile in registers (never a dequantised
// copy in memory, cf. "Profiling down to the register ...", Phase 4);
// k_scale is folded into the score multiplier and v_scale applied once to
// the output ("Sparse paged GQA decode attention ...", Implementations).
//
// The waves of a workgroup merge their (max, sum, acc) in LDS.  With one
// split the workgroup writes the final bf16 O (times sigmoid(gate)) and the
// natural-log LSE; otherwise it writes an fp32 partial (o_s, log2-sum-exp)
// and the combine kernel merges the splits.

#include <math.h>
#include "gqa_device.h"

namespace gqa {

// Shared-memory footprint of the partial kernel.
__host__ __device__ constexpr int vstage_bytes(int D) { return kWaves * kTile * D * 2; }
__host__ __device__ constexpr int merge_bytes(int D) { return kWaves * 16 * D * 4 + 2 * kWaves * 16 * 4; }

template <int D, bool FP8>
struct TileShape {
  static constexpr int ESZ = FP8 ? 1 : 2;
  static constexpr int KK = D / 32;            // MFMA k-steps over d
  static constexpr int NB = D / 16;            // 16-wide d blocks of O
  static constexpr int LD = D * ESZ / 64;      // 16-byte loads per token per lane
};

// Element d of the QK contraction that (k-step kk, lane group qd, element j)
// stands for.  bf16: each 16-byte load is one k-step; FP8: one 16-byte load
// (16 codes) feeds two consecutive k-steps.
template <bool FP8>
__device__ __forceinline__ int qk_d(int kk, int qd) {
  return FP8 ? (64 * (kk >> 1) + 16 * qd + 8 * (kk & 1)) : (32 * kk + 8 * qd);
}

template <int D, bool FP8, bool INDIRECT, int MB>
__global__ void __launch_bounds__(kThreads) gqa_partial_kernel(DecodeArgs a) {
  using TS = TileShape<D, FP8>;
  constexpr int KK = TS::KK, NB = TS::NB, LD = TS::LD, ESZ = TS::ESZ;
  constexpr int R = MB * 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m16 = lane & 15;
  const int qd = lane >> 4;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;

  const int n = seq_len(a, b);
  const int L = list_len(a, n);
  const int start = split * a.chunk;
  if (a.num_splits > 1 && start >= L) return;  // nothing in this split; the combine skips it
  const int end = min(L, start + a.chunk);
  const int ntiles = end > start ? (end - start + kTile - 1) / kTile : 0;
  const int64_t base = row_base(a, b);

  int32_t* trow = reinterpret_cast<int32_t*>(smem + vstage_bytes(D));
  int32_t* ttok = trow + a.chunk;
  if constexpr (INDIRECT) {
    // Resolve every slot of the chunk once: physical row and logical token
    // (-1 = masked).  Slots past the end are masked.
    for (int p = threadIdx.x; p < a.chunk; p += kThreads) {
      const int pos = start + p;
      int t = -1;
      int64_t row = 0;
      if (pos < end) {
        t = slot_token(a, b, n, pos);
        if (t >= 0) row = token_row(a, b, t, base);
      }
      trow[p] = (int32_t)row;
      ttok[p] = t;
    }
    __syncthreads();
  }

  // Q as the B operand of S^T = K Q^T: lane = query row, 8 d per k-step.
  // Row r of the group is (query token i = r / G, head g*G + r % G).
  u32x4 qop[MB][KK];
  int lim[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = mb * 16 + m16;
    const int rr = min(r, a.rows - 1);
    const int i = rr / a.group;
    lim[mb] = a.causal ? (n - a.s_q + i) : 0x7fffffff;
    if (r < a.rows) {
      const int h = g * a.group + (r - i * a.group);
      const uint16_t* qrow = a.q + ((int64_t)(b * a.s_q + i) * a.h_q + h) * D;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        qop[mb][kk] = *reinterpret_cast<const u32x4*>(qrow + qk_d<FP8>(kk, qd));
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qop[mb][kk] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  float sc = a.scale_log2;
  if constexpr (FP8) sc *= a.k_scale[b * a.h_kv + g];

  f32x4 acc[MB][NB];
  float mrun[MB], lrun[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    mrun[mb] = -INFINITY;
    lrun[mb] = 0.f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  uint16_t* vs = reinterpret_cast<uint16_t*>(smem) + wave * kTile * D;
  const size_t head_off = (size_t)g * D * ESZ;
  const size_t row_bytes = (size_t)a.h_kv * D * ESZ;

  // Issue the 16-byte loads of one tile: lane (m16, qd) fetches, for tokens
  // m16 and 16 + m16 of the tile, bytes [64 j + 16 qd, +16) of the KV head.
  auto load_tile = [&](int tile, u32x4 (&kr)[2][LD], u32x4 (&vr)[2][LD]) {
    const int tb = start + tile * kTile;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int p = tb + hb * 16 + m16;
      int64_t row;
      if constexpr (INDIRECT) {
        row = trow[p - start];
      } else {
        row = token_row(a, b, p < end ? p : 0, base);
      }
      const size_t off = (size_t)row * row_bytes + head_off + 16 * qd;
      const uint8_t* kp = a.k + off;
      const uint8_t* vp = a.v + off;
#pragma unroll
      for (int j = 0; j < LD; ++j) kr[hb][j] = *reinterpret_cast<const u32x4*>(kp + 64 * j);
#pragma unroll
      for (int j = 0; j < LD; ++j) vr[hb][j] = *reinterpret_cast<const u32x4*>(vp + 64 * j);
    }
  };

  auto compute_tile = [&](int tile, const u32x4 (&kr)[2][LD], const u32x4 (&vr)[2][LD]) {
    const int tb = start + tile * kTile;

    // K operands (bf16), unpacking FP8 in registers.
    u32x4 kop[2][KK];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
      for (int j = 0; j < LD; ++j) {
        if constexpr (FP8) {
          uint32_t x0, x1, x2, x3, y0, y1, y2, y3;
          fp8x4_to_bf16x4(kr[hb][j][0], x0, x1);
          fp8x4_to_bf16x4(kr[hb][j][1], x2, x3);
          fp8x4_to_bf16x4(kr[hb][j][2], y0, y1);
          fp8x4_to_bf16x4(kr[hb][j][3], y2, y3);
          kop[hb][2 * j] = u32x4{x0, x1, x2, x3};
          kop[hb][2 * j + 1] = u32x4{y0, y1, y2, y3};
        } else {
          kop[hb][j] = kr[hb][j];
        }
      }
    }

    // S^T for both 16-token halves and every row block.
    f32x4 s[2][MB];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) c = mfma_16x16x32(kop[hb][kk], qop[mb][kk], c);
        s[hb][mb] = c * sc;
      }
    }

    // Stage V (as bf16) in this wave's LDS tile: row = token, 16-element
    // blocks XOR-swizzled by (token / 4) % 4 so the transposed reads below
    // hit four different bank groups.
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int tok = hb * 16 + m16;
      const int swz = ((tok >> 2) & 3) << 4;
      uint16_t* vrow = vs + tok * D;
#pragma unroll
      for (int j = 0; j < LD; ++j) {
        if constexpr (FP8) {
          const int d0 = 64 * j + 16 * qd;
          uint32_t x0, x1, x2, x3, y0, y1, y2, y3;
          fp8x4_to_bf16x4(vr[hb][j][0], x0, x1);
          fp8x4_to_bf16x4(vr[hb][j][1], x2, x3);
          fp8x4_to_bf16x4(vr[hb][j][2], y0, y1);
          fp8x4_to_bf16x4(vr[hb][j][3], y2, y3);
          *reinterpret_cast<u32x4*>(vrow + (d0 ^ swz)) = u32x4{x0, x1, x2, x3};
          *reinterpret_cast<u32x4*>(vrow + ((d0 + 8) ^ swz)) = u32x4{y0, y1, y2, y3};
        } else {
          const int d0 = 32 * j + 8 * qd;
          *reinterpret_cast<u32x4*>(vrow + (d0 ^ swz)) = vr[hb][j];
        }
      }
    }

    // Masking: slots past the end, masked top-K entries, causal tail.
    const bool need_mask = INDIRECT || (tb + kTile > end) || (a.causal && tb + kTile - 1 > n - a.s_q);
    if (need_mask) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int p = tb + hb * 16 + 4 * qd + i;
          int t;
          bool ok;
          if constexpr (INDIRECT) {
            t = ttok[p - start];
            ok = t >= 0;
          } else {
            t = p;
            ok = p < end;
          }
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            if (!ok || t > lim[mb]) s[hb][mb][i] = -INFINITY;
        }
      }
    }

    // Online softmax (base 2) per query row.  The row sum uses the fp32
    // weights (it sets the LSE); P is rounded to bf16 only as the MFMA
    // operand of the PV product.
    u32x4 pB[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      float mx = fmaxf(fmaxf(fmaxf(s[0][mb][0], s[0][mb][1]), fmaxf(s[0][mb][2], s[0][mb][3])),
                       fmaxf(fmaxf(s[1][mb][0], s[1][mb][1]), fmaxf(s[1][mb][2], s[1][mb][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mrun[mb], mx);
      const float muse = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = fast_exp2(mrun[mb] - muse);
      float pf[2][4];
      float ps = 0.f;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pf[hb][i] = fast_exp2(s[hb][mb][i] - muse);
          ps += pf[hb][i];
        }
      uint32_t pk[4];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        pk[2 * hb] = pack_bf16(pf[hb][0], pf[hb][1]);
        pk[2 * hb + 1] = pack_bf16(pf[hb][2], pf[hb][3]);
      }
      lrun[mb] = lrun[mb] * alpha + ps;
      mrun[mb] = mnew;
      pB[mb] = u32x4{pk[0], pk[1], pk[2], pk[3]};
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[mb][nb] *= alpha;
    }

    // LDS writes above must land before other lanes read them; a wave's LDS
    // operations execute in order, so a compiler barrier suffices.
    __builtin_amdgcn_wave_barrier();
    __asm__ __volatile__("" ::: "memory");

    // V^T operand: lane (m16, qd) takes column d = 16 nb + m16 for tokens
    // 4 qd + j and 16 + 4 qd + j (j < 4), matching P's k-slot order.
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = ((nb ^ qd) << 4) + m16;
      uint32_t w[4];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int t0 = 4 * qd + 2 * jj;
        const uint32_t a0 = vs[(t0)*D + col];
        const uint32_t a1 = vs[(t0 + 1) * D + col];
        const uint32_t b0 = vs[(16 + t0) * D + col];
        const uint32_t b1 = vs[(16 + t0 + 1) * D + col];
        w[jj] = a0 | (a1 << 16);
        w[2 + jj] = b0 | (b1 << 16);
      }
      const u32x4 av = {w[0], w[1], w[2], w[3]};
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb][nb] = mfma_16x16x32(av, pB[mb], acc[mb][nb]);
    }
    __builtin_amdgcn_wave_barrier();
    __asm__ __volatile__("" ::: "memory");
  };

  // Software pipeline: the next tile's loads are in flight while this one
  // is computed.
  {
    u32x4 kA[2][LD], vA[2][LD], kB[2][LD], vB[2][LD];
    int tile = wave;
    if (tile < ntiles) load_tile(tile, kA, vA);
    while (tile < ntiles) {
      int nxt = tile + kWaves;
      if (nxt < ntiles) load_tile(nxt, kB, vB);
      compute_tile(tile, kA, vA);
      tile = nxt;
      if (tile >= ntiles) break;
      nxt = tile + kWaves;
      if (nxt < ntiles) load_tile(nxt, kA, vA);
      compute_tile(tile, kB, vB);
      tile = nxt;
    }
  }

  // Row sums over the four lane groups.
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    lrun[mb] += __shfl_xor(lrun[mb], 16);
    lrun[mb] += __shfl_xor(lrun[mb], 32);
  }

  // Merge the four waves, one 16-row block at a time.
  float* wm = reinterpret_cast<float*>(smem);
  float* wl = wm + kWaves * 16;
  float* wacc = wl + kWaves * 16;
  const float vsc = FP8 ? a.v_scale[b * a.h_kv + g] : 1.f;
  const bool final_out = (a.num_splits == 1);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (mb * 16 >= a.rows) break;
    __syncthreads();
    if (qd == 0) {
      wm[wave * 16 + m16] = mrun[mb];
      wl[wave * 16 + m16] = lrun[mb];
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      *reinterpret_cast<f32x4*>(wacc + (wave * 16 + m16) * D + 16 * nb + 4 * qd) = acc[mb][nb];
    __syncthreads();

    const int nrow = min(16, a.rows - mb * 16);
    for (int it = threadIdx.x; it < nrow * (D / 8); it += kThreads) {
      const int rl = it / (D / 8);
      const int d8 = it - rl * (D / 8);
      const int r = mb * 16 + rl;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wm[w * 16 + rl]);
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = 0.f;
      float lse2 = -INFINITY;
      if (M != -INFINITY) {
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float e = fast_exp2(wm[w * 16 + rl] - M);
          sum += e * wl[w * 16 + rl];
          const float* src = wacc + (w * 16 + rl) * D + d8 * 8;
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
          const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            o[c] += e * x0[c];
            o[4 + c] += e * x1[c];
          }
        }
        const float inv = vsc / sum;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= inv;
        lse2 = M + __log2f(sum);
      }
      const int i = r / a.group;
      const int h = g * a.group + (r - i * a.group);
      if (final_out) {
        const int64_t oidx = ((int64_t)(b * a.s_q + i) * a.h_q + h) * D + d8 * 8;
        if (a.gate_mode == kGateElementwise) {
          const u32x4 gw = *reinterpret_cast<const u32x4*>(a.gate + oidx);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            o[2 * c] *= sigmoidf_(bf16_lo(gw[c]));
            o[2 * c + 1] *= sigmoidf_(bf16_hi(gw[c]));
          }
        } else if (a.gate_mode == kGateHeadwise) {
          const uint32_t gb = a.gate[(int64_t)(b * a.s_q + i) * a.h_q + h];
          const float sg = sigmoidf_(bf16_lo(gb));
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] *= sg;
        }
        const u32x4 ov = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]), pack_bf16(o[4], o[5]),
                          pack_bf16(o[6], o[7])};
        *reinterpret_cast<u32x4*>(a.o + oidx) = ov;
        if (d8 == 0) a.lse[((int64_t)b * a.h_q + h) * a.s_q + i] = lse2 * 0.69314718055994530942f;
      } else {
        const int64_t prow = ((int64_t)(b * a.h_kv + g) * a.num_splits + split) * a.rows + r;
        float* dst = a.o_part + prow * D + d8 * 8;
        *reinterpret_cast<f32x4*>(dst) = f32x4{o[0], o[1], o[2], o[3]};
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4], o[5], o[6], o[7]};
        if (d8 == 0) a.lse_part[prow] = lse2;
      }
    }
  }
}

// LSE combine: one workgroup per (query row of the group, KV head, request).
// With M = max_s lse_s (base 2), O = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M)
// and LSE = ln 2 * (M + log2 sum_s 2^(lse_s - M)); empty splits (-inf) weigh 0.
template <int D>
__global__ void __launch_bounds__(kThreads) gqa_combine_kernel(DecodeArgs a) {
  constexpr int Q4 = D / 4;          // float4 columns
  constexpr int SG = kThreads / Q4;  // split lanes
  __shared__ f32x4 red[SG][Q4];
  const int r = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int n = seq_len(a, b);
  const int L = list_len(a, n);
  const int nsp = min(a.num_splits, (L + a.chunk - 1) / a.chunk);
  const int64_t first = (int64_t)(b * a.h_kv + g) * a.num_splits;
  const float* lsep = a.lse_part + first * a.rows + r;
  const float* op = a.o_part + (first * a.rows + r) * D;

  float M = -INFINITY;
  for (int s = lane; s < nsp; s += 64) M = fmaxf(M, lsep[(int64_t)s * a.rows]);
  M = wave_max(M);
  float S = 0.f;
  if (M != -INFINITY)
    for (int s = lane; s < nsp; s += 64) S += fast_exp2(lsep[(int64_t)s * a.rows] - M);
  S = wave_sum(S);

  const int d4 = threadIdx.x % Q4;
  const int sg = threadIdx.x / Q4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
    for (int s = sg; s < nsp; s += SG) {
      const float w = fast_exp2(lsep[(int64_t)s * a.rows] - M);
      const f32x4 x = *reinterpret_cast<const f32x4*>(op + (int64_t)s * a.rows * D + d4 * 4);
      acc += w * x;
    }
  }
  red[sg][d4] = acc;
  __syncthreads();
  if (sg == 0) {
    for (int k = 1; k < SG; ++k) acc += red[k][d4];
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
      const float inv = 1.f / S;
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = acc[c] * inv;
    }
    const int i = r / a.group;
    const int h = g * a.group + (r - i * a.group);
    const int64_t oidx = ((int64_t)(b * a.s_q + i) * a.h_q + h) * D + d4 * 4;
    if (a.gate_mode == kGateElementwise) {
      const uint2 gw = *reinterpret_cast<const uint2*>(a.gate + oidx);
      o[0] *= sigmoidf_(bf16_lo(gw.x));
      o[1] *= sigmoidf_(bf16_hi(gw.x));
      o[2] *= sigmoidf_(bf16_lo(gw.y));
      o[3] *= sigmoidf_(bf16_hi(gw.y));
    } else if (a.gate_mode == kGateHeadwise) {
      const float sgm = sigmoidf_(bf16_lo(a.gate[(int64_t)(b * a.s_q + i) * a.h_q + h]));
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] *= sgm;
    }
    *reinterpret_cast<uint2*>(a.o + oidx) = uint2{pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
    if (d4 == 0)
      a.lse[((int64_t)b * a.h_q + h) * a.s_q + i] =
          (M == -INFINITY) ? -INFINITY : (M + __log2f(S)) * 0.69314718055994530942f;
  }
}

// Address resolution only, through the same slot_token / token_row the
// partial kernel uses.  out[b, i, p] = physical row or -1.
__global__ void __launch_bounds__(kThreads) gqa_resolve_kernel(DecodeArgs a, int64_t* out, int list_cap) {
  const int p = blockIdx.x * kThreads + threadIdx.x;
  const int i = blockIdx.y, b = blockIdx.z;
  if (p >= list_cap) return;
  const int n = seq_len(a, b);
  const int L = list_len(a, n);
  int64_t v = -1;
  if (p < L) {
    const int t = slot_token(a, b, n, p);
    if (t >= 0 && (!a.causal || t <= n - a.s_q + i)) v = token_row(a, b, t, row_base(a, b));
  }
  out[((int64_t)b * a.s_q + i) * list_cap + p] = v;
}

// ---------------------------------------------------------------------------
// Host-side launchers (called from the C ABI in gqa_api.cpp).
// ---------------------------------------------------------------------------

template <int D, bool FP8, bool IND, int MB>
static hipError_t launch_partial_t(const DecodeArgs& a, dim3 grid, hipStream_t st) {
  size_t lds = (size_t)vstage_bytes(D) + (IND ? (size_t)a.chunk * 8 : 0);
  lds = lds > (size_t)merge_bytes(D) ? lds : (size_t)merge_bytes(D);
  hipLaunchKernelGGL((gqa_partial_kernel<D, FP8, IND, MB>), grid, dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <int D, bool FP8, bool IND>
static hipError_t launch_mb(const DecodeArgs& a, int mb, dim3 grid, hipStream_t st) {
  switch (mb) {
    case 1: return launch_partial_t<D, FP8, IND, 1>(a, grid, st);
    case 2: return launch_partial_t<D, FP8, IND, 2>(a, grid, st);
    default: return launch_partial_t<D, FP8, IND, 4>(a, grid, st);
  }
}

size_t partial_lds_bytes(int D, bool indirect, int chunk) {
  size_t lds = (size_t)vstage_bytes(D) + (indirect ? (size_t)chunk * 8 : 0);
  return lds > (size_t)merge_bytes(D) ? lds : (size_t)merge_bytes(D);
}

hipError_t launch_partial(const DecodeArgs& a, int D, bool fp8, bool indirect, int mb, dim3 grid,
                          hipStream_t st) {
  if (D == 128) {
    if (fp8) return indirect ? launch_mb<128, true, true>(a, mb, grid, st) : launch_mb<128, true, false>(a, mb, grid, st);
    return indirect ? launch_mb<128, false, true>(a, mb, grid, st) : launch_mb<128, false, false>(a, mb, grid, st);
  }
  if (fp8) return indirect ? launch_mb<64, true, true>(a, mb, grid, st) : launch_mb<64, true, false>(a, mb, grid, st);
  return indirect ? launch_mb<64, false, true>(a, mb, grid, st) : launch_mb<64, false, false>(a, mb, grid, st);
}

hipError_t launch_combine(const DecodeArgs& a, int D, dim3 grid, hipStream_t st) {
  if (D == 128)
    hipLaunchKernelGGL((gqa_combine_kernel<128>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((gqa_combine_kernel<64>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_resolve(const DecodeArgs& a, int64_t* out, int list_cap, hipStream_t st) {
  dim3 grid((list_cap + kThreads - 1) / kThreads, a.s_q, a.batch);
  hipLaunchKernelGGL(gqa_resolve_kernel, grid, dim3(kThreads), 0, st, a, out, list_cap);
  return hipGetLastError();
}

}  // namespace gqa
