// GQA decode kernels for gfx950 (MI355X).
//
// Split-KV partial kernel.  A workgroup of 4 wave64s covers one list chunk
// of one request for HPW consecutive KV heads (HPW = 4 when H_kv allows,
// else 2 or 1; paged and top-K lists can take eight, one wave each, in a
// workgroup of 8 wave64s -- WIDE below).  Wave w works on head g0 + w % HPW;
// the waves that share a head take alternate 32-position tiles of the chunk
// and are merged in LDS at the end.  With HPW = 4 the workgroup reads, for every token, a
// contiguous 1 KiB of the cache (four heads' K or V), which is what lets
// HBM run close to its streaming rate.  Groups of more than 16 query rows
// per KV head can instead split the rows over the waves of a head (two,
// four, or eight in a workgroup of 8 wave64s), which share each tile
// through LDS (SHARE below).
//
// Each K/V tile of a head is loaded from HBM once and serves every query row
// of the head's group: G = H_q / H_kv query heads times S_q query tokens,
// padded to 16-row MFMA blocks.  This is the load sharing the grouped
// kernels of "Sparse paged GQA decode attention with FP8 KV cache on SM89"
// leave open ("Open problem"); K/V are never expanded to H_q heads ("When
// the K/V copy costs more than the attention").
//
//   S^T (tokens x rows) = K (tokens x d) . Q^T (d x rows)         MFMA
//   online softmax in base 2, scale folded into one multiplier
//   O^T (d x rows)     += V^T (d x tokens) . P^T (tokens x rows)  MFMA
//
// Loads are whole cache rows: one wave-wide 16-byte load covers 4 tokens x
// 256 B (bf16, d=128), non-temporal since K/V are read once.  Both tiles
// pass through per-wave LDS: K is re-read in the MFMA A-operand layout
// (lane = token, 8 consecutive contraction slots; the contraction order
// over d is free as long as Q uses the same one), V is read transposed
// with ds_read_b64_tr_b16.  The QK result already sits in the layout the PV
// B operand needs (lane = query row, 4 + 4 tokens), so P never leaves
// registers.
//
// FP8 E4M3FN K/V are unpacked tile by tile (never a dequantised copy in
// memory, cf. "Profiling down to the register, then an extension ...",
// Phase 4); k_scale is folded into the score multiplier and v_scale is
// applied once to the output ("Sparse paged GQA decode attention ...",
// Implementations).
//
// With one split the workgroup writes the final bf16 O (times
// sigmoid(gate)) and the natural-log LSE; otherwise each head writes an
// fp32 partial (o_s, log2-sum-exp) and the combine kernel merges the splits.

#include <hip/hip_ext.h>
#include <math.h>
#include "gqa_device.h"

namespace gqa {

template <int D, bool Q8>
struct TileShape {
  static constexpr int ESZ = Q8 ? 1 : 2;
  static constexpr int RB = D * ESZ;          // bytes of one head in one token row
  static constexpr int CPR = RB / 16;         // 16-byte chunks per row (16, 8 or 4)
  static constexpr int TPI = 64 / CPR;        // tokens per wave-wide load (4, 8 or 16)
  static constexpr int NLD = kTile / TPI;     // wave-wide loads per tile per tensor
  static constexpr int KK = D / 32;           // MFMA k-steps over d
  static constexpr int NB = D / 16;           // 16-wide d blocks of O
  // Loads are issued and staged in NPART parts per tile: d = 256 rows are
  // 512 B, and a whole 32-token tile per register buffer would take 128
  // VGPRs; in halves it takes 64, like d = 128.
  static constexpr int NPART = (D == 256) ? 2 : 1;
  static constexpr int NLDP = NLD / NPART;    // wave-wide loads per part per tensor
};

// Contraction slot -> d.  K-step kk, lane group qd covers d = qk_d(kk, qd)
// .. +7.  bf16: one 16-byte chunk per k-step (chunk 4 kk + qd); FP8: one
// 16-byte chunk (16 codes, chunk 4 (kk / 2) + qd) feeds two k-steps.
template <bool Q8>
__device__ __forceinline__ int qk_d(int kk, int qd) {
  return Q8 ? (64 * (kk >> 1) + 16 * qd + 8 * (kk & 1)) : (32 * kk + 8 * qd);
}

// Physical 16-byte chunk of logical chunk c in the K tile row of token tok:
// XOR by a token-dependent value so that the 16 rows one A-operand read
// touches fall on distinct LDS banks (rows of 16 or 32 chunks: by the token;
// of 8 or 4 chunks, where two or four rows share a bank sweep: by the token
// divided by 2 or 4).
template <int CPR>
__device__ __forceinline__ int kchunk(int c, int tok) {
  return c ^ ((tok >> (CPR >= 16 ? 0 : (CPR == 8 ? 1 : 2))) & (CPR - 1));
}

// Physical 16-element block of logical block blk in the V tile row of token
// tok: the XOR spreads the 16 rows one transposed read touches over all
// bank groups (d=128: a row is 8 blocks, one bank sweep; d=64: two rows
// share a sweep).
template <int D>
__device__ __forceinline__ int vblk(int blk, int tok) {
  return D >= 128 ? (blk ^ (tok & 7)) : (blk ^ ((tok >> 1) & 3));
}

// How a partial workgroup finds its work.
//   kDense    one chunk of one request's list (contiguous / ragged cache),
//             addresses computed from the position;
//   kIndirect the same through a block table and / or a top-K list, resolved
//             into an LDS row table first;
//   kPacked   one chunk of the packed rows of a ragged cache: the chunk is cut
//             at request boundaries into segments, each computed like a
//             kDense chunk of its request.  Every workgroup then gets the same
//             number of rows, however the lengths vary.
constexpr int kDense = 0, kIndirect = 1, kPacked = 2;

// Largest base-2 exponent that a softmax weight may reach before the MFMA
// path moves its running maximum (weights below 2^8 keep bf16 P and the fp32
// sums far from overflow).
constexpr float kLazyRescale = 8.f;

// Waves of a partial workgroup: kPWaves, or eight -- for row sharing over
// eight waves, or (WIDE) for eight KV heads, one wave each -- two per SIMD
// in one workgroup.
template <int SHARE, bool WIDE = false>
constexpr int partial_waves() { return SHARE == 8 || WIDE ? 8 : kPWaves; }

// The launch bound's second value is waves per SIMD.
template <int D, bool Q8, int MB, int RV, int SHARE, bool WIDE = false>
constexpr int partial_min_waves() {
  return WIDE ? 2 : partial_wgs_per_cu(D, Q8, MB, RV, SHARE) * partial_waves<SHARE>() / 4;
}

// MB: 16-row MFMA blocks (RV = 0).  RV > 0 selects the VALU variant for up
// to RV query rows (MB = 1): the same loads, LDS staging and pipeline, with
// the two products done by v_dot2_f32_bf16 and fp32 FMAs instead of MFMA.
//   QK: lane (token slot l / CPR, chunk c = l % CPR) dots its ELT elements
//       of K with the same elements of each Q row; a DPP sum over the CPR
//       lanes of the token completes the score in all of them.
//   PV: the lane accumulates p x V over its own token slot for its ELT
//       columns; the token slots are summed once, after the last tile.
// SHARE = 2, 4 or 8 (row sharing): the SHARE waves of a head split the rows
// instead of the tiles.  Each computes MB 16-row blocks over every tile of
// the chunk, and each loads and stages 1/SHARE of every tile into a
// head-wide, double-buffered LDS tile (an LDS-only barrier per tile).  HBM
// still reads each tile once per workgroup, and a wave's registers are
// those of a one- or two-block kernel.  Used for d = 256 with 17 to 32 rows
// (two blocks of d = 256 in one wave do not fit) and for every group of
// more than 32 rows; a workgroup covers SHARE * MB * 16 rows (row group
// blockIdx.y / (H_kv / HPW)), and a group of up to 512 rows takes several
// row groups, each reading the chunk.  SHARE = 8 is a workgroup of eight
// waves, two per SIMD, for one head: 128 or 256 rows read each tile once,
// and while one wave of a SIMD runs its softmax the other's MFMAs run.
// WIDE: a workgroup of eight waves, one per KV head (HPW = 8), for the
// one-block variants whose registers fit two waves per SIMD (one-byte tiles
// at d <= 128, bf16 at d = 64).  A CU then runs one workgroup whose eight
// waves stream alike, where two four-wave workgroups per CU stream unequally
// (the older one's waves win the CU's issue arbitration); a top-K or paged
// request's row table is resolved once for all eight heads.
template <int D, int KVT, int MODE, int MB, int RV, int SHARE, bool WIDE = false>
__global__ void __launch_bounds__((64 * partial_waves<SHARE, WIDE>()),
                                  (partial_min_waves<D, KVT != kKvBf16, MB, RV, SHARE, WIDE>()))
    gqa_partial_kernel(DecodeArgs a) {
  constexpr bool Q8 = KVT != kKvBf16;          // one-byte codes (FP8 or int8) with scales
  using TS = TileShape<D, Q8>;
  constexpr int RB = TS::RB, CPR = TS::CPR, TPI = TS::TPI, NLD = TS::NLD, KK = TS::KK, NB = TS::NB;
  constexpr bool SHARED = SHARE > 1;
  constexpr int NPART = TS::NPART;
  // Loads per part: a shared tile is loaded in SHARE parts, one per wave;
  // with fewer loads per tile than waves (eight waves over one-byte or
  // d = 64 tiles), the first NLD waves load one each and the rest none.
  constexpr int NLDP = SHARED ? (NLD >= SHARE ? NLD / SHARE : 1) : NLD / NPART;
  constexpr int NLOADERS = SHARED ? NLD / NLDP : 1;
  static_assert(RV == 0 || D <= 128, "the VALU variant is built for d <= 128");
  static_assert(SHARE == 1 || ((SHARE == 2 || SHARE == 4 || SHARE == 8) && RV == 0 && MB <= 2 &&
                                (NLD % SHARE == 0 || SHARE % NLD == 0)),
                "row sharing: 2, 4 or 8 waves per head, one or two blocks per wave");
  static_assert(!WIDE || (SHARE == 1 && RV == 0 && MB == 1), "eight heads: one block, waves split the tiles");
  constexpr int NW = partial_waves<SHARE, WIDE>();  // waves of this workgroup
  constexpr int NT = 64 * NW;
  // LDS tiles: one per wave, or two per head (row sharing; eight waves
  // cover one head)
  constexpr int NTILE = SHARE == 8 ? 2 : (SHARED ? kPWaves : NW);
  constexpr bool INDIRECT = MODE == kIndirect;
  constexpr bool PACKED = MODE == kPacked;
  constexpr bool VALU = RV > 0;
  constexpr int ELT = Q8 ? 16 : 8;             // elements of one 16-byte chunk
  constexpr int NR = VALU ? RV : MB;            // running-state rows per lane
  static_assert(!VALU || MB == 1, "the VALU variant computes one block of at most 16 rows");
  // Row stride (floats) of the accumulators the waves of a head merge
  // through LDS after the tile loop: four floats of padding put the 16 rows
  // one store covers on different banks.
  constexpr int WST = D + 4;
  static_assert(SHARED || NW * 16 * WST * 4 <= NTILE * wave_tile_bytes(D, Q8), "accumulators fit in the tiles");
  // Lazy rescaling (below) keeps a tile's scores live across a branch; the
  // variants with the most accumulators (four blocks, or two of d = 256)
  // would spill for it, and rescale at every tile instead.
  constexpr bool LAZY = MB * D <= 256;
  // Two 16-row blocks of bf16 d = 256 per wave keep Q in LDS (the host plans
  // them with one KV head per workgroup): Q's 64 VGPRs of MFMA operands would
  // otherwise spill the wave's registers.
  constexpr bool QLDS = q_in_lds(D, KVT != kKvBf16, MB, RV, SHARE) && !WIDE;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ __attribute__((aligned(16))) unsigned char tiles[NTILE * wave_tile_bytes(D, Q8)];
  __shared__ float wstat[2 * NW * 16];
  __shared__ u32x4 qbuf[QLDS ? MB * KK * 64 : 1];  // Q operands, lane-major (QLDS)

  const int lane = threadIdx.x & 63;
  // Wave index as a scalar: tile-level control flow is then uniform, which
  // keeps branches scalar and the compiler's memory-counter waits precise.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m16 = lane & 15;
  const int qd = lane >> 4;
  const int hpw = a.heads_per_wg;
  const int wph = NW / hpw;                      // waves per head
  const int hs = wave % hpw;                    // head slot of this wave
  const int sub = wave / hpw;                   // this wave's share of the head's tiles (or rows)
  const int hgroups = a.h_kv / hpw;             // head groups in grid.y (times the row groups)
  // The row groups of one chunk read the same tiles.  Given consecutive
  // dispatch slots on one XCD (workgroups i and i + 8k share an XCD), they
  // run together and the XCD's L2 serves the group behind: the chunk is
  // fetched from HBM about once.  Workgroup L takes XCD L mod 8, row group
  // (L / 8) mod R and unit ((L / 8) / R) * 8 + L mod 8 of the units
  // (split, head group, request); the host sets R (xcd_rows) only when the
  // grid divides into 8 R.  On MI355X, 64 query tokens of 64/8 heads over
  // 128K tokens (two row groups): FETCH 2.02 -> 1.04 times the K/V bytes,
  // 333.5 -> 304.6 us.
  unsigned bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
  if (a.xcd_rows > 1) {
    const unsigned R = (unsigned)a.xcd_rows;
    const unsigned L = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const unsigned k = L / kXcds, u = (k / R) * kXcds + L % kXcds;
    bx = u % gridDim.x;
    const unsigned rest = u / gridDim.x;
    by = (k % R) * (unsigned)hgroups + rest % (unsigned)hgroups;
    bz = rest / (unsigned)hgroups;
  }
  const int rgroup = __builtin_amdgcn_readfirstlane(by / hgroups);
  const int rbase = SHARED ? (rgroup * SHARE + sub) * MB * 16 : 0;  // first query row of this wave's blocks
  const int g0 = __builtin_amdgcn_readfirstlane((by - rgroup * hgroups) * hpw);
  const int g = g0 + hs;
  const int split = __builtin_amdgcn_readfirstlane(bx);

  // Packed rows [x0, x1) of this workgroup and the first request they meet.
  int64_t x0 = 0, x1 = 0;
  int bnext = 0;
  if constexpr (PACKED) {
    x0 = (int64_t)split * a.chunk;
    x1 = x0 + a.chunk;
    bnext = __builtin_amdgcn_readfirstlane(packed_request(a, x0, lane));
  }

  // One pass per segment: list positions [start, end) of request b, written
  // as partial `split` of b, or as the final output when the segment is b's
  // whole list (fin).  Only the packed mode has more than one.
  for (;;) {
  int b, n, start, end;
  bool fin;
  if constexpr (PACKED) {
    if (bnext >= a.batch) break;
    const int64_t s0 = __builtin_amdgcn_readfirstlane(a.cu_seqlens[bnext]);
    if (s0 >= x1) break;
    b = bnext++;
    n = __builtin_amdgcn_readfirstlane(seq_len(a, b));
    start = (int)min<int64_t>(max<int64_t>(x0 - s0, 0), n);
    end = (int)max<int64_t>(min<int64_t>(x1 - s0, n), 0);
    if (start >= end) continue;
    fin = (start == 0 && end == n);
  } else {
    b = __builtin_amdgcn_readfirstlane(bz);
    n = seq_len(a, b);
    const int L = list_len(a, n);
    start = split * a.chunk;
    if (a.num_splits > 1 && start >= L) return;  // nothing in this split; the combine skips it
    end = min(L, start + a.chunk);
    fin = (a.num_splits == 1);
  }
  const int ntiles = end > start ? (end - start + kTile - 1) / kTile : 0;
  const int64_t base = row_base(a, b);

  // Paged and top-K chunks: every slot of the chunk is resolved once into an
  // LDS table of physical rows and logical tokens (-1 = masked; slots past
  // the end are masked).  The loads are ordered for their in-order return:
  // a thread's top-K entries first, then Q, the scales and the gate (which
  // do not depend on the table), then the block-table entries, so that each
  // wait covers only loads issued before what it waits for.  A paged top-K
  // list whose request has at most kBtCache pages loads the request's whole
  // block-table row next to its top-K entries (the two do not depend on each
  // other) and looks pages up in LDS: one dependent HBM round trip fewer
  // before the first tile's loads.
  int32_t* trow = reinterpret_cast<int32_t*>(smem);
  int32_t* ttok = trow + a.chunk;
  int32_t* btc = ttok + a.chunk;                  // the block-table row (paged top-K lists)
  constexpr int RPT = INDIRECT ? 4096 / NT : 1;   // slots per thread at the largest chunk
  constexpr int BTR = INDIRECT ? kBtCache / NT : 1;
  int tk[RPT];
  int btv[BTR];
  int npg = 0;
  bool btc_on = false;
  if constexpr (INDIRECT) {
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int p = threadIdx.x + k * NT;
      tk[k] = (p < a.chunk && start + p < end) ? slot_token(a, b, n, start + p) : -1;
    }
    const int64_t pages = ((int64_t)n + (1 << a.page_shift) - 1) >> a.page_shift;  // no int overflow near 2^31
    btc_on = a.layout == kLayoutPaged && a.topk_len > 0 && pages <= kBtCache;
    npg = btc_on ? (int)pages : 0;
#pragma unroll
    for (int k = 0; k < BTR; ++k) {
      const int p = threadIdx.x + k * NT;
      btv[k] = (btc_on && p < npg) ? a.block_table[(int64_t)b * a.max_pages + p] : 0;
    }
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  }

  // Q, the scales and (one-byte one-block variants) an elementwise gate:
  // loaded while the row table's loads are in flight.
  // Q as the B operand of S^T = K Q^T: lane = query row, 8 d per k-step.
  // Row r of the group is (query token i = r / G, head g*G + r % G).
  // VALU: every lane holds the ELT elements of its chunk for all RV rows.
  u32x4 qop[VALU ? 1 : MB][KK];
  uint32_t qv[VALU ? RV : 1][ELT / 2];
  int lim[NR];
  if constexpr (VALU) {
#pragma unroll
    for (int r = 0; r < RV; ++r) {
      const int rr = min(r, a.rows - 1);
      const int i = rr / a.group;
      lim[r] = a.causal ? (n - a.s_q + i) : 0x7fffffff;
      const int h = g * a.group + (rr - i * a.group);
      const uint16_t* qrow = a.q + ((int64_t)(b * a.s_q + i) * a.h_q + h) * D + (lane % CPR) * ELT;
#pragma unroll
      for (int j = 0; j < ELT / 8; ++j) {
        const u32x4 v = r < a.rows ? *reinterpret_cast<const u32x4*>(qrow + 8 * j) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int c = 0; c < 4; ++c) qv[r][4 * j + c] = v[c];
      }
    }
  }
#pragma unroll
  for (int mb = 0; mb < (VALU ? 0 : MB); ++mb) {
    const int r = rbase + mb * 16 + m16;
    const int rr = min(r, a.rows - 1);
    const int i = rr / a.group;
    lim[mb] = a.causal ? (n - a.s_q + i) : 0x7fffffff;
    if (r < a.rows) {
      const int h = g * a.group + (r - i * a.group);
      const uint16_t* qrow = a.q + ((int64_t)(b * a.s_q + i) * a.h_q + h) * D;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        qop[mb][kk] = *reinterpret_cast<const u32x4*>(qrow + qk_d<Q8>(kk, qd));
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qop[mb][kk] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  float sc = a.scale_log2;
  if constexpr (Q8) sc *= a.k_scale[b * a.h_kv + g];
  const float vsc = Q8 ? a.v_scale[b * a.h_kv + g] : 1.f;

  // Elementwise gate of this wave's rows (final output only), for the
  // variants that write O from registers and have registers to spare:
  // loaded here, used in the epilogue.
  constexpr bool GATE_AHEAD = Q8 && !VALU && MB == 1 && LAZY;
  uint2 gpre[GATE_AHEAD ? NB : 1];
  if constexpr (GATE_AHEAD) {
    const int r = rbase + m16;
    const int i = min(r, a.rows - 1) / a.group;
    const int h = g * a.group + (min(r, a.rows - 1) - i * a.group);
    const bool want = fin && a.gate_mode == kGateElementwise && r < a.rows && (SHARED || wph == 1);
    const int64_t obase = ((int64_t)(b * a.s_q + i) * a.h_q + h) * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      gpre[nb] = want ? *reinterpret_cast<const uint2*>(a.gate + obase + 16 * nb + 4 * qd) : uint2{0u, 0u};
  }

  if constexpr (INDIRECT) {
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (btc_on) {
#pragma unroll
      for (int k = 0; k < BTR; ++k) {
        const int p = threadIdx.x + k * NT;
        if (p < npg) btc[p] = btv[k];
      }
      __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int p = threadIdx.x + k * NT;
      if (p < a.chunk) {
        int32_t row = 0;
        if (tk[k] >= 0) {
          if (btc_on) {
            const int64_t r = ((int64_t)btc[tk[k] >> a.page_shift] << a.page_shift) +
                              (tk[k] & ((1 << a.page_shift) - 1));
            row = (int32_t)min(max(r, (int64_t)0), a.kv_rows - 1);
          } else {
            row = (int32_t)token_row(a, b, tk[k], base);
          }
        }
        trow[p] = row;
        ttok[p] = tk[k];
      }
    }
    __syncthreads();
  }

  if constexpr (LAZY && !VALU) {
    // LAZY variants apply the multiplier inside the exponent (one FMA per
    // score), which needs it positive: a negative one moves its sign into Q
    // (exact for bf16), and a zero one (a zero k_scale) becomes the smallest
    // normal float, which leaves every score zero to within rounding.
    if (sc < 0.f) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qop[mb][kk] ^= 0x80008000u;
      sc = -sc;
    }
    sc = fmaxf(sc, 1.17549435e-38f);
  }
  if constexpr (QLDS) {
    // Lane `lane` of k-step kk of block mb reads its B operand from
    // qbuf[(mb * KK + kk) * 64 + lane]: 16 consecutive bytes per lane, no
    // bank conflicts.  One wave of the head writes it (the other waves hold
    // the same values).
    if (sub == 0) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qbuf[(mb * KK + kk) * 64 + lane] = qop[mb][kk];
    }
    __syncthreads();
  }

  f32x4 acc[VALU ? 1 : MB][NB];
  float accv[VALU ? RV : 1][ELT];
  float mrun[NR], lrun[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    mrun[r] = -INFINITY;
    lrun[r] = 0.f;
  }
#pragma unroll
  for (int mb = 0; mb < (VALU ? 1 : MB); ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < (VALU ? RV : 1); ++r)
#pragma unroll
    for (int e = 0; e < ELT; ++e) accv[r][e] = 0.f;

  // Staged K and V tiles: one per wave, or (rows shared) two per head,
  // alternating by tile parity.
  unsigned char* wtiles = tiles + (SHARED ? 2 * hs : wave) * wave_tile_bytes(D, Q8);
  u32x4* kt = reinterpret_cast<u32x4*>(wtiles);
  uint16_t* vt = reinterpret_cast<uint16_t*>(wtiles + ktile_chunks(D, Q8) * 16);
  auto use_buffer = [&](int parity) __attribute__((always_inline)) {
    unsigned char* t = tiles + (2 * hs + parity) * wave_tile_bytes(D, Q8);
    kt = reinterpret_cast<u32x4*>(t);
    vt = reinterpret_cast<uint16_t*>(t + ktile_chunks(D, Q8) * 16);
  };
  const size_t head_off = (size_t)g * RB;
  const size_t row_bytes = (size_t)a.h_kv * RB;
  const int ltok = lane / CPR;                  // token of this lane within a wave-wide load
  const int lch = lane % CPR;                   // 16-byte chunk of this lane

  // Every helper lambda below is forced inline: one left out of line is
  // called with its captures in a stack frame, and every pointer it reads
  // from there is generic -- flat loads for HBM and LDS alike.
  auto row_of = [&](int p) __attribute__((always_inline)) -> int64_t {
    if constexpr (INDIRECT) {
      return trow[p - start];
    } else {
      return dense_row(a, p < end ? p : 0, base);
    }
  };

  // Issue one tile's loads: NLD wave-wide 16-byte loads each for K and V,
  // load i covering tokens i*TPI .. +TPI-1 of the tile in whole rows.  A
  // non-real tile (the prefetch slot after a wave's last tile) reads one
  // 16-byte location with every lane: no branch, no HBM traffic to speak of.
  auto load_tile = [&](int tile, u32x4 (&kr)[NLDP], u32x4 (&vr)[NLDP], bool real, int part = 0)
      __attribute__((always_inline)) {
    if (NLOADERS < SHARE && part >= NLOADERS) return;   // a wave with no part of the tile
    const int tb = start + tile * kTile;
    const int lane_on = real ? 1 : 0;
#pragma unroll
    for (int ii = 0; ii < NLDP; ++ii) {
      const int i = part * NLDP + ii;
      const int64_t row = row_of(real ? tb + i * TPI + ltok : start);
      const size_t off = (size_t)row * row_bytes + head_off + (size_t)(16 * lch * lane_on);
      kr[ii] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.k + off));
      vr[ii] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.v + off));
    }
  };

  // Stage a tile's K (raw chunks) and V (bf16) in this wave's LDS tiles.
  auto stage_tile = [&](const u32x4 (&kr)[NLDP], const u32x4 (&vr)[NLDP], int part = 0)
      __attribute__((always_inline)) {
#pragma unroll
    for (int ii = 0; ii < ((NLOADERS < SHARE && part >= NLOADERS) ? 0 : NLDP); ++ii) {
      const int i = part * NLDP + ii;
      const int tok = i * TPI + ltok;
      kt[tok * CPR + kchunk<CPR>(lch, tok)] = kr[ii];
      uint16_t* vrow = vt + tok * D;
      if constexpr (Q8) {
        // 16 codes = d [16 lch, +16) = one 16-element block
        uint32_t x0, x1, x2, x3, y0, y1, y2, y3;
        codes4_to_bf16x4<KVT>(vr[ii][0], x0, x1);
        codes4_to_bf16x4<KVT>(vr[ii][1], x2, x3);
        codes4_to_bf16x4<KVT>(vr[ii][2], y0, y1);
        codes4_to_bf16x4<KVT>(vr[ii][3], y2, y3);
        uint16_t* dst = vrow + 16 * vblk<D>(lch, tok);
        *reinterpret_cast<u32x4*>(dst) = u32x4{x0, x1, x2, x3};
        *reinterpret_cast<u32x4*>(dst + 8) = u32x4{y0, y1, y2, y3};
      } else {
        // 8 elements = d [8 lch, +8) = half of block lch / 2
        *reinterpret_cast<u32x4*>(vrow + 16 * vblk<D>(lch >> 1, tok) + 8 * (lch & 1)) = vr[ii];
      }
    }
    // The writes above must land before other lanes read them; a wave's LDS
    // operations execute in order, so a compiler barrier suffices.
    __builtin_amdgcn_wave_barrier();
    __asm__ __volatile__("" ::: "memory");
  };

  // Compute one staged tile (from LDS only).
  auto compute_tile = [&](int tile) __attribute__((always_inline)) {
    const int tb = start + tile * kTile;

    // S^T for both 16-token halves and every row block.  K operands: lane
    // (m16, qd) reads token 16 hb + m16, contraction chunk of k-step kk;
    // FP8 chunks are unpacked to bf16 in registers.  Wide heads (d = 256)
    // take the halves one after the other, so that only one half's operands
    // are live (their registers would otherwise spill).
    f32x4 s[2][MB];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int tok = hb * 16 + m16;
      u32x4 kop[KK];
#pragma unroll
      for (int j = 0; j < (Q8 ? KK / 2 : KK); ++j) {
        const u32x4 c = kt[tok * CPR + kchunk<CPR>(4 * j + qd, tok)];
        if constexpr (Q8) {
          uint32_t x0, x1, x2, x3, y0, y1, y2, y3;
          codes4_to_bf16x4<KVT>(c[0], x0, x1);
          codes4_to_bf16x4<KVT>(c[1], x2, x3);
          codes4_to_bf16x4<KVT>(c[2], y0, y1);
          codes4_to_bf16x4<KVT>(c[3], y2, y3);
          kop[2 * j] = u32x4{x0, x1, x2, x3};
          kop[2 * j + 1] = u32x4{y0, y1, y2, y3};
        } else {
          kop[j] = c;
        }
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          if constexpr (QLDS)
            c = mfma_16x16x32(kop[kk], qbuf[(mb * KK + kk) * 64 + lane], c);
          else
            c = mfma_16x16x32(kop[kk], qop[mb][kk], c);
        }
        s[hb][mb] = LAZY ? c : c * sc;        // LAZY: unscaled, sc > 0 is applied in the exponent
      }
      if constexpr (D == 256) __builtin_amdgcn_sched_barrier(0);
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
    // operand of the PV product.  LAZY variants move the running maximum
    // that the weights are taken against only when a tile's maximum exceeds
    // it by more than kLazyRescale (base 2): the weights then stay below
    // 2^kLazyRescale, and most tiles skip the rescale of the accumulators.
    // Any reference value gives the same O and LSE up to rounding, since l
    // and O are both taken against it; the decision is made for the whole
    // wave at once.
    u32x4 pB[MB];
    // Weights of one block against the reference -nmuse: fp32 row sum into
    // lrun, bf16 pairs into pB.
    auto weights = [&](int mb, float nmuse) __attribute__((always_inline)) {
      float pf[2][4];
      float ps = 0.f;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pf[hb][i] = fast_exp2(LAZY ? fmaf(s[hb][mb][i], sc, nmuse) : s[hb][mb][i] + nmuse);
          ps += pf[hb][i];
        }
      lrun[mb] += ps;
      pB[mb] = u32x4{pack_bf16(pf[0][0], pf[0][1]), pack_bf16(pf[0][2], pf[0][3]),
                     pack_bf16(pf[1][0], pf[1][1]), pack_bf16(pf[1][2], pf[1][3])};
    };
    auto tile_max = [&](int mb) __attribute__((always_inline)) -> float {
      const float mx = fmaxf(fmaxf(fmaxf(s[0][mb][0], s[0][mb][1]), fmaxf(s[0][mb][2], s[0][mb][3])),
                             fmaxf(fmaxf(s[1][mb][0], s[1][mb][1]), fmaxf(s[1][mb][2], s[1][mb][3])));
      const float m = max_xor32(max_xor16(mx));  // over the four lane groups of the column
      return LAZY ? m * sc : m;
    };
    if constexpr (LAZY) {
      float mt[MB];
      bool grow = false;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        mt[mb] = tile_max(mb);
        grow |= mt[mb] > mrun[mb] + kLazyRescale;
      }
      if (__any(grow)) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const float mnew = fmaxf(mrun[mb], mt[mb]);
          const float alpha = fast_exp2(mrun[mb] - (mnew == -INFINITY ? 0.f : mnew));
          lrun[mb] *= alpha;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc[mb][nb] *= alpha;
          mrun[mb] = mnew;
        }
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) weights(mb, mrun[mb] == -INFINITY ? 0.f : -mrun[mb]);
    } else {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const float mnew = fmaxf(mrun[mb], tile_max(mb));
        const float muse = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = fast_exp2(mrun[mb] - muse);
        lrun[mb] *= alpha;
        mrun[mb] = mnew;
        weights(mb, -muse);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] *= alpha;
      }
    }

    // V^T operand: lane (m16, qd) needs column d = 16 nb + m16 for tokens
    // 4 qd + k and 16 + 4 qd + k (k < 4), matching P's k-slot order.  One
    // ds_read_b64_tr_b16 delivers four of them: within each 16-lane group,
    // lane r supplies the address of 4 consecutive bf16 of row
    // M[r] = V[tok(r)][16 nb + 4 (r & 3) .. +3], tok(r) = 4 qd + r / 4, and
    // lane i receives M[4 k + i / 4][i % 4] = V[4 qd + k][16 nb + i].
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      uint32_t w[4];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int tok = 16 * hf + 4 * qd + (m16 >> 2);
        const uint2 t = lds_read_tr16(vt + tok * D + 16 * vblk<D>(nb, tok) + 4 * (m16 & 3));
        w[2 * hf] = t.x;
        w[2 * hf + 1] = t.y;
      }
      const u32x4 av = {w[0], w[1], w[2], w[3]};
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb][nb] = mfma_16x16x32(av, pB[mb], acc[mb][nb]);
    }
    // All reads of this tile's LDS are done before the next tile is staged.
    __builtin_amdgcn_wave_barrier();
    __asm__ __volatile__("" ::: "memory");
  };

  // VALU variant of compute_tile (RV rows).  Lane (ltok, lch) reads, for
  // each wave-wide row group i, chunk lch of token i*TPI + ltok from the
  // staged K and V tiles.
  auto compute_tile_valu = [&](int tile) __attribute__((always_inline)) {
    const int tb = start + tile * kTile;
    float sv[NLD][VALU ? RV : 1];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int tok = i * TPI + ltok;
      const u32x4 c = kt[tok * CPR + kchunk<CPR>(lch, tok)];
      uint32_t kp[ELT / 2];
      if constexpr (Q8) {
#pragma unroll
        for (int w = 0; w < 4; ++w) codes4_to_bf16x4<KVT>(c[w], kp[2 * w], kp[2 * w + 1]);
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) kp[w] = c[w];
      }
#pragma unroll
      for (int r = 0; r < RV; ++r) {
        float d = 0.f;
#pragma unroll
        for (int j = 0; j < ELT / 2; ++j) d = dot2_bf16(kp[j], qv[r][j], d);
        sv[i][r] = sum_low_lanes<CPR>(d) * sc;
      }
    }

    const bool need_mask = INDIRECT || (tb + kTile > end) || (a.causal && tb + kTile - 1 > n - a.s_q);
    if (need_mask) {
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int p = tb + i * TPI + ltok;
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
        for (int r = 0; r < RV; ++r)
          if (!ok || t > lim[r]) sv[i][r] = -INFINITY;
      }
    }

    // Online softmax per row: the tile maximum over every token slot; each
    // lane's sum covers its own slot (slots are summed after the last tile).
#pragma unroll
    for (int r = 0; r < RV; ++r) {
      float mx = sv[0][r];
#pragma unroll
      for (int i = 1; i < NLD; ++i) mx = fmaxf(mx, sv[i][r]);
      mx = max_high_lanes<CPR>(mx);
      const float mnew = fmaxf(mrun[r], mx);
      const float muse = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = fast_exp2(mrun[r] - muse);
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        sv[i][r] = fast_exp2(sv[i][r] - muse);
        ps += sv[i][r];
      }
      lrun[r] = lrun[r] * alpha + ps;
      mrun[r] = mnew;
#pragma unroll
      for (int e = 0; e < ELT; ++e) accv[r][e] *= alpha;
    }

    // PV: columns [ELT lch, +ELT) of each of the lane's tokens (bf16 in LDS).
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int tok = i * TPI + ltok;
      float vf[ELT];
#pragma unroll
      for (int h = 0; h < ELT / 8; ++h) {
        const int col = ELT * lch + 8 * h;     // first column of this 8-element half block
        const u32x4 w = *reinterpret_cast<const u32x4*>(vt + tok * D + 16 * vblk<D>(col >> 4, tok) + (col & 8));
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          vf[8 * h + 2 * c] = bf16_lo(w[c]);
          vf[8 * h + 2 * c + 1] = bf16_hi(w[c]);
        }
      }
#pragma unroll
      for (int r = 0; r < RV; ++r)
#pragma unroll
        for (int e = 0; e < ELT; ++e) accv[r][e] = fmaf(sv[i][r], vf[e], accv[r][e]);
    }
    __builtin_amdgcn_wave_barrier();
    __asm__ __volatile__("" ::: "memory");
  };

  auto compute = [&](int tile) __attribute__((always_inline)) {
    if constexpr (VALU)
      compute_tile_valu(tile);
    else
      compute_tile(tile);
  };

  // Keeps every load issued so far above this point: no IR pass may sink a
  // load past a possible memory write, and the machine scheduler may not
  // move instructions across the barrier.
  auto issue_fence = []() __attribute__((always_inline)) {
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // Software pipeline over the wave's tiles (tile, tile + wph, ...), two
  // register buffers: each step stages the current tile's registers into
  // LDS, at once refills the same registers with the tile two steps ahead
  // (a dummy past the end), then computes from LDS -- so two tiles of loads
  // are in flight while a tile is computed.  Every step is one straight-line
  // block, so the compiler cannot hoist work above the loads.  A pass takes
  // two real tiles and the loop has one exit test: every path back to the
  // loop head then has the same loads in flight (A older than B), which is
  // what lets the compiler's counter waits keep the younger tile in flight
  // (an exit between the two steps gives the loop a path on which A's
  // loads are the youngest, and every pass then waits for all loads).
  if constexpr (SHARED) {
    // Rows shared by the SHARE waves of a head: all walk every tile of the
    // chunk; wave `sub` loads and stages part `sub` of each tile into the
    // head's LDS buffer of the tile's parity (waves past NLOADERS have no
    // part and only compute).  A step stages the next tile's
    // part into the buffer the previous tile used, refills the staged
    // registers with the tile two beyond it, and computes the current tile;
    // the LDS-only barrier that ends the step makes the staged parts
    // visible and frees the computed buffer, while both register buffers
    // stay in flight.  Two tiles per pass, one exit test, and a tail for an
    // odd last tile.
    u32x4 kA[NLDP], vA[NLDP], kB[NLDP], vB[NLDP];
    if (ntiles > 0) {
      load_tile(0, kA, vA, true, sub);
      issue_fence();
      load_tile(1 < ntiles ? 1 : 0, kB, vB, 1 < ntiles, sub);
      issue_fence();
      use_buffer(0);
      stage_tile(kA, vA, sub);
      issue_fence();
      load_tile(2 < ntiles ? 2 : 0, kA, vA, 2 < ntiles, sub);
      issue_fence();
      lds_barrier();
      int tile = 0;
      // B holds tile + 1, A holds tile + 2 (dummies past the end); the
      // buffer of tile's parity holds tile.
      while (tile + 1 < ntiles) {
        use_buffer((tile + 1) & 1);
        stage_tile(kB, vB, sub);
        issue_fence();
        load_tile(tile + 3 < ntiles ? tile + 3 : 0, kB, vB, tile + 3 < ntiles, sub);
        issue_fence();
        use_buffer(tile & 1);
        compute(tile);
        issue_fence();
        lds_barrier();
        use_buffer(tile & 1);                       // tile + 2 has tile's parity
        stage_tile(kA, vA, sub);
        issue_fence();
        load_tile(tile + 4 < ntiles ? tile + 4 : 0, kA, vA, tile + 4 < ntiles, sub);
        issue_fence();
        use_buffer((tile + 1) & 1);
        compute(tile + 1);
        issue_fence();
        lds_barrier();
        tile += 2;
      }
      if (tile < ntiles) {
        use_buffer(tile & 1);
        compute(tile);
        issue_fence();
      }
    }
  } else if constexpr (NPART == 2) {
    // d = 256: the two register buffers hold the two halves of a tile.  Each
    // step stages both halves of the current tile, refilling each buffer at
    // once with the same half of the next tile, then computes -- so the
    // next tile (32 KiB of K and V per wave, as two d = 128 tiles) is in
    // flight while a tile is computed.  One exit test per step.
    u32x4 kA[NLDP], vA[NLDP], kB[NLDP], vB[NLDP];
    int tile = sub;
    if (tile < ntiles) {
      load_tile(tile, kA, vA, true, 0);
      issue_fence();
      load_tile(tile, kB, vB, true, 1);
      issue_fence();
      while (true) {
        const int next = tile + wph;
        const bool real = next < ntiles;
        stage_tile(kA, vA, 0);
        issue_fence();
        load_tile(real ? next : tile, kA, vA, real, 0);
        issue_fence();
        stage_tile(kB, vB, 1);
        issue_fence();
        load_tile(real ? next : tile, kB, vB, real, 1);
        issue_fence();
        compute(tile);
        issue_fence();
        if (!real) break;
        tile = next;
      }
    }
  } else {
    u32x4 kA[NLD], vA[NLD], kB[NLD], vB[NLD];
    int tile = sub;
    if (tile < ntiles) {
      load_tile(tile, kA, vA, true);
      issue_fence();  // keep the first tile's loads older than the second's
      const bool second = tile + wph < ntiles;
      load_tile(second ? tile + wph : tile, kB, vB, second);
      issue_fence();
      while (tile + wph < ntiles) {  // A holds `tile`, B holds `tile + wph`, both real
        stage_tile(kA, vA);
        issue_fence();  // the staged registers are dead before they are refilled
        int ahead = tile + 2 * wph;
        bool real = ahead < ntiles;
        load_tile(real ? ahead : tile, kA, vA, real);
        issue_fence();
        compute(tile);
        issue_fence();
        stage_tile(kB, vB);
        issue_fence();
        ahead = tile + 3 * wph;
        real = ahead < ntiles;
        load_tile(real ? ahead : tile, kB, vB, real);
        issue_fence();
        compute(tile + wph);
        issue_fence();
        tile += 2 * wph;
      }
      if (tile < ntiles) {  // an odd last tile, in A (B holds a dummy)
        stage_tile(kA, vA);
        issue_fence();
        compute(tile);
        issue_fence();
      }
    }
  }

  // Row sums over the four lane groups (MFMA) or over the token slots
  // (VALU, which also sums its accumulators over them).
  if constexpr (VALU) {
#pragma unroll
    for (int r = 0; r < RV; ++r) {
      lrun[r] = sum_high_lanes<CPR>(lrun[r]);
#pragma unroll
      for (int e = 0; e < ELT; ++e) accv[r][e] = sum_high_lanes<CPR>(accv[r][e]);
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) lrun[mb] = sum_xor32(sum_xor16(lrun[mb]));
  }

  if (SHARED || (!VALU && LAZY && wph == 1)) {
    // Each wave holds complete rows (MB blocks of 16 of its head's group):
    // with rows shared, or with one wave per head (HPW = 4), no merge is
    // needed (the variants with the most accumulators keep the merge, whose
    // code they are built around).  Normalise and write them from
    // registers.  Lane (m16, qd) of block mb has row rbase + 16 mb + m16,
    // columns 16 nb + 4 qd .. +3.
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = rbase + mb * 16 + m16;
      if (r >= a.rows) continue;
      const float m = mrun[mb], l = lrun[mb];
      const bool empty = (m == -INFINITY);
      const float inv = empty ? 0.f : vsc / l;
      const float lse2 = empty ? -INFINITY : m + __log2f(l);
      const int i = r / a.group;
      const int h = g * a.group + (r - i * a.group);
      if (fin) {
        const int64_t obase = ((int64_t)(b * a.s_q + i) * a.h_q + h) * D;
        const float sgh =
            a.gate_mode == kGateHeadwise ? sigmoidf_(bf16_lo(a.gate[(int64_t)(b * a.s_q + i) * a.h_q + h])) : 1.f;
        // Elementwise gates: every load issued before the first is used
        // (or loaded before the tile loop).
        uint2 gw[NB];
        const bool egate = a.gate_mode == kGateElementwise;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          if constexpr (GATE_AHEAD)
            gw[nb] = gpre[nb];
          else
            gw[nb] = egate ? *reinterpret_cast<const uint2*>(a.gate + obase + 16 * nb + 4 * qd) : uint2{0u, 0u};
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int col = 16 * nb + 4 * qd;
          float o[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) o[c] = acc[mb][nb][c] * inv * sgh;
          if (egate) {
            o[0] *= sigmoidf_(bf16_lo(gw[nb].x));
            o[1] *= sigmoidf_(bf16_hi(gw[nb].x));
            o[2] *= sigmoidf_(bf16_lo(gw[nb].y));
            o[3] *= sigmoidf_(bf16_hi(gw[nb].y));
          }
          *reinterpret_cast<uint2*>(a.o + obase + col) = uint2{pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
        }
        if (qd == 0) a.lse[((int64_t)b * a.h_q + h) * a.s_q + i] = lse2 * 0.69314718055994530942f;
      } else {
        const int64_t prow = b * a.part_sb + g * a.part_sg + split * a.part_ss + r;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          *reinterpret_cast<f32x4*>(a.o_part + prow * D + 16 * nb + 4 * qd) = acc[mb][nb] * inv;
        if (qd == 0) a.lse_part[prow] = lse2;
      }
    }
  } else {
    // Merge the waves of each head, one 16-row block at a time, and write.
    float* wacc = reinterpret_cast<float*>(tiles);
    float* wm = wstat;
    float* wl = wstat + NW * 16;
    const bool final_out = fin;
    constexpr int D8 = D / 8;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb * 16 >= a.rows) break;
      __syncthreads();
      if constexpr (VALU) {
        if (lane == 0) {
#pragma unroll
          for (int r = 0; r < RV; ++r) {
            wm[wave * 16 + r] = mrun[r];
            wl[wave * 16 + r] = lrun[r];
          }
        }
        if (ltok == 0) {
#pragma unroll
          for (int r = 0; r < RV; ++r)
#pragma unroll
            for (int e = 0; e < ELT; e += 4)
              *reinterpret_cast<f32x4*>(wacc + (wave * 16 + r) * WST + ELT * lch + e) =
                  f32x4{accv[r][e], accv[r][e + 1], accv[r][e + 2], accv[r][e + 3]};
        }
      } else {
        if (qd == 0) {
          wm[wave * 16 + m16] = mrun[mb];
          wl[wave * 16 + m16] = lrun[mb];
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          *reinterpret_cast<f32x4*>(wacc + (wave * 16 + m16) * WST + 16 * nb + 4 * qd) = acc[mb][nb];
      }
      __syncthreads();

      const int nrow = min(16, a.rows - mb * 16);
      for (int it = threadIdx.x; it < hpw * nrow * D8; it += NT) {
        const int hh = it / (nrow * D8);
        const int rem = it - hh * (nrow * D8);
        const int rl = rem / D8;
        const int d8 = rem - rl * D8;
        const int r = mb * 16 + rl;
        const int gg = g0 + hh;
        float M = -INFINITY;
        for (int k = 0; k < wph; ++k) M = fmaxf(M, wm[(hh + k * hpw) * 16 + rl]);
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = 0.f;
        float lse2 = -INFINITY;
        if (M != -INFINITY) {
          float sum = 0.f;
          for (int k = 0; k < wph; ++k) {
            const int w = hh + k * hpw;
            const float e = fast_exp2(wm[w * 16 + rl] - M);
            sum += e * wl[w * 16 + rl];
            const float* src = wacc + (w * 16 + rl) * WST + d8 * 8;
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              o[c] += e * x0[c];
              o[4 + c] += e * x1[c];
            }
          }
          const float inv = (Q8 ? a.v_scale[b * a.h_kv + gg] : 1.f) / sum;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] *= inv;
          lse2 = M + __log2f(sum);
        }
        const int i = r / a.group;
        const int h = gg * a.group + (r - i * a.group);
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
          const int64_t prow = b * a.part_sb + gg * a.part_sg + split * a.part_ss + r;
          float* dst = a.o_part + prow * D + d8 * 8;
          *reinterpret_cast<f32x4*>(dst) = f32x4{o[0], o[1], o[2], o[3]};
          *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4], o[5], o[6], o[7]};
          if (d8 == 0) a.lse_part[prow] = lse2;
        }
      }
    }
  }
  if constexpr (!PACKED) break;
  __syncthreads();  // the next segment stages tiles where the merge just read
  }
}

// LSE combine.  With M = max_s lse_s (base 2),
// O = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M) and
// LSE = ln 2 * (M + log2 sum_s 2^(lse_s - M)); empty splits (-inf) weigh 0.
// A workgroup takes rows [rb * (x / cb), +rb) of one (KV head, request) and
// column slice x % cb (D / cb columns); its threads are (split lane sg, row,
// column quad), the column quad fastest, so a wave-wide load reads whole
// 16-quad runs of a partial row.  Thread sg owns splits sg, sg + SG, ...: it
// issues all their loads at once and merges them with a private running
// maximum.  The split lanes inside a wave are then merged with cross-lane
// swaps, and the (at most four) wave results through LDS.  The host sizes
// rb, cb (and so SG) so that a thread has at most 16 splits.
template <int D>
__global__ void __launch_bounds__(kThreads) gqa_combine_kernel(DecodeArgs a) {
  constexpr int UNROLL = 8;          // splits per thread per round
  __shared__ f32x4 racc[kThreads];
  __shared__ float rm[kThreads], rsum[kThreads];
  const int cb = a.comb_cols, rb = a.comb_rows;
  const int q4c = D / 4 / cb;        // column quads per workgroup (8 or more)
  const int W = rb * q4c;            // (row, quad) items, a power of two
  const int SG = kThreads / W;       // split lanes
  const int tid = threadIdx.x;
  const int d4 = (blockIdx.x % cb) * q4c + tid % q4c;
  const int r = (blockIdx.x / cb) * rb + (tid / q4c) % rb;
  const int sg = tid / W;
  const int g = blockIdx.y, b = blockIdx.z;
  const int n = seq_len(a, b);
  // Splits [s_lo, s_lo + nsp) of request b.  Packed: the chunks its rows
  // meet; a request inside one chunk was finished by the partial kernel.
  int s_lo = 0, nsp;
  if (a.packed) {
    const int64_t r0 = a.cu_seqlens[b];
    const int64_t w0 = r0 >= 0 ? r0 / a.chunk : 0;
    const int64_t w1 = r0 >= 0 ? (r0 + n - 1) / a.chunk : 0;
    if (n > 0 && r0 >= 0 && w0 == w1 && w0 < a.num_splits) return;
    s_lo = (int)min<int64_t>(w0, a.num_splits - 1);
    nsp = n > 0 ? (int)(min<int64_t>(max<int64_t>(w1, w0), a.num_splits - 1) - s_lo + 1) : 0;
  } else {
    nsp = min(a.num_splits, (list_len(a, n) + a.chunk - 1) / a.chunk);
  }
  const bool live = r < a.rows;
  const int64_t first = b * a.part_sb + g * a.part_sg + s_lo * a.part_ss + (live ? r : 0);
  const float* lsep = a.lse_part + first;
  const float* op = a.o_part + first * D;

  float m = -INFINITY, l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = sg; s0 < nsp; s0 += SG * UNROLL) {
    float ls[UNROLL];
    f32x4 x[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t sidx = min(s0 + u * SG, nsp - 1);
      ls[u] = lsep[sidx * a.part_ss];
      x[u] = *reinterpret_cast<const f32x4*>(op + sidx * a.part_ss * D + d4 * 4);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      if (s0 + u * SG >= nsp) ls[u] = -INFINITY;
    float mx = m;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) mx = fmaxf(mx, ls[u]);
    // No branch on mx: a branch lets the compiler sink the row loads below
    // the LSE loads' wait.  Splits in [0, nsp) hold finite rows (an empty
    // one holds zeros), so a zero weight contributes exactly zero.
    const float mref = mx == -INFINITY ? 0.f : mx;
    const float alpha = fast_exp2(m - mref);
    acc *= alpha;
    l *= alpha;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const float w = fast_exp2(ls[u] - mref);
      l += w;
      acc += w * x[u];
    }
    m = mx;
  }

  // Split lanes of one item inside a wave sit at lane strides W .. 32.
  float M = m;
  for (int st = W; st < 64; st *= 2) M = max_lanes_xor(M, st);
  {
    const float w = (M == -INFINITY) ? 0.f : fast_exp2(m - M);
    l *= w;
    acc *= w;
  }
  for (int st = W; st < 64; st *= 2) {
    l = sum_lanes_xor(l, st);
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = sum_lanes_xor(acc[c], st);
  }
  // Wave results: item t's copies are at t + k * max(W, 64).
  const int layer = W > 64 ? W : 64;
  const int K = kThreads / layer;
  if (K > 1) {
    racc[tid] = acc;
    rm[tid] = M;
    rsum[tid] = l;
    __syncthreads();
    if (tid >= W) return;
    float MM = -INFINITY;
    for (int k = 0; k < K; ++k) MM = fmaxf(MM, rm[tid + k * layer]);
    l = 0.f;
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
    if (MM != -INFINITY) {
      for (int k = 0; k < K; ++k) {
        const float w = fast_exp2(rm[tid + k * layer] - MM);
        l += w * rsum[tid + k * layer];
        acc += w * racc[tid + k * layer];
      }
    }
    M = MM;
  }
  if (sg != 0 || !live) return;
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  float lse2 = -INFINITY;
  if (M != -INFINITY) {
    const float inv = 1.f / l;
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = acc[c] * inv;
    lse2 = M + __log2f(l);
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
  if (d4 == 0) a.lse[((int64_t)b * a.h_q + h) * a.s_q + i] = lse2 * 0.69314718055994530942f;
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

// ev0 / ev1 (may be null): events stamped by the dispatch itself at the
// kernel's start and end, so they time the kernel alone.
template <int D, int KVT, int MODE, int MB, int RV, int SHARE = 1, bool WIDE = false>
static hipError_t launch_partial_t(const DecodeArgs& a, dim3 grid, hipStream_t st, hipEvent_t ev0,
                                   hipEvent_t ev1) {
  const size_t lds = table_bytes(MODE == kIndirect, a.chunk);
  hipExtLaunchKernelGGL((gqa_partial_kernel<D, KVT, MODE, MB, RV, SHARE, WIDE>), grid,
                        dim3(64 * partial_waves<SHARE, WIDE>()), lds, st, ev0, ev1, 0, a);
  return hipGetLastError();
}

// rv > 0: the VALU variant for up to rv rows (1, 2, 4 or 8); share = 2, 4
// or 8: that many waves per head split the rows, mb 16-row blocks each;
// else mb MFMA blocks per wave, the waves of a head splitting the tiles
// (eight waves for eight heads when a.heads_per_wg is 8).
template <int D, int KVT, int MODE>
static hipError_t launch_mb(const DecodeArgs& a, int mb, int rv, int share, dim3 grid, hipStream_t st,
                            hipEvent_t ev0, hipEvent_t ev1) {
  // Row sharing: the combinations the planner picks (plan_tiling in the
  // host code) and no others.
  constexpr int NLD = TileShape<D, KVT != kKvBf16>::NLD;
  if (share == 2) {
    if constexpr (D == 256) return launch_partial_t<D, KVT, MODE, 1, 0, 2>(a, grid, st, ev0, ev1);
    if constexpr (NLD == 2) return launch_partial_t<D, KVT, MODE, 2, 0, 2>(a, grid, st, ev0, ev1);
    return hipErrorInvalidValue;
  }
  if (share == 4) {
    if constexpr (NLD % 4 == 0) {
      if (mb == 1) return launch_partial_t<D, KVT, MODE, 1, 0, 4>(a, grid, st, ev0, ev1);
      if constexpr (D <= 128) return launch_partial_t<D, KVT, MODE, 2, 0, 4>(a, grid, st, ev0, ev1);
    }
    return hipErrorInvalidValue;
  }
  if (share == 8) {
    if (mb == 1) return launch_partial_t<D, KVT, MODE, 1, 0, 8>(a, grid, st, ev0, ev1);
    if constexpr (D <= 128) return launch_partial_t<D, KVT, MODE, 2, 0, 8>(a, grid, st, ev0, ev1);
    return hipErrorInvalidValue;
  }
  // Q kept in LDS holds one KV head.
  if (q_in_lds(D, KVT != kKvBf16, mb, rv, share) && a.heads_per_wg != 1) return hipErrorInvalidValue;
  if (a.heads_per_wg == 8) {
    if constexpr (wide_fits(D, KVT != kKvBf16))
      if (mb == 1 && rv == 0) return launch_partial_t<D, KVT, MODE, 1, 0, 1, true>(a, grid, st, ev0, ev1);
    return hipErrorInvalidValue;
  }
  if constexpr (D <= 128) {
    if (rv > 0) {
      switch (rv) {
        case 1: return launch_partial_t<D, KVT, MODE, 1, 1>(a, grid, st, ev0, ev1);
        case 2: return launch_partial_t<D, KVT, MODE, 1, 2>(a, grid, st, ev0, ev1);
        case 4: return launch_partial_t<D, KVT, MODE, 1, 4>(a, grid, st, ev0, ev1);
        default: return launch_partial_t<D, KVT, MODE, 1, 8>(a, grid, st, ev0, ev1);
      }
    }
  }
  switch (mb) {
    case 1: return launch_partial_t<D, KVT, MODE, 1, 0>(a, grid, st, ev0, ev1);
    case 2: return launch_partial_t<D, KVT, MODE, 2, 0>(a, grid, st, ev0, ev1);
    default: return launch_partial_t<D, KVT, MODE, 4, 0>(a, grid, st, ev0, ev1);
  }
}

template <int D, int KVT>
static hipError_t launch_mode(const DecodeArgs& a, int mode, int mb, int rv, int share, dim3 grid,
                              hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  switch (mode) {
    case kIndirect: return launch_mb<D, KVT, kIndirect>(a, mb, rv, share, grid, st, ev0, ev1);
    case kPacked: return launch_mb<D, KVT, kPacked>(a, mb, rv, share, grid, st, ev0, ev1);
    default: return launch_mb<D, KVT, kDense>(a, mb, rv, share, grid, st, ev0, ev1);
  }
}

template <int D>
static hipError_t launch_kvt(const DecodeArgs& a, int kvt, int mode, int mb, int rv, int share, dim3 grid,
                             hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  switch (kvt) {
    case kKvFp8: return launch_mode<D, kKvFp8>(a, mode, mb, rv, share, grid, st, ev0, ev1);
    case kKvInt8: return launch_mode<D, kKvInt8>(a, mode, mb, rv, share, grid, st, ev0, ev1);
    default: return launch_mode<D, kKvBf16>(a, mode, mb, rv, share, grid, st, ev0, ev1);
  }
}

// mode: 0 dense, 1 indirect (paged / top-K), 2 packed ragged.  kvt: the
// stored K/V type (kKvBf16, kKvFp8, kKvInt8).
hipError_t launch_partial(const DecodeArgs& a, int D, int kvt, int mode, int mb, int rv, int share, dim3 grid,
                          hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (D == 256) return launch_kvt<256>(a, kvt, mode, mb, rv, share, grid, st, ev0, ev1);
  if (D == 128) return launch_kvt<128>(a, kvt, mode, mb, rv, share, grid, st, ev0, ev1);
  return launch_kvt<64>(a, kvt, mode, mb, rv, share, grid, st, ev0, ev1);
}

hipError_t launch_combine(const DecodeArgs& a, int D, dim3 grid, hipStream_t st) {
  if (D == 256)
    hipLaunchKernelGGL((gqa_combine_kernel<256>), grid, dim3(kThreads), 0, st, a);
  else if (D == 128)
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
