"""Seeded synthetic inputs for GQA decode over a KV cache.

This module is the only code shared by the CPU oracle (``oracle/``) and the
HIP path (``gqa_kv_cache_amd``).  It draws random numbers and encodes them
into the storage formats the decode step consumes (bf16 bit patterns, FP8
E4M3FN codes with per-(request, KV head) scales, ragged offsets, block
tables, top-K lists).  It contains no attention arithmetic: no head map, no
address resolution, no softmax, no decoding of stored values.

Workload shapes follow the pages:
  * "When the K/V copy costs more than the attention" (results table):
    batch 1, 64/8 heads, d=128, S_q=2, a 128K cache.
  * "Attention Kernel Portability Across GPU Architectures" (Decode):
    H_kv=8, d=128, KV length 512..16384, batch up to 64.
  * "Sparse paged GQA decode attention with FP8 KV cache on SM89" (Workload):
    256 requests, 32/8 heads, d=128, top-K 512, page 16, 32 pages/request,
    FP8 E4M3FN K/V, bf16 query/gate/output.

Every array is produced by ``numpy.random.Generator(PCG64(SeedSequence([seed,
stream])))`` with the fixed stream ids below, so a workload is a pure
function of its spec and seed.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

# Stream ids: one independent generator per input tensor.
STREAM_Q = 0
STREAM_K = 1
STREAM_V = 2
STREAM_GATE = 3
STREAM_LENGTHS = 4
STREAM_PAGES = 5
STREAM_TOPK = 6

LAYOUT_CONTIGUOUS = "contiguous"
LAYOUT_RAGGED = "ragged"
LAYOUT_PAGED = "paged"

KV_BF16 = "bf16"
KV_FP8 = "fp8_e4m3fn"
KV_INT8 = "int8"
INT8_MAX = 127.0

E4M3FN_MAX = 448.0


def stream_rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(stream)])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even) and
    return the 16-bit patterns as uint16.  Inputs are finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def normal_bf16_bits(rng: np.random.Generator, shape, chunk: int = 1 << 26,
                     mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """N(mean, std^2) float32 draws rounded to bf16, generated in chunks so
    multi-GiB caches do not need a float32 copy of the whole array."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        if mean != 0.0:
            x += np.float32(mean)
        out[s:e] = f32_to_bf16_bits(x)
    return out.reshape(shape)


def quantize_e4m3fn(x: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Encode float32 values x / scale as OCP FP8 E4M3FN codes (uint8), with
    round to nearest even and saturation to +-448.  ``scale`` broadcasts
    against ``x``.  Uses torch's CPU float8 cast for the rounding; values are
    clamped first so its overflow behaviour is never relied on."""
    import torch

    y = np.clip(np.asarray(x, np.float32) / np.asarray(scale, np.float32),
                -E4M3FN_MAX, E4M3FN_MAX).astype(np.float32)
    t = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def quantize_int8(x: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Encode float32 values x / scale as int8 codes (returned as their
    uint8 bytes): float32 quotient, clamp to +-127, round half to even."""
    y = np.clip(np.asarray(x, np.float32) / np.asarray(scale, np.float32), -INT8_MAX, INT8_MAX)
    return np.rint(y).astype(np.int8).view(np.uint8)


@dataclasses.dataclass
class Spec:
    """Shape and structure of one decode call."""
    name: str
    batch: int
    h_q: int
    h_kv: int
    head_dim: int
    s_q: int = 1
    seqlen: int = 1024                 # KV length when lengths are uniform
    min_len: Optional[int] = None      # ragged: lengths ~ U{min_len..max_len}
    max_len: Optional[int] = None
    layout: str = LAYOUT_CONTIGUOUS
    causal: bool = False
    page_size: int = 16
    pages_per_seq: Optional[int] = None  # paged: block-table width
    pool_pages: Optional[int] = None     # paged: physical pool size
    topk: int = 0                      # 0 = dense attention over the request
    topk_mode: str = "permutation"     # permutation | prefix | random_masked
    kv_dtype: str = KV_BF16
    gate: bool = False
    capacity: Optional[int] = None     # contiguous: S_cap >= max length
    v_mean: float = 0.0                # stress variant: V ~ N(v_mean, 1)
    q_std: float = 1.0                 # stress variant: sharper softmax
    fixed_lengths: Optional[tuple] = None  # explicit per-request lengths


@dataclasses.dataclass
class Workload:
    spec: Spec
    seed: int
    q: np.ndarray                       # uint16 bf16 bits [B, S_q, H_q, d]
    k_cache: np.ndarray                 # uint16 (bf16) or uint8 (fp8) codes
    v_cache: np.ndarray
    seqlens: np.ndarray                 # int32 [B]
    cu_seqlens: Optional[np.ndarray]    # int32 [B+1] (ragged)
    block_table: Optional[np.ndarray]   # int32 [B, pages_per_seq] (paged)
    topk_idx: Optional[np.ndarray]      # int32 [B, K] (sparse)
    k_scale: Optional[np.ndarray]       # float32 [B, H_kv] (fp8)
    v_scale: Optional[np.ndarray]
    gate: Optional[np.ndarray]          # uint16 bf16 bits [B, S_q, H_q, d]

    @property
    def max_seqlen(self) -> int:
        return int(self.seqlens.max()) if self.seqlens.size else 0

    def arrays(self) -> Dict[str, Optional[np.ndarray]]:
        return dict(q=self.q, k_cache=self.k_cache, v_cache=self.v_cache,
                    seqlens=self.seqlens, cu_seqlens=self.cu_seqlens,
                    block_table=self.block_table, topk_idx=self.topk_idx,
                    k_scale=self.k_scale, v_scale=self.v_scale, gate=self.gate)

    def params(self) -> Dict[str, object]:
        s = self.spec
        return dict(h_q=s.h_q, h_kv=s.h_kv, head_dim=s.head_dim, s_q=s.s_q,
                    layout=s.layout, causal=s.causal, page_size=s.page_size,
                    kv_dtype=s.kv_dtype)


def _lengths(spec: Spec, seed: int) -> np.ndarray:
    if spec.fixed_lengths is not None:
        ls = np.asarray(spec.fixed_lengths, dtype=np.int64)
        assert ls.shape == (spec.batch,)
        return ls.astype(np.int32)
    if spec.min_len is not None:
        rng = stream_rng(seed, STREAM_LENGTHS)
        return rng.integers(spec.min_len, spec.max_len, size=spec.batch,
                            endpoint=True).astype(np.int32)
    return np.full(spec.batch, spec.seqlen, dtype=np.int32)


def build(spec: Spec, seed: int) -> Workload:
    """Generate every input of one decode call from (spec, seed)."""
    B, Hq, Hkv, d, Sq = spec.batch, spec.h_q, spec.h_kv, spec.head_dim, spec.s_q
    lens = _lengths(spec, seed)
    q = normal_bf16_bits(stream_rng(seed, STREAM_Q), (B, Sq, Hq, d), std=spec.q_std)
    gate = normal_bf16_bits(stream_rng(seed, STREAM_GATE), (B, Sq, Hq, d)) if spec.gate else None
    rk = stream_rng(seed, STREAM_K)
    rv = stream_rng(seed, STREAM_V)
    cu = None
    bt = None
    k_scale = v_scale = None
    fp8 = spec.kv_dtype in (KV_FP8, KV_INT8)   # one-byte codes with per-(request, head) scales
    qmax, quant = (INT8_MAX, quantize_int8) if spec.kv_dtype == KV_INT8 else (E4M3FN_MAX, quantize_e4m3fn)

    if spec.layout == LAYOUT_CONTIGUOUS:
        cap = spec.capacity if spec.capacity is not None else max(int(lens.max()), 1)
        assert cap >= lens.max()
        shape = (B, cap, Hkv, d)
        token_groups = [(b, (slice(b, b + 1), slice(0, int(lens[b])))) for b in range(B)]
    elif spec.layout == LAYOUT_RAGGED:
        cu = np.zeros(B + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lens.astype(np.int64)).astype(np.int32)
        shape = (max(int(cu[-1]), 1), Hkv, d)
        token_groups = [(b, (slice(int(cu[b]), int(cu[b + 1])),)) for b in range(B)]
    elif spec.layout == LAYOUT_PAGED:
        P = spec.page_size
        need = int(max(1, -(-int(lens.max()) // P)))
        pps = spec.pages_per_seq if spec.pages_per_seq is not None else need
        assert pps >= need
        pool = spec.pool_pages if spec.pool_pages is not None else B * pps
        assert pool >= B * pps, "pool must hold every request's pages"
        perm = stream_rng(seed, STREAM_PAGES).permutation(pool).astype(np.int32)
        bt = np.ascontiguousarray(perm[: B * pps].reshape(B, pps))
        shape = (pool, P, Hkv, d)
        token_groups = None
    else:
        raise ValueError(spec.layout)

    if not fp8:
        kc = normal_bf16_bits(rk, shape)
        vc = normal_bf16_bits(rv, shape, mean=spec.v_mean)
    else:
        kf = rk.standard_normal(shape, dtype=np.float32)
        vf = rv.standard_normal(shape, dtype=np.float32)
        if spec.v_mean:
            vf += np.float32(spec.v_mean)
        k_scale = np.ones((B, Hkv), dtype=np.float32)
        v_scale = np.ones((B, Hkv), dtype=np.float32)
        kc = np.zeros(shape, dtype=np.uint8)
        vc = np.zeros(shape, dtype=np.uint8)
        for b in range(B):
            n = int(lens[b])
            if spec.layout == LAYOUT_PAGED:
                pages = bt[b, : -(-n // spec.page_size)] if n else bt[b, :0]
                sel = (pages,)
            else:
                sel = token_groups[b][1]
            for src, dst, sc in ((kf, kc, k_scale), (vf, vc, v_scale)):
                blk = src[sel]  # request b's storage (may include unused tail slots)
                if spec.layout == LAYOUT_PAGED:
                    flat = blk.reshape(-1, Hkv, d)[:n]
                elif spec.layout == LAYOUT_CONTIGUOUS:
                    flat = blk.reshape(-1, Hkv, d)[:n]
                else:
                    flat = blk.reshape(-1, Hkv, d)
                amax = np.abs(flat).max(axis=(0, 2)) if n else np.zeros(Hkv, np.float32)
                s = np.where(amax > 0, amax / np.float32(qmax), np.float32(1.0)).astype(np.float32)
                sc[b] = s
                dst[sel] = quant(blk, s[None, :, None] if blk.ndim == 3 else s[None, None, :, None])
        del kf, vf

    topk = None
    if spec.topk:
        K = spec.topk
        rng = stream_rng(seed, STREAM_TOPK)
        topk = np.full((B, K), -1, dtype=np.int32)
        for b in range(B):
            n = int(lens[b])
            if spec.topk_mode == "permutation":
                assert K == n, "a permutation top-K list covers every token"
                topk[b] = rng.permutation(n).astype(np.int32)
            elif spec.topk_mode == "prefix":
                m = min(K, n)
                topk[b, :m] = rng.choice(n, size=m, replace=False).astype(np.int32) if n else []
            elif spec.topk_mode == "random_masked":
                # indices drawn with replacement from [-2, n+2): exercises
                # masked entries (negative / out of range) and duplicates
                topk[b] = rng.integers(-2, n + 2, size=K).astype(np.int32)
            else:
                raise ValueError(spec.topk_mode)

    return Workload(spec=spec, seed=seed, q=q, k_cache=kc, v_cache=vc,
                    seqlens=lens.astype(np.int32), cu_seqlens=cu,
                    block_table=bt, topk_idx=topk, k_scale=k_scale,
                    v_scale=v_scale, gate=gate)


# ---------------------------------------------------------------------------
# The named workloads.  Seeds: 1, 2, 3, 33, 4, 5.
# ---------------------------------------------------------------------------

TINY = Spec(name="tiny_8x1_d64_1k", batch=1, h_q=8, h_kv=1, head_dim=64, s_q=1,
            seqlen=1024)
LONG_128K = Spec(name="long_64x8_d128_sq2_128k", batch=1, h_q=64, h_kv=8, head_dim=128,
                 s_q=2, seqlen=131072, causal=True)
RAGGED_B64 = Spec(name="ragged_b64_32x8_d128_512to16k", batch=64, h_q=32, h_kv=8,
                  head_dim=128, s_q=1, min_len=512, max_len=16384,
                  layout=LAYOUT_RAGGED)
RAGGED_B32_SQ8 = Spec(name="ragged_b32_32x8_d128_sq8_8k", batch=32, h_q=32, h_kv=8,
                      head_dim=128, s_q=8, seqlen=8192, layout=LAYOUT_RAGGED,
                      causal=True)
PAGED_B32 = Spec(name="paged_b32_64x8_d128_32k_p16", batch=32, h_q=64, h_kv=8,
                 head_dim=128, s_q=1, seqlen=32768, layout=LAYOUT_PAGED,
                 page_size=16, pages_per_seq=2048, pool_pages=65536)
SPARSE_FP8 = Spec(name="sparse_paged_fp8_gated_b256_32x8_top512", batch=256, h_q=32,
                  h_kv=8, head_dim=128, s_q=1, seqlen=512, layout=LAYOUT_PAGED,
                  page_size=16, pages_per_seq=32, pool_pages=8192, topk=512,
                  topk_mode="permutation", kv_dtype=KV_FP8, gate=True)

# The other shapes of the batch-1, S_q 2, 128K-token results table in "When
# the K/V copy costs more than the attention" (64/8 d128 is LONG_128K).
LONG_32X8 = Spec(name="long_32x8_d128_sq2_128k", batch=1, h_q=32, h_kv=8, head_dim=128,
                 s_q=2, seqlen=131072, causal=True)
LONG_8X1 = Spec(name="long_8x1_d128_sq2_128k", batch=1, h_q=8, h_kv=1, head_dim=128,
                s_q=2, seqlen=131072, causal=True)
LONG_64X8_D64 = Spec(name="long_64x8_d64_sq2_128k", batch=1, h_q=64, h_kv=8, head_dim=64,
                     s_q=2, seqlen=131072, causal=True)
LONG_32X2_D256 = Spec(name="long_32x2_d256_sq2_128k", batch=1, h_q=32, h_kv=2, head_dim=256,
                      s_q=2, seqlen=131072, causal=True)
# Multi-token query blocks: speculative verification of 16 draft tokens
# over the ragged S_q 8 batch's caches, and a 64-token prefill chunk
# against a 128K-token cache (512 query rows per KV head).
RAGGED_B32_SQ16 = Spec(name="ragged_b32_32x8_d128_sq16_8k", batch=32, h_q=32, h_kv=8,
                       head_dim=128, s_q=16, seqlen=8192, layout=LAYOUT_RAGGED, causal=True)
LONG_SQ64 = Spec(name="long_64x8_d128_sq64_128k", batch=1, h_q=64, h_kv=8, head_dim=128,
                 s_q=64, seqlen=131072, causal=True)

# The sparse FP8 workload's shape with an int8 cache (absmax/127 scales).
SPARSE_INT8 = dataclasses.replace(SPARSE_FP8, name="sparse_paged_int8_gated_b256_32x8_top512", kv_dtype=KV_INT8)

NAMED = {
    "tiny": (TINY, 1),
    "long128k": (LONG_128K, 2),
    "ragged": (RAGGED_B64, 3),
    "ragged_sq8": (RAGGED_B32_SQ8, 33),
    "paged": (PAGED_B32, 4),
    "sparse_fp8": (SPARSE_FP8, 5),
    "long_32x8": (LONG_32X8, 6),
    "long_8x1": (LONG_8X1, 7),
    "long_64x8_d64": (LONG_64X8_D64, 8),
    "long_32x2_d256": (LONG_32X2_D256, 9),
    "ragged_sq16": (RAGGED_B32_SQ16, 34),
    "long_sq64": (LONG_SQ64, 35),
    "sparse_int8": (SPARSE_INT8, 36),
}


def named(name: str) -> Workload:
    spec, seed = NAMED[name]
    return build(spec, seed)


def scaled(spec: Spec, **changes) -> Spec:
    """A smaller copy of a named spec (same heads, d, layout and dtype)."""
    return dataclasses.replace(spec, **changes)


# ---------------------------------------------------------------------------
# K/V append inputs: the new rows a model step produces, and the paged pool
# they are written into.
# ---------------------------------------------------------------------------

STREAM_SCALES = 7


@dataclasses.dataclass
class AppendWorkload:
    name: str
    seed: int
    k_new: np.ndarray          # uint16 bf16 bits [B, S, H_kv, d]
    v_new: np.ndarray
    seqlens: np.ndarray        # int32 [B], lengths before the append
    block_table: np.ndarray    # int32 [B, pages_per_seq]
    pool_pages: int
    page_size: int
    k_scale: np.ndarray        # float32 [B, H_kv] (used by the given-scale policy)
    v_scale: np.ndarray
    policy: str                # "given" or "first_block"


# name: (batch, new tokens, H_kv, d, existing tokens, pages per request, policy, seed)
APPEND_NAMED = {
    # one decode step of the sparse FP8 workload's cache: token 512 of each
    # of 256 requests (511 stored), 8 KV heads, d 128, pages of 16
    "append_decode": (256, 1, 8, 128, 511, 32, "given", 10),
    # a prefill-sized append: 32 empty requests receive 8192 rows each
    # (the ragged S_q 8 batch's cache), scales from the block
    "append_prefill": (32, 8192, 8, 128, 0, 512, "first_block", 11),
}


def append_named(name: str) -> AppendWorkload:
    B, S, Hkv, d, n0, pps, policy, seed = APPEND_NAMED[name]
    P = 16
    k_new = normal_bf16_bits(stream_rng(seed, STREAM_K), (B, S, Hkv, d))
    v_new = normal_bf16_bits(stream_rng(seed, STREAM_V), (B, S, Hkv, d))
    pool = B * pps
    bt = stream_rng(seed, STREAM_PAGES).permutation(pool).reshape(B, pps).astype(np.int32)
    # given scales: an absmax/448-sized scale for N(0, 1) rows, per (request, head)
    rs = stream_rng(seed, STREAM_SCALES)
    ks = (rs.uniform(4.0, 5.0, size=(B, Hkv)) / E4M3FN_MAX).astype(np.float32)
    vs = (rs.uniform(4.0, 5.0, size=(B, Hkv)) / E4M3FN_MAX).astype(np.float32)
    return AppendWorkload(name=name, seed=seed, k_new=k_new, v_new=v_new,
                          seqlens=np.full(B, n0, dtype=np.int32), block_table=bt, pool_pages=pool,
                          page_size=P, k_scale=ks, v_scale=vs, policy=policy)
