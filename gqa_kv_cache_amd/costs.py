"""Byte and FLOP accounting for GQA decode (pure Python, no device code).

* K/V footprint of one decode step, ``2 * B * H_kv * N * D * s`` (K and V,
  batch B, KV heads H_kv, length N, head dim D, s bytes per element) —
  "Attention Kernel Portability Across GPU Architectures", Decode section
  (the byte model; bandwidth = bytes / measured time).
* The K/V expansion the method avoids, ``2 * N * H_q * D * s`` per request —
  "When the K/V copy costs more than the attention", "The change, and how I
  measured it" (4 GiB per call at 64 query heads, d=128, 128K).
* Nominal FLOPs ``4 * B * TopK * H_q * D`` — "Sparse paged GQA decode
  attention with FP8 KV cache on SM89", Workload.

``minimum_bytes`` adds everything else a decode call must touch once: the
query, the output, the LSE, lengths / offsets / block-table entries /
top-K lists, FP8 scales and the gate.
"""

from __future__ import annotations

from typing import Optional, Sequence


def kv_bytes(batch: int, h_kv: int, n: int, d: int, s: int) -> int:
    return 2 * batch * h_kv * n * d * s


def expansion_bytes(n: int, h_q: int, d: int, s: int) -> int:
    return 2 * n * h_q * d * s


def nominal_flops(batch: int, topk: int, h_q: int, d: int) -> int:
    return 4 * batch * topk * h_q * d


def rate(bytes_or_flops: float, seconds: float) -> float:
    return bytes_or_flops / seconds


def kv_tokens(lengths: Sequence[int], topk: int = 0, distinct: Optional[Sequence[int]] = None) -> int:
    """K/V rows one KV head must read: every token of every request for
    dense attention; for a top-K list, its distinct valid entries."""
    if distinct is not None:
        return int(sum(distinct))
    if topk:
        return int(sum(min(int(n), topk) for n in lengths))
    return int(sum(int(n) for n in lengths))


def minimum_bytes(*, batch: int, s_q: int, h_q: int, h_kv: int, d: int,
                  kv_elem_bytes: int, tokens: int, layout: str,
                  pages_touched: int = 0, topk: int = 0, fp8_scales: bool = False,
                  gate: bool = False) -> int:
    """Bytes a decode call must move at least once (HBM roofline numerator).

    ``tokens`` is the number of K/V token rows read per KV head (summed over
    requests)."""
    kv = 2 * tokens * h_kv * d * kv_elem_bytes
    q = batch * s_q * h_q * d * 2
    o = batch * s_q * h_q * d * 2
    lse = batch * h_q * s_q * 4
    meta = 0
    if layout == "ragged":
        meta += (batch + 1) * 4
    else:
        meta += batch * 4
    if layout == "paged":
        meta += pages_touched * 4
    if topk:
        meta += batch * topk * 4
    if fp8_scales:
        meta += 2 * batch * h_kv * 4
    g = batch * s_q * h_q * d * 2 if gate else 0
    return kv + q + o + lse + meta + g


def decode_flops(*, tokens: int, h_q: int, d: int, s_q: int) -> int:
    """QK and PV multiply-adds, 2 FLOPs each: 4 * tokens * H_q * d * S_q
    (the causal tail is counted as dense)."""
    return 4 * tokens * h_q * d * s_q
