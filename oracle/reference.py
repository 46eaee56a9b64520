"""CPU oracle for grouped-query attention at decode over a KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP path; both sides read their inputs from ``gqa_inputs``.

Everything here is plain float64 NumPy, written to be checked by eye against
the pages, with no blocking, fusion or reordering beyond the definition:

* head map ``g = h // (H_q // H_kv)`` — "When the K/V copy costs more than
  the attention", section "What I was looking at" (the kernels' own
  ``kv_head_idx``) and the head-mapping table in "Why it closed, and the
  tests that merged";
* native GQA equals the same inputs pre-expanded to H_q heads and run as
  multi-head attention — same page, "The change, and how I measured it" (the
  66-case bitwise check).  The oracle performs that expansion explicitly: for
  every query head it copies its KV head's visible rows into a private fp64
  array before computing anything;
* sparse attention over a per-request list of selected token positions, then
  a sigmoid gate on the output — "Sparse paged GQA decode attention with FP8
  KV cache on SM89", sections "Workload" and "Implementations" (the eager
  version gathers K/V, then runs matmul, softmax and the gate);
* FP8 E4M3FN K/V with one scale per (request, KV head): the stored value
  means ``code_value * scale`` (same page, "Implementations": the fused
  kernels fold ``k_scale`` into the score scale and apply ``v_scale`` once
  at the end, which is the same quantity in exact arithmetic);
* paging with 16-token pages addressed through a block table (same page,
  "Workload");
* an int8 K/V cache, dequantised inside attention rather than as a whole
  -- "Profiling down to the register, then an extension that broke my
  assumptions twice", int8 KV-cache section.  The page gives no encoding;
  the reading taken is the FP8 one with the integer format: a stored code
  (two's complement int8) means ``code * scale`` with one scale per
  (request, KV head).

Readings where the pages are silent (each is listed with its reason in the
design notes): LSE is the natural log-sum-exp of the *scaled* scores; a
query block of S_q tokens is aligned bottom-right (query i sits at position
n - S_q + i and sees tokens t <= n - S_q + i); a row with nothing visible
gives O = 0 and LSE = -inf; top-K entries outside [0, n) are masked and
duplicates count once per occurrence; the gate is elementwise with O's shape
(a headwise gate broadcasts over d); the paged pool is laid out
[pages, page_size, H_kv, d].

Parity pins for every function here live in ``tests/test_oracle_*.py``:
every branch -- each layout, top-K masking, causal blocks, FP8 and int8
codes, a given (also negative) softmax scale, the elementwise and the
headwise gate -- is checked against an independently written brute force
on tiny inputs, and planted bugs in each of them fail at least one pin.
Which gate shape the pages mean is still a reading (they name a gate
tensor beside the query and output, and a sigmoid after attention); both
shapes are built and pinned.
"""

from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

CONTIGUOUS = "contiguous"
RAGGED = "ragged"
PAGED = "paged"

FP8 = "fp8_e4m3fn"
INT8 = "int8"
BF16 = "bf16"


# ---------------------------------------------------------------------------
# Storage decoding (exact)
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 is the top half of an IEEE binary32: shift the 16 stored bits up
    and reinterpret.  Exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3fn_value(code: int) -> float:
    """Value of one OCP FP8 E4M3FN code: 1 sign bit, 4 exponent bits with
    bias 7, 3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); there is
    no infinity and S.1111.111 is NaN, so the largest finite value is 448."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    sign = -1.0 if s else 1.0
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3fn_table() -> np.ndarray:
    return np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


_E4M3FN = None


def int8_codes_to_f64(codes: np.ndarray) -> np.ndarray:
    """Two's complement bytes: 0x00..0x7F are 0..127, 0x80..0xFF are
    -128..-1.  Exact."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c >= 128, c - 256, c).astype(np.float64)


def fp8_codes_to_f64(codes: np.ndarray) -> np.ndarray:
    global _E4M3FN
    if _E4M3FN is None:
        _E4M3FN = e4m3fn_table()
    return _E4M3FN[np.asarray(codes, dtype=np.uint8)]


# ---------------------------------------------------------------------------
# Addressing
# ---------------------------------------------------------------------------

def kv_head(h: int, h_q: int, h_kv: int) -> int:
    """KV head shared by query head h: the group of G = H_q / H_kv
    consecutive query heads h = g*G .. g*G+G-1 reads KV head g."""
    return h // (h_q // h_kv)


def seq_length(b: int, layout: str, seqlens, cu_seqlens) -> int:
    if layout == RAGGED:
        return int(cu_seqlens[b + 1]) - int(cu_seqlens[b])
    return int(seqlens[b])


def physical_row(b: int, t: int, layout: str, *, capacity: int = 0,
                 cu_seqlens=None, block_table=None, page_size: int = 16) -> int:
    """Token row (index into the cache's leading token axes, before the KV
    head axis) holding logical token t of request b."""
    if layout == CONTIGUOUS:        # cache [B, S_cap, H_kv, d]
        return b * capacity + t
    if layout == RAGGED:            # cache [sum n_b, H_kv, d]
        return int(cu_seqlens[b]) + t
    if layout == PAGED:             # cache [pages, P, H_kv, d]
        return int(block_table[b, t // page_size]) * page_size + t % page_size
    raise ValueError(layout)


def visible_positions(b: int, i: int, n: int, s_q: int, causal: bool,
                      topk_idx=None) -> List[Tuple[int, int]]:
    """(list slot, logical token) pairs that query i of request b attends to.

    Dense: every token 0..n-1.  Sparse: the request's top-K list in order,
    dropping entries outside [0, n); duplicates stay.  Causal with S_q query
    tokens: query i sits at position n - S_q + i and sees t <= that."""
    if topk_idx is None:
        cand = [(t, t) for t in range(n)]
    else:
        cand = [(k, int(t)) for k, t in enumerate(topk_idx[b]) if 0 <= int(t) < n]
    if causal:
        last = n - s_q + i
        cand = [(k, t) for (k, t) in cand if t <= last]
    return cand


def resolve_rows(*, batch: int, s_q: int, layout: str, seqlens=None,
                 cu_seqlens=None, block_table=None, topk_idx=None,
                 page_size: int = 16, capacity: int = 0, causal: bool = False,
                 list_len: Optional[int] = None) -> np.ndarray:
    """int64 [B, S_q, L]: physical token row of each list slot, -1 where the
    slot is masked.  L = K for sparse lists, else the longest request."""
    if list_len is None:
        if topk_idx is not None:
            list_len = topk_idx.shape[1]
        else:
            list_len = max([seq_length(b, layout, seqlens, cu_seqlens) for b in range(batch)] + [0])
    out = np.full((batch, s_q, list_len), -1, dtype=np.int64)
    for b in range(batch):
        n = seq_length(b, layout, seqlens, cu_seqlens)
        for i in range(s_q):
            for k, t in visible_positions(b, i, n, s_q, causal, topk_idx):
                out[b, i, k] = physical_row(b, t, layout, capacity=capacity,
                                            cu_seqlens=cu_seqlens,
                                            block_table=block_table,
                                            page_size=page_size)
    return out


# ---------------------------------------------------------------------------
# Attention for one (request, query position, query head)
# ---------------------------------------------------------------------------

def softmax_attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Plain scaled-dot-product attention of one query vector over the rows
    of K and V (fp64).  Returns (out [d], lse) with lse = log sum exp of the
    scaled scores; an empty K gives (0, -inf)."""
    d = q.shape[0]
    if K.shape[0] == 0:
        return np.zeros(d, dtype=np.float64), -math.inf
    x = scale * (K @ q)
    m = x.max()
    w = np.exp(x - m)
    l = w.sum()
    out = (w @ V) / l
    return out, float(m + math.log(l))


def sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def score_scale(head_dim: int, softmax_scale: Optional[float] = None) -> float:
    """Multiplier of q.k: the caller's scale when one is given (None or 0
    means none), else 1/sqrt(d) -- the tiny workload's definition.  Any
    other value, negative ones included, is used as given: the pages fold
    one multiplier into the scores ("Sparse paged GQA decode attention with
    FP8 KV cache on SM89", section "Implementations") and nothing there
    restricts its sign."""
    return (1.0 / math.sqrt(head_dim)) if not softmax_scale else float(softmax_scale)


def gate_factor(gate, gate_mode: str, b: int, i: int, h: int):
    """sigmoid(gate) for the output row of request b, query i, head h: the
    d values gate[b, i, h, :] (elementwise gate, O's shape) or the one value
    gate[b, i, h] (headwise gate [B, S_q, H_q], the same for every column).
    Same page, section "Workload": a sigmoid gate applied after attention."""
    if gate_mode == "headwise":
        return sigmoid(bf16_bits_to_f64(gate[b, i, h]))
    return sigmoid(bf16_bits_to_f64(gate[b, i, h, :]))


def reference_decode(*, q, k_cache, v_cache, h_q: int, h_kv: int, head_dim: int,
                     s_q: int, layout: str, seqlens=None, cu_seqlens=None,
                     block_table=None, page_size: int = 16, topk_idx=None,
                     kv_dtype: str = BF16, k_scale=None, v_scale=None,
                     gate=None, gate_mode: str = "elementwise",
                     causal: bool = False, softmax_scale: Optional[float] = None,
                     rows: Optional[Iterable[Tuple[int, int, int]]] = None):
    """fp64 reference for one decode call.

    q: bf16 bits [B, S_q, H_q, d].  k_cache / v_cache: bf16 bits, or FP8 or
    int8 codes, in the layout named by ``layout``.  Returns (O [B, S_q, H_q, d] float64,
    LSE [B, H_q, S_q] float64).  ``rows`` restricts the work to a list of
    (b, i, h); other entries are left NaN."""
    B = q.shape[0]
    d = head_dim
    assert q.shape == (B, s_q, h_q, d)
    assert h_q % h_kv == 0
    scale = score_scale(d, softmax_scale)
    fp8 = kv_dtype == FP8
    int8 = kv_dtype == INT8
    capacity = k_cache.shape[1] if layout == CONTIGUOUS else 0
    # flatten the token axes: row-major [rows, H_kv, d]
    kf = k_cache.reshape(-1, h_kv, d)
    vf = v_cache.reshape(-1, h_kv, d)
    if rows is None:
        rows = [(b, i, h) for b in range(B) for i in range(s_q) for h in range(h_q)]
    O = np.full((B, s_q, h_q, d), np.nan, dtype=np.float64)
    LSE = np.full((B, h_q, s_q), np.nan, dtype=np.float64)
    for (b, i, h) in rows:
        g = kv_head(h, h_q, h_kv)
        n = seq_length(b, layout, seqlens, cu_seqlens)
        vis = visible_positions(b, i, n, s_q, causal, topk_idx)
        phys = [physical_row(b, t, layout, capacity=capacity, cu_seqlens=cu_seqlens,
                             block_table=block_table, page_size=page_size)
                for (_, t) in vis]
        idx = np.asarray(phys, dtype=np.int64)
        # explicit expansion: this query head's private copy of its KV rows
        if fp8:
            Kh = fp8_codes_to_f64(kf[idx, g, :]) * float(k_scale[b, g])
            Vh = fp8_codes_to_f64(vf[idx, g, :]) * float(v_scale[b, g])
        elif int8:
            Kh = int8_codes_to_f64(kf[idx, g, :]) * float(k_scale[b, g])
            Vh = int8_codes_to_f64(vf[idx, g, :]) * float(v_scale[b, g])
        else:
            Kh = bf16_bits_to_f64(kf[idx, g, :])
            Vh = bf16_bits_to_f64(vf[idx, g, :])
        qv = bf16_bits_to_f64(q[b, i, h, :])
        out, lse = softmax_attend(qv, Kh, Vh, scale)
        if gate is not None:
            out = out * gate_factor(gate, gate_mode, b, i, h)
        O[b, i, h, :] = out
        LSE[b, h, i] = lse
    return O, LSE


# ---------------------------------------------------------------------------
# Combining results over disjoint parts of a visible list
# ---------------------------------------------------------------------------

def combine(parts: Sequence[Tuple[np.ndarray, float]]):
    """Merge (out_s, lse_s) computed over disjoint subsets of one row's
    visible list into the result over their union: with M = max lse_s,
    LSE = M + log sum_s exp(lse_s - M) and out = sum_s exp(lse_s - LSE) out_s.
    Parts with lse = -inf (empty subsets) carry zero weight; if all are
    empty the result is (0, -inf)."""
    if not parts:
        raise ValueError("combine needs at least one part")
    d = parts[0][0].shape[0]
    live = [(o, l) for (o, l) in parts if l != -math.inf]
    if not live:
        return np.zeros(d, dtype=np.float64), -math.inf
    M = max(l for (_, l) in live)
    tot = sum(math.exp(l - M) for (_, l) in live)
    LSE = M + math.log(tot)
    out = np.zeros(d, dtype=np.float64)
    for (o, l) in live:
        out += math.exp(l - LSE) * o
    return out, LSE
