"""CPU oracle for appending new K/V rows to a cache, with FP8 E4M3FN or
int8 quantisation on write.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP path.

What the pages fix, and what is read into them:

* The cache stores FP8 E4M3FN codes with one scale per (request, KV head),
  a stored code meaning ``value(code) * scale`` -- "Sparse paged GQA decode
  attention with FP8 KV cache on SM89", sections "Workload" and
  "Implementations".  The decode oracle reads them that way.
* A quantised cache has to be written somewhere, and dequantising the whole
  cache for every step is the mistake "Profiling down to the register, then
  an extension that broke my assumptions twice" reports in its int8 KV-cache
  section: the fix it names is to convert tile by tile.  The write side
  here therefore touches only the appended rows, never rows already stored.
* Quantisation (a reading; the pages give no formula): ``code =
  RNE_e4m3fn(clamp(x / scale, -448, 448))`` with the quotient taken in
  IEEE float32, as the kernel computes it, because it decides an integer
  code.  Ties go to the code with an even mantissa; a value that rounds to
  zero keeps its sign (code 0x80 for negative).
* Int8 (a reading; the int8 KV-cache section of "Profiling down to the
  register, then an extension that broke my assumptions twice" gives no
  encoding): ``code = clamp(RNE_int(x / scale), -127, 127)``, the quotient
  again in IEEE float32, ties to the even integer; ``first_block`` scales
  are ``absmax / 127``.  The decode path reads any two's-complement code
  (-128 included) as ``code * scale``; the append never writes -128.
* Scale policies (a reading of a "streaming" scale): ``given`` -- the
  caller's scales are used as they are; ``first_block`` -- a request whose
  cache is empty before the append (n_b = 0) takes, per KV head, ``scale =
  absmax / 448`` over the rows it appends (float32 division; 1 when the
  absmax is 0), and every later append to it reuses that scale, clamping
  what falls outside +-448 * scale.  Stored codes are never re-scaled.
* Rows go to logical positions n_b .. n_b + S - 1 of request b, through the
  same physical-row map the decode path reads (contiguous or paged), and
  the new length is n_b + S.  A position with no row of its own -- past
  the request's capacity (contiguous), past its block-table row (paged),
  or mapped outside the cache -- is not written (the library's contract;
  the pages say nothing about overflow).

Parity pins live in ``tests/test_oracle_append.py``.
"""

from __future__ import annotations

import numpy as np

from .reference import CONTIGUOUS, PAGED, FP8, INT8, BF16, e4m3fn_value, physical_row

E4M3FN_MAX = 448.0
INT8_MAX = 127.0

_POS = None  # (values, codes) of the 127 finite non-negative E4M3FN codes, ascending


def _positive_codes():
    global _POS
    if _POS is None:
        codes = np.arange(0x7F, dtype=np.int64)          # 0x00 .. 0x7E (0x7F is NaN)
        vals = np.array([e4m3fn_value(int(c)) for c in codes], dtype=np.float64)
        assert np.all(np.diff(vals) > 0)
        _POS = (vals, codes)
    return _POS


def e4m3fn_encode(y: np.ndarray) -> np.ndarray:
    """Round finite float values with |y| <= 448 to the nearest E4M3FN code,
    ties to the code with an even mantissa (low bit 0).  The magnitude is
    rounded; the sign bit is copied from y (so -0.0 and negative values
    that round to zero give 0x80)."""
    vals, codes = _positive_codes()
    y = np.asarray(y, dtype=np.float64)
    if np.any(~np.isfinite(y)) or np.any(np.abs(y) > E4M3FN_MAX):
        raise ValueError("e4m3fn_encode takes finite values within +-448")
    mag = np.abs(y)
    hi = np.searchsorted(vals, mag, side="left")         # first value >= mag
    hi = np.minimum(hi, len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - vals[lo]
    d_hi = vals[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    exact = vals[hi] == mag
    c = np.where(exact | pick_hi, codes[hi], codes[lo])
    sign = np.signbit(y).astype(np.int64) << 7
    return (c | sign).astype(np.uint8)


def quantize(x_f32: np.ndarray, scale: float) -> np.ndarray:
    """FP8 codes of float32 values x under one scale: float32 quotient,
    clamp to +-448, round to nearest even."""
    with np.errstate(over="ignore"):          # an infinite quotient saturates below
        y = np.asarray(x_f32, dtype=np.float32) / np.float32(scale)
    y = np.clip(y, np.float32(-E4M3FN_MAX), np.float32(E4M3FN_MAX))
    return e4m3fn_encode(y.astype(np.float64))


def quantize_int8(x_f32: np.ndarray, scale: float) -> np.ndarray:
    """Int8 codes (as uint8 bytes, two's complement) of float32 values x under
    one scale: float32 quotient, round to the nearest integer with ties to
    even, clamp to +-127."""
    with np.errstate(over="ignore"):
        y = np.asarray(x_f32, dtype=np.float32) / np.float32(scale)
    r = np.clip(np.rint(y.astype(np.float64)), -INT8_MAX, INT8_MAX)
    return r.astype(np.int64).astype(np.int8).view(np.uint8)


def first_block_scale(x_f32: np.ndarray, qmax: float = E4M3FN_MAX) -> np.float32:
    """absmax / qmax in float32 (448 for FP8, 127 for int8), or 1 when every
    value is zero."""
    amax = np.float32(np.max(np.abs(np.asarray(x_f32, dtype=np.float32)))) if np.size(x_f32) else np.float32(0)
    return np.float32(amax / np.float32(qmax)) if amax > 0 else np.float32(1.0)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def reference_append(*, k_cache, v_cache, k_new, v_new, seqlens, layout: str, kv_dtype: str,
                     capacity: int = 0, block_table=None, page_size: int = 16,
                     k_scale=None, v_scale=None, policy: str = "given"):
    """Append k_new / v_new (bf16 bits [B, S, H_kv, d]) after each request's
    current length.  Returns new copies (k_cache, v_cache, k_scale, v_scale,
    seqlens_out); the inputs are not modified.

    Caches are token-row arrays as the decode path reads them: contiguous
    [B, S_cap, H_kv, d] or paged [pages, P, H_kv, d] (bf16 bits or FP8
    codes).  Logical token t of request b lives in physical row
    ``physical_row(b, t, ...)`` of the cache viewed as [rows, H_kv, d]."""
    if layout not in (CONTIGUOUS, PAGED):
        raise ValueError("append writes contiguous or paged caches")
    if kv_dtype not in (BF16, FP8, INT8):
        raise ValueError(kv_dtype)
    q8 = kv_dtype in (FP8, INT8)
    if policy not in ("given", "first_block"):
        raise ValueError(policy)
    k_new = np.asarray(k_new, dtype=np.uint16)
    v_new = np.asarray(v_new, dtype=np.uint16)
    B, S, Hkv, d = k_new.shape
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    rows_k = kc.reshape(-1, Hkv, d)
    rows_v = vc.reshape(-1, Hkv, d)
    ks = None if k_scale is None else np.array(k_scale, dtype=np.float32, copy=True)
    vs = None if v_scale is None else np.array(v_scale, dtype=np.float32, copy=True)
    lens = np.asarray(seqlens, dtype=np.int64)
    for b in range(B):
        n = int(lens[b])
        for g in range(Hkv):
            for new, rows, sc in ((k_new, rows_k, ks), (v_new, rows_v, vs)):
                block = new[b, :, g, :]                      # [S, d] bf16 bits
                if q8:
                    x = bf16_bits_to_f32(block)
                    if policy == "first_block" and n == 0:
                        sc[b, g] = first_block_scale(x, E4M3FN_MAX if kv_dtype == FP8 else INT8_MAX)
                    codes = quantize(x, float(sc[b, g])) if kv_dtype == FP8 else quantize_int8(x, float(sc[b, g]))
                for j in range(S):
                    t = n + j
                    if t < 0 or (layout == CONTIGUOUS and t >= capacity):
                        continue
                    if layout == PAGED and t // page_size >= np.asarray(block_table).shape[1]:
                        continue
                    r = physical_row(b, t, layout, capacity=capacity, block_table=block_table,
                                     page_size=page_size)
                    if not 0 <= r < rows.shape[0]:
                        continue
                    rows[r, g, :] = codes[j] if q8 else block[j]
    return kc, vc, ks, vs, (lens + S).astype(np.int32)
