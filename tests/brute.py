"""Brute-force decode attention for tiny inputs, written independently of
``oracle/`` so that it can pin it.

Differences from the oracle, on purpose:
  * stored values are decoded with torch's bfloat16 / float8_e4m3fn casts
    (library routines), not with bit arithmetic or a formula table;
  * the visible set is found by walking every *physical* cache row and
    mapping it back to (request, logical token) — the inverse of the
    oracle's forward address map;
  * the KV head of a query head comes from splitting the H_q heads into
    H_kv equal consecutive groups;
  * softmax is evaluated without max subtraction, LSE directly as
    log(sum exp), using ``math.fsum`` over Python floats;
  * a headwise gate is widened to the elementwise shape before use.
"""

from __future__ import annotations

import math
from collections import Counter

import numpy as np
import torch


def _decode_bf16(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def _decode_fp8(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _decode_int8(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.int8)
    return t.to(torch.float64).numpy()


def _inverse_rows(w):
    """Map every physical token row to (request, logical token) or None."""
    s = w.spec
    out = {}
    if s.layout == "contiguous":
        B, cap = w.k_cache.shape[0], w.k_cache.shape[1]
        for r in range(B * cap):
            b, t = divmod(r, cap)
            out[r] = (b, t)
    elif s.layout == "ragged":
        cu = w.cu_seqlens
        total = int(cu[-1])
        for r in range(total):
            b = int(np.searchsorted(cu, r, side="right")) - 1
            out[r] = (b, r - int(cu[b]))
    elif s.layout == "paged":
        P = s.page_size
        owner = {}
        for b in range(w.block_table.shape[0]):
            for j, p in enumerate(w.block_table[b]):
                owner[int(p)] = (b, j)
        pool = w.k_cache.shape[0]
        for p in range(pool):
            for slot in range(P):
                if p in owner:
                    b, j = owner[p]
                    out[p * P + slot] = (b, j * P + slot)
    return out


def brute_decode(w, softmax_scale=None, headwise_gate=None):
    """fp64 outputs (O [B, S_q, H_q, d], LSE [B, H_q, S_q]) of workload w.

    softmax_scale: the score multiplier (None: 1/sqrt(d)).  headwise_gate:
    bf16 bits [B, S_q, H_q] used instead of w.gate, one value per head; it
    is widened here to an elementwise gate by repeating each head's value
    over the d columns, so both gate shapes go through the same loop."""
    s = w.spec
    B, Sq, Hq, Hkv, d = s.batch, s.s_q, s.h_q, s.h_kv, s.head_dim
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    groups = np.array_split(np.arange(Hq), Hkv)
    head_of = {int(h): gi for gi, grp in enumerate(groups) for h in grp}
    dec = {"fp8_e4m3fn": _decode_fp8, "int8": _decode_int8}.get(s.kv_dtype, _decode_bf16)
    K = dec(w.k_cache).reshape(-1, Hkv, d)
    V = dec(w.v_cache).reshape(-1, Hkv, d)
    q = _decode_bf16(w.q)
    if headwise_gate is not None:
        assert headwise_gate.shape == (B, Sq, Hq)
        gate = np.repeat(_decode_bf16(headwise_gate)[:, :, :, None], d, axis=3)
    else:
        gate = _decode_bf16(w.gate) if w.gate is not None else None
    lens = w.seqlens if s.layout != "ragged" else np.diff(w.cu_seqlens)
    inv = _inverse_rows(w)
    mult = None
    if w.topk_idx is not None:
        mult = [Counter(int(t) for t in w.topk_idx[b]) for b in range(B)]
    O = np.zeros((B, Sq, Hq, d))
    LSE = np.zeros((B, Hq, Sq))
    for b in range(B):
        n = int(lens[b])
        for i in range(Sq):
            for h in range(Hq):
                g = head_of[h]
                terms = []  # (score, v_row)
                for r, bt in inv.items():
                    rb, t = bt
                    if rb != b or not (0 <= t < n):
                        continue
                    if s.causal and t > n - Sq + i:
                        continue
                    c = mult[b][t] if mult is not None else 1
                    if c == 0:
                        continue
                    kr = K[r, g]
                    vr = V[r, g]
                    if w.k_scale is not None:
                        kr = kr * float(w.k_scale[b, g])
                        vr = vr * float(w.v_scale[b, g])
                    x = scale * math.fsum(float(a) * float(bb) for a, bb in zip(q[b, i, h], kr))
                    for _ in range(c):
                        terms.append((x, vr))
                if not terms:
                    O[b, i, h] = 0.0
                    LSE[b, h, i] = -math.inf
                    continue
                den = math.fsum(math.exp(x) for x, _ in terms)
                LSE[b, h, i] = math.log(den)
                for c_ in range(d):
                    O[b, i, h, c_] = math.fsum(math.exp(x) * float(vr[c_]) for x, vr in terms) / den
                if gate is not None:
                    for c_ in range(d):
                        O[b, i, h, c_] *= 1.0 / (1.0 + math.exp(-gate[b, i, h, c_]))
    return O, LSE
