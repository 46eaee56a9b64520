"""Planted bugs in the oracle (on the CPU): each mutation must make at least
one pin fail.  This is the planted-bug method of "When the K/V copy costs
more than the attention" ("Why it closed, and the tests that merged"),
applied to the checker itself: the pins are only trusted if plausible
mistakes — a wrong head map, a swapped page/slot, a causal off-by-one, a
dropped term, a wrong sign or exponent bias — cannot pass them.
"""

import math

import numpy as np
import pytest

import oracle.reference as R
import pins

_orig_softmax = R.softmax_attend
_orig_phys = R.physical_row
_orig_vis = R.visible_positions
_orig_scale = R.score_scale
_orig_gate = R.gate_factor


def _lse_without_max(q, K, V, scale):
    o, lse = _orig_softmax(q, K, V, scale)
    if K.shape[0] == 0:
        return o, lse
    x = scale * (K @ q)
    return o, lse - float(x.max())   # forgot "+ m"


def _unnormalised(q, K, V, scale):
    o, lse = _orig_softmax(q, K, V, scale)
    if K.shape[0] == 0:
        return o, lse
    x = scale * (K @ q)
    return o * np.exp(x - x.max()).sum(), lse


def _swap_page_slot(b, t, layout, **kw):
    if layout == "paged":
        P = kw["page_size"]
        bt = kw["block_table"]
        return int(bt[b, t % P]) * P + t // P if t % P < bt.shape[1] else 0
    return _orig_phys(b, t, layout, **kw)


def _causal_off_by_one(b, i, n, s_q, causal, topk_idx=None):
    vis = _orig_vis(b, i, n, s_q, False, topk_idx)
    if causal:
        vis = [(k, t) for (k, t) in vis if t < n - s_q + i]
    return vis


def _combine_no_max(parts):
    d = parts[0][0].shape[0]
    live = [(o, l) for (o, l) in parts if l != -math.inf]
    if not live:
        return np.zeros(d), -math.inf
    tot = sum(math.exp(l) for (_, l) in live)
    out = sum(math.exp(l) * o for (o, l) in live)   # weights exp(lse_s), unnormalised
    return out, math.log(tot)


def _fp8_bias8(code):
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 15 and m == 7:
        return float("nan")
    sign = -1.0 if s else 1.0
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 8)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 8)


def _bf16_wrong_shift(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
    return b.view(np.float32).astype(np.float64)


def _int8_unsigned(codes):
    return np.asarray(codes, dtype=np.uint8).astype(np.float64)   # sign ignored


def _scale_ignored(head_dim, softmax_scale=None):
    return 1.0 / math.sqrt(head_dim)                # the caller's scale dropped


def _scale_abs(head_dim, softmax_scale=None):
    return abs(_orig_scale(head_dim, softmax_scale))  # sign of a given scale dropped


def _headwise_gate_b_h_i(gate, gate_mode, b, i, h):
    if gate_mode == "headwise":
        B, Sq, Hq = gate.shape
        flat = np.asarray(gate).reshape(B, Hq, Sq)    # read as [B, H_q, S_q]
        return R.sigmoid(R.bf16_bits_to_f64(flat[b, h, i]))
    return _orig_gate(gate, gate_mode, b, i, h)


def _headwise_gate_skipped(gate, gate_mode, b, i, h):
    if gate_mode == "headwise":
        return 1.0                                    # only the elementwise gate applied
    return _orig_gate(gate, gate_mode, b, i, h)


MUTATIONS = {
    "kv_head_(h//Hkv)%Hkv": ("kv_head", lambda h, hq, hkv: (h // hkv) % hkv),
    "kv_head_h//Hkv": ("kv_head", lambda h, hq, hkv: min(h // hkv, hkv - 1)),
    "kv_head_h%Hkv": ("kv_head", lambda h, hq, hkv: h % hkv),
    "paged_page_slot_swapped": ("physical_row", _swap_page_slot),
    "causal_off_by_one": ("visible_positions", _causal_off_by_one),
    "lse_missing_max": ("softmax_attend", _lse_without_max),
    "output_not_normalised": ("softmax_attend", _unnormalised),
    "combine_weights_exp_lse": ("combine", _combine_no_max),
    "sigmoid_sign_flipped": ("sigmoid", lambda x: 1.0 / (1.0 + np.exp(x))),
    "fp8_exponent_bias_8": ("e4m3fn_value", _fp8_bias8),
    "bf16_decode_shift_15": ("bf16_bits_to_f64", _bf16_wrong_shift),
    "int8_read_unsigned": ("int8_codes_to_f64", _int8_unsigned),
    "softmax_scale_ignored": ("score_scale", _scale_ignored),
    "softmax_scale_sign_dropped": ("score_scale", _scale_abs),
    "headwise_gate_read_b_h_i": ("gate_factor", _headwise_gate_b_h_i),
    "headwise_gate_not_applied": ("gate_factor", _headwise_gate_skipped),
}


@pytest.mark.parametrize("mut", sorted(MUTATIONS))
def test_mutation_is_caught(mut, monkeypatch):
    attr, fn = MUTATIONS[mut]
    monkeypatch.setattr(R, attr, fn)
    monkeypatch.setattr(R, "_E4M3FN", None)      # rebuild the FP8 table from the mutated formula
    failed = pins.failing_checks()
    assert failed, f"planted bug {mut} passed every pin"


def test_unmutated_oracle_passes_every_pin():
    assert pins.failing_checks() == []
