"""Pins for the append oracle (``oracle/append.py``): the E4M3FN encoder
against the format's own values and torch's independent float8 cast, the
int8 quantiser against hand-worked ties and clamps and a half-step error
bound, the first-block scales against their closed form, and the append
against caches the input generator builds directly."""

import numpy as np
import pytest
import torch

import gqa_inputs as gi
from oracle import append as A
from oracle import reference as R


def torch_e4m3fn(y_f32):
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(y_f32, np.float32))).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = np.array([R.e4m3fn_value(int(c)) for c in codes])
    vals[codes == 0x80] = -0.0
    assert np.array_equal(A.e4m3fn_encode(vals), codes)


def test_midpoints_go_to_even_mantissa():
    vals, codes = A._positive_codes()
    mids = (vals[:-1] + vals[1:]) / 2          # exact in float64
    got = A.e4m3fn_encode(mids)
    want = np.where(codes[:-1] % 2 == 0, codes[:-1], codes[1:])
    assert np.array_equal(got, want.astype(np.uint8))
    assert np.array_equal(A.e4m3fn_encode(-mids), (want | 0x80).astype(np.uint8))


def test_encoder_matches_torch_cast_on_every_bf16_value():
    # every finite bf16 bit pattern within +-448 (the cast's own domain here)
    x = A.bf16_bits_to_f32(np.arange(1 << 16, dtype=np.uint32).astype(np.uint16))
    x = x[np.isfinite(x) & (np.abs(x) <= 448)]
    assert np.array_equal(A.e4m3fn_encode(x.astype(np.float64)), torch_e4m3fn(x))


def test_quantize_matches_torch_cast_on_random_quotients():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200_000) * rng.choice([1e-3, 0.1, 1, 30], 200_000)).astype(np.float32)
    for s in (np.float32(0.0071), np.float32(1.0), np.float32(3.3e-3)):
        y = np.clip(x / s, np.float32(-448), np.float32(448))
        assert np.array_equal(A.quantize(x, float(s)), torch_e4m3fn(y))


def test_quantize_saturates():
    x = np.array([1e6, -1e6, 448.0 * 2, -448.0 * 2, 448.0, -448.0], dtype=np.float32)
    assert list(A.quantize(x, 1.0)) == [0x7E, 0xFE, 0x7E, 0xFE, 0x7E, 0xFE]
    assert list(A.quantize(x, 2.0)) == [0x7E, 0xFE, 0x7E, 0xFE, 0x76, 0xF6]   # 224: exponent field 14, mantissa 6


def test_first_block_scale_closed_form():
    x = np.array([[0.5, -3.0, 2.0], [1.0, 0.0, -0.25]], dtype=np.float32)
    s = A.first_block_scale(x)
    assert s == np.float32(3.0) / np.float32(448.0)
    codes = A.quantize(x, float(s))
    assert codes[0, 1] == 0xFE                 # the absmax element lands on -448
    assert A.first_block_scale(np.zeros((3, 4), np.float32)) == np.float32(1.0)


def test_int8_quantize_ties_to_even_and_clamps():
    # x / s exactly halfway between integers goes to the even one; beyond
    # +-127 clamps; a negative value that rounds to zero is code 0
    x = np.array([2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5, 126.5, 127.5, 300.0, -300.0, -0.4, 0.0],
                 dtype=np.float32)
    want = [2, 4, -2, -4, 0, 0, 2, 126, 127, 127, -127, 0, 0]
    assert A.quantize_int8(x, 1.0).view(np.int8).tolist() == want
    # the same through a scale: 5 / 2 = 2.5 -> 2, 7 / 2 = 3.5 -> 4
    assert A.quantize_int8(np.array([5.0, 7.0, -5.0], np.float32), 2.0).view(np.int8).tolist() == [2, 4, -2]


def test_int8_round_trip_error_within_half_a_step():
    # brute force over a range of bf16 values: |code * s - x| <= s / 2 inside
    # the representable range, and codes are monotone in x
    x = A.bf16_bits_to_f32(np.arange(1 << 16, dtype=np.uint32).astype(np.uint16))
    x = np.sort(x[np.isfinite(x) & (np.abs(x) <= 2.0)])
    s = np.float32(2.0 / 127)
    codes = A.quantize_int8(x, float(s)).view(np.int8).astype(np.int64)
    inside = np.abs(x.astype(np.float64)) <= 127 * float(s)
    err = np.abs(codes * np.float64(s) - x.astype(np.float64))
    assert np.all(err[inside] <= float(s) / 2 * (1 + 1e-6))
    assert np.all(np.diff(codes) >= 0)
    assert codes.min() == -127 and codes.max() == 127


def test_int8_first_block_scale_closed_form():
    x = np.array([[0.5, -3.0, 2.0], [1.0, 0.0, -0.25]], dtype=np.float32)
    s = A.first_block_scale(x, A.INT8_MAX)
    assert s == np.float32(3.0) / np.float32(127.0)
    codes = A.quantize_int8(x, float(s)).view(np.int8)
    assert codes[0, 1] == -127                 # the absmax element lands on -127
    assert A.first_block_scale(np.zeros((3, 4), np.float32), A.INT8_MAX) == np.float32(1.0)


def test_int8_append_is_read_back_by_the_decode_oracle_within_half_a_step():
    rng = np.random.default_rng(4)
    B, S, Hkv, d, cap = 2, 5, 3, 64, 8
    x = rng.standard_normal((B, S, Hkv, d)).astype(np.float32)
    k_new = gi.f32_to_bf16_bits(x)
    v_new = gi.f32_to_bf16_bits(-x)
    kc = np.zeros((B, cap, Hkv, d), np.uint8)
    kc2, vc2, ks, vs, lens = A.reference_append(k_cache=kc, v_cache=kc.copy(), k_new=k_new, v_new=v_new,
                                                seqlens=np.zeros(B, np.int32), layout=R.CONTIGUOUS,
                                                kv_dtype=R.INT8, capacity=cap, k_scale=np.zeros((B, Hkv), np.float32),
                                                v_scale=np.zeros((B, Hkv), np.float32), policy="first_block")
    assert lens.tolist() == [S, S]
    xb = A.bf16_bits_to_f32(k_new).astype(np.float64)
    back = R.int8_codes_to_f64(kc2[:, :S]) * ks[:, None, :, None]
    assert np.all(np.abs(back - xb) <= ks[:, None, :, None] / 2 * (1 + 1e-6))
    assert np.array_equal(kc2[:, S:], np.zeros_like(kc2[:, S:]))    # rows past the append untouched


def _split(w: gi.Workload, n_keep):
    """A cache holding only the first n_keep[b] tokens of each request of w,
    the rest of every row left as a sentinel, and the rows that follow."""
    s = w.spec
    B, Hkv, d = s.batch, s.h_kv, s.head_dim
    rows_k = w.k_cache.reshape(-1, Hkv, d)
    rows_v = w.v_cache.reshape(-1, Hkv, d)
    sentinel = 0x7F if s.kv_dtype == gi.KV_FP8 else 0x7FC0
    kc = np.full_like(w.k_cache, sentinel)
    vc = np.full_like(w.v_cache, sentinel)
    kr, vr = kc.reshape(-1, Hkv, d), vc.reshape(-1, Hkv, d)
    cap = w.k_cache.shape[1] if s.layout == gi.LAYOUT_CONTIGUOUS else 0
    for b in range(B):
        for t in range(int(n_keep[b])):
            r = R.physical_row(b, t, s.layout, capacity=cap, block_table=w.block_table, page_size=s.page_size)
            kr[r] = rows_k[r]
            vr[r] = rows_v[r]
    return kc, vc, cap


@pytest.mark.parametrize("layout", [gi.LAYOUT_CONTIGUOUS, gi.LAYOUT_PAGED])
def test_append_rebuilds_generated_bf16_cache(layout):
    # A cache of n tokens per request, with the last S of them taken out and
    # appended again, is the generator's cache row for row.
    S = 3
    spec = gi.Spec(name="app", batch=3, h_q=8, h_kv=2, head_dim=16, layout=layout, page_size=4,
                   fixed_lengths=(9, 3, 14))
    w = gi.build(spec, seed=11)
    n = w.seqlens.astype(np.int64)
    kc, vc, cap = _split(w, n - S)
    Hkv, d = spec.h_kv, spec.head_dim
    cap_w = w.k_cache.shape[1] if layout == gi.LAYOUT_CONTIGUOUS else 0
    k_new = np.zeros((spec.batch, S, Hkv, d), np.uint16)
    v_new = np.zeros_like(k_new)
    for b in range(spec.batch):
        for j in range(S):
            r = R.physical_row(b, int(n[b]) - S + j, layout, capacity=cap_w, block_table=w.block_table,
                               page_size=spec.page_size)
            k_new[b, j] = w.k_cache.reshape(-1, Hkv, d)[r]
            v_new[b, j] = w.v_cache.reshape(-1, Hkv, d)[r]
    k2, v2, _, _, lens = A.reference_append(k_cache=kc, v_cache=vc, k_new=k_new, v_new=v_new,
                                            seqlens=(n - S).astype(np.int32), layout=layout, kv_dtype=R.BF16,
                                            capacity=cap, block_table=w.block_table, page_size=spec.page_size)
    assert np.array_equal(lens, w.seqlens)
    full_k, full_v, _ = _split(w, n)
    assert np.array_equal(k2, full_k) and np.array_equal(v2, full_v)


def test_first_block_append_matches_generator_quantiser():
    # FP8: appending a whole block to empty requests gives the generator's
    # absmax/448 quantisation of the same values (torch's cast does the
    # rounding there).
    rng = np.random.default_rng(3)
    B, S, Hkv, d = 2, 40, 3, 32
    bits = gi.f32_to_bf16_bits(rng.standard_normal((B, S, Hkv, d)).astype(np.float32))
    vbits = gi.f32_to_bf16_bits((rng.standard_normal((B, S, Hkv, d)) * 7).astype(np.float32))
    cap = 64
    kc = np.zeros((B, cap, Hkv, d), np.uint8)
    vc = np.zeros_like(kc)
    k2, v2, ks, vs, lens = A.reference_append(
        k_cache=kc, v_cache=vc, k_new=bits, v_new=vbits, seqlens=np.zeros(B, np.int32), layout=R.CONTIGUOUS,
        kv_dtype=R.FP8, capacity=cap, k_scale=np.full((B, Hkv), 5.0, np.float32),
        v_scale=np.full((B, Hkv), 5.0, np.float32), policy="first_block")
    for src, out, sc in ((bits, k2, ks), (vbits, v2, vs)):
        x = A.bf16_bits_to_f32(src)
        amax = np.abs(x).max(axis=(1, 3))
        want_s = (amax / np.float32(448)).astype(np.float32)
        assert np.array_equal(sc, want_s)
        want = gi.quantize_e4m3fn(x, want_s[:, None, :, None])
        assert np.array_equal(out[:, :S], want)
        assert not out[:, S:].any()
    assert list(lens) == [S, S]


def test_later_appends_keep_the_scale_and_clamp():
    B, Hkv, d = 1, 1, 8
    kc = np.zeros((B, 8, Hkv, d), np.uint8)
    first = gi.f32_to_bf16_bits(np.full((B, 2, Hkv, d), 2.0, np.float32))
    k1, v1, ks, vs, lens = A.reference_append(k_cache=kc, v_cache=kc, k_new=first, v_new=first,
                                              seqlens=[0], layout=R.CONTIGUOUS, kv_dtype=R.FP8, capacity=8,
                                              k_scale=np.ones((1, 1), np.float32), v_scale=np.ones((1, 1), np.float32),
                                              policy="first_block")
    assert ks[0, 0] == np.float32(2.0) / np.float32(448)
    big = gi.f32_to_bf16_bits(np.full((B, 1, Hkv, d), 10.0, np.float32))
    k2, _, ks2, _, lens2 = A.reference_append(k_cache=k1, v_cache=v1, k_new=big, v_new=big, seqlens=lens,
                                              layout=R.CONTIGUOUS, kv_dtype=R.FP8, capacity=8, k_scale=ks,
                                              v_scale=vs, policy="first_block")
    assert ks2[0, 0] == ks[0, 0]                 # n > 0: the scale stays
    assert np.all(k2[0, 2] == 0x7E)              # 10 / (2/448) > 448: saturated
    assert np.array_equal(k2[0, :2], k1[0, :2])  # stored rows untouched
    assert list(lens2) == [3]


def test_append_writes_only_target_rows_paged():
    P, Hkv, d = 4, 2, 8
    pool = np.full((6, P, Hkv, d), 0x55, np.uint8)
    bt = np.array([[5, 2, 0], [1, 3, 4]], np.int32)
    k_new = gi.f32_to_bf16_bits(np.ones((2, 3, Hkv, d), np.float32))
    k2, _, _, _, _ = A.reference_append(k_cache=pool, v_cache=pool, k_new=k_new, v_new=k_new, seqlens=[3, 4],
                                        layout=R.PAGED, kv_dtype=R.FP8, block_table=bt, page_size=P,
                                        k_scale=np.ones((2, Hkv), np.float32), v_scale=np.ones((2, Hkv), np.float32))
    # request 0: tokens 3,4,5 -> page 5 slot 3, page 2 slots 0,1; request 1: 4,5,6 -> page 3 slots 0,1,2
    written = {(5, 3), (2, 0), (2, 1), (3, 0), (3, 1), (3, 2)}
    one = R.e4m3fn_value(0x38)
    assert one == 1.0
    for pg in range(6):
        for sl in range(P):
            want = 0x38 if (pg, sl) in written else 0x55
            assert np.all(k2[pg, sl] == want), (pg, sl)


def test_positions_without_a_row_are_not_written():
    B, Hkv, d, cap = 2, 1, 8, 4
    cache = np.full((B, cap, Hkv, d), 0x5555, np.uint16)
    new = np.full((B, 3, Hkv, d), 0x3F80, np.uint16)          # 1.0
    k2, _, _, _, lens = A.reference_append(k_cache=cache, v_cache=cache, k_new=new, v_new=new, seqlens=[2, 4],
                                           layout=R.CONTIGUOUS, kv_dtype=R.BF16, capacity=cap)
    assert np.all(k2[0, 2:] == 0x3F80) and np.all(k2[0, :2] == 0x5555)   # request 0: slots 2, 3; slot 4 is past
    assert np.all(k2[1] == 0x5555)                                       # request 1 is full: nothing written
    assert list(lens) == [5, 7]
    P = 2
    pool = np.full((3, P, Hkv, d), 0x5555, np.uint16)
    bt = np.array([[2, 9], [1, 0]], np.int32)                             # page 9 is outside the pool
    k3, _, _, _, _ = A.reference_append(k_cache=pool, v_cache=pool, k_new=new, v_new=new, seqlens=[1, 3],
                                        layout=R.PAGED, kv_dtype=R.BF16, block_table=bt, page_size=P)
    assert np.all(k3[2, 1] == 0x3F80)                                    # request 0, token 1
    assert np.all(k3[0, 1] == 0x3F80)                                    # request 1, token 3 (page 0, slot 1)
    assert np.all(k3[1] == 0x5555) and np.all(k3[2, 0] == 0x5555) and np.all(k3[0, 0] == 0x5555)


# ---------------------------------------------------------------------------
# Planted bugs in the append oracle: each must fail at least one pin above.
# ---------------------------------------------------------------------------

_PINS = [test_every_finite_code_round_trips, test_midpoints_go_to_even_mantissa,
         test_encoder_matches_torch_cast_on_every_bf16_value, test_quantize_matches_torch_cast_on_random_quotients,
         test_quantize_saturates, test_first_block_scale_closed_form,
         lambda: test_append_rebuilds_generated_bf16_cache(gi.LAYOUT_CONTIGUOUS),
         lambda: test_append_rebuilds_generated_bf16_cache(gi.LAYOUT_PAGED),
         test_first_block_append_matches_generator_quantiser, test_later_appends_keep_the_scale_and_clamp,
         test_append_writes_only_target_rows_paged, test_positions_without_a_row_are_not_written,
         test_int8_quantize_ties_to_even_and_clamps, test_int8_round_trip_error_within_half_a_step,
         test_int8_first_block_scale_closed_form, test_int8_append_is_read_back_by_the_decode_oracle_within_half_a_step]

_orig_encode = A.e4m3fn_encode
_orig_quantize = A.quantize
_orig_scale = A.first_block_scale
_orig_phys = A.physical_row


def _ties_away(y):
    vals, codes = A._positive_codes()
    y = np.asarray(y, dtype=np.float64)
    mag = np.abs(y)
    hi = np.minimum(np.searchsorted(vals, mag, side="left"), len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    c = np.where(vals[hi] - mag <= mag - vals[lo], codes[hi], codes[lo])
    return (c | (np.signbit(y).astype(np.int64) << 7)).astype(np.uint8)


def _truncate(y):
    vals, codes = A._positive_codes()
    y = np.asarray(y, dtype=np.float64)
    mag = np.abs(y)
    idx = np.searchsorted(vals, mag, side="right") - 1
    return (codes[idx] | (np.signbit(y).astype(np.int64) << 7)).astype(np.uint8)


def _no_sign(y):
    return _orig_encode(np.abs(np.asarray(y, dtype=np.float64)))


def _multiply_scale(x, scale):
    y = np.clip(np.asarray(x, np.float32) * np.float32(scale), -448, 448)
    return _orig_encode(y.astype(np.float64))


def _scale_over_max_code(x, qmax=A.E4M3FN_MAX):
    amax = np.float32(np.max(np.abs(np.asarray(x, np.float32))))
    return np.float32(amax / np.float32(240.0)) if amax > 0 else np.float32(1.0)


def _zero_scale_kept(x, qmax=A.E4M3FN_MAX):
    amax = np.float32(np.max(np.abs(np.asarray(x, np.float32))))
    return np.float32(amax / np.float32(qmax)) if amax > 0 else np.float32(0.0)


def _int8_ties_away(x, scale):
    y = (np.asarray(x, np.float32) / np.float32(scale)).astype(np.float64)
    r = np.clip(np.sign(y) * np.floor(np.abs(y) + 0.5), -127, 127)
    return r.astype(np.int64).astype(np.int8).view(np.uint8)


def _int8_clamp_128(x, scale):
    y = (np.asarray(x, np.float32) / np.float32(scale)).astype(np.float64)
    return np.clip(np.rint(y), -128, 127).astype(np.int64).astype(np.int8).view(np.uint8)


def _one_past(b, t, layout, **kw):
    return _orig_phys(b, t + 1, layout, **kw)


MUTATIONS = {
    "ties away from zero": ("e4m3fn_encode", _ties_away),
    "truncation": ("e4m3fn_encode", _truncate),
    "sign dropped": ("e4m3fn_encode", _no_sign),
    "scale multiplied": ("quantize", _multiply_scale),
    "scale over the wrong maximum": ("first_block_scale", _scale_over_max_code),
    "zero block gets scale 0": ("first_block_scale", _zero_scale_kept),
    "written one token late": ("physical_row", _one_past),
    "int8 ties away from zero": ("quantize_int8", _int8_ties_away),
    "int8 clamps to -128": ("quantize_int8", _int8_clamp_128),
}


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_append_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(A, attr, fn)
    failed = 0
    for pin in _PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError, ZeroDivisionError, FloatingPointError):
            failed += 1
    assert failed > 0, f"planted bug '{name}' passed every pin"
