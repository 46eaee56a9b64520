"""Checks that pin the oracle to facts outside itself.

Each check raises AssertionError when the oracle disagrees.  They are kept
as plain functions so the mutation tests can run the same checks against an
oracle with a planted bug and confirm that at least one of them fails.
All oracle calls go through the module object so that monkeypatched
internals take effect.
"""

from __future__ import annotations

import dataclasses
import math
import os

import numpy as np
import torch

import gqa_inputs as gi
import oracle.reference as R
from brute import brute_decode

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def run_oracle(w, **kw):
    return R.reference_decode(**w.arrays(), **w.params(), **kw)


def tiny_spec(layout="contiguous", h_q=8, h_kv=4, d=8, s_q=1, causal=False,
              lengths=(5, 13), kv_dtype="bf16", topk=0, topk_mode="permutation",
              gate=False, page_size=4, capacity=None):
    B = len(lengths)
    kw = dict(name="tiny", batch=B, h_q=h_q, h_kv=h_kv, head_dim=d, s_q=s_q,
              layout=layout, causal=causal, kv_dtype=kv_dtype, topk=topk,
              topk_mode=topk_mode, gate=gate, page_size=page_size,
              fixed_lengths=tuple(lengths))
    if layout == "contiguous":
        kw["capacity"] = capacity if capacity is not None else max(lengths) + 3
    if layout == "paged":
        pps = -(-max(lengths) // page_size) + 1
        kw["pages_per_seq"] = pps
        kw["pool_pages"] = B * pps + 3
    return gi.Spec(**kw)


# ---------------------------------------------------------------------------

def check_head_map_truth_table():
    path = os.path.join(GOLDEN, "head_map_truth_table.txt")
    rows = 0
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        ratio, correct, buggy, same = [c.strip() for c in line.split("|")]
        hq, hkv = (int(x) for x in ratio.split("/"))
        want = [int(x) for x in correct.split()]
        got = [R.kv_head(h, hq, hkv) for h in range(hq)]
        assert got == want, (ratio, got, want)
        bug = [int(x) for x in buggy.split()]
        assert bug == [(h // hkv) % hkv for h in range(hq)]
        assert (want == bug) == (same == "yes")
        rows += 1
    assert rows == 4


def check_brute(spec, seed=0, atol=1e-12, softmax_scale=None, gate_mode="elementwise"):
    """Oracle against the brute force on one tiny workload.  A headwise gate
    takes each head's first gate value ([B, S_q, H_q])."""
    w = gi.build(spec, seed)
    if gate_mode == "headwise":
        hw = np.ascontiguousarray(w.gate[..., 0])
        O, L = R.reference_decode(**dict(w.arrays(), gate=hw), **w.params(), gate_mode="headwise",
                                  softmax_scale=softmax_scale)
        Ob, Lb = brute_decode(w, softmax_scale=softmax_scale, headwise_gate=hw)
    else:
        O, L = run_oracle(w, softmax_scale=softmax_scale)
        Ob, Lb = brute_decode(w, softmax_scale=softmax_scale)
    assert np.array_equal(np.isneginf(L), np.isneginf(Lb))
    fin = np.isfinite(Lb)
    assert np.allclose(L[fin], Lb[fin], rtol=0, atol=atol), np.abs(L[fin] - Lb[fin]).max()
    assert np.allclose(O, Ob, rtol=0, atol=atol), np.abs(O - Ob).max()


def _expand_to_mha(w):
    """Same inputs with K/V repeated so every query head has its own copy:
    query head h reads copy h of the repeated heads (numpy.repeat keeps the
    G copies of KV head g adjacent)."""
    s = w.spec
    G = s.h_q // s.h_kv
    axis = w.k_cache.ndim - 2
    k = np.ascontiguousarray(np.repeat(w.k_cache, G, axis=axis))
    v = np.ascontiguousarray(np.repeat(w.v_cache, G, axis=axis))
    ks = vs = None
    if w.k_scale is not None:
        ks = np.repeat(w.k_scale, G, axis=1)
        vs = np.repeat(w.v_scale, G, axis=1)
    w2 = dataclasses.replace(w, spec=dataclasses.replace(s, h_kv=s.h_q), k_cache=k,
                             v_cache=v, k_scale=ks, v_scale=vs)
    return w2


def check_gqa_equals_mha(spec, seed=0):
    w = gi.build(spec, seed)
    O, L = run_oracle(w)
    O2, L2 = run_oracle(_expand_to_mha(w))
    assert np.array_equal(O, O2, equal_nan=True)
    assert np.array_equal(L, L2, equal_nan=True)


def check_single_key(d=8):
    spec = tiny_spec(lengths=(1,), h_q=4, h_kv=2, d=d)
    w = gi.build(spec, 7)
    O, L = run_oracle(w)
    k = torch.from_numpy(w.k_cache.view(np.int16)).view(torch.bfloat16).double().numpy()
    v = torch.from_numpy(w.v_cache.view(np.int16)).view(torch.bfloat16).double().numpy()
    q = torch.from_numpy(w.q.view(np.int16)).view(torch.bfloat16).double().numpy()
    for h in range(4):
        g = [0, 0, 1, 1][h]
        assert np.array_equal(O[0, 0, h], v[0, 0, g]), "one visible key: O is that key's V row exactly"
        x = float(np.dot(q[0, 0, h], k[0, 0, g])) / math.sqrt(d)
        assert abs(L[0, h, 0] - x) < 1e-12


def check_zero_query():
    spec = tiny_spec(lengths=(9, 4))
    w = gi.build(spec, 3)
    w.q[...] = 0
    O, L = run_oracle(w)
    v = torch.from_numpy(w.v_cache.view(np.int16)).view(torch.bfloat16).double().numpy()
    for b, n in enumerate((9, 4)):
        for h in range(8):
            g = h // 2
            assert abs(L[b, h, 0] - math.log(n)) < 1e-12
            assert np.allclose(O[b, 0, h], v[b, :n, g].mean(axis=0), rtol=0, atol=1e-14)


def check_uniform_v():
    spec = tiny_spec(lengths=(11, 6))
    w = gi.build(spec, 4)
    w.v_cache[:] = w.v_cache[:, :1]          # every token row equal to row 0
    O, _ = run_oracle(w)
    v = torch.from_numpy(w.v_cache.view(np.int16)).view(torch.bfloat16).double().numpy()
    for b in range(2):
        for h in range(8):
            assert np.allclose(O[b, 0, h], v[b, 0, h // 2], rtol=1e-14, atol=0)


def check_gate_zero():
    spec = tiny_spec(lengths=(7, 3), gate=True)
    w = gi.build(spec, 5)
    w.gate[...] = 0                          # sigmoid(0) = 1/2 exactly
    O, L = run_oracle(w)
    wn = dataclasses.replace(w, gate=None)
    O0, L0 = run_oracle(wn)
    assert np.array_equal(O, O0 / 2)
    assert np.array_equal(L, L0)


def check_combine_partition(seed=11):
    rng = np.random.default_rng(seed)
    d, n = 8, 37
    q = rng.standard_normal(d)
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    o_ref, l_ref = R.softmax_attend(q, K, V, 0.4)
    for cuts in ([0, n], [0, 1, n], [0, 16, 17, 32, n], sorted(set([0, n] + list(rng.integers(0, n, 6))))):
        parts = [R.softmax_attend(q, K[a:b], V[a:b], 0.4) for a, b in zip(cuts[:-1], cuts[1:])]
        parts.append(R.softmax_attend(q, K[:0], V[:0], 0.4))  # an empty split
        o, l = R.combine(parts)
        assert abs(l - l_ref) < 1e-12
        assert np.allclose(o, o_ref, rtol=0, atol=1e-12)
    o, l = R.combine([R.softmax_attend(q, K[:0], V[:0], 0.4)] * 3)
    assert l == -math.inf and np.all(o == 0)


def check_page_permutation(seed=8):
    spec = tiny_spec(layout="paged", lengths=(9, 14), page_size=4)
    w = gi.build(spec, seed)
    O, L = run_oracle(w)
    pool = w.k_cache.shape[0]
    perm = np.random.default_rng(seed).permutation(pool)   # new slot of each page
    k2 = np.empty_like(w.k_cache)
    v2 = np.empty_like(w.v_cache)
    k2[perm] = w.k_cache
    v2[perm] = w.v_cache
    bt2 = perm[w.block_table].astype(np.int32)
    w2 = dataclasses.replace(w, k_cache=k2, v_cache=v2, block_table=bt2)
    O2, L2 = run_oracle(w2)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


def check_topk_identity_and_permutation(seed=9):
    spec = tiny_spec(layout="paged", lengths=(12, 12), page_size=4)
    w = gi.build(spec, seed)
    O, L = run_oracle(w)
    ident = np.tile(np.arange(12, dtype=np.int32), (2, 1))
    O1, L1 = run_oracle(dataclasses.replace(w, topk_idx=ident))
    assert np.array_equal(O, O1) and np.array_equal(L, L1)
    rng = np.random.default_rng(seed)
    perm = np.stack([rng.permutation(12) for _ in range(2)]).astype(np.int32)
    O2, L2 = run_oracle(dataclasses.replace(w, topk_idx=perm))
    assert np.allclose(O, O2, rtol=0, atol=1e-13) and np.allclose(L, L2, rtol=0, atol=1e-13)


def check_causal_prefix(seed=10):
    """Query i of an S_q block sees exactly the first n - S_q + i + 1 tokens:
    compare with a non-causal call on a shortened cache."""
    Sq = 3
    spec = tiny_spec(lengths=(8, 5), s_q=Sq, causal=True)
    w = gi.build(spec, seed)
    O, L = run_oracle(w)
    for i in range(Sq):
        lens = np.array([8 - Sq + i + 1, 5 - Sq + i + 1], dtype=np.int32)
        wi = dataclasses.replace(w, spec=dataclasses.replace(w.spec, causal=False),
                                 seqlens=lens)
        Oi, Li = run_oracle(wi)
        assert np.array_equal(O[:, i], Oi[:, i]) and np.array_equal(L[:, :, i], Li[:, :, i])


def check_fp8_table():
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = R.fp8_codes_to_f64(codes)
    assert np.array_equal(np.isnan(lib), np.isnan(tab))
    ok = ~np.isnan(lib)
    assert np.array_equal(lib[ok], tab[ok])
    assert np.nanmax(tab) == 448.0 and np.isnan(tab[0x7F]) and np.isnan(tab[0xFF])


def check_fp8_brute(seed=12):
    spec = tiny_spec(layout="paged", lengths=(16, 16), page_size=4, kv_dtype="fp8_e4m3fn",
                     topk=16, gate=True)
    check_brute(spec, seed)


def check_int8_table():
    # every byte against torch's int8 view of it (two's complement)
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.int8).to(torch.float64).numpy()
    assert np.array_equal(R.int8_codes_to_f64(codes), lib)
    assert R.int8_codes_to_f64(np.array([0x7F, 0x80, 0xFF], np.uint8)).tolist() == [127.0, -128.0, -1.0]


def check_int8_brute(seed=14):
    spec = tiny_spec(layout="paged", lengths=(16, 11), page_size=4, kv_dtype="int8", topk=16,
                     topk_mode="random_masked", gate=True, s_q=2, causal=True)
    check_brute(spec, seed)


def check_int8_quantiser_round_trip():
    # the generator's int8 codes times their scale recover every input within
    # half a step, and the absmax element lands exactly on +-127
    rng = np.random.default_rng(15)
    x = rng.standard_normal((64, 3, 16)).astype(np.float32)
    amax = np.abs(x).max(axis=(0, 2))
    s = (amax / np.float32(127.0)).astype(np.float32)
    codes = gi.quantize_int8(x, s[None, :, None])
    back = R.int8_codes_to_f64(codes) * s[None, :, None]
    assert np.all(np.abs(back - x) <= s[None, :, None] * 0.5 + 1e-6)
    assert set(np.abs(R.int8_codes_to_f64(codes)).max(axis=(0, 2)).tolist()) == {127.0}


def check_resolve_rows(seed=13):
    """resolve_rows agrees with the physical rows found by the brute force's
    inverse map, for every layout and with causal masking and top-K."""
    from brute import _inverse_rows
    cases = [
        tiny_spec(layout="contiguous", lengths=(5, 9), s_q=2, causal=True),
        tiny_spec(layout="ragged", lengths=(6, 0, 4)),
        tiny_spec(layout="paged", lengths=(9, 14), page_size=4, s_q=2, causal=True),
        tiny_spec(layout="paged", lengths=(9, 14), page_size=4, topk=10, topk_mode="random_masked"),
    ]
    for spec in cases:
        w = gi.build(spec, seed)
        s = w.spec
        cap = w.k_cache.shape[1] if s.layout == "contiguous" else 0
        rows = R.resolve_rows(batch=s.batch, s_q=s.s_q, layout=s.layout, seqlens=w.seqlens,
                              cu_seqlens=w.cu_seqlens, block_table=w.block_table,
                              topk_idx=w.topk_idx, page_size=s.page_size, capacity=cap,
                              causal=s.causal)
        inv = _inverse_rows(w)
        fwd = {v: k for k, v in inv.items()}
        lens = w.seqlens if s.layout != "ragged" else np.diff(w.cu_seqlens)
        for b in range(s.batch):
            n = int(lens[b])
            for i in range(s.s_q):
                for kslot in range(rows.shape[2]):
                    t = int(w.topk_idx[b, kslot]) if w.topk_idx is not None else kslot
                    vis = 0 <= t < n and (not s.causal or t <= n - s.s_q + i)
                    want = fwd[(b, t)] if vis else -1
                    assert rows[b, i, kslot] == want, (spec.layout, b, i, kslot)


ALL_CHECKS = [
    ("head_map_truth_table", check_head_map_truth_table),
    ("brute_contig_8x4", lambda: check_brute(tiny_spec(h_q=8, h_kv=4))),
    ("brute_contig_8x2_causal", lambda: check_brute(tiny_spec(h_q=8, h_kv=2, s_q=3, causal=True, lengths=(6, 2)))),
    ("brute_ragged", lambda: check_brute(tiny_spec(layout="ragged", h_q=8, h_kv=2, lengths=(3, 0, 17)))),
    ("brute_paged", lambda: check_brute(tiny_spec(layout="paged", lengths=(9, 14), page_size=4))),
    ("brute_sparse_masked", lambda: check_brute(tiny_spec(layout="paged", lengths=(9, 14), page_size=4, topk=12, topk_mode="random_masked"))),
    ("brute_gate", lambda: check_brute(tiny_spec(lengths=(4, 7), gate=True))),
    ("brute_fp8", check_fp8_brute),
    # a given softmax scale, positive and negative ("Sparse paged GQA decode
    # attention with FP8 KV cache on SM89", "Implementations": one folded
    # score multiplier), on causal, paged top-K and FP8 cases
    ("brute_scale_0.3_causal", lambda: check_brute(tiny_spec(h_q=8, h_kv=2, s_q=2, causal=True, lengths=(6, 9)),
                                                   seed=16, softmax_scale=0.3)),
    ("brute_scale_neg_fp8_sparse", lambda: check_brute(tiny_spec(layout="paged", lengths=(16, 13), page_size=4,
                                                                 kv_dtype="fp8_e4m3fn", topk=16,
                                                                 topk_mode="random_masked", gate=True),
                                                       seed=17, softmax_scale=-0.11)),
    # a headwise gate [B, S_q, H_q] (same page, "Workload": sigmoid gate
    # after attention), with S_q > 1 so that its two leading axes cannot be
    # confused, bf16 and FP8
    ("brute_headwise_gate_causal", lambda: check_brute(tiny_spec(h_q=8, h_kv=2, s_q=3, causal=True, gate=True,
                                                                 lengths=(7, 4)), seed=18, gate_mode="headwise")),
    ("brute_headwise_gate_fp8_scale", lambda: check_brute(tiny_spec(layout="paged", h_q=4, h_kv=2, s_q=2,
                                                                    causal=True, gate=True, lengths=(9, 12),
                                                                    page_size=4, kv_dtype="fp8_e4m3fn"),
                                                          seed=19, gate_mode="headwise", softmax_scale=0.21)),
    ("gqa_equals_mha_8x4", lambda: check_gqa_equals_mha(tiny_spec(h_q=8, h_kv=4))),
    ("gqa_equals_mha_8x2", lambda: check_gqa_equals_mha(tiny_spec(h_q=8, h_kv=2))),
    ("gqa_equals_mha_8x1", lambda: check_gqa_equals_mha(tiny_spec(h_q=8, h_kv=1))),
    ("gqa_equals_mha_32x8", lambda: check_gqa_equals_mha(tiny_spec(h_q=32, h_kv=8, lengths=(3, 4)))),
    ("gqa_equals_mha_paged_fp8", lambda: check_gqa_equals_mha(tiny_spec(layout="paged", h_q=8, h_kv=2, kv_dtype="fp8_e4m3fn", lengths=(9, 5)))),
    ("single_key", check_single_key),
    ("zero_query", check_zero_query),
    ("uniform_v", check_uniform_v),
    ("gate_zero", check_gate_zero),
    ("combine_partition", check_combine_partition),
    ("page_permutation", check_page_permutation),
    ("topk_identity_permutation", check_topk_identity_and_permutation),
    ("causal_prefix", check_causal_prefix),
    ("fp8_table", check_fp8_table),
    ("int8_table", check_int8_table),
    ("brute_int8", check_int8_brute),
    ("int8_quantiser_round_trip", check_int8_quantiser_round_trip),
    ("gqa_equals_mha_paged_int8", lambda: check_gqa_equals_mha(tiny_spec(layout="paged", h_q=8, h_kv=2, kv_dtype="int8", lengths=(9, 5)))),
    ("resolve_rows", check_resolve_rows),
]


def failing_checks():
    """Names of the checks that fail against the oracle as it currently is."""
    bad = []
    for name, fn in ALL_CHECKS:
        try:
            fn()
        except AssertionError:
            bad.append(name)
        except Exception as e:  # a crash also counts as a detection
            bad.append(f"{name} ({type(e).__name__})")
    return bad
