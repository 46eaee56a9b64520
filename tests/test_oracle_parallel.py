"""The oracle's process-pool driver (CPU only): it changes nothing in what
the oracle computes.  Every row it returns equals the serial oracle's bit
for bit, a budget returns a subset of whole rows, and the append mode equals
the serial append oracle byte for byte."""

import dataclasses

import numpy as np

import gqa_inputs as gi
import oracle.reference as R
from oracle import append as A
from oracle import parallel as OP
from pins import tiny_spec


def test_pool_equals_serial_bitwise():
    w = gi.build(tiny_spec(layout="paged", h_q=8, h_kv=2, s_q=2, causal=True, lengths=(13, 30, 7), page_size=4,
                           kv_dtype="fp8_e4m3fn", topk=16, topk_mode="random_masked", gate=True), 21)
    O, L = R.reference_decode(**w.arrays(), **w.params())
    rows, Op, Lp, secs, workers = OP.reference_rows(w, workers=3, chunk=5)
    assert workers == 3 and len(rows) == 3 * 2 * 8
    assert sorted(map(tuple, rows.tolist())) == OP.all_rows(w)
    b, i, h = rows[:, 0], rows[:, 1], rows[:, 2]
    assert np.array_equal(Op, O[b, i, h]) and np.array_equal(Lp, L[b, h, i], equal_nan=False)


def test_pool_budget_gives_whole_rows():
    w = gi.build(tiny_spec(h_q=8, h_kv=4, lengths=(50, 60)), 22)
    O, L = R.reference_decode(**w.arrays(), **w.params())
    rows, Op, Lp, _, _ = OP.reference_rows(w, workers=2, chunk=1, budget_core_seconds=0.0)
    assert 1 <= len(rows) <= len(OP.all_rows(w))
    b, i, h = rows[:, 0], rows[:, 1], rows[:, 2]
    assert np.array_equal(Op, O[b, i, h]) and np.array_equal(Lp, L[b, h, i])


def test_append_pool_equals_serial():
    rng = np.random.default_rng(23)
    B, S, H, d, P, pps = 3, 5, 2, 64, 4, 4
    w = gi.AppendWorkload(name="small", seed=0,
                          k_new=gi.f32_to_bf16_bits(rng.standard_normal((B, S, H, d)).astype(np.float32)),
                          v_new=gi.f32_to_bf16_bits(rng.standard_normal((B, S, H, d)).astype(np.float32)),
                          seqlens=np.array([0, 3, 13], np.int32),
                          block_table=rng.permutation(B * pps).reshape(B, pps).astype(np.int32),
                          pool_pages=B * pps, page_size=P,
                          k_scale=np.full((B, H), 0.02, np.float32), v_scale=np.full((B, H), 0.03, np.float32),
                          policy="first_block")
    for kvd in (R.FP8, R.INT8):
        done, _, _ = OP.reference_append_requests(w, "first_block", kvd, workers=2)
        assert [x[0] for x in done] == [0, 1, 2]
        pool = np.zeros((B * pps, P, H, d), np.uint8)
        kc, vc, ks, vs, lens = A.reference_append(k_cache=pool, v_cache=pool, k_new=w.k_new, v_new=w.v_new,
                                                  seqlens=w.seqlens, layout=R.PAGED, kv_dtype=kvd,
                                                  block_table=w.block_table, page_size=P, k_scale=w.k_scale,
                                                  v_scale=w.v_scale, policy="first_block")
        for b, K, V, kb, vb, n in done:
            tok = np.arange(w.seqlens[b], w.seqlens[b] + S)
            keep = tok // P < pps             # request 2's last rows fall past its pages and are not written
            pages = w.block_table[b][tok[keep] // P]
            assert np.array_equal(kc[pages, tok[keep] % P], K[keep])
            assert np.array_equal(vc[pages, tok[keep] % P], V[keep])
            assert np.array_equal(ks[b], kb) and np.array_equal(vs[b], vb) and lens[b] == n
