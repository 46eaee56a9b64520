"""The eight-head workgroup (eight waves, one KV head each) against the fp64
oracle (needs a gfx950 GPU).

Paged and top-K lists with up to 16 query rows per KV head and H_kv a
multiple of 8 take it for one-byte K/V at d <= 128 and for bf16 at d = 64.
The cases cover both head dims and all three stored types, paged and top-K
lists (permuted, prefix-padded, and with out-of-range and masked entries),
causal query blocks, gates, ragged lengths with empty requests, one split
(final output from the partial kernel) and several (partials plus the
combine), and two head groups per request (H_kv = 16).  Each case also
checks that the plan really is the eight-head one: the partial grid holds
H_kv / 8 head groups per (split, request).
"""

import numpy as np
import pytest

import gqa_inputs as gi
from gpu_common import Uploaded, compare, oracle

pytestmark = pytest.mark.gpu

# (h_q, h_kv, s_q, d, kv dtype, layout, topk, topk mode, lengths, causal, gate, chunk)
CASES = [
    (32, 8, 1, 128, gi.KV_FP8, "paged", 0, "permutation", (300, 77, 0, 513), False, True, 0),
    (32, 8, 2, 128, gi.KV_FP8, "paged", 0, "permutation", (300, 77, 0, 513), True, False, 64),
    (64, 8, 2, 128, gi.KV_INT8, "paged", 0, "permutation", (129, 1, 250), True, True, 0),
    (32, 8, 1, 128, gi.KV_FP8, "paged", 96, "permutation", (96, 96, 96), False, True, 0),
    (32, 8, 1, 128, gi.KV_INT8, "paged", 96, "prefix", (200, 96, 31), False, False, 32),
    (16, 8, 5, 128, gi.KV_FP8, "contiguous", 64, "random_masked", (180, 70), True, True, 0),
    (128, 16, 2, 128, gi.KV_FP8, "paged", 0, "permutation", (400, 33), True, False, 0),
    (32, 16, 1, 64, gi.KV_FP8, "paged", 0, "permutation", (257, 3, 64), False, True, 64),
    (64, 8, 1, 64, gi.KV_INT8, "ragged", 128, "prefix", (300, 128, 5), False, False, 0),
    (64, 8, 2, 64, gi.KV_BF16, "paged", 0, "permutation", (333, 0, 90), True, False, 0),
    (8, 8, 3, 64, gi.KV_BF16, "contiguous", 50, "random_masked", (120, 60), True, False, 32),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_eight_heads_per_workgroup(case):
    h_q, h_kv, s_q, d, kvd, layout, topk, mode, lengths, causal, gate, chunk = CASES[case]
    s = gi.Spec(name=f"wide{case}", batch=len(lengths), h_q=h_q, h_kv=h_kv, s_q=s_q, head_dim=d, kv_dtype=kvd,
                layout=layout, fixed_lengths=lengths, causal=causal, gate=gate, page_size=16,
                topk=topk, topk_mode=mode)
    w = gi.build(s, seed=7700 + case)
    gate_mode = ("headwise" if case % 2 else "elementwise") if gate else None
    up = Uploaded(w, kv_chunk=chunk, gate_mode=gate_mode)
    plan = up.plan
    assert plan["rows"] <= 16 and plan["math"] == 1
    assert plan["partial_workgroups"] == plan["num_splits"] * (h_kv // 8) * len(lengths), plan
    up.run()
    O, LSE = up.result()
    Oref, Lref = oracle(w, gate_mode=up.gate_mode)
    compare(O, LSE, Oref, Lref, fp8=kvd in (gi.KV_FP8, gi.KV_INT8),
            label=f"wide {case}: {h_q}/{h_kv} S_q={s_q} d={d} {kvd} {layout} topk={topk}/{mode} "
                  f"lengths={lengths} chunk={chunk} gate={up.gate_mode}")


def test_dense_lists_keep_four_heads():
    # A dense list with the same shape keeps four heads per workgroup.
    s = gi.Spec(name="dense8", batch=2, h_q=32, h_kv=8, s_q=1, head_dim=128, kv_dtype=gi.KV_FP8,
                layout="contiguous", fixed_lengths=(300, 77))
    up = Uploaded(gi.build(s, seed=7799))
    plan = up.plan
    assert plan["partial_workgroups"] == plan["num_splits"] * 2 * 2, plan
