"""Paged top-K lists on both sides of the block-table cache (needs a gfx950
GPU).

A paged top-K list whose request spans at most 1024 pages has its
block-table row copied to LDS and its pages looked up there; a longer row
(here: pages of one token and more than 1024 tokens) takes the pages from
HBM slot by slot.  Both must give the oracle's result, for the four-wave
kernels (bf16 d = 128, H_kv = 4) and the eight-head ones (FP8 and int8,
H_kv = 8), with requests on either side of the limit in one batch, masked
and out-of-range list entries, and one or several splits.
"""

import pytest

import gqa_inputs as gi
from gpu_common import check_workload

pytestmark = pytest.mark.gpu

# (h_q, h_kv, d, kv dtype, page size, lengths, topk, topk mode, chunk)
CASES = [
    (16, 4, 128, gi.KV_BF16, 16, (1500, 700, 0), 600, "prefix", 0),       # cached rows (94 pages)
    (16, 4, 128, gi.KV_BF16, 1, (1500, 700, 3), 600, "prefix", 0),        # 1500 pages: from HBM
    (16, 4, 128, gi.KV_BF16, 1, (1500, 700), 400, "random_masked", 128),  # mixed, several splits
    (32, 8, 128, gi.KV_FP8, 1, (1100, 1030, 1024), 512, "prefix", 0),     # eight heads, both sides
    (32, 8, 128, gi.KV_INT8, 4, (4200, 90), 512, "random_masked", 64),    # 1050 and 23 pages
    (64, 8, 64, gi.KV_FP8, 2, (2049, 2048, 5), 256, "prefix", 0),         # 1025 and 1024 pages
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_paged_topk_block_table_cache(case):
    h_q, h_kv, d, kvd, ps, lengths, topk, mode, chunk = CASES[case]
    s = gi.Spec(name=f"ptk{case}", batch=len(lengths), h_q=h_q, h_kv=h_kv, s_q=1, head_dim=d, kv_dtype=kvd,
                layout="paged", fixed_lengths=lengths, page_size=ps, topk=topk, topk_mode=mode,
                gate=kvd != gi.KV_BF16)
    check_workload(gi.build(s, seed=8800 + case), kv_chunk=chunk,
                   label=f"paged top-K {case}: {h_q}/{h_kv} d={d} {kvd} page={ps} lengths={lengths} "
                         f"topk={topk}/{mode} chunk={chunk}")
