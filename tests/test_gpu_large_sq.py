"""Multi-token query blocks of 16 to 64 tokens (chunked prefill, speculative
verification): 17 to 512 query rows per KV head, against the fp64 oracle
(needs a gfx950 GPU).

These rows are laid over a KV head's two, four or eight waves, which split
the rows and share every tile through LDS (one or two 16-row blocks each;
with eight waves over small tiles only the first waves load), and over
several row groups when a group has more rows than a workgroup covers.
The cases cross every such tiling with the cache layouts, FP8, int8 and
the gates, forced splits, and the causal alignment of the query block.
"""

import numpy as np
import pytest

import gqa_inputs as gi
from gpu_common import check_workload

pytestmark = pytest.mark.gpu


def spec(**kw):
    base = dict(name="large-sq", batch=2, h_q=8, h_kv=2, head_dim=128, s_q=16, causal=True,
                layout="contiguous")
    base.update(kw)
    if "fixed_lengths" in base:
        base["batch"] = len(base["fixed_lengths"])
    return gi.Spec(**base)


# (h_q, h_kv, s_q, d): rows = h_q / h_kv * s_q
SHAPES = [
    (4, 2, 16, 128),    # 32 rows: two blocks in one wave
    (6, 2, 16, 128),    # 48 rows: four waves, one block each
    (8, 2, 16, 128),    # 64 rows
    (10, 2, 13, 128),   # 65 rows: eight waves, one block each
    (16, 2, 16, 128),   # 128 rows
    (18, 2, 16, 128),   # 144 rows: eight waves of two blocks
    (64, 8, 64, 128),   # 512 rows: two row groups of 256
    (8, 1, 64, 64),     # 512 rows, d 64
    (8, 8, 16, 64),     # 16 rows, d 64
    (12, 4, 16, 64),    # 48 rows, d 64
    (6, 2, 16, 256),    # 48 rows, d 256: four waves, one block each
    (16, 2, 16, 256),   # 128 rows, d 256: eight waves, one block each
    (64, 8, 64, 256),   # 512 rows, d 256: four row groups of 128
]


@pytest.mark.parametrize("hq,hkv,sq,d", SHAPES)
def test_large_sq_contiguous(hq, hkv, sq, d):
    s = spec(h_q=hq, h_kv=hkv, s_q=sq, head_dim=d, fixed_lengths=(700, sq, sq + 37))
    check_workload(gi.build(s, seed=hq * 7 + hkv + sq + d), label=f"{hq}/{hkv} S_q={sq} d={d}")


@pytest.mark.parametrize("hq,hkv,sq", [(4, 2, 16), (8, 2, 16), (16, 2, 16), (64, 8, 32)])
def test_large_sq_packed_ragged(hq, hkv, sq):
    s = spec(layout="ragged", h_q=hq, h_kv=hkv, s_q=sq, fixed_lengths=(sq, 1000, 0, 77, 3000, sq + 1))
    check_workload(gi.build(s, seed=300 + hq + sq), label=f"packed {hq}/{hkv} S_q={sq}")


@pytest.mark.parametrize("chunk", [0, 32, 96])
def test_large_sq_packed_forced_chunks(chunk):
    s = spec(layout="ragged", h_q=16, h_kv=2, s_q=16, fixed_lengths=(40, 500, 16, 250))
    check_workload(gi.build(s, seed=400 + chunk), kv_chunk=chunk, label=f"packed S_q=16 chunk {chunk}")


@pytest.mark.parametrize("page", [16, 1])
def test_large_sq_paged(page):
    s = spec(layout="paged", h_q=16, h_kv=4, s_q=32, page_size=page, fixed_lengths=(900, 64, 333))
    check_workload(gi.build(s, seed=500 + page), label=f"paged P={page} S_q=32")


@pytest.mark.parametrize("gate_mode,mode", [("elementwise", "permutation"), ("headwise", "random_masked")])
def test_large_sq_fp8_sparse_gated(gate_mode, mode):
    lengths = (512, 512) if mode == "permutation" else (512, 300)
    s = spec(layout="paged", h_q=32, h_kv=8, s_q=16, page_size=16, topk=512, topk_mode=mode,
             kv_dtype=gi.KV_FP8, gate=True, fixed_lengths=lengths)
    check_workload(gi.build(s, seed=600), gate_mode=gate_mode, label=f"fp8 sparse S_q=16 {gate_mode}")


@pytest.mark.parametrize("hq,hkv,d", [(16, 2, 64), (12, 3, 64), (16, 2, 128), (16, 2, 256)])
def test_large_sq_fp8(hq, hkv, d):
    # FP8 d 64 has two loads per tile and tensor: two waves per head split the
    # rows (even H_kv), or one wave takes four blocks (odd H_kv, <= 64 rows)
    s = spec(h_q=hq, h_kv=hkv, s_q=16, head_dim=d, kv_dtype=gi.KV_FP8, gate=True, fixed_lengths=(800, 40))
    check_workload(gi.build(s, seed=700 + hq + d), label=f"fp8 {hq}/{hkv} S_q=16 d={d}")


@pytest.mark.parametrize("chunk", [32, 64, 4096])
def test_large_sq_forced_splits(chunk):
    s = spec(h_q=32, h_kv=4, s_q=32, fixed_lengths=(1200, 31, 97))
    check_workload(gi.build(s, seed=800 + chunk), kv_chunk=chunk, label=f"256 rows kv_chunk {chunk}")


def test_large_sq_non_causal_and_stress():
    s = spec(h_q=16, h_kv=2, s_q=16, causal=False, v_mean=1.0, q_std=4.0, fixed_lengths=(600, 17))
    check_workload(gi.build(s, seed=900), label="S_q=16 non-causal stress")


def test_large_sq_query_block_longer_than_cache():
    # S_q larger than n: the first S_q - n queries see nothing (O = 0, LSE = -inf)
    s = spec(h_q=8, h_kv=2, s_q=64, fixed_lengths=(20, 64, 1))
    check_workload(gi.build(s, seed=901), label="S_q=64 over short caches")


# Eight waves over tiles of fewer than eight loads per tensor (FP8 and int8,
# bf16 at d 64 beyond 256 rows): the first four or two waves load and stage
# each tile, and all eight compute on it.
SMALL_TILES = [
    # (kv_dtype, h_q, h_kv, s_q, d)
    (gi.KV_FP8, 32, 2, 16, 128),    # 256 rows: two blocks per wave, four loading waves
    (gi.KV_INT8, 16, 2, 16, 128),   # 128 rows: one block per wave
    (gi.KV_FP8, 80, 1, 2, 64),      # 160 rows, odd H_kv: two loading waves
    (gi.KV_INT8, 40, 1, 8, 64),     # 320 rows: two row groups of 256
    (gi.KV_BF16, 40, 1, 8, 64),     # 320 rows, bf16 d 64: eight waves, two row groups
    (gi.KV_BF16, 80, 1, 2, 64),     # 160 rows, bf16 d 64: four waves, three row groups
    (gi.KV_FP8, 16, 1, 16, 256),    # 256 rows, d 256: two row groups of 128
]


@pytest.mark.parametrize("kvd,hq,hkv,sq,d", SMALL_TILES)
def test_large_sq_small_tiles(kvd, hq, hkv, sq, d):
    s = spec(h_q=hq, h_kv=hkv, s_q=sq, head_dim=d, kv_dtype=kvd, gate=kvd != gi.KV_BF16,
             fixed_lengths=(700, sq, sq + 37))
    check_workload(gi.build(s, seed=1000 + hq + sq + d), label=f"{kvd} {hq}/{hkv} S_q={sq} d={d}")


@pytest.mark.parametrize("layout", ["ragged", "paged"])
@pytest.mark.parametrize("kvd", [gi.KV_FP8, gi.KV_INT8])
def test_large_sq_small_tiles_layouts(layout, kvd):
    s = spec(layout=layout, h_q=64, h_kv=4, s_q=8, head_dim=128, kv_dtype=kvd, gate=True, page_size=16,
             fixed_lengths=(333, 8, 1000, 0, 65))
    check_workload(gi.build(s, seed=1100), gate_mode="headwise", label=f"{kvd} {layout} 128 rows")


# 512 rows per KV head in two row groups (d 128) or four (d 256) that share
# their chunks on one XCD: every layout, and chunk sizes whose grids do and
# do not divide into 8 x row groups (the planner falls back to the plain
# workgroup order for the latter).
XCD_CASES = [(gi.KV_BF16, 128, 0), (gi.KV_BF16, 128, 96), (gi.KV_FP8, 128, 0), (gi.KV_BF16, 256, 0)]


@pytest.mark.parametrize("layout", ["contiguous", "ragged", "paged"])
@pytest.mark.parametrize("kvd,d,chunk", XCD_CASES)
def test_row_groups_on_one_xcd(layout, kvd, d, chunk):
    s = spec(layout=layout, h_q=64, h_kv=8, s_q=64, head_dim=d, kv_dtype=kvd, page_size=16,
             gate=kvd != gi.KV_BF16, fixed_lengths=(600, 64, 250))
    check_workload(gi.build(s, seed=1200 + d), kv_chunk=chunk, label=f"xcd row groups {layout} {kvd} d={d} chunk={chunk}")
