"""HIP path vs the fp64 oracle on the same seeded inputs (needs a gfx950 GPU).

Sizes are small enough for the oracle to finish in seconds while spanning
several 32-position tiles, several splits and a ragged tail.  Lengths that
are not multiples of the tile or split size are there on purpose: a short
last block mis-split was one of the planted bugs that the old suite missed
in "When the K/V copy costs more than the attention" ("Why it closed, and
the tests that merged").
"""

import dataclasses

import numpy as np
import pytest

import gqa_inputs as gi
from gpu_common import check_workload, log

pytestmark = pytest.mark.gpu

LENGTHS = (1, 2, 15, 16, 17, 63, 64, 65, 1000, 4097)


def spec(**kw):
    base = dict(name="t", batch=2, h_q=8, h_kv=4, head_dim=128, s_q=1, layout="contiguous")
    base.update(kw)
    if "fixed_lengths" in base:
        base["batch"] = len(base["fixed_lengths"])
    return gi.Spec(**base)


# Head ratios from the head-mapping table (8/4 and 8/2 separate a correct map
# from (h // H_kv) % H_kv; 4/2 and 16/4 do not), plus the workloads' ratios
# and plain MHA.
@pytest.mark.parametrize("hq,hkv", [(8, 4), (8, 2), (4, 2), (16, 4), (8, 1), (32, 8), (64, 8), (32, 32)])
def test_head_ratios(hq, hkv):
    w = gi.build(spec(h_q=hq, h_kv=hkv, fixed_lengths=(17, 300, 1)), seed=hq * 100 + hkv)
    check_workload(w, label=f"ratio {hq}/{hkv}")


@pytest.mark.parametrize("n", LENGTHS)
def test_lengths_contiguous(n):
    w = gi.build(spec(h_q=32, h_kv=8, fixed_lengths=(n, max(1, n // 3))), seed=n)
    check_workload(w, label=f"len {n}")


@pytest.mark.parametrize("d", [64, 128])
def test_head_dims(d):
    w = gi.build(spec(h_q=8, h_kv=1, head_dim=d, fixed_lengths=(1024,)), seed=d)
    check_workload(w, label=f"d{d}")


@pytest.mark.parametrize("sq", [1, 2, 3, 4, 5, 6, 7, 8])
def test_multi_token_causal(sq):
    w = gi.build(spec(h_q=32, h_kv=8, s_q=sq, causal=True, fixed_lengths=(100, sq, 37)), seed=sq)
    check_workload(w, label=f"s_q {sq} causal")


def test_multi_token_not_causal():
    w = gi.build(spec(h_q=16, h_kv=4, s_q=4, causal=False, fixed_lengths=(70, 5)), seed=44)
    check_workload(w, label="s_q 4 non-causal")


@pytest.mark.parametrize("hq,hkv,sq", [(64, 8, 4), (32, 8, 8), (64, 8, 8), (8, 1, 8), (64, 1, 1)])
def test_row_blocks(hq, hkv, sq):
    # 32 and 64 query rows per KV head: two and four 16-row MFMA blocks
    w = gi.build(spec(h_q=hq, h_kv=hkv, s_q=sq, causal=True, fixed_lengths=(129, 40)), seed=hq + sq)
    check_workload(w, label=f"rows {hq // hkv * sq}")


def test_ragged_with_empty_requests():
    w = gi.build(spec(layout="ragged", h_q=32, h_kv=8, fixed_lengths=(0, 33, 1, 0, 700, 64)), seed=5)
    check_workload(w, label="ragged with empties")


def test_ragged_seeded_lengths():
    w = gi.build(gi.scaled(gi.RAGGED_B64, batch=6, min_len=1, max_len=3000), seed=3)
    check_workload(w, label="ragged U[1,3000]")


# A ragged cache without top-K is cut into equal chunks of packed rows, each
# split at request boundaries.  With 32- and 64-row chunks these lengths put
# several requests (and empty ones) inside one chunk, requests that start or
# end exactly on a chunk boundary, and requests over many chunks.
PACKED_LENGTHS = (5, 0, 40, 1, 0, 0, 77, 32, 31, 33, 64, 3, 0, 128, 64, 0, 500, 2)


@pytest.mark.parametrize("chunk", [32, 64, 96])
def test_packed_ragged_segments(chunk):
    s = spec(layout="ragged", h_q=32, h_kv=8, fixed_lengths=PACKED_LENGTHS)
    check_workload(gi.build(s, seed=40 + chunk), kv_chunk=chunk, label=f"packed segments, chunk {chunk}")


@pytest.mark.parametrize("chunk", [32, 64])
def test_packed_ragged_causal_multi_token(chunk):
    s = spec(layout="ragged", h_q=16, h_kv=4, s_q=4, causal=True, fixed_lengths=(3, 64, 0, 65, 200, 4))
    check_workload(gi.build(s, seed=50 + chunk), kv_chunk=chunk, label=f"packed causal S_q=4, chunk {chunk}")


def test_packed_ragged_all_empty():
    s = spec(layout="ragged", h_q=8, h_kv=2, fixed_lengths=(0, 0, 0))
    check_workload(gi.build(s, seed=61), label="packed, every request empty")


@pytest.mark.parametrize("chunk", [0, 64])
def test_packed_ragged_offset_and_slack(chunk):
    """Packed rows that start after row 0 and a cache with unused rows at
    both ends: offsets are taken as given, and the unused rows are read by
    no request (they hold large values that would show if they were)."""
    s = spec(layout="ragged", h_q=32, h_kv=8, fixed_lengths=(70, 0, 1, 300, 33))
    w = gi.build(s, seed=62)
    head, tail = 45, 130
    pad = lambda c, n: np.full((n,) + c.shape[1:], 0x4480, dtype=c.dtype)   # bf16 1024.0
    w2 = dataclasses.replace(
        w, k_cache=np.concatenate([pad(w.k_cache, head), w.k_cache, pad(w.k_cache, tail)]),
        v_cache=np.concatenate([pad(w.v_cache, head), w.v_cache, pad(w.v_cache, tail)]),
        cu_seqlens=(w.cu_seqlens + head).astype(np.int32))
    check_workload(w2, kv_chunk=chunk, label=f"packed offset + slack, chunk {chunk}")


@pytest.mark.parametrize("chunk", [32, 128])
def test_packed_ragged_fp8(chunk):
    s = spec(layout="ragged", h_q=32, h_kv=8, kv_dtype=gi.KV_FP8, gate=True,
             fixed_lengths=(100, 0, 31, 257, 1))
    check_workload(gi.build(s, seed=70 + chunk), kv_chunk=chunk, label=f"packed fp8 gated, chunk {chunk}")


@pytest.mark.parametrize("d", [64, 128])
def test_packed_ragged_d64_one_head_group(d):
    # H_kv = 1 (one head per workgroup) and H_kv = 2 (two)
    for hkv in (1, 2):
        s = spec(layout="ragged", h_q=8, h_kv=hkv, head_dim=d, fixed_lengths=(40, 0, 129, 7))
        check_workload(gi.build(s, seed=80 + hkv), kv_chunk=32, label=f"packed d={d} h_kv={hkv}")


def test_contiguous_capacity_larger_than_lengths():
    w = gi.build(spec(h_q=16, h_kv=2, fixed_lengths=(10, 200, 0), capacity=300), seed=9)
    check_workload(w, label="capacity 300")


@pytest.mark.parametrize("page", [16, 4, 1, 64])
def test_paged(page):
    w = gi.build(spec(layout="paged", h_q=64, h_kv=8, page_size=page, fixed_lengths=(50, 513, 16)), seed=page)
    check_workload(w, label=f"paged P={page}")


def test_paged_causal_sq2():
    w = gi.build(spec(layout="paged", h_q=64, h_kv=8, s_q=2, causal=True, fixed_lengths=(333, 2)), seed=7)
    check_workload(w, label="paged causal s_q=2")


@pytest.mark.parametrize("mode", ["permutation", "prefix", "random_masked"])
def test_sparse_topk(mode):
    if mode == "permutation":
        s = spec(layout="paged", h_q=32, h_kv=8, topk=96, topk_mode=mode, fixed_lengths=(96, 96, 96))
    else:
        s = spec(layout="paged", h_q=32, h_kv=8, topk=80, topk_mode=mode, fixed_lengths=(50, 200, 0))
    w = gi.build(s, seed=len(mode))
    check_workload(w, label=f"top-K {mode}")


def test_sparse_over_contiguous_layout():
    s = spec(layout="contiguous", h_q=8, h_kv=2, topk=40, topk_mode="random_masked", fixed_lengths=(30, 77))
    check_workload(gi.build(s, seed=21), label="top-K over contiguous")


@pytest.mark.parametrize("gate_mode", ["elementwise", "headwise"])
def test_fp8_gated_sparse_paged(gate_mode):
    s = gi.scaled(gi.SPARSE_FP8, batch=5, pool_pages=5 * 32 + 7)
    check_workload(gi.build(s, seed=5), gate_mode=gate_mode, label=f"fp8 sparse gated {gate_mode}")


def test_fp8_dense_contiguous_d64():
    s = spec(h_q=8, h_kv=1, head_dim=64, kv_dtype="fp8_e4m3fn", fixed_lengths=(300, 33))
    check_workload(gi.build(s, seed=6), label="fp8 contiguous d64")


def test_bf16_gate_only():
    s = spec(h_q=16, h_kv=4, gate=True, fixed_lengths=(90, 3))
    check_workload(gi.build(s, seed=8), label="bf16 gate")


@pytest.mark.parametrize("chunk", [32, 64, 96, 160, 1024])
def test_forced_splits(chunk):
    # many splits, a short last split, and splits past the end of short requests
    s = spec(layout="ragged", h_q=32, h_kv=8, s_q=2, causal=True, fixed_lengths=(1000, 31, 97, 0))
    check_workload(gi.build(s, seed=chunk), kv_chunk=chunk, label=f"kv_chunk {chunk}")


@pytest.mark.parametrize("chunk", [32, 128])
def test_forced_splits_paged_fp8(chunk):
    s = gi.scaled(gi.SPARSE_FP8, batch=3, pool_pages=100)
    check_workload(gi.build(s, seed=chunk), kv_chunk=chunk, label=f"fp8 sparse kv_chunk {chunk}")


def test_softmax_scale_override():
    s = spec(h_q=8, h_kv=2, fixed_lengths=(200,))
    check_workload(gi.build(s, seed=77), softmax_scale=0.3, label="scale 0.3")


@pytest.mark.parametrize("variant", ["v_mean1", "q_std4"])
def test_stress_values(variant):
    # |O| near 1 (V ~ N(1,1)) makes the absolute tolerance meaningful;
    # q * 4 makes the softmax sharp.
    kw = dict(v_mean=1.0) if variant == "v_mean1" else dict(q_std=4.0)
    s = spec(h_q=64, h_kv=8, s_q=2, causal=True, fixed_lengths=(3000, 77), **kw)
    check_workload(gi.build(s, seed=31), label=variant)


def _many_lengths(batch, seed, hi, long):
    """Mostly short requests (0 .. hi-1 tokens, empties among them) with a few
    long ones at given positions."""
    lens = np.random.default_rng(seed).integers(0, hi, size=batch)
    for pos, n in long.items():
        lens[pos] = n
    return tuple(int(x) for x in lens)


@pytest.mark.parametrize("batch", [300, 5000])
def test_packed_ragged_many_requests(batch):
    """Thousands of requests in one packed cache: a workgroup's chunk holds
    hundreds of segments, and finding the first request of a chunk takes two
    (over 64 requests) or three (over 4096) rounds of the 64-way search."""
    lens = _many_lengths(batch, batch, 4, {7: 700, batch // 2: 1500, batch - 1: 65})
    s = spec(layout="ragged", h_q=8, h_kv=2, fixed_lengths=lens)
    check_workload(gi.build(s, seed=90), label=f"packed, {batch} requests")


def test_packed_ragged_max_batch():
    lens = _many_lengths(65535, 1, 3, {0: 300, 4095: 129, 4096: 1, 40000: 1000, 65534: 33})
    s = spec(layout="ragged", h_q=4, h_kv=1, head_dim=64, fixed_lengths=lens)
    check_workload(gi.build(s, seed=91), label="packed, 65535 requests")


def test_paged_max_batch():
    # one workgroup row per request along the grid's third dimension
    lens = _many_lengths(65535, 2, 33, {0: 32, 65534: 17})
    s = spec(layout="paged", h_q=4, h_kv=1, head_dim=64, page_size=16, fixed_lengths=lens)
    check_workload(gi.build(s, seed=92), label="paged, 65535 requests")
