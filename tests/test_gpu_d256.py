"""Head dim 256 (MFMA path; loads staged in half tiles) against the fp64
oracle on every layout, FP8 with the gate, causal multi-token queries with
16 and 32 rows per KV head, forced splits, and one-hot addressing probes
(needs a gfx950 GPU).
"""

import numpy as np
import pytest
import torch

import gqa_inputs as gi
from gpu_common import Uploaded, check_workload, log

pytestmark = pytest.mark.gpu


def spec(**kw):
    base = dict(name="t", batch=2, h_q=16, h_kv=2, head_dim=256, s_q=1, layout="contiguous")
    base.update(kw)
    if "fixed_lengths" in base:
        base["batch"] = len(base["fixed_lengths"])
    return gi.Spec(**base)


@pytest.mark.parametrize("hq,hkv", [(32, 2), (8, 8), (16, 4), (8, 1)])
def test_d256_head_ratios(hq, hkv):
    check_workload(gi.build(spec(h_q=hq, h_kv=hkv, fixed_lengths=(1000, 65)), seed=hq + hkv), label=f"d256 {hq}/{hkv}")


@pytest.mark.parametrize("n", [1, 17, 4097])
def test_d256_lengths(n):
    check_workload(gi.build(spec(fixed_lengths=(n, 33)), seed=n), label=f"d256 n={n}")


@pytest.mark.parametrize("sq,hq", [(2, 16), (2, 32), (8, 4)])
def test_d256_multi_token_causal(sq, hq):
    # 16 rows (one MFMA block), 32 rows (two), 8 rows
    s = spec(h_q=hq, h_kv=2, s_q=sq, causal=True, fixed_lengths=(600, 9))
    check_workload(gi.build(s, seed=sq * 100 + hq), label=f"d256 {hq}/2 S_q={sq} causal")


@pytest.mark.parametrize("chunk", [0, 32, 96])
def test_d256_ragged_packed(chunk):
    s = spec(layout="ragged", h_q=16, h_kv=4, fixed_lengths=(5, 0, 40, 77, 32, 500, 2))
    check_workload(gi.build(s, seed=200 + chunk), kv_chunk=chunk, label=f"d256 packed chunk {chunk}")


@pytest.mark.parametrize("page", [16, 1])
def test_d256_paged(page):
    s = spec(layout="paged", h_q=32, h_kv=2, page_size=page, fixed_lengths=(700, 129))
    check_workload(gi.build(s, seed=300 + page), label=f"d256 paged P={page}")


@pytest.mark.parametrize("mode", ["permutation", "random_masked"])
def test_d256_sparse_fp8_gated(mode):
    lengths = (512, 512) if mode == "permutation" else (512, 300)
    s = spec(layout="paged", h_q=16, h_kv=4, page_size=16, topk=512, topk_mode=mode, kv_dtype=gi.KV_FP8,
             gate=True, fixed_lengths=lengths)
    check_workload(gi.build(s, seed=400), label=f"d256 fp8 sparse {mode}")


def test_d256_fp8_dense_two_blocks():
    s = spec(h_q=32, h_kv=2, s_q=2, causal=True, kv_dtype=gi.KV_FP8, fixed_lengths=(900, 40))
    check_workload(gi.build(s, seed=500), label="d256 fp8 32 rows")


@pytest.mark.parametrize("chunk", [32, 64, 4096])
def test_d256_forced_splits(chunk):
    s = spec(layout="ragged", h_q=32, h_kv=2, s_q=2, causal=True, fixed_lengths=(1000, 31, 97, 0))
    check_workload(gi.build(s, seed=600 + chunk), kv_chunk=chunk, label=f"d256 kv_chunk {chunk}")


@pytest.mark.parametrize("chunk", [0, 32])
def test_d256_one_hot_rows(chunk):
    # every visible token of one KV head is made the unique maximum in turn
    # for a sample of rows: O must equal that V row exactly (bf16 integers)
    s = spec(h_q=8, h_kv=2, fixed_lengths=(300, 77))
    w = gi.build(s, seed=700)
    rng = np.random.default_rng(chunk)
    B, Hkv, d = 2, 2, 256
    kf = w.k_cache.reshape(-1, Hkv, d)
    vf = w.v_cache.reshape(-1, Hkv, d)
    kf[...] = 0
    digits = (np.arange(kf.shape[0])[:, None, None] * 3 + np.arange(d)[None, None, :] + np.arange(Hkv)[None, :, None]) % 61
    vf[...] = gi.f32_to_bf16_bits(digits.astype(np.float32))
    w.q[...] = gi.f32_to_bf16_bits(np.full(w.q.shape, 8.0, dtype=np.float32))
    cap = w.k_cache.shape[1]
    targets = {}
    for b in range(B):
        for g in range(Hkv):
            t = int(rng.integers(w.seqlens[b]))
            row = b * cap + t
            kf[row, g, :] = gi.f32_to_bf16_bits(np.full(d, 1.0, dtype=np.float32))
            targets[(b, g)] = row
    up = Uploaded(w, kv_chunk=chunk)
    up.run()
    torch.cuda.synchronize()
    O = up.o.view(torch.int16).cpu().numpy().view(np.uint16)
    for (b, g), row in targets.items():
        for h in range(g * 4, g * 4 + 4):
            assert np.array_equal(O[b, 0, h], vf[row, g]), f"(b={b}, h={h}) expected row {row}"
    log(f"  d256 one-hot chunk={chunk}: exact")


# 17 to 32 rows with an even H_kv: the two waves of a head take one 16-row
# block each and share every tile through LDS.  Odd H_kv keeps two blocks
# in one wave.
@pytest.mark.parametrize("hq,hkv,sq", [(24, 1, 1), (48, 2, 1), (16, 2, 3), (20, 4, 4), (34, 2, 1), (32, 1, 1),
                                       (96, 3, 1)])
def test_d256_shared_rows_dense(hq, hkv, sq):
    s = spec(h_q=hq, h_kv=hkv, s_q=sq, causal=sq > 1, fixed_lengths=(1500, 33, 1))
    check_workload(gi.build(s, seed=800 + hq + hkv + sq), label=f"d256 shared {hq}/{hkv} S_q={sq}")


@pytest.mark.parametrize("kvd", [gi.KV_FP8, gi.KV_INT8])
@pytest.mark.parametrize("hq,hkv,sq", [(48, 2, 1), (24, 1, 1), (16, 2, 3)])
def test_d256_17_to_32_rows_one_byte(kvd, hq, hkv, sq):
    s = spec(h_q=hq, h_kv=hkv, s_q=sq, causal=sq > 1, kv_dtype=kvd, gate=True, fixed_lengths=(1200, 40, 1))
    check_workload(gi.build(s, seed=850 + hq + hkv + sq), label=f"d256 {kvd} {hq}/{hkv} S_q={sq}")


@pytest.mark.parametrize("layout,chunk", [("ragged", 0), ("ragged", 64), ("paged", 0), ("paged", 32),
                                          ("contiguous", 32)])
def test_d256_shared_rows_layouts(layout, chunk):
    s = spec(layout=layout, h_q=48, h_kv=2, s_q=1, page_size=16, fixed_lengths=(5, 0, 400, 97))
    check_workload(gi.build(s, seed=900 + chunk), kv_chunk=chunk, label=f"d256 shared {layout} chunk {chunk}")


@pytest.mark.parametrize("gate_mode,mode", [("elementwise", "permutation"), ("headwise", "random_masked")])
def test_d256_shared_rows_fp8_sparse_gated(gate_mode, mode):
    lengths = (256, 256) if mode == "permutation" else (256, 100)
    s = spec(layout="paged", h_q=24, h_kv=2, s_q=2, causal=True, page_size=16, topk=256, topk_mode=mode,
             kv_dtype=gi.KV_FP8, gate=True, fixed_lengths=lengths)
    check_workload(gi.build(s, seed=1000), gate_mode=gate_mode, label=f"d256 shared fp8 sparse {gate_mode}")


def test_d256_shared_rows_headwise_gate_bf16():
    s = spec(h_q=64, h_kv=2, s_q=1, gate=True, fixed_lengths=(777, 64))
    check_workload(gi.build(s, seed=1100), gate_mode="headwise", label="d256 shared bf16 headwise gate")
