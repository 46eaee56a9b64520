"""The VALU variant of the partial kernel (v_dot2_f32_bf16 and fp32 FMAs in
place of MFMA, for at most 8 query rows per KV head) against the fp64
oracle: every layout, both head dims, FP8 with the gate, the causal
multi-token case, forced splits and stress values (needs a gfx950 GPU).
"""

import numpy as np
import pytest

import gqa_inputs as gi
from gpu_common import check_workload

pytestmark = pytest.mark.gpu


def spec(**kw):
    base = dict(name="t", batch=2, h_q=8, h_kv=4, head_dim=128, s_q=1, layout="contiguous")
    base.update(kw)
    if "fixed_lengths" in base:
        base["batch"] = len(base["fixed_lengths"])
    return gi.Spec(**base)


@pytest.mark.parametrize("hq,hkv", [(8, 4), (8, 2), (4, 2), (8, 1), (32, 8), (64, 8), (32, 32)])
def test_valu_head_ratios(hq, hkv):
    s = spec(h_q=hq, h_kv=hkv, fixed_lengths=(1000, 65))
    check_workload(gi.build(s, seed=hq * 10 + hkv), math="valu", label=f"valu {hq}/{hkv}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [1, 17, 4097])
def test_valu_lengths_and_dims(d, n):
    s = spec(h_q=16, h_kv=4, head_dim=d, fixed_lengths=(n, 33))
    check_workload(gi.build(s, seed=n + d), math="valu", label=f"valu d={d} n={n}")


@pytest.mark.parametrize("sq,hq", [(2, 16), (4, 8), (8, 4)])
def test_valu_multi_token_causal(sq, hq):
    s = spec(h_q=hq, h_kv=4, s_q=sq, causal=True, fixed_lengths=(300, 9))
    check_workload(gi.build(s, seed=sq), math="valu", label=f"valu S_q={sq} causal")


@pytest.mark.parametrize("chunk", [0, 32, 96])
def test_valu_ragged_packed(chunk):
    s = spec(layout="ragged", h_q=32, h_kv=8, fixed_lengths=(5, 0, 40, 1, 0, 77, 32, 31, 33, 64, 500, 2))
    check_workload(gi.build(s, seed=90 + chunk), kv_chunk=chunk, math="valu", label=f"valu packed chunk {chunk}")


@pytest.mark.parametrize("page", [16, 1, 64])
def test_valu_paged(page):
    s = spec(layout="paged", h_q=64, h_kv=8, page_size=page, fixed_lengths=(700, 129))
    check_workload(gi.build(s, seed=page), math="valu", label=f"valu paged P={page}")


@pytest.mark.parametrize("mode", ["permutation", "prefix", "random_masked"])
def test_valu_sparse(mode):
    lengths = (200, 200) if mode == "permutation" else (250, 180)   # a permutation covers every token
    s = spec(layout="paged", h_q=32, h_kv=8, page_size=16, topk=200, topk_mode=mode, fixed_lengths=lengths)
    check_workload(gi.build(s, seed=3), math="valu", label=f"valu top-K {mode}")


@pytest.mark.parametrize("gate_mode,mode", [("elementwise", "permutation"), ("headwise", "permutation"),
                                            ("elementwise", "random_masked")])
def test_valu_fp8_gated_sparse_paged(gate_mode, mode):
    lengths = (512, 512) if mode == "permutation" else (512, 300)
    s = spec(layout="paged", h_q=32, h_kv=8, page_size=16, topk=512, topk_mode=mode,
             kv_dtype=gi.KV_FP8, gate=True, fixed_lengths=lengths)
    check_workload(gi.build(s, seed=5), gate_mode=gate_mode, math="valu", label=f"valu fp8 gate {gate_mode}")


@pytest.mark.parametrize("d", [64, 128])
def test_valu_fp8_dense(d):
    s = spec(h_q=16, h_kv=2, head_dim=d, kv_dtype=gi.KV_FP8, fixed_lengths=(900, 40))
    check_workload(gi.build(s, seed=d), math="valu", label=f"valu fp8 dense d={d}")


@pytest.mark.parametrize("chunk", [32, 64, 4096])
def test_valu_forced_splits(chunk):
    s = spec(layout="contiguous", h_q=16, h_kv=4, s_q=2, causal=True, fixed_lengths=(1000, 31, 97, 0))
    check_workload(gi.build(s, seed=chunk), kv_chunk=chunk, math="valu", label=f"valu kv_chunk {chunk}")


@pytest.mark.parametrize("variant", ["v_mean", "q_sharp"])
def test_valu_stress(variant):
    kw = dict(v_mean=1.0) if variant == "v_mean" else dict(q_std=4.0)
    s = spec(h_q=32, h_kv=8, fixed_lengths=(3000, 5), **kw)
    check_workload(gi.build(s, seed=21), math="valu", label=f"valu stress {variant}")
