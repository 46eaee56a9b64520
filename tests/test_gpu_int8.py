"""The int8 K/V cache (codes times a per-(request, KV head) scale, converted
to bf16 tile by tile in registers) against the fp64 oracle fed the same
codes and scales, on every layout, head dim and tiling, both math paths,
with both gates; and one-hot probes that must return a V row bit for bit
(needs a gfx950 GPU)."""

import numpy as np
import pytest
import torch

import gqa_inputs as gi
from gpu_common import Uploaded, check_workload, log
from test_gpu_exact import _probe

pytestmark = pytest.mark.gpu


def spec(**kw):
    base = dict(name="int8", batch=2, h_q=8, h_kv=2, head_dim=128, s_q=1, layout="contiguous", kv_dtype=gi.KV_INT8)
    base.update(kw)
    if "fixed_lengths" in base:
        base["batch"] = len(base["fixed_lengths"])
    return gi.Spec(**base)


@pytest.mark.parametrize("hq,hkv,sq,d", [(8, 4, 1, 128), (8, 8, 1, 64), (32, 8, 1, 128), (64, 8, 2, 128),
                                         (32, 2, 2, 256), (16, 2, 4, 64), (8, 1, 16, 128), (64, 8, 16, 64),
                                         (16, 2, 16, 256)])
def test_int8_shapes(hq, hkv, sq, d):
    s = spec(h_q=hq, h_kv=hkv, s_q=sq, head_dim=d, causal=sq > 1, fixed_lengths=(1100, 33, 1))
    check_workload(gi.build(s, seed=hq + hkv + sq + d), label=f"int8 {hq}/{hkv} S_q={sq} d={d}")


@pytest.mark.parametrize("math", ["valu", "mfma"])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 4), (8, 2), (8, 1)])
def test_int8_math_paths(math, hq, hkv):
    s = spec(h_q=hq, h_kv=hkv, fixed_lengths=(900, 70))
    check_workload(gi.build(s, seed=50 + hq // hkv), math=math, label=f"int8 {hq}/{hkv} {math}")


@pytest.mark.parametrize("layout,chunk", [("ragged", 0), ("ragged", 64), ("paged", 0), ("paged", 32)])
def test_int8_layouts(layout, chunk):
    s = spec(layout=layout, h_q=32, h_kv=8, s_q=2, causal=True, page_size=16, fixed_lengths=(5, 0, 800, 97, 2048))
    check_workload(gi.build(s, seed=60 + chunk), kv_chunk=chunk, label=f"int8 {layout} chunk {chunk}")


@pytest.mark.parametrize("gate_mode,mode", [("elementwise", "permutation"), ("headwise", "random_masked")])
def test_int8_sparse_gated(gate_mode, mode):
    lengths = (512, 512, 512) if mode == "permutation" else (512, 300, 1)
    s = spec(layout="paged", h_q=32, h_kv=8, page_size=16, topk=512, topk_mode=mode, gate=True, fixed_lengths=lengths)
    check_workload(gi.build(s, seed=70), gate_mode=gate_mode, label=f"int8 sparse {gate_mode}")


def test_int8_stress_values():
    s = spec(h_q=16, h_kv=2, s_q=2, causal=True, v_mean=1.0, q_std=4.0, fixed_lengths=(2000, 8))
    check_workload(gi.build(s, seed=80), label="int8 stress")


@pytest.mark.parametrize("layout,chunk,math", [("contiguous", 0, "mfma"), ("paged", 32, "mfma"),
                                               ("paged", 96, "valu"), ("ragged", 32, "mfma")])
def test_int8_one_hot_probe(layout, chunk, math):
    s = spec(layout=layout, h_q=8 if math == "valu" else 32, h_kv=8, page_size=16, fixed_lengths=(700, 1, 1300))
    w = gi.build(s, seed=90)
    expect = _probe(w, np.random.default_rng(chunk + 3), int8=True)
    up = Uploaded(w, kv_chunk=chunk, math=math)
    up.run()
    torch.cuda.synchronize()
    O = up.o.view(torch.int16).cpu().numpy().view(np.uint16)
    vf = w.v_cache.reshape(-1, s.h_kv, s.head_dim)
    Gq = s.h_q // s.h_kv
    checked = 0
    for (b, g), target in expect.items():
        want = gi.f32_to_bf16_bits(vf[target, g].view(np.int8).astype(np.float32))
        for h in range(g * Gq, (g + 1) * Gq):
            assert np.array_equal(O[b, 0, h], want), f"(b={b}, h={h}) expected row {target}"
            checked += 1
    log(f"  int8 probe {layout} chunk={chunk} {math}: {checked} rows exact")
    assert checked > 0
