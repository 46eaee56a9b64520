"""The running maximum of the online softmax, against the fp64 oracle (needs
a gfx950 GPU).

The MFMA kernels with at most 256 accumulator columns per lane move the
maximum that softmax weights are taken against only when a tile's maximum
exceeds it by more than 2^8, and apply the score multiplier inside the
exponent, which needs it positive (a negative one is moved into Q).  These
inputs drive both: scores that rise along the sequence (the reference moves
many times, with weights up to 2^8 in between), fall, or go up and down;
negative softmax scales and negative or zero K scales; across the tilings
(one and two blocks per wave, rows shared by four and eight waves, d 256
with one and two blocks).  Every result is exact softmax up to rounding,
whatever reference the kernel keeps, so the oracle and tolerances are the
usual ones.
"""

import dataclasses

import numpy as np
import pytest

import gqa_inputs as gi
from gpu_common import check_workload

pytestmark = pytest.mark.gpu

# (h_q, h_kv, s_q, d): rows = h_q / h_kv * s_q
TILINGS = [
    (8, 8, 2, 128),     # 2 rows, one block
    (32, 8, 4, 128),    # 16 rows
    (32, 8, 8, 128),    # 32 rows, two blocks per wave
    (16, 4, 16, 128),   # 64 rows, four waves share the rows
    (16, 2, 16, 128),   # 128 rows, eight waves
    (32, 2, 16, 128),   # 256 rows, eight waves of two blocks
    (8, 2, 8, 256),     # 32 rows, d 256, two waves share the rows
    (8, 1, 4, 256),     # 32 rows, d 256, odd H_kv: two blocks (rescaled every tile)
]


def spec(hq, hkv, sq, d, n=1500, **kw):
    base = dict(name="running-max", batch=2, h_q=hq, h_kv=hkv, head_dim=d, s_q=sq, causal=True,
                layout="contiguous", fixed_lengths=(n, n // 3 + 5))
    base.update(kw)
    return gi.Spec(**base)


def with_ramp(w: gi.Workload, profile: str, height: float = 10.0) -> gi.Workload:
    """Give every key a component along the queries' mean direction that
    follows `profile` over the tokens, so that the scores of every row do
    the same (rising by about `height` times sqrt(d) over the sequence)."""
    s = w.spec
    q = np.ones((s.batch, s.s_q, s.h_q, s.head_dim), dtype=np.float32)
    q += 0.25 * np.random.default_rng(5).standard_normal(q.shape).astype(np.float32)
    k = 0.1 * (w.k_cache.astype(np.uint32) << 16).view(np.float32)
    cap = k.shape[1]
    t = np.arange(cap, dtype=np.float32) / max(1, cap - 1)
    if profile == "rise":
        r = t
    elif profile == "fall":
        r = 1.0 - t
    else:  # up and down three times
        r = np.abs(np.sin(3 * np.pi * t))
    k = k + (height * r)[None, :, None, None]
    return dataclasses.replace(w, q=gi.f32_to_bf16_bits(q), k_cache=gi.f32_to_bf16_bits(k))


@pytest.mark.parametrize("profile", ["rise", "fall", "saw"])
@pytest.mark.parametrize("hq,hkv,sq,d", TILINGS)
def test_score_profiles(hq, hkv, sq, d, profile):
    w = with_ramp(gi.build(spec(hq, hkv, sq, d), seed=hq + sq + d), profile)
    check_workload(w, label=f"{profile} {hq}/{hkv} S_q={sq} d={d}")


@pytest.mark.parametrize("chunk", [64, 256])
def test_score_rise_across_splits(chunk):
    # the reference moves inside every split, and the combine meets splits
    # whose references differ by far more than 2^8
    w = with_ramp(gi.build(spec(32, 2, 16, 128, n=3000), seed=3), "rise", height=30.0)
    check_workload(w, kv_chunk=chunk, label=f"rise, kv_chunk {chunk}")


@pytest.mark.parametrize("hq,hkv,sq,d", TILINGS)
def test_negative_softmax_scale(hq, hkv, sq, d):
    w = gi.build(spec(hq, hkv, sq, d, n=700), seed=11 + hq)
    check_workload(w, softmax_scale=-0.11, label=f"scale -0.11 {hq}/{hkv} S_q={sq} d={d}")


@pytest.mark.parametrize("kv_dtype", [gi.KV_FP8, gi.KV_INT8])
@pytest.mark.parametrize("hq,hkv,sq", [(32, 8, 1), (32, 8, 4), (16, 2, 16)])
def test_negative_and_zero_k_scale(kv_dtype, hq, hkv, sq):
    """k_scale < 0 flips every score of its head; k_scale = 0 makes them all
    zero (uniform weights over the visible tokens)."""
    w = gi.build(spec(hq, hkv, sq, 128, n=900, kv_dtype=kv_dtype), seed=21 + sq)
    ks = np.array(w.k_scale, copy=True)
    ks[0, 0] = -ks[0, 0]
    ks[1, -1] = -ks[1, -1]
    ks[0, 1] = 0.0
    check_workload(dataclasses.replace(w, k_scale=ks), label=f"{kv_dtype} k_scale signs {hq}/{hkv} S_q={sq}")
