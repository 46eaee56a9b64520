"""A seeded sweep over the planner's tilings against the fp64 oracle (needs a
gfx950 GPU).

Each case draws a head ratio, S_q, head dim, stored type, cache layout and a
few ragged lengths from a fixed generator, so that the row counts fall on
and between every tiling boundary (16, 32, 64, 128, 256 rows; one, two,
four and eight waves per head; one or several row groups; tiles that only
some waves load) in combinations the targeted tests do not name.
"""

import numpy as np
import pytest

import gqa_inputs as gi
from gpu_common import check_workload

pytestmark = pytest.mark.gpu

N_CASES = 48


def draw(i):
    rng = np.random.default_rng(9000 + i)
    h_kv = int(rng.choice([1, 2, 3, 4, 8]))
    group = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16]))
    s_q = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 24, 32, 48, 64]))
    while group * s_q > 512:
        s_q = max(1, s_q // 2)
    d = int(rng.choice([64, 128, 256]))
    kvd = str(rng.choice([gi.KV_BF16, gi.KV_FP8, gi.KV_INT8]))
    layout = str(rng.choice(["contiguous", "ragged", "paged"]))
    batch = int(rng.integers(1, 4))
    lengths = tuple(int(x) for x in rng.integers(0, 200, size=batch))
    if max(lengths) == 0:
        lengths = (s_q + 7,) + lengths[1:]
    chunk = int(rng.choice([0, 0, 32, 64]))
    return dict(h_q=group * h_kv, h_kv=h_kv, s_q=s_q, head_dim=d, kv_dtype=kvd, layout=layout,
                fixed_lengths=lengths, causal=bool(s_q > 1 and rng.random() < 0.8),
                gate=bool(kvd != gi.KV_BF16 and rng.random() < 0.5)), chunk


@pytest.mark.parametrize("i", range(N_CASES))
def test_tiling_sweep(i):
    kw, chunk = draw(i)
    s = gi.Spec(name=f"sweep{i}", batch=len(kw["fixed_lengths"]), page_size=16, **kw)
    label = (f"sweep {i}: {kw['h_q']}/{kw['h_kv']} S_q={kw['s_q']} d={kw['head_dim']} {kw['kv_dtype']} "
             f"{kw['layout']} lengths={kw['fixed_lengths']} chunk={chunk}")
    check_workload(gi.build(s, seed=9100 + i), kv_chunk=chunk, label=label)
