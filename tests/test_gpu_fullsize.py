"""The named workloads at full size on the GPU, in the planner's default
launch configuration (the one bench.py times) and, where both apply, with the
other math path, checked against the fp64
oracle on a seeded sample of output rows computed one by one.  Needs a
gfx950 GPU; the largest (paged, 4 GiB of K/V) takes about a minute.
"""

import numpy as np
import pytest
import torch

import gqa_inputs as gi
import gqa_kv_cache_amd as G
from gpu_common import Uploaded, compare, log, oracle

pytestmark = pytest.mark.gpu

SAMPLE_ROWS = 48


def _sample_rows(w, k, seed):
    s = w.spec
    rng = np.random.default_rng(seed)
    rows = set()
    # always include the first and last query head of the first and last request
    for b in (0, s.batch - 1):
        for h in (0, s.h_q - 1):
            rows.add((b, s.s_q - 1, h))
    while len(rows) < min(k, s.batch * s.s_q * s.h_q):
        rows.add((int(rng.integers(s.batch)), int(rng.integers(s.s_q)), int(rng.integers(s.h_q))))
    return sorted(rows)


# Every workload with the planner's choice; those with at most 8 query rows
# per KV head also with the other math path.
FULL_CASES = [(n, "auto") for n in ("tiny", "long128k", "ragged", "ragged_sq8", "paged", "sparse_fp8",
                                     "long_32x8", "long_8x1", "long_64x8_d64", "long_32x2_d256",
                                     "ragged_sq16", "long_sq64", "sparse_int8")] + \
             [(n, "other") for n in ("tiny", "ragged", "paged", "sparse_fp8")]


@pytest.mark.parametrize("name,which", FULL_CASES, ids=[f"{n}-{m}" for n, m in FULL_CASES])
def test_named_workload_full_size(name, which):
    log(f"[fullsize] {name} ({which}): generating")
    w = gi.named(name)
    math = "auto"
    if which == "other":
        s = w.spec
        shape = G.make_params(batch=1, s_q=s.s_q, h_q=s.h_q, h_kv=s.h_kv, head_dim=s.head_dim, kv_dtype=s.kv_dtype,
                              max_seqlen_kv=1, seq_capacity=1, kv_rows=1, num_cus=256)
        math = "valu" if G.gqa_decode_make_plan(shape)["math"] == 1 else "mfma"
    up = Uploaded(w, math=math)
    log(f"[fullsize] {name}: plan {up.plan}")
    up.run()
    O, LSE = up.result()
    rows = _sample_rows(w, SAMPLE_ROWS, seed=len(name))
    Oref, Lref = oracle(w, gate_mode=up.gate_mode, rows=rows)
    idx_b = np.array([r[0] for r in rows])
    idx_i = np.array([r[1] for r in rows])
    idx_h = np.array([r[2] for r in rows])
    stats = compare(O[idx_b, idx_i, idx_h], LSE[idx_b, idx_h, idx_i], Oref[idx_b, idx_i, idx_h],
                    Lref[idx_b, idx_h, idx_i], fp8=w.spec.kv_dtype in (gi.KV_FP8, gi.KV_INT8), label=f"{name} (sampled)")
    # Properties of every row at any size: finite, and each output is a
    # convex combination of V rows (times a sigmoid <= 1), so |O| never
    # exceeds the largest |V| of its KV head and column (plus bf16 rounding).
    assert np.isfinite(O).all() and np.isfinite(LSE).all()
    s = w.spec
    G_ = s.h_q // s.h_kv
    if s.kv_dtype in (gi.KV_FP8, gi.KV_INT8):
        code_max = 448.0 if s.kv_dtype == gi.KV_FP8 else 128.0
        bound = np.full((s.batch, s.h_kv, s.head_dim), code_max) * w.v_scale[:, :, None]
    else:
        vmax = up.v.reshape(-1, s.h_kv, s.head_dim).float().abs().amax(dim=0).cpu().numpy()
        bound = np.broadcast_to(vmax[None], (s.batch, s.h_kv, s.head_dim))
    bound_q = np.repeat(bound, G_, axis=1)[:, None, :, :]          # [B, 1, H_q, d]
    assert (np.abs(O) <= bound_q * (1 + 2 ** -8) + 1e-6).all(), f"{name}: |O| exceeds max |V|"
    del up
    torch.cuda.empty_cache()
