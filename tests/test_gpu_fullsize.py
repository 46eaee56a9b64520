"""The named workloads at full size on the GPU, in the planner's default
launch configuration (the one bench.py times) and, where both apply, with the
other math path, checked against the fp64 oracle on EVERY output row.

The oracle runs row by row over a process pool in a child process
(``python -m oracle.parallel``) that regenerates the same seeded workload and
never touches the GPU; it works while this process uploads and runs the HIP
path.  Needs a gfx950 GPU; the largest (paged, 4 GiB of K/V) takes about a
minute.
"""

import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import gqa_inputs as gi
import gqa_kv_cache_amd as G
from gpu_common import Uploaded, compare, log

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

NAMES = ["tiny", "long128k", "ragged", "ragged_sq8", "paged", "sparse_fp8", "long_32x8", "long_8x1",
         "long_64x8_d64", "long_32x2_d256", "ragged_sq16", "long_sq64", "sparse_int8"]
# workloads with at most 8 query rows per KV head also run with the other math path
BOTH_PATHS = {"tiny", "ragged", "paged", "sparse_fp8"}


def _bound_check(name, w, up, O):
    # Every output is a convex combination of V rows (times a sigmoid <= 1),
    # so |O| never exceeds the largest |V| of its KV head and column (plus
    # bf16 rounding): a property of every row at any size.
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


@pytest.mark.parametrize("name", NAMES)
def test_named_workload_full_size(name, tmp_path):
    log(f"[fullsize] {name}: oracle started in a child process")
    out = tmp_path / "oracle"
    with open(tmp_path / "oracle.log", "w") as olog:
        child = subprocess.Popen([sys.executable, "-m", "oracle.parallel", "--workload", name, "--out", str(out)],
                                 cwd=ROOT, stdout=olog, stderr=subprocess.STDOUT)
    try:
        w = gi.named(name)
        s = w.spec
        paths = ["auto"]
        if name in BOTH_PATHS:
            shape = G.make_params(batch=1, s_q=s.s_q, h_q=s.h_q, h_kv=s.h_kv, head_dim=s.head_dim,
                                  kv_dtype=s.kv_dtype, max_seqlen_kv=1, seq_capacity=1, kv_rows=1, num_cus=256)
            paths.append("valu" if G.gqa_decode_make_plan(shape)["math"] == 1 else "mfma")
        results = {}
        for math in paths:
            up = Uploaded(w, math=math)
            log(f"[fullsize] {name} ({math}): plan {up.plan}")
            up.run()
            O, LSE = up.result()
            assert np.isfinite(O).all() and np.isfinite(LSE).all()
            _bound_check(name, w, up, O)
            results[math] = (O, LSE)
            del up
            torch.cuda.empty_cache()
        rc = child.wait(timeout=900)
    finally:
        if child.poll() is None:
            child.kill()
            child.wait()
    assert rc == 0, open(tmp_path / "oracle.log").read()[-3000:]
    meta = json.load(open(out / "meta.json"))
    log(f"[fullsize] {name}: oracle {meta}")
    rows = np.load(out / "rows.npy")
    Oref = np.load(out / "O.npy")
    Lref = np.load(out / "LSE.npy")
    assert len(rows) == s.batch * s.s_q * s.h_q == meta["rows_total"], "the oracle covered every row"
    b, i, h = rows[:, 0], rows[:, 1], rows[:, 2]
    fp8 = s.kv_dtype in (gi.KV_FP8, gi.KV_INT8)
    for math, (O, LSE) in results.items():
        compare(O[b, i, h], LSE[b, h, i], Oref, Lref, fp8=fp8, label=f"{name} {math}, all {len(rows)} rows")
