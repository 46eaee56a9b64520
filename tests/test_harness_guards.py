"""The checking harness cannot pass on broken results (CPU only): the GPU
tests' comparison fails on NaN, on a missing -inf and on an all-zero output
at long context (which the absolute tolerance alone would accept); the
bench's own check flags NaN; bench.py exits non-zero when it cannot run as
asked; and the binding raises when the library is missing (there is no
fallback path)."""

import os
import subprocess
import sys

import numpy as np
import pytest

import gqa_kv_cache_amd as G
from gpu_common import compare

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _reference(rows=64, d=128, n=131072, seed=0):
    # |O| ~ sqrt(e / n) as for N(0, 1) inputs at 128K tokens; LSE ~ ln n
    rng = np.random.default_rng(seed)
    Oref = rng.standard_normal((1, 1, rows, d)) * np.sqrt(np.e / n)
    Lref = np.full((1, rows, 1), np.log(n)) + rng.standard_normal((1, rows, 1)) * 1e-3
    return Oref, Lref


def test_compare_accepts_the_reference_itself():
    Oref, Lref = _reference()
    compare(Oref.astype(np.float32).astype(np.float64), Lref, Oref, Lref, label="self")


def test_compare_rejects_all_zero_output_at_long_context():
    Oref, Lref = _reference()
    assert np.abs(Oref).max() < 2e-2                 # inside the absolute O tolerance ...
    with pytest.raises(AssertionError):              # ... so the relative L2 / cosine gates must catch it
        compare(np.zeros_like(Oref), Lref, Oref, Lref, label="zeros")


def test_compare_rejects_nan():
    Oref, Lref = _reference()
    O = Oref.copy()
    O[0, 0, 3, 5] = np.nan
    with pytest.raises(AssertionError):
        compare(O, Lref, Oref, Lref, label="nan")


def test_compare_rejects_finite_lse_where_nothing_is_visible():
    Oref, Lref = _reference()
    Lref = Lref.copy()
    Oref = Oref.copy()
    Lref[0, 7, 0] = -np.inf
    Oref[0, 0, 7, :] = 0.0
    with pytest.raises(AssertionError):
        compare(Oref, np.where(np.isinf(Lref), 0.0, Lref), Oref, Lref, label="lse")


def test_bench_check_flags_nan():
    import torch
    sys.path.insert(0, ROOT)
    import bench
    Oref, Lref = _reference(rows=4, d=8)
    rows = np.array([(0, 0, h) for h in range(4)], np.int64)     # (b, i, h) of each oracle row
    Orows, Lrows = Oref[0, 0], Lref[0, :, 0]                        # [4, d] and [4]
    o = torch.from_numpy(Oref.astype(np.float32))
    o[0, 0, 2, 1] = float("nan")
    lse = torch.from_numpy(Lref.astype(np.float32))
    assert bench.check_against_oracle(o, lse, rows, Orows, Lrows, False)["ok"] is False
    good = torch.from_numpy(Oref.astype(np.float32))
    assert bench.check_against_oracle(good, lse, rows, Orows, Lrows, False)["ok"] is True
    assert bench.check_against_oracle(torch.zeros_like(good), lse, rows, Orows, Lrows, False)["ok"] is False
    assert bench.check_against_oracle(good, lse, rows[:0], Orows[:0], Lrows[:0], False)["ok"] is False


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr


def test_bench_fails_without_a_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "1", "--warmup", "0"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and not r.stdout.strip()


def test_binding_raises_without_the_library(tmp_path):
    with pytest.raises(RuntimeError):
        G.load_library(str(tmp_path / "libgqa_decode.so"))
