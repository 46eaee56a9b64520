"""The oracle over a process pool, row by row -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` use this module.  It changes nothing in what the oracle
computes: every output row (request b, query i, head h) is an independent
call of ``reference.reference_decode`` restricted to that row, exactly as in
a serial run, so the results are identical to the serial oracle's, bit for
bit.  Rows are dealt to worker processes in chunks; each worker runs NumPy
with one BLAS thread.

Run as a program, it regenerates a named workload from its seed (the same
arrays the GPU side uploads), computes all its rows or as many as a CPU-time
budget allows, and writes them with the oracle's own wall time:

    python -m oracle.parallel --workload long128k --out DIR [--workers N]
                              [--budget-core-seconds S]

DIR/rows.npy (int64 [k, 3]: b, i, h), DIR/O.npy (float64 [k, d]),
DIR/LSE.npy (float64 [k]) and DIR/meta.json (seconds, workers, rows).
For an append workload (``append_*``, with --append-policy and
--append-dtype) it runs the append oracle request by request instead and
writes the codes of each finished request's new rows (K.npy, V.npy
[k, S, H_kv, d]), its scales and new length.
A program of its own so that the process that owns the GPU never forks:
the pool's workers are children of a process that has not touched it.
"""

from __future__ import annotations

import argparse
import json
import multiprocessing as mp
import os
import sys
import time
from typing import List, Optional, Sequence, Tuple

import numpy as np

from . import reference as R

_W = None          # the workload, inherited by forked workers
_GATE = "elementwise"
_SCALE = None


def host_cores(cap: int = 16) -> int:
    """Worker processes for this host: the cores this process may run on,
    at most ``cap`` (a shared GPU machine grants one GPU's share of its CPUs)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, cap))


def all_rows(w) -> List[Tuple[int, int, int]]:
    s = w.spec
    return [(b, i, h) for b in range(s.batch) for i in range(s.s_q) for h in range(s.h_q)]


def _init(w, gate_mode, softmax_scale):
    global _W, _GATE, _SCALE
    _W, _GATE, _SCALE = w, gate_mode, softmax_scale


def _rows_job(rows: Sequence[Tuple[int, int, int]]):
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        O, L = R.reference_decode(**_W.arrays(), **_W.params(), rows=rows, gate_mode=_GATE,
                                  softmax_scale=_SCALE)
    b = np.array([r[0] for r in rows])
    i = np.array([r[1] for r in rows])
    h = np.array([r[2] for r in rows])
    return np.asarray(rows, dtype=np.int64), O[b, i, h].copy(), L[b, h, i].copy()


def reference_rows(w, rows: Optional[Sequence[Tuple[int, int, int]]] = None, *, workers: Optional[int] = None,
                   gate_mode: str = "elementwise", softmax_scale=None, chunk: Optional[int] = None,
                   budget_core_seconds: Optional[float] = None):
    """Oracle outputs of the given rows (default: all), computed by a pool
    of forked workers.  Returns (rows int64 [k, 3], O [k, d], LSE [k],
    seconds, workers).  With a budget, chunks stop being started once the
    pool has used about that much CPU time (wall time x workers); the rows
    returned are those finished, in the order given."""
    rows = list(all_rows(w) if rows is None else rows)
    workers = workers or host_cores()
    if chunk is None:
        chunk = max(1, min(64, len(rows) // (4 * workers) or 1))
    chunks = [rows[k:k + chunk] for k in range(0, len(rows), chunk)]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    done = []
    with ctx.Pool(workers, initializer=_init, initargs=(w, gate_mode, softmax_scale)) as pool:
        if budget_core_seconds is None:
            done = pool.map(_rows_job, chunks)
        else:
            pending = []
            it = iter(chunks)
            for c in it:                     # keep every worker busy, one chunk queued behind each
                pending.append(pool.apply_async(_rows_job, (c,)))
                if len(pending) >= 2 * workers:
                    break
            k = 0
            while k < len(pending):
                done.append(pending[k].get())
                k += 1
                if (time.perf_counter() - t0) * workers < budget_core_seconds:
                    c = next(it, None)
                    if c is not None:
                        pending.append(pool.apply_async(_rows_job, (c,)))
            pool.terminate()
    seconds = time.perf_counter() - t0
    if not done:
        d = w.spec.head_dim
        return np.zeros((0, 3), np.int64), np.zeros((0, d)), np.zeros(0), seconds, workers
    r = np.concatenate([x[0] for x in done])
    O = np.concatenate([x[1] for x in done])
    L = np.concatenate([x[2] for x in done])
    return r, O, L, seconds, workers


# ---- the K/V append oracle, request by request -----------------------------

_AW = None   # (append workload, scale policy, code type), inherited by forked workers


def _init_append(w, policy, kv_dtype):
    global _AW
    _AW = (w, policy, kv_dtype)


def _append_job(b: int):
    """Request b of an append workload on a compact pool of its own pages
    (block-table row 0..pps-1): the oracle's codes for its S new rows [S,
    H_kv, d] (K and V), its scales and its new length."""
    from threadpoolctl import threadpool_limits
    from . import append as A
    w, policy, kvd = _AW
    B, S, Hkv, d = w.k_new.shape
    P, pps = w.page_size, w.block_table.shape[1]
    bt = np.arange(pps, dtype=np.int32)[None, :]
    dt = np.uint8 if kvd in (R.FP8, R.INT8) else np.uint16
    zero = np.zeros((pps, P, Hkv, d), dt)
    with threadpool_limits(1):
        kc, vc, ks, vs, lens = A.reference_append(
            k_cache=zero, v_cache=zero, k_new=w.k_new[b:b + 1], v_new=w.v_new[b:b + 1],
            seqlens=w.seqlens[b:b + 1], layout=R.PAGED, kv_dtype=kvd, block_table=bt, page_size=P,
            k_scale=w.k_scale[b:b + 1], v_scale=w.v_scale[b:b + 1], policy=policy)
    n0 = int(w.seqlens[b])
    tok = np.arange(n0, n0 + S)
    keep = tok // P < pps                                  # positions with a row of their own
    K = np.zeros((S, Hkv, d), dt)
    V = np.zeros((S, Hkv, d), dt)
    K[keep] = kc[tok[keep] // P, tok[keep] % P]
    V[keep] = vc[tok[keep] // P, tok[keep] % P]
    return b, K, V, ks[0].copy(), vs[0].copy(), int(lens[0])


def reference_append_requests(w, policy: str, kv_dtype: str, *, workers: Optional[int] = None,
                              budget_core_seconds: Optional[float] = None):
    """The append oracle over a pool, one request per job, in request order
    until about budget_core_seconds of CPU time.  Returns (list of
    _append_job results, seconds, workers)."""
    workers = workers or host_cores()
    B = w.k_new.shape[0]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    done = []
    with ctx.Pool(workers, initializer=_init_append, initargs=(w, policy, kv_dtype)) as pool:
        pending = [pool.apply_async(_append_job, (b,)) for b in range(min(B, 2 * workers))]
        nxt = len(pending)
        k = 0
        while k < len(pending):
            done.append(pending[k].get())
            k += 1
            if nxt < B and (budget_core_seconds is None or (time.perf_counter() - t0) * workers < budget_core_seconds):
                pending.append(pool.apply_async(_append_job, (nxt,)))
                nxt += 1
        pool.terminate()
    return done, time.perf_counter() - t0, workers


def main(argv=None):
    ap = argparse.ArgumentParser(description="the oracle over a process pool, for one named workload")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--workers", type=int, default=0)
    ap.add_argument("--budget-core-seconds", type=float, default=None)
    ap.add_argument("--gate-mode", default="elementwise")
    ap.add_argument("--append-policy", default=None, help="append workloads: given or first_block")
    ap.add_argument("--append-dtype", default=R.FP8, help="append workloads: fp8_e4m3fn or int8")
    args = ap.parse_args(argv)
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import gqa_inputs as gi
    os.makedirs(args.out, exist_ok=True)
    if args.workload.startswith("append_"):
        t = time.perf_counter()
        w = gi.append_named(args.workload)
        gen = time.perf_counter() - t
        done, seconds, workers = reference_append_requests(w, args.append_policy or w.policy, args.append_dtype,
                                                           workers=args.workers or None,
                                                           budget_core_seconds=args.budget_core_seconds)
        np.save(os.path.join(args.out, "requests.npy"), np.array([x[0] for x in done], np.int64))
        np.save(os.path.join(args.out, "K.npy"), np.stack([x[1] for x in done]))
        np.save(os.path.join(args.out, "V.npy"), np.stack([x[2] for x in done]))
        np.save(os.path.join(args.out, "k_scale.npy"), np.stack([x[3] for x in done]))
        np.save(os.path.join(args.out, "v_scale.npy"), np.stack([x[4] for x in done]))
        np.save(os.path.join(args.out, "lens.npy"), np.array([x[5] for x in done], np.int64))
        meta = {"workload": args.workload, "seconds": seconds, "workers": workers, "requests": len(done),
                "requests_total": int(w.k_new.shape[0]), "generate_seconds": gen}
        with open(os.path.join(args.out, "meta.json"), "w") as f:
            json.dump(meta, f)
        print(json.dumps(meta), flush=True)
        return
    t = time.perf_counter()
    w = gi.named(args.workload)
    gen = time.perf_counter() - t
    rows, O, L, seconds, workers = reference_rows(w, workers=args.workers or None, gate_mode=args.gate_mode,
                                                  budget_core_seconds=args.budget_core_seconds)
    np.save(os.path.join(args.out, "rows.npy"), rows)
    np.save(os.path.join(args.out, "O.npy"), O)
    np.save(os.path.join(args.out, "LSE.npy"), L)
    meta = {"workload": args.workload, "seconds": seconds, "workers": workers, "rows": int(len(rows)),
            "rows_total": len(all_rows(w)), "generate_seconds": gen}
    with open(os.path.join(args.out, "meta.json"), "w") as f:
        json.dump(meta, f)
    print(json.dumps(meta), flush=True)


if __name__ == "__main__":
    main()
