#!/usr/bin/env python3
"""Benchmark of GQA decode over a KV cache on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long128k]

A step is one decode call (split-KV partial kernel + LSE combine) over the
resident synthetic inputs of the workload.  The default workload is the
long-context decode: batch 1, 64 query / 8 KV heads, d=128, S_q=2 causal,
a 128K-token bf16 cache (512 MiB of K+V) — the shape of the results table
in "When the K/V copy costs more than the attention".

Prints one JSON line: achieved bandwidth over the minimum bytes a call must
move (K/V + Q + O + LSE + lengths) divided by the measured time per call,
the roofline of the partial kernel (algorithmic K/V bytes per launch over
its event-timed duration, against 8 TB/s), and the CPU oracle timed on a
bounded sample of the same workload.  Progress goes to stderr.

    python bench.py --op append [--workload append_decode|append_prefill]
                    [--scale-policy given|first_block]

times the K/V append with FP8 quantisation on write instead: a step is one
append of every request's new rows into the paged FP8 pool; the line
reports GB/s over the bytes the append must move (bf16 rows read, codes
written) and the append kernel's roofline.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import shutil
import statistics
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/call and achieved HBM GB/s (% of peak), GQA decode 64/8 d128 128K KV"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix peak of MI355X
KERNEL_SOURCES = ["gqa_kv_cache_amd/csrc/gqa_kernels.hip", "gqa_kv_cache_amd/csrc/gqa_device.h"]


def say(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per partial-kernel launch from the committed rocprofv3
    counter summary, or None if absent or taken on other kernel source."""
    path = os.path.join(ROOT, "profiles", f"gqa_partial_kernel_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    try:
        if kv.get("kernel_source_sha256") != kernel_source_hash():
            return None
        fetch = float(kv["FETCH_SIZE_KiB_per_dispatch"]) * float(kv["fetch_scale"])
        write = float(kv["WRITE_SIZE_KiB_per_dispatch"]) * float(kv["write_scale"])
        return (fetch + write) * 1024.0
    except (KeyError, ValueError):
        return None


def workload_bytes(w):
    """(minimum bytes per call, algorithmic K/V bytes per partial launch)."""
    from gqa_kv_cache_amd import costs
    s = w.spec
    es = 1 if s.kv_dtype in ("fp8_e4m3fn", "int8") else 2
    if s.topk:
        tokens = sum(len(set(int(t) for t in w.topk_idx[b] if 0 <= t < w.seqlens[b])) for b in range(s.batch))
    else:
        tokens = int(w.seqlens.astype("int64").sum())
    pages = 0
    if s.layout == "paged":
        pages = sum(-(-int(n) // s.page_size) for n in w.seqlens)
    mb = costs.minimum_bytes(batch=s.batch, s_q=s.s_q, h_q=s.h_q, h_kv=s.h_kv, d=s.head_dim,
                             kv_elem_bytes=es, tokens=tokens, layout=s.layout, pages_touched=pages,
                             topk=s.topk, fp8_scales=s.kv_dtype in ("fp8_e4m3fn", "int8"), gate=w.gate is not None)
    kv = 2 * tokens * s.h_kv * s.head_dim * es
    return mb, kv, tokens


def host_info():
    """CPU model and host RAM of this machine, from /proc."""
    model, ram = platform.machine(), None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
        for line in open("/proc/meminfo"):
            if line.startswith("MemTotal"):
                ram = round(int(line.split()[1]) / 2 ** 20, 1)
                break
    except OSError:
        pass
    return model, ram


def cpu_baseline(workload: str, min_bytes: int, wall_budget_s: float = 20.0):
    """The fp64 oracle, as it is, on this host's cores: ``python -m
    oracle.parallel`` in a child process (which regenerates the same seeded
    workload and never touches the GPU) deals the output rows to one worker
    process per core, each with one BLAS thread, until about wall_budget_s
    of wall time is used.  Throughput is the minimum bytes scaled to the
    share of rows computed, over the oracle's own wall time (generation
    excluded).  Also returns the oracle's rows and outputs."""
    import tempfile
    from oracle.parallel import host_cores
    workers = host_cores()
    out = tempfile.mkdtemp(prefix="gqa_oracle_")
    cmd = [sys.executable, "-m", "oracle.parallel", "--workload", workload, "--out", out,
           "--workers", str(workers), "--budget-core-seconds", str(wall_budget_s * workers)]
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("oracle run failed: " + r.stdout[-2000:] + r.stderr[-2000:])
    meta = json.load(open(os.path.join(out, "meta.json")))
    rows, O, L = (np.load(os.path.join(out, f)) for f in ("rows.npy", "O.npy", "LSE.npy"))
    shutil.rmtree(out, ignore_errors=True)
    dt = meta["seconds"]
    frac = meta["rows"] / meta["rows_total"]
    model, ram = host_info()
    res = {"value": round(min_bytes * frac / dt / 1e9, 4), "unit": "GB/s", "cores": meta["workers"],
           "kind": "oracle",
           "sample": f"{meta['rows']} of {meta['rows_total']} query rows ({100 * frac:.0f}% of the workload), "
                     f"{dt:.2f} s wall over {meta['workers']} worker processes with one BLAS thread each",
           "seconds": round(dt, 3), "cpu_model": model, "host_ram_gb": ram}
    return res, rows, O, L


def check_against_oracle(o_gpu, lse_gpu, rows, Oref, Lref, fp8):
    """Max errors of the GPU outputs on the rows the oracle computed
    (rows int64 [k, 3] of (b, i, h); Oref [k, d], Lref [k])."""
    b, i, h = rows[:, 0], rows[:, 1], rows[:, 2]
    O = o_gpu.float().cpu().numpy()[b, i, h].astype(np.float64)
    L = lse_gpu.cpu().numpy()[b, h, i].astype(np.float64)
    Or, Lr = Oref, Lref
    fin = np.isfinite(Lr)
    o_err = float(np.abs(O - Or).max()) if O.size else 0.0
    l_err = float(np.abs(L[fin] - Lr[fin]).max()) if fin.any() else 0.0
    nref = float(np.linalg.norm(Or))
    rel = float(np.linalg.norm(O - Or) / nref) if nref > 0 else 0.0
    na = float(np.linalg.norm(O))
    cos = float((O.ravel() @ Or.ravel()) / (na * nref)) if na > 0 and nref > 0 else 1.0
    ok = (len(rows) > 0 and o_err <= (6e-2 if fp8 else 2e-2) and l_err <= 1e-3 and
          np.array_equal(np.isneginf(L), np.isneginf(Lr)) and (nref <= 1e-6 or (rel <= 1e-2 and cos >= 0.9999)))
    return {"rows": len(rows), "o_max_abs_err": o_err, "lse_max_abs_err": l_err, "o_rel_l2": rel,
            "o_cosine": cos, "ok": bool(ok)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # Untimed steps before the timed ones.  The GPU reaches its steady
    # clocks only after tens of milliseconds of sustained load: measured on
    # MI355X, the sparse top-512 FP8 call took 49.2, 46.4 and 44.9 us after
    # 20, 200 and 1000 warm-up calls, the 128K call 89.6, 88.0 and 87.9 us;
    # calls of 0.65 ms did not change.  The default warms up for 1000 calls.
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--op", default="decode", choices=["decode", "append"])
    ap.add_argument("--workload", default=None,
                    choices=["tiny", "long128k", "ragged", "ragged_sq8", "paged", "sparse_fp8",
                             "long_32x8", "long_8x1", "long_64x8_d64", "long_32x2_d256",
                             "ragged_sq16", "long_sq64", "sparse_int8", "append_decode", "append_prefill"])
    ap.add_argument("--scale-policy", default=None, choices=["given", "first_block"],
                    help="append: scale policy (default: the workload's)")
    ap.add_argument("--kv-chunk", type=int, default=0, help="force list positions per workgroup")
    ap.add_argument("--append-dtype", default="fp8_e4m3fn", choices=["fp8_e4m3fn", "int8"],
                    help="--op append: the code type written to the cache")
    ap.add_argument("--math", default="auto", choices=["auto", "mfma", "valu"],
                    help="math path of the partial kernel (auto: the planner's measured choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold", action="store_true", help="also time single calls after a 1 GiB cache flush")
    ap.add_argument("--graph", action="store_true",
                    help="also time K replays of a HIP graph holding one call (launch cost off the host)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="(kept for old command lines: the 512 MiB device-to-device copy is always timed)")
    ap.add_argument("--h-q", type=int, default=0, help="override the workload's query heads (shape sweeps)")
    ap.add_argument("--s-q", type=int, default=0, help="override the workload's query tokens per request")
    ap.add_argument("--head-dim", type=int, default=0, help="override the workload's head dim")
    ap.add_argument("--kv-dtype", default=None, choices=["bf16", "fp8_e4m3fn", "int8"],
                    help="override the workload's stored K/V type")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the decode path has no multi-GPU mode in this build", file=sys.stderr)
        sys.exit(2)

    import torch

    import gqa_inputs as gi
    import gqa_kv_cache_amd as G

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    G.load_library()
    if args.op == "append":
        return bench_append(args)
    if args.workload is None:
        args.workload = "long128k"
    if args.workload.startswith("append_"):
        print("append workloads need --op append", file=sys.stderr)
        sys.exit(2)

    say(f"generating workload {args.workload}")
    t = time.perf_counter()
    over = {k: v for k, v in (("h_q", args.h_q), ("s_q", args.s_q), ("head_dim", args.head_dim),
                              ("kv_dtype", args.kv_dtype)) if v}
    if over:
        # a variant of a named shape, for sweeps (no oracle run: the oracle
        # child regenerates named workloads only)
        spec, seed = gi.NAMED[args.workload]
        name = spec.name + "".join(f"_{k}={v}" for k, v in over.items())
        w = gi.build(gi.scaled(spec, name=name, **over), seed)
        args.no_cpu_baseline = True
    else:
        w = gi.named(args.workload)
    s = w.spec
    say(f"  generated in {time.perf_counter() - t:.1f} s")
    min_bytes, kv_bytes, tokens = workload_bytes(w)

    dev = "cuda"

    def bf16(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    fp8 = s.kv_dtype in ("fp8_e4m3fn", "int8")   # one-byte codes with scales
    q = bf16(w.q)
    k = torch.from_numpy(w.k_cache).to(dev) if fp8 else bf16(w.k_cache)
    v = torch.from_numpy(w.v_cache).to(dev) if fp8 else bf16(w.v_cache)
    i32 = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    f32 = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    seqlens = i32(w.seqlens) if s.layout != "ragged" else None
    cu, bt, topk = i32(w.cu_seqlens), i32(w.block_table), i32(w.topk_idx)
    ks, vs = f32(w.k_scale), f32(w.v_scale)
    gate = bf16(w.gate) if w.gate is not None else None
    if s.layout == "contiguous":
        cap, kv_rows, mpp = w.k_cache.shape[1], w.k_cache.shape[0] * w.k_cache.shape[1], 0
    elif s.layout == "ragged":
        cap, kv_rows, mpp = 0, w.k_cache.shape[0], 0
    else:
        cap, kv_rows, mpp = 0, w.k_cache.shape[0] * s.page_size, w.block_table.shape[1]
    params = G.make_params(batch=s.batch, s_q=s.s_q, h_q=s.h_q, h_kv=s.h_kv, head_dim=s.head_dim,
                           layout=s.layout, kv_dtype=s.kv_dtype, causal=s.causal,
                           max_seqlen_kv=w.max_seqlen, seq_capacity=cap, kv_rows=kv_rows,
                           page_size=s.page_size, max_pages_per_seq=mpp, topk=s.topk,
                           gate_mode="elementwise" if gate is not None else "none", kv_chunk=args.kv_chunk,
                           math=args.math)
    plan = G.gqa_decode_make_plan(params)
    ws = torch.empty(max(plan["workspace_bytes"], 16), dtype=torch.uint8, device=dev)
    o = torch.empty((s.batch, s.s_q, s.h_q, s.head_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((s.batch, s.h_q, s.s_q), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    say(f"plan {plan}")

    # The call's arguments are checked once and kept as device pointers, as a
    # serving loop that reuses its buffers would: a step only enqueues it.
    call = G.DecodeCall(params, q, k, v, seqlens, cu, bt, topk, ks, vs, gate, o, lse, ws, ws.numel())

    def step():
        call.run(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: exactly K back-to-back calls, as a caller makes them.
    K = args.steps
    say(f"timing {K} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Kernel duration: K more calls whose partial-kernel dispatch stamps a
    # pair of events (recorded by the library on the launch stream).  Kept
    # out of the timed region above: the stamps add packets to every call.
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    for e in ev0 + ev1:
        e.record(stream)            # creates the underlying hipEvent
    torch.cuda.synchronize()
    for i in range(K):
        params.partial_event_begin = ev0[i].cuda_event
        params.partial_event_end = ev1[i].cuda_event
        step()
    torch.cuda.synchronize()
    params.partial_event_begin = None
    params.partial_event_end = None
    partial_ms = [ev0[i].elapsed_time(ev1[i]) for i in range(K)]
    ms_per_step = wall * 1e3 / K
    partial_us = statistics.mean(partial_ms) * 1e3
    us_per_call = ms_per_step * 1e3
    value = min_bytes / (us_per_call * 1e-6) / 1e9
    achieved = kv_bytes / (partial_us * 1e-6) / 1e9
    say(f"  {us_per_call:.2f} us/call, partial kernel {partial_us:.2f} us, {value:.1f} GB/s, "
        f"partial {achieved:.1f} GB/s ({achieved / HBM_PEAK_GBPS:.1%} of 8 TB/s)")

    extra = {}
    if args.cold:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cold = []
        for _ in range(20):
            flush.zero_()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step()
            b.record(stream)
            torch.cuda.synchronize()
            cold.append(a.elapsed_time(b) * 1e3)
        extra["us_per_call_cold_median"] = round(statistics.median(cold), 3)
        del flush
    if args.graph:
        # One call captured into a graph on torch's capture stream (the
        # binding takes the current stream when none is given), replayed K
        # times back to back.
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            G.gqa_decode_run(params, q, k, v, seqlens, cu, bt, topk, ks, vs, gate, o, lse, ws, ws.numel(), None)
        stream.wait_stream(side)
        with torch.cuda.graph(graph):
            G.gqa_decode_run(params, q, k, v, seqlens, cu, bt, topk, ks, vs, gate, o, lse, ws, ws.numel(), None)
        for _ in range(10):
            graph.replay()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(K):
            graph.replay()
        torch.cuda.synchronize()
        extra["us_per_call_graph"] = round((time.perf_counter() - t) / K * 1e6, 3)
        del graph
    # The achievable-bandwidth reference: a 512 MiB device-to-device copy
    # ("Attention Kernel Portability Across GPU Architectures", section
    # "Experimental setup", measures a GPU's bandwidth this way).
    extra["d2d_copy_512MiB_GBps"] = calibrate_copy(torch, stream)

    traffic = None if over else read_traffic(args.workload)
    # The partial kernel's binding roofline: HBM, unless its matrix work per
    # K/V byte exceeds the ridge (peak FLOP/s over peak bytes/s), as for
    # query blocks of hundreds of rows per KV head.
    from gqa_kv_cache_amd import costs
    flops = costs.decode_flops(tokens=tokens, h_q=s.h_q, d=s.head_dim, s_q=s.s_q)
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    if flops / kv_bytes > ridge:
        tflops = flops / (partial_us * 1e-6) / 1e12
        roofline = {"bound": "mfma", "kernel": "gqa_partial_kernel", "achieved": round(tflops, 2),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                    "traffic": None if traffic is None else int(traffic), "algorithmic_flops_per_launch": flops,
                    "algorithmic_bytes_per_launch": kv_bytes, "kv_GBps": round(achieved, 2),
                    "kernel_us": round(partial_us, 3)}
    else:
        roofline = {"bound": "hbm", "kernel": "gqa_partial_kernel", "achieved": round(achieved, 2),
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                    "traffic": None if traffic is None else int(traffic), "algorithmic_bytes_per_launch": kv_bytes,
                    "kernel_us": round(partial_us, 3)}
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{s.kv_dtype}->bf16" if fp8 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": s.name, "batch": s.batch, "h_q": s.h_q, "h_kv": s.h_kv, "head_dim": s.head_dim,
            "s_q": s.s_q, "kv_tokens": tokens, "layout": s.layout, "causal": s.causal, "topk": s.topk,
            "kv_dtype": s.kv_dtype, "gate": w.gate is not None, "seed": w.seed,
            "kv_chunk": plan["kv_chunk"], "num_splits": plan["num_splits"],
            "math": {1: "mfma", 2: "valu"}[plan["math"]],
        },
        "us_per_call": round(us_per_call, 3),
        "min_bytes_per_call": min_bytes,
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "roofline": roofline,
        **extra,
    }
    ok = True
    if not args.no_cpu_baseline:
        say("timing the CPU oracle on this host's cores (a bounded sample)")
        res, rows, Oref, Lref = cpu_baseline(args.workload, min_bytes)
        line["cpu_baseline"] = res
        line["check"] = check_against_oracle(o, lse, rows, Oref, Lref, fp8)
        ok = line["check"]["ok"]
    print(json.dumps(line), flush=True)
    if not ok:
        say("GPU output does not match the oracle on the sampled rows")
        sys.exit(1)


def calibrate_copy(torch, stream) -> float:
    """A 512 MiB device-to-device copy (its counters scale FETCH_SIZE /
    WRITE_SIZE of the same profiled run); returns its GB/s."""
    src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(10):
        dst.copy_(src)
    b.record(stream)
    torch.cuda.synchronize()
    t_copy = a.elapsed_time(b) / 10 * 1e-3
    del src, dst
    return round(2 * (512 << 20) / t_copy / 1e9, 1)


APPEND_METRIC = "GB/s over the bytes moved, K/V append with quantise-on-write (paged pool)"


def bench_append(args):
    """One step = one gqa_kv_append of every request's new rows."""
    import torch

    import gqa_inputs as gi
    import gqa_kv_cache_amd as G

    name = args.workload or "append_decode"
    if not name.startswith("append_"):
        print("--op append takes --workload append_decode or append_prefill", file=sys.stderr)
        sys.exit(2)
    say(f"generating append workload {name}")
    w = gi.append_named(name)
    policy = args.scale_policy or w.policy
    B, S, Hkv, d = w.k_new.shape
    P, pps = w.page_size, w.block_table.shape[1]
    dev = "cuda"
    elems = B * S * Hkv * d
    bf16 = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev)
    kn, vn = bf16(w.k_new), bf16(w.v_new)
    kc = torch.zeros((w.pool_pages, P, Hkv, d), dtype=torch.uint8, device=dev)
    vc = torch.zeros_like(kc)
    sl = torch.from_numpy(w.seqlens).to(dev)
    so = torch.empty_like(sl)
    bt = torch.from_numpy(w.block_table).to(dev)
    ks = torch.from_numpy(w.k_scale).to(dev)
    vs = torch.from_numpy(w.v_scale).to(dev)
    kvd = args.append_dtype
    p = G.make_append_params(batch=B, s_new=S, h_kv=Hkv, head_dim=d, layout="paged", kv_dtype=kvd,
                             scale_policy=policy, kv_rows=w.pool_pages * P, page_size=P, max_pages_per_seq=pps)
    wsb = G.gqa_kv_append_workspace_size(p)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    call = G.AppendCall(p, kn, vn, sl, so, bt, kc, vc, ks, vs, ws, wsb)

    def step():
        call.run(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    say(f"timing {K} appends ({B} x {S} rows, policy {policy})")
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # Per-call device time: events around each call on the launch stream
    # (with the given policy a call is one dispatch of the append kernel).
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    dev_us = statistics.mean(a.elapsed_time(b) for a, b in ev) * 1e3
    two_pass = wsb > 0
    # bytes: bf16 K and V read, codes written, lengths and scales.  The
    # roofline counts the method's bytes only -- each row read once, each
    # code written once -- although the first-block policy over several
    # workgroups reads every row a second time (from the MALL when a
    # request group fits it).
    pages_touched = B * (-(-S // P) + 1)
    min_bytes = elems * 2 * (2 + 1) + B * 4 * 2 + B * Hkv * 4 * 2 + pages_touched * 4
    alg = elems * 2 * (2 + 1)
    launches = 2 if two_pass else 1
    us_per_call = wall / K * 1e6
    value = min_bytes / (us_per_call * 1e-6) / 1e9
    achieved = alg / (dev_us * 1e-6) / 1e9
    say(f"  {us_per_call:.2f} us/call, device {dev_us:.2f} us, {value:.1f} GB/s, kernel {achieved:.1f} GB/s")
    extra = {"d2d_copy_512MiB_GBps": calibrate_copy(torch, stream)}

    line = {
        "metric": APPEND_METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"bf16->{kvd}",
        "data": "synthetic",
        "config": {"workload": name, "batch": B, "new_tokens": S, "h_kv": Hkv, "head_dim": d, "kv_dtype": kvd,
                   "stored_tokens": int(w.seqlens[0]), "layout": "paged", "page_size": P,
                   "scale_policy": policy, "seed": w.seed, "launches": launches},
        "us_per_call": round(us_per_call, 3),
        "min_bytes_per_call": int(min_bytes),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": "gqa_append_kernel" + (" (maxima launch + write launch)" if two_pass else ""),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": None,
            "algorithmic_bytes_per_launch": int(alg),
            "kernel_us": round(dev_us, 3),
        },
        **extra,
    }
    ok = True
    if not args.no_cpu_baseline:
        say("timing the CPU append oracle on a bounded sample and checking sampled requests")
        res, chk = append_baseline_and_check(w, policy, kc, vc, ks, vs, so, kv_dtype=kvd)
        line["cpu_baseline"] = res
        line["check"] = chk
        ok = chk["ok"]
    print(json.dumps(line), flush=True)
    if not ok:
        say("GPU append does not match the oracle on the sampled requests")
        sys.exit(1)


def append_baseline_and_check(w, policy, kc, vc, ks, vs, so, kv_dtype="fp8_e4m3fn", wall_budget_s: float = 20.0):
    """The append oracle on this host's cores: ``python -m oracle.parallel``
    in a child process runs it request by request (each on a compact pool
    of its own pages) over one worker per core until about wall_budget_s;
    time it, and compare every byte of those requests' new rows and their
    scales and lengths with the GPU's."""
    import tempfile
    from oracle.parallel import host_cores
    B, S, Hkv, d = w.k_new.shape
    P = w.page_size
    workers = host_cores()
    out = tempfile.mkdtemp(prefix="gqa_append_oracle_")
    cmd = [sys.executable, "-m", "oracle.parallel", "--workload", w.name, "--out", out, "--workers", str(workers),
           "--budget-core-seconds", str(wall_budget_s * workers), "--append-policy", policy,
           "--append-dtype", kv_dtype]
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("append oracle run failed: " + r.stdout[-2000:] + r.stderr[-2000:])
    meta = json.load(open(os.path.join(out, "meta.json")))
    req, K, V, rks, rvs, lens = (np.load(os.path.join(out, f)) for f in
                                 ("requests.npy", "K.npy", "V.npy", "k_scale.npy", "v_scale.npy", "lens.npy"))
    shutil.rmtree(out, ignore_errors=True)
    gk, gv = kc.cpu().numpy(), vc.cpu().numpy()
    gks, gvs, gso = ks.cpu().numpy(), vs.cpu().numpy(), so.cpu().numpy()
    pps = w.block_table.shape[1]
    mism = 0
    for j, b in enumerate(req):
        n0 = int(w.seqlens[b])
        tok = np.arange(n0, n0 + S)
        keep = tok // P < pps
        pages = w.block_table[b][tok[keep] // P]
        slots = tok[keep] % P
        # only the appended slots are compared (the pool's other slots keep
        # whatever the GPU pool held)
        if not (np.array_equal(gk[pages, slots], K[j][keep]) and np.array_equal(gv[pages, slots], V[j][keep])):
            mism += 1
        if not (np.array_equal(gks[b], rks[j]) and np.array_equal(gvs[b], rvs[j]) and gso[b] == lens[j]):
            mism += 1
    done = len(req)
    t_oracle = meta["seconds"]
    rows = done * S
    moved = rows * Hkv * d * 2 * 3
    model, ram = host_info()
    res = {"value": round(moved / t_oracle / 1e9, 4), "unit": "GB/s", "cores": meta["workers"], "kind": "oracle",
           "sample": f"{done} of {B} requests ({rows} of {B * S} new rows), {t_oracle:.2f} s wall over "
                     f"{meta['workers']} worker processes with one BLAS thread each",
           "seconds": round(t_oracle, 3), "cpu_model": model, "host_ram_gb": ram}
    return res, {"requests": done, "mismatches": mism, "ok": bool(mism == 0)}


if __name__ == "__main__":
    main()
