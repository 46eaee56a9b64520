"""Time the two math paths of the split-KV partial kernel against each other.

    python -m gqa_kv_cache_amd.crossover [--rows 1,2,4,8,16] [--tokens 131072]
                                         [--shapes bf16-d128,bf16-d64,fp8-d128]

For each shape and row count (query rows per KV head = H_q / H_kv at S_q = 1,
over H_kv = 8 heads and one request of `--tokens` tokens), it times the
partial kernel alone (events stamped by its dispatch, median of --calls) and
the whole call, for MFMA and -- up to 8 rows -- for VALU.  The planner's
GQA_MATH_AUTO choice comes from this measurement.  Inputs are random and made
on the device: only their size and shape matter here, not their values.
Needs a GPU and the built library.
"""

import argparse
import statistics
import time

HBM_PEAK_GBPS = 8000.0


def _time(G, torch, params, args, calls, stream):
    plan = G.gqa_decode_make_plan(params)
    ws = torch.empty(max(plan["workspace_bytes"], 16), dtype=torch.uint8, device="cuda")
    run = lambda: G.gqa_decode_run(params, *args, ws, ws.numel(), stream)
    for _ in range(10):
        run()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(calls):
        run()
    torch.cuda.synchronize()
    call_us = (time.perf_counter() - t) / calls * 1e6
    e0 = [torch.cuda.Event(enable_timing=True) for _ in range(calls)]
    e1 = [torch.cuda.Event(enable_timing=True) for _ in range(calls)]
    for e in e0 + e1:
        e.record(stream)
    torch.cuda.synchronize()
    for i in range(calls):
        params.partial_event_begin, params.partial_event_end = e0[i].cuda_event, e1[i].cuda_event
        run()
    torch.cuda.synchronize()
    params.partial_event_begin = params.partial_event_end = None
    kernel_us = statistics.median(e0[i].elapsed_time(e1[i]) for i in range(calls)) * 1e3
    return call_us, kernel_us


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--rows", default="1,2,4,8,16")
    ap.add_argument("--tokens", type=int, default=131072)
    ap.add_argument("--shapes", default="bf16-d128,bf16-d64,fp8-d128")
    ap.add_argument("--calls", type=int, default=50)
    args = ap.parse_args()

    import torch
    import gqa_kv_cache_amd as G

    G.load_library()
    torch.manual_seed(0)
    stream = torch.cuda.current_stream()
    n, hkv = args.tokens, 8
    for shape in args.shapes.split(","):
        dt, dd = shape.split("-")
        fp8, d = dt == "fp8", int(dd[1:])
        if fp8:
            mk = lambda: (torch.randn(n, hkv, d, device="cuda") * 100).clamp(-448, 448).to(
                torch.float8_e4m3fn).view(torch.uint8)
        else:
            mk = lambda: torch.randn(n, hkv, d, device="cuda").to(torch.bfloat16)
        k, v = mk(), mk()
        kv_bytes = 2 * n * hkv * d * (1 if fp8 else 2)
        seqlens = torch.tensor([n], dtype=torch.int32, device="cuda")
        scale = torch.ones(1, hkv, device="cuda") if fp8 else None
        for rows in (int(r) for r in args.rows.split(",")):
            hq = hkv * rows
            q = torch.randn(1, 1, hq, d, device="cuda").to(torch.bfloat16)
            o = torch.empty(1, 1, hq, d, dtype=torch.bfloat16, device="cuda")
            lse = torch.empty(1, hq, 1, device="cuda")
            cols = []
            for math in (("mfma", "valu") if rows <= 8 else ("mfma",)):
                p = G.make_params(batch=1, s_q=1, h_q=hq, h_kv=hkv, head_dim=d,
                                  kv_dtype="fp8_e4m3fn" if fp8 else "bf16", max_seqlen_kv=n, seq_capacity=n,
                                  kv_rows=n, math=math)
                call_us, kernel_us = _time(G, torch, p, (q, k, v, seqlens, None, None, None, scale, scale, None, o,
                                                          lse), args.calls, stream)
                frac = kv_bytes / (kernel_us * 1e-6) / 1e9 / HBM_PEAK_GBPS
                cols.append(f"{math}: kernel {kernel_us:8.2f} us ({frac:6.1%})  call {call_us:8.2f} us")
            print(f"{shape:9s} {hq:3d}/{hkv} rows={rows:2d} | " + " | ".join(cols), flush=True)
        del k, v
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
