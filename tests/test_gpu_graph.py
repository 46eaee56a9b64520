"""Calls captured into a HIP graph and replayed (needs a gfx950 GPU).

The library enqueues only kernel launches on the caller's stream (no
allocation, no memset, no synchronisation), so a call can be captured.  Each
case replays the graph several times with eager work of the program in
between (refilling the outputs with NaN, an eager call of another workload,
synchronisations) and checks every replay bit for bit against the eager
result of the same call.
"""

import numpy as np
import pytest
import torch

import gqa_inputs as gi
from gpu_common import Uploaded, log

pytestmark = pytest.mark.gpu


def spec(**kw):
    base = dict(name="t", batch=2, h_q=8, h_kv=4, head_dim=128, s_q=1, layout="contiguous")
    base.update(kw)
    if "fixed_lengths" in base:
        base["batch"] = len(base["fixed_lengths"])
    return gi.Spec(**base)


CASES = {
    "split_contiguous": (spec(h_q=64, h_kv=8, s_q=2, causal=True, fixed_lengths=(3000, 40)), 256),
    "packed_ragged": (spec(layout="ragged", h_q=32, h_kv=8, fixed_lengths=(700, 0, 33, 2049)), 64),
    "sparse_fp8_one_split": (spec(layout="paged", h_q=32, h_kv=8, page_size=16, topk=512, topk_mode="permutation",
                                  kv_dtype=gi.KV_FP8, gate=True, fixed_lengths=(512, 512)), 0),
    "valu_one_row": (spec(h_q=8, h_kv=8, fixed_lengths=(1000, 77)), 128),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replay_matches_eager(name):
    s, chunk = CASES[name]
    w = gi.build(s, seed=31)
    up = Uploaded(w, kv_chunk=chunk)
    other = Uploaded(gi.build(spec(layout="ragged", h_q=16, h_kv=4, fixed_lengths=(300, 5)), seed=32))
    up.run()
    torch.cuda.synchronize()
    ref_o = up.o.view(torch.int16).clone()
    ref_l = up.lse.clone()

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        up.run()                       # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        up.run()                       # stream None: the capture stream
    for rep in range(4):
        up.o.fill_(float("nan"))
        up.lse.fill_(float("nan"))
        other.run()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(up.o.view(torch.int16), ref_o), f"{name}: replay {rep} O differs"
        assert torch.equal(up.lse, ref_l), f"{name}: replay {rep} LSE differs"
    log(f"  graph {name}: 4 replays bitwise equal to eager (plan {up.plan})")
