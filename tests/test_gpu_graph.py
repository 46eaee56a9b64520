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


@pytest.mark.parametrize("policy,S", [("given", 1), ("first_block", 700)])
def test_graph_replay_of_append(policy, S):
    # the append enqueues one kernel, or three (first-block scales over
    # several workgroups per request); replays after the caches, scales,
    # lengths and workspace are reset must write them exactly as the eager
    # call did
    import gqa_kv_cache_amd as G
    rng = np.random.default_rng(5)
    B, H, d, P, pps = 4, 8, 128, 16, 48
    dev = "cuda"
    k_new = torch.from_numpy(gi.f32_to_bf16_bits(rng.standard_normal((B, S, H, d)).astype(np.float32)).view(np.int16)).to(dev)
    v_new = torch.from_numpy(gi.f32_to_bf16_bits(rng.standard_normal((B, S, H, d)).astype(np.float32)).view(np.int16)).to(dev)
    seqlens = torch.tensor([0, 5, 0, 40], dtype=torch.int32, device=dev)
    bt = torch.from_numpy(rng.permutation(B * pps).reshape(B, pps).astype(np.int32)).to(dev)
    kc = torch.full((B * pps, P, H, d), 0x55, dtype=torch.uint8, device=dev)   # rows not appended keep 0x55
    vc = torch.full_like(kc, 0x55)
    ks = torch.full((B, H), 0.02, device=dev)
    vs = torch.full((B, H), 0.03, device=dev)
    so = torch.empty_like(seqlens)
    p = G.make_append_params(batch=B, s_new=S, h_kv=H, head_dim=d, layout="paged", kv_dtype="fp8_e4m3fn",
                             scale_policy=policy, kv_rows=B * pps * P, page_size=P, max_pages_per_seq=pps)
    wsb = G.gqa_kv_append_workspace_size(p)
    ws = torch.empty(max(wsb, 4), dtype=torch.uint8, device=dev)
    ks0, vs0 = ks.clone(), vs.clone()

    def call(stream=None):
        G.gqa_kv_append(p, k_new, v_new, seqlens, so, bt, kc, vc, ks, vs, ws, wsb, stream)

    call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (kc, vc, ks, vs, so)]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        call()
    for rep in range(4):
        kc.fill_(0x55)
        vc.fill_(0x55)
        ks.copy_(ks0)
        vs.copy_(vs0)
        so.fill_(-1)
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, r, name in zip((kc, vc, ks, vs, so), ref, ("k_cache", "v_cache", "k_scale", "v_scale", "seqlens_out")):
            assert torch.equal(t, r), f"append {policy}: replay {rep} {name} differs"
    log(f"  graph append {policy} S={S}: 4 replays equal to eager (workspace {wsb} B)")
