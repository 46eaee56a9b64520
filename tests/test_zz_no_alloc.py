"""The decode entry point that allocates nothing (gqa_decode_run_noalloc),
called through the C ABI on the GPU: its outputs equal gqa_decode_run's
with a caller workspace, bit for bit (the same plan and kernels, the partials
in the library's scratch array instead), and both match the fp64 oracle.
Two calls in a row, the second with a smaller input than the first, show
that nothing a call leaves in the shared array reaches the next.  A plan
whose partials exceed the array is refused and writes nothing."""

import numpy as np
import pytest
import torch

import gqa_inputs as gi
import gqa_kv_cache_amd as G
from gpu_common import Uploaded, compare, log, oracle

pytestmark = pytest.mark.gpu


def _spec(**kw):
    base = dict(name="noalloc", batch=2, h_q=16, h_kv=4, head_dim=128, s_q=2, causal=True, seqlen=9000)
    base.update(kw)
    return gi.Spec(**base)


def _noalloc(up):
    o = torch.full_like(up.o, float("nan"))
    lse = torch.full_like(up.lse, float("nan"))
    G.gqa_decode_run_noalloc(up.params, up.q, up.k, up.v, up.seqlens, up.cu, up.bt, up.topk, up.ks, up.vs,
                             up.gate, o, lse)
    torch.cuda.synchronize()
    return o, lse


CASES = [
    # (first call, second call): each pair shrinks, and every call splits its
    # KV walk (so the partials go through the scratch array)
    ("contiguous then ragged", _spec(), 101,
     _spec(layout="ragged", batch=3, h_q=8, h_kv=2, s_q=1, causal=False, min_len=100, max_len=3000), 102),
    ("paged fp8 gated then contiguous", _spec(layout="paged", batch=4, seqlen=6000, page_size=16,
                                               kv_dtype="fp8_e4m3fn", gate=True, pages_per_seq=400),
     103, _spec(batch=1, seqlen=700, h_q=8, h_kv=8, s_q=1, causal=False), 104),
]


@pytest.mark.parametrize("label,spec1,seed1,spec2,seed2", CASES, ids=[c[0] for c in CASES])
def test_noalloc_equals_workspace_call(label, spec1, seed1, spec2, seed2):
    for spec, seed, chunk in ((spec1, seed1, 256), (spec2, seed2, 128)):
        w = gi.build(spec, seed)
        up = Uploaded(w, kv_chunk=chunk)
        assert up.plan["combine"] == 1 and 0 < up.plan["workspace_bytes"] <= G.NOALLOC_SCRATCH_BYTES
        log(f"[noalloc] {label}: {spec.layout} B={spec.batch} plan {up.plan}")
        up.run()
        torch.cuda.synchronize()
        o, lse = _noalloc(up)
        assert torch.equal(o, up.o) and torch.equal(lse, up.lse), "differs from the call with a workspace"
        O, LSE = o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
        Oref, Lref = oracle(w, gate_mode=up.gate_mode)
        compare(O, LSE, Oref, Lref, fp8=spec.kv_dtype != "bf16", label=f"noalloc {label} B={spec.batch}")


def test_noalloc_refuses_a_plan_beyond_the_array():
    # 64/8 heads at S_q 64 over 128K tokens: 512 rows per KV head, about
    # 68 MB of partials
    w = gi.build(_spec(batch=1, h_q=64, h_kv=8, s_q=64, seqlen=131072), 105)
    up = Uploaded(w)
    assert up.plan["workspace_bytes"] > G.NOALLOC_SCRATCH_BYTES
    o = torch.full_like(up.o, 7.0)
    with pytest.raises(G.GqaError) as e:
        G.gqa_decode_run_noalloc(up.params, up.q, up.k, up.v, up.seqlens, o=o, lse=up.lse)
    assert e.value.status == 4 and "no-allocation" in str(e.value)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()), "a refused call wrote its output"
