"""The Python binding's argument checks (CPU only).

The C ABI receives plain pointers and cannot tell an int64 index array from
an int32 one, a strided view from a packed tensor, or a short buffer from a
long one; the binding checks those before anything reaches the library.
Each case here must raise GqaError(GQA_ERR_INVALID_ARG) with CPU tensors.
Wrong types, strides and sizes are found before the device check, and
correct CPU tensors fail only on the device.
"""

import pytest
import torch

import gqa_kv_cache_amd as G

B, SQ, HQ, HKV, D, N = 2, 1, 8, 2, 64, 40


def _params(**kw):
    base = dict(batch=B, s_q=SQ, h_q=HQ, h_kv=HKV, head_dim=D, layout="contiguous", max_seqlen_kv=N,
                seq_capacity=N, kv_rows=B * N, num_cus=256)
    base.update(kw)
    return G.make_params(**base)


def _args():
    return dict(
        q=torch.zeros(B, SQ, HQ, D, dtype=torch.bfloat16),
        k_cache=torch.zeros(B, N, HKV, D, dtype=torch.bfloat16),
        v_cache=torch.zeros(B, N, HKV, D, dtype=torch.bfloat16),
        seqlens=torch.full((B,), N, dtype=torch.int32),
        o=torch.empty(B, SQ, HQ, D, dtype=torch.bfloat16),
        lse=torch.empty(B, HQ, SQ, dtype=torch.float32),
    )


def _run(params, a, **over):
    a = dict(a, **over)
    G.gqa_decode_run(params, a["q"], a["k_cache"], a["v_cache"], seqlens=a["seqlens"], o=a["o"], lse=a["lse"],
                     **{k: v for k, v in a.items() if k not in ("q", "k_cache", "v_cache", "seqlens", "o", "lse")})


def _expect(msg, fn):
    with pytest.raises(G.GqaError) as e:
        fn()
    assert e.value.status == 1
    assert msg in str(e.value), str(e.value)


CASES = {
    "int64 seqlens": (dict(seqlens=torch.full((B,), N, dtype=torch.int64)), "seqlens: dtype"),
    "float32 q": (dict(q=torch.zeros(B, SQ, HQ, D)), "q: dtype"),
    "fp16 k_cache": (dict(k_cache=torch.zeros(B, N, HKV, D, dtype=torch.float16)), "k_cache: dtype"),
    "bf16 lse": (dict(lse=torch.empty(B, HQ, SQ, dtype=torch.bfloat16)), "lse: dtype"),
    "fp32 out": (dict(o=torch.empty(B, SQ, HQ, D)), "o: dtype"),
    "strided q": (dict(q=torch.zeros(B, SQ, HQ, 2 * D, dtype=torch.bfloat16)[..., ::2]), "q: tensor is not contiguous"),
    "transposed o": (dict(o=torch.empty(B, SQ, D, HQ, dtype=torch.bfloat16).transpose(2, 3)), "o: tensor is not contiguous"),
    "short o": (dict(o=torch.empty(B, SQ, HQ, D - 1, dtype=torch.bfloat16)), "o: "),
    "short lse": (dict(lse=torch.empty(B, HQ, SQ + 1, dtype=torch.float32)), "lse: "),
    "short seqlens": (dict(seqlens=torch.full((B - 1,), N, dtype=torch.int32)), "seqlens: "),
    "short cache": (dict(v_cache=torch.zeros(B, N - 1, HKV, D, dtype=torch.bfloat16)), "v_cache: "),
    "elementwise gate of headwise size": (dict(gate=torch.zeros(B, SQ, HQ, dtype=torch.bfloat16)), "gate: "),
    "numpy q": (dict(q=torch.zeros(B, SQ, HQ, D, dtype=torch.int16).numpy()), "q: expected a torch tensor"),
    "cpu tensors": ({}, "not on a CUDA device"),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_decode_rejects(case):
    over, msg = CASES[case]
    gm = "elementwise" if "gate" in over else "none"
    _expect(msg, lambda: _run(_params(gate_mode=gm), _args(), **over))


def test_fp8_cache_types():
    p = _params(kv_dtype="fp8_e4m3fn")
    a = _args()
    codes = dict(k_cache=torch.zeros(B, N, HKV, D, dtype=torch.uint8), v_cache=torch.zeros(B, N, HKV, D, dtype=torch.uint8),
                 k_scale=torch.ones(B, HKV), v_scale=torch.ones(B, HKV))
    _expect("not on a CUDA device", lambda: _run(p, a, **codes))     # accepted up to the device
    _expect("k_cache: dtype", lambda: _run(p, a, **dict(codes, k_cache=torch.zeros(B, N, HKV, D, dtype=torch.bfloat16))))
    _expect("k_scale: dtype", lambda: _run(p, a, **dict(codes, k_scale=torch.ones(B, HKV, dtype=torch.float64))))
    _expect("v_scale: ", lambda: _run(p, a, **dict(codes, v_scale=torch.ones(B, HKV - 1))))


def test_int_workspace_needs_its_size():
    p = _params(kv_chunk=32)                # 40 tokens in chunks of 32: two splits, a workspace
    _expect("needs workspace_bytes", lambda: G.gqa_decode_run(p, 0, 0, 0, seqlens=0, o=0, lse=0, workspace=4096))


def test_resolve_rows_rejects_int32_output():
    p = _params()
    _expect("rows_out: dtype", lambda: G.gqa_resolve_rows(p, seqlens=torch.full((B,), N, dtype=torch.int32),
                                                           rows_out=torch.empty(B, SQ, N, dtype=torch.int32)))


def test_append_rejects():
    p = G.make_append_params(batch=B, s_new=3, h_kv=HKV, head_dim=D, layout="paged", kv_dtype="fp8_e4m3fn",
                             kv_rows=64, page_size=16, max_pages_per_seq=2)
    good = dict(k_new=torch.zeros(B, 3, HKV, D, dtype=torch.int16), v_new=torch.zeros(B, 3, HKV, D, dtype=torch.int16),
                seqlens=torch.zeros(B, dtype=torch.int32), seqlens_out=torch.zeros(B, dtype=torch.int32),
                block_table=torch.zeros(B, 2, dtype=torch.int32), k_cache=torch.zeros(4, 16, HKV, D, dtype=torch.uint8),
                v_cache=torch.zeros(4, 16, HKV, D, dtype=torch.uint8), k_scale=torch.ones(B, HKV),
                v_scale=torch.ones(B, HKV))
    run = lambda **o: G.gqa_kv_append(p, **dict(good, **o))
    _expect("not on a CUDA device", lambda: run())
    _expect("block_table: dtype", lambda: run(block_table=torch.zeros(B, 2, dtype=torch.int64)))
    _expect("k_new: dtype", lambda: run(k_new=torch.zeros(B, 3, HKV, D)))
    _expect("v_cache: ", lambda: run(v_cache=torch.zeros(3, 16, HKV, D, dtype=torch.uint8)))
    _expect("seqlens_out: ", lambda: run(seqlens_out=torch.zeros(B, dtype=torch.int32)[:1]))


class _Recorder:
    """Stands in for the loaded library: records the workspace size that
    gqa_decode_run would hand to the C call."""

    def __init__(self):
        self.ws_bytes = None

    def gqa_decode_run(self, *args):
        self.ws_bytes = args[-2].value
        return 0


def test_workspace_size_is_the_buffers_own(monkeypatch):
    rec = _Recorder()
    monkeypatch.setattr(G, "load_library", lambda path=None: rec)
    monkeypatch.setattr(G._Checked, "same_cuda_device", lambda self: None)
    a = _args()
    ws = torch.empty(100, dtype=torch.float32)       # 400 bytes
    _run(_params(), a, workspace=ws, stream=0)
    assert rec.ws_bytes == 400
    # decode() passes a caller's workspace on with its own size, whatever the
    # plan needs (the C call then rejects one that is too small)
    monkeypatch.setattr(G, "gqa_decode_workspace_size", lambda p: 1 << 20)
    G.decode(a["q"], a["k_cache"], a["v_cache"], seqlens=a["seqlens"], workspace=torch.empty(24, dtype=torch.uint8),
             stream=0)
    assert rec.ws_bytes == 24


def test_prepared_calls_check_once(monkeypatch):
    # DecodeCall / AppendCall run the same checks at construction ...
    a = _args()
    _expect("seqlens: dtype", lambda: G.DecodeCall(_params(), a["q"], a["k_cache"], a["v_cache"],
                                                   seqlens=torch.zeros(B, dtype=torch.int64), o=a["o"], lse=a["lse"]))
    _expect("not on a CUDA device", lambda: G.DecodeCall(_params(), a["q"], a["k_cache"], a["v_cache"],
                                                         seqlens=a["seqlens"], o=a["o"], lse=a["lse"]))
    # ... and then only enqueue, with the buffers' own workspace size
    rec = _Recorder()
    monkeypatch.setattr(G, "load_library", lambda path=None: rec)
    monkeypatch.setattr(G._Checked, "same_cuda_device", lambda self: None)
    call = G.DecodeCall(_params(), a["q"], a["k_cache"], a["v_cache"], seqlens=a["seqlens"], o=a["o"], lse=a["lse"],
                        workspace=torch.empty(40, dtype=torch.int16))
    call.run(stream=0)
    assert rec.ws_bytes == 80
