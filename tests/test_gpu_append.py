"""K/V append with FP8 or int8 quantise-on-write, through the C ABI, against
the append oracle: every byte of both caches, the scales and the new lengths
bit for bit (needs a gfx950 GPU).  Cases cover contiguous and paged caches,
bf16, FP8 and int8, both scale policies, single- and multi-workgroup
requests, positions past the capacity, every finite bf16 value through the
encoders, and an append followed by a decode."""

import numpy as np
import pytest
import torch

import gqa_inputs as gi
import gqa_kv_cache_amd as G
from gpu_common import Uploaded, compare, log, oracle
from oracle import append as A
from oracle import reference as R

pytestmark = pytest.mark.gpu

DEV = "cuda"


def dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def host(t, dtype):
    return t.cpu().numpy().view(dtype)


def new_rows(rng, B, S, Hkv, d, spread=True):
    """bf16 bits with magnitudes over many binades (and exact zeros)."""
    x = rng.standard_normal((B, S, Hkv, d)).astype(np.float32)
    if spread:
        x *= np.float32(2.0) ** rng.integers(-12, 6, size=x.shape).astype(np.float32)
        x[rng.random(x.shape) < 0.01] = 0.0
    return gi.f32_to_bf16_bits(x)


def run_case(*, layout, kv_dtype, policy, B, S, Hkv, d, lens, cap=0, P=16, pages_per_seq=0, scales=None,
             seed=0, k_new=None, v_new=None):
    rng = np.random.default_rng(seed)
    fp8 = kv_dtype in (R.FP8, R.INT8)    # one-byte codes with scales
    esz = np.uint8 if fp8 else np.uint16
    if layout == R.CONTIGUOUS:
        shape = (B, cap, Hkv, d)
        bt = None
    else:
        pool = B * pages_per_seq + 3
        shape = (pool, P, Hkv, d)
        bt = rng.permutation(pool)[: B * pages_per_seq].reshape(B, pages_per_seq).astype(np.int32)
    kc = rng.integers(0, 256 if fp8 else 1 << 16, size=shape).astype(esz)
    if kv_dtype == R.FP8:
        kc[(kc & 0x7F) == 0x7F] = 0      # keep the sentinel bytes finite codes
    vc = rng.integers(0, 256 if fp8 else 1 << 16, size=shape).astype(esz)
    if kv_dtype == R.FP8:
        vc[(vc & 0x7F) == 0x7F] = 0
    k_new = new_rows(rng, B, S, Hkv, d) if k_new is None else k_new
    v_new = new_rows(rng, B, S, Hkv, d) if v_new is None else v_new
    seqlens = np.asarray(lens, np.int32)
    if scales is None:
        scales = rng.uniform(0.001, 0.05, size=(B, Hkv)).astype(np.float32)
    ks = np.array(scales, np.float32)
    vs = np.array(scales[::-1] if scales.shape[0] > 1 else scales, np.float32)

    want = A.reference_append(k_cache=kc, v_cache=vc, k_new=k_new, v_new=v_new, seqlens=seqlens, layout=layout,
                              kv_dtype=kv_dtype, capacity=cap, block_table=bt, page_size=P,
                              k_scale=ks if fp8 else None, v_scale=vs if fp8 else None, policy=policy)

    kv_rows = int(np.prod(shape[:-2]))
    p = G.make_append_params(batch=B, s_new=S, h_kv=Hkv, head_dim=d, layout=layout, kv_dtype=kv_dtype,
                             scale_policy=policy, seq_capacity=cap, kv_rows=kv_rows, page_size=P,
                             max_pages_per_seq=pages_per_seq)
    ws_bytes = G.gqa_kv_append_workspace_size(p)
    t = dict(kn=dev(k_new.view(np.int16)), vn=dev(v_new.view(np.int16)), sl=dev(seqlens),
             so=torch.full((B,), -7, dtype=torch.int32, device=DEV), bt=dev(bt),
             kc=dev(kc.view(np.int8) if fp8 else kc.view(np.int16)), vc=dev(vc.view(np.int8) if fp8 else vc.view(np.int16)),
             ks=dev(ks) if fp8 else None, vs=dev(vs) if fp8 else None,
             ws=torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device=DEV))
    log(f"  append {layout} {kv_dtype} {policy} B={B} S={S} H_kv={Hkv} d={d} ws={ws_bytes}")
    G.gqa_kv_append(p, t["kn"], t["vn"], t["sl"], t["so"], t["bt"], t["kc"], t["vc"], t["ks"], t["vs"], t["ws"],
                    ws_bytes)
    torch.cuda.synchronize()
    got_k = host(t["kc"], esz).reshape(shape)
    got_v = host(t["vc"], esz).reshape(shape)
    assert np.array_equal(got_k, want[0]), f"K cache differs at {np.argwhere(got_k != want[0])[:5].tolist()}"
    assert np.array_equal(got_v, want[1]), f"V cache differs at {np.argwhere(got_v != want[1])[:5].tolist()}"
    if fp8:
        assert np.array_equal(host(t["ks"], np.float32), want[2])
        assert np.array_equal(host(t["vs"], np.float32), want[3])
    assert np.array_equal(host(t["so"], np.int32), want[4])
    return want


@pytest.mark.parametrize("layout", [R.CONTIGUOUS, R.PAGED])
@pytest.mark.parametrize("kv_dtype", [R.BF16, R.FP8, R.INT8])
@pytest.mark.parametrize("S", [1, 3, 40])
def test_append_given_scales(layout, kv_dtype, S):
    B, Hkv, d = 5, 4, 128
    lens = [0, 7, 15, 16, 100]
    run_case(layout=layout, kv_dtype=kv_dtype, policy="given", B=B, S=S, Hkv=Hkv, d=d, lens=lens, cap=160,
             pages_per_seq=10, seed=S)


@pytest.mark.parametrize("kv_dtype", [R.FP8, R.INT8])
@pytest.mark.parametrize("layout", [R.CONTIGUOUS, R.PAGED])
@pytest.mark.parametrize("S", [1, 8, 33, 700])
def test_append_first_block(layout, S, kv_dtype):
    # 700 new tokens of 8 heads x d 128 span several workgroups per request:
    # the per-workgroup maxima go through the workspace
    B, Hkv, d = 4, 8, 128
    lens = [0, 5, 0, 64]
    run_case(layout=layout, kv_dtype=kv_dtype, policy="first_block", B=B, S=S, Hkv=Hkv, d=d, lens=lens, cap=800,
             pages_per_seq=52, seed=100 + S)


@pytest.mark.parametrize("kv_dtype", [R.FP8, R.INT8])
@pytest.mark.parametrize("d,Hkv", [(64, 1), (64, 3), (256, 2), (256, 8)])
def test_append_head_shapes(d, Hkv, kv_dtype):
    for policy in ("given", "first_block"):
        run_case(layout=R.PAGED, kv_dtype=kv_dtype, policy=policy, B=3, S=21, Hkv=Hkv, d=d, lens=[0, 3, 40],
                 pages_per_seq=5, P=16, seed=d + Hkv)


def test_append_first_block_all_zero_rows():
    B, S, Hkv, d = 2, 4, 2, 64
    z = np.zeros((B, S, Hkv, d), np.uint16)
    want = run_case(layout=R.CONTIGUOUS, kv_dtype=R.FP8, policy="first_block", B=B, S=S, Hkv=Hkv, d=d,
                    lens=[0, 0], cap=8, k_new=z, v_new=z)
    assert np.all(want[2] == 1.0)


def test_append_past_capacity_is_not_written():
    # contiguous: request 1 is 2 short of its capacity; paged: request 0's
    # block-table row ends, request 2 points outside the pool
    run_case(layout=R.CONTIGUOUS, kv_dtype=R.FP8, policy="given", B=3, S=5, Hkv=2, d=64, lens=[0, 30, 32], cap=32)
    run_case(layout=R.PAGED, kv_dtype=R.BF16, policy="given", B=3, S=6, Hkv=2, d=64, lens=[13, 0, 4],
             P=4, pages_per_seq=4)


def test_append_page_size_one_and_large():
    run_case(layout=R.PAGED, kv_dtype=R.FP8, policy="first_block", B=2, S=9, Hkv=4, d=128, lens=[0, 17],
             P=1, pages_per_seq=40, seed=5)
    run_case(layout=R.PAGED, kv_dtype=R.FP8, policy="given", B=2, S=9, Hkv=4, d=128, lens=[250, 3],
             P=256, pages_per_seq=2, seed=6)


def _every_bf16_row():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    bits[~np.isfinite(A.bf16_bits_to_f32(bits))] = 0       # NaN and infinity replaced by zero
    return bits


@pytest.mark.parametrize("kv_dtype", [R.FP8, R.INT8])
@pytest.mark.parametrize("scale", [1.0, 0.125, 0.0137, 3.0])
def test_encoder_on_every_bf16_value(scale, kv_dtype):
    # one token row of 256 heads x d 256 = 65536 elements: every bf16 bit
    # pattern once, under one scale
    k_new = _every_bf16_row().reshape(1, 1, 256, 256)
    v_new = k_new[:, :, ::-1, ::-1].copy()
    run_case(layout=R.CONTIGUOUS, kv_dtype=kv_dtype, policy="given", B=1, S=1, Hkv=256, d=256, lens=[0], cap=2,
             scales=np.full((1, 256), scale, np.float32), k_new=k_new, v_new=v_new)


@pytest.mark.parametrize("kv_dtype", [R.FP8, R.INT8])
def test_encoder_on_every_bf16_value_under_many_scales(kv_dtype):
    # 32 requests x 256 heads of per-head scales -- log-uniform over 2^-40 ..
    # 2^40, powers of two (exact quotients, many exact ties), and the ends:
    # a subnormal scale whose reciprocal overflows, a subnormal one whose
    # reciprocal does not, and huge ones.  Each request holds every bf16
    # value once, rotated so that each value meets other heads.
    B, H, d = 32, 256, 256
    rng = np.random.default_rng(77)
    scales = np.exp2(rng.uniform(-40, 40, size=(B, H))).astype(np.float32)
    scales[0, :64] = np.exp2(np.arange(-32, 32)).astype(np.float32)
    scales[1, :8] = np.array([1e-40, 5e-39, 1.2e-38, 1e30, 3e38, 1.0, 448.0, 1 / 448], np.float32)
    row = _every_bf16_row()
    k_new = np.stack([np.roll(row, 997 * b) for b in range(B)]).reshape(B, 1, H, d)
    v_new = k_new[:, :, ::-1, ::-1].copy()
    run_case(layout=R.CONTIGUOUS, kv_dtype=kv_dtype, policy="given", B=B, S=1, Hkv=H, d=d, lens=[0] * B, cap=1,
             scales=scales, k_new=k_new, v_new=v_new)


@pytest.mark.parametrize("kv_dtype", [R.FP8, R.INT8])
def test_append_then_decode(kv_dtype):
    # A decode step: the new token's K/V are appended (first-block scales
    # for the empty request), then attention runs over the cache -- against
    # the oracle's decode of the oracle's appended cache.
    rng = np.random.default_rng(9)
    B, Hq, Hkv, d, P, pps = 3, 16, 4, 128, 16, 8
    lens = np.array([0, 37, 100], np.int32)
    S = 2
    pool = B * pps
    bt = rng.permutation(pool).reshape(B, pps).astype(np.int32)
    shape = (pool, P, Hkv, d)
    kc = np.zeros(shape, np.uint8)
    vc = np.zeros(shape, np.uint8)
    # the stored part: random codes under known scales
    ks = rng.uniform(0.005, 0.02, (B, Hkv)).astype(np.float32)
    vs = rng.uniform(0.005, 0.02, (B, Hkv)).astype(np.float32)
    for b in range(B):
        for t in range(int(lens[b])):
            r = bt[b, t // P] * P + t % P
            qz = A.quantize if kv_dtype == R.FP8 else A.quantize_int8
            kc.reshape(-1, Hkv, d)[r] = qz(rng.standard_normal((Hkv, d)).astype(np.float32) * 0.5, 0.01)
            vc.reshape(-1, Hkv, d)[r] = qz(rng.standard_normal((Hkv, d)).astype(np.float32) * 0.5, 0.01)
    k_new = new_rows(rng, B, S, Hkv, d, spread=False)
    v_new = new_rows(rng, B, S, Hkv, d, spread=False)
    kc2, vc2, ks2, vs2, lens2 = run_case(layout=R.PAGED, kv_dtype=kv_dtype, policy="first_block", B=B, S=S, Hkv=Hkv,
                                         d=d, lens=lens, P=P, pages_per_seq=pps, scales=ks, k_new=k_new, v_new=v_new)
    # decode over the appended cache (the oracle's bytes, which the GPU
    # matched exactly above)
    q = gi.f32_to_bf16_bits(rng.standard_normal((B, S, Hq, d)).astype(np.float32))
    spec = gi.Spec(name="append-decode", batch=B, h_q=Hq, h_kv=Hkv, head_dim=d, s_q=S, causal=True,
                   layout=gi.LAYOUT_PAGED, page_size=P, kv_dtype=kv_dtype, fixed_lengths=tuple(int(x) for x in lens2))
    w = gi.Workload(spec=spec, seed=0, q=q, k_cache=kc2, v_cache=vc2, seqlens=lens2, cu_seqlens=None,
                    block_table=bt, topk_idx=None, k_scale=ks2, v_scale=vs2, gate=None)
    up = Uploaded(w)
    up.run()
    O, LSE = up.result()
    Oref, Lref = oracle(w)
    compare(O, LSE, Oref, Lref, fp8=True, label="append then decode")
