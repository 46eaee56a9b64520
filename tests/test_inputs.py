"""The seeded input generators (CPU)."""

import numpy as np
import torch

import gqa_inputs as gi


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000).astype(np.float32)
    # explicit ties: low 16 bits exactly 0x8000, both parities of bit 16
    ties = (np.arange(64, dtype=np.uint32) << np.uint32(17)) | np.uint32(0x3F808000)
    ties2 = ties | np.uint32(1 << 16)
    x = np.concatenate([x, ties.view(np.float32), ties2.view(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gi.f32_to_bf16_bits(x), want)


def test_build_is_deterministic():
    spec = gi.scaled(gi.RAGGED_B64, batch=4, min_len=5, max_len=40)
    a = gi.build(spec, 3)
    b = gi.build(spec, 3)
    for k, v in a.arrays().items():
        if v is not None:
            assert np.array_equal(v, b.arrays()[k]), k
    c = gi.build(spec, 4)
    assert not np.array_equal(a.q, c.q)


def test_ragged_lengths_and_offsets():
    spec = gi.scaled(gi.RAGGED_B64, batch=64)
    lens = gi._lengths(spec, 3)
    assert lens.min() >= 512 and lens.max() <= 16384
    spec_small = gi.scaled(gi.RAGGED_B64, batch=6, min_len=1, max_len=20)
    w = gi.build(spec_small, 3)
    assert w.cu_seqlens[0] == 0 and np.array_equal(np.diff(w.cu_seqlens), w.seqlens)
    assert w.k_cache.shape == (int(w.cu_seqlens[-1]), 8, 128)


def test_paged_block_table_is_a_permutation():
    spec = gi.scaled(gi.PAGED_B32, batch=4, seqlen=100, pages_per_seq=8, pool_pages=40)
    w = gi.build(spec, 4)
    bt = w.block_table
    assert bt.shape == (4, 8)
    assert len(set(bt.ravel().tolist())) == bt.size and bt.min() >= 0 and bt.max() < 40
    assert w.k_cache.shape == (40, 16, 8, 128)


def test_sparse_fp8_inputs():
    spec = gi.scaled(gi.SPARSE_FP8, batch=3)
    w = gi.build(spec, 5)
    assert w.k_cache.dtype == np.uint8 and w.k_cache.shape == (8192, 16, 8, 128)
    for b in range(3):
        assert sorted(w.topk_idx[b].tolist()) == list(range(512))
        pages = w.block_table[b]
        for cache, scale in ((w.k_cache, w.k_scale), (w.v_cache, w.v_scale)):
            vals = torch.from_numpy(cache[pages]).view(torch.float8_e4m3fn).float().numpy()
            amax = np.abs(vals).max(axis=(0, 1, 3))
            assert np.all(amax == 448.0)           # absmax maps to the largest code
            assert np.all(scale[b] > 0)
    # the stored value times its scale reproduces the N(0,1) draw to FP8 precision
    rk = gi.stream_rng(5, gi.STREAM_K)
    kf = rk.standard_normal((8192, 16, 8, 128), dtype=np.float32)
    b = 0
    pages = w.block_table[b]
    deq = torch.from_numpy(w.k_cache[pages]).view(torch.float8_e4m3fn).float().numpy() * w.k_scale[b][None, None, :, None]
    assert np.allclose(deq, kf[pages], rtol=0.0625, atol=w.k_scale[b].max() * 2 ** -9)


def test_named_specs_shapes():
    assert gi.LONG_128K.seqlen * gi.LONG_128K.h_kv * gi.LONG_128K.head_dim * 2 * 2 == 512 * 2**20
    assert gi.PAGED_B32.pool_pages == 32 * 2048
    s = gi.SPARSE_FP8
    assert s.pages_per_seq * s.page_size == s.topk == 512
