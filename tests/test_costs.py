"""The byte / FLOP model against the numbers printed on the pages."""

import os

from gqa_kv_cache_amd import costs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.txt")


def _golden():
    out = {}
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            k, v = (x.strip() for x in line.split("="))
            out[k] = float(v)
    return out


def test_worked_examples():
    g = _golden()
    assert costs.expansion_bytes(131072, 64, 128, 2) == g["expansion_bytes_64x8_d128_128k"]
    b = costs.kv_bytes(32, 8, 16384, 128, 2)
    assert b == g["kv_bytes_b32_hkv8_n16384_d128_bf16"]
    assert round(costs.rate(b, 863.7e-6) / 1e9) == g["kv_gbps_b32_at_863p7us"]
    assert round(costs.kv_bytes(1, 32, 16384, 128, 2) / 1e6) == g["kv_mb_b1_hkv32_n16384"]
    assert round(costs.kv_bytes(1, 8, 16384, 128, 2) / 1e6) == g["kv_mb_b1_hkv8_n16384"]
    # 256 requests x 32 pages x 16 tokens = 512 tokens each, FP8 (1 byte)
    assert costs.kv_bytes(256, 8, 512, 128, 1) / 2**20 == g["kv_mib_b256_32pages_16tok_hkv8_d128_fp8"]
    f = costs.nominal_flops(256, 512, 32, 128)
    assert round(f / 1e9, 2) == g["nominal_gflop_b256_top512_hq32_d128"]
    assert round(costs.rate(f, 2.1641e-3) / 1e12, 3) == g["tflops_at_2p1641ms"]
    assert round(costs.rate(f, 2.4420e-3) / 1e12, 3) == g["tflops_at_2p4420ms"]


def test_minimum_bytes_long_context():
    # batch 1, 64/8, d128, S_q=2, 128K contiguous: 512 MiB of K/V plus
    # q, o (bf16), lse (fp32) and one length
    m = costs.minimum_bytes(batch=1, s_q=2, h_q=64, h_kv=8, d=128, kv_elem_bytes=2,
                            tokens=131072, layout="contiguous")
    assert m == 536870912 + 2 * 2 * 64 * 128 * 2 + 64 * 2 * 4 + 4


def test_decode_flops_matches_nominal_for_sq1():
    assert costs.decode_flops(tokens=256 * 512, h_q=32, d=128, s_q=1) == costs.nominal_flops(256, 512, 32, 128)
