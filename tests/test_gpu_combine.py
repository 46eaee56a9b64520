"""LSE combine over many split counts, against the fp64 oracle.

The combine's workgroup shape follows the split count: with few splits a
workgroup merges several rows, with many it takes a slice of the columns,
and its split lanes are merged at lane strides 8 to 32 and across waves.
Each case forces a chunk size that lands on another of those shapes
(needs a gfx950 GPU).
"""

import pytest

import gqa_inputs as gi
from gpu_common import check_workload

pytestmark = pytest.mark.gpu


# (head_dim, h_q, h_kv, s_q, lengths, chunk): the split count is about
# max(lengths) / chunk
CASES = [
    (64, 8, 1, 1, (16384, 100), 32),     # 512 splits: column slices of 8 quads, strides 8-32
    (128, 8, 1, 1, (4096, 5), 32),       # 128 splits: one row, all columns, stride 32
    (128, 16, 1, 1, (2048, 2047), 32),   # 64 splits: two rows per workgroup, waves only
    (128, 16, 4, 1, (1024, 3), 128),     # 8 splits: four rows per workgroup
    (128, 32, 8, 4, (700, 650), 128),    # 6 splits, 16 rows: eight rows, one split lane
    (256, 32, 1, 1, (16384, 31), 32),    # 512 splits, 32 rows, d 256: eight column slices
    (256, 4, 2, 1, (512, 511), 32),      # 16 splits, 2 rows
    (128, 64, 8, 2, (4097, 1), 32),      # 129 splits, causal, 16 rows: two column slices
    (64, 8, 8, 1, (33, 0, 64), 32),      # 2 splits and an empty request
]


@pytest.mark.parametrize("d,hq,hkv,sq,lengths,chunk", CASES)
def test_combine_shapes(d, hq, hkv, sq, lengths, chunk):
    s = gi.Spec(name="combine", batch=len(lengths), h_q=hq, h_kv=hkv, head_dim=d, s_q=sq, causal=sq > 1,
                layout="contiguous", fixed_lengths=lengths)
    check_workload(gi.build(s, seed=d + hq + chunk), kv_chunk=chunk,
                   label=f"combine d{d} {hq}/{hkv} S_q={sq} n={lengths} chunk {chunk}")


@pytest.mark.parametrize("chunk", [64, 512])
def test_combine_packed_many_chunks(chunk):
    # packed ragged rows: a long request spans many chunks, short ones one
    s = gi.Spec(name="combine-packed", batch=5, h_q=32, h_kv=8, head_dim=128, s_q=2, causal=True,
                layout="ragged", fixed_lengths=(6000, 40, 1, 900, 2))
    check_workload(gi.build(s, seed=chunk), kv_chunk=chunk, label=f"combine packed chunk {chunk}")
