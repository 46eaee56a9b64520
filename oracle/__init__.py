"""CPU oracle for GQA decode over a KV cache — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg import this package.  The HIP library and its Python binding never do.
"""

from .reference import (  # noqa: F401
    BF16, CONTIGUOUS, FP8, PAGED, RAGGED,
    bf16_bits_to_f64, combine, e4m3fn_table, e4m3fn_value, fp8_codes_to_f64,
    kv_head, physical_row, reference_decode, resolve_rows, seq_length,
    sigmoid, softmax_attend, visible_positions,
)
