"""CPU fp64 oracle: TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The device library never imports, links or calls it, and this
package imports nothing from the device library.
"""
from .attention import (  # noqa: F401
    BLOCK,
    append_kv,
    block_table_from_csr,
    chunk_prefill,
    bf16_to_f64,
    cu_seqlens_from_lengths,
    e4m3fn_table,
    e4m3fn_to_f64,
    gather_kv_rows,
    paged_decode,
    quantize_e4m3fn,
    ragged_prefill,
    ragged_prefill_fp8,
    ragged_prefill_rope_fp8,
    widen,
)
