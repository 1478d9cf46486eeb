"""CPU fp64 oracle for paged grouped-query attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the library.
"""
from .paged_attention import (  # noqa: F401
    BLOCK,
    bf16_bits_to_f64,
    bf16_ulp,
    causal_visible,
    combine_partials,
    copy_blocks,
    decode,
    decode_multi,
    decode_multi_partials,
    decode_partials,
    f64_to_bf16_f64,
    gather_sequence,
    kv_head_of,
    prefill,
    scores,
    softmax_rows,
    write_kv,
)
from .prefix_cache import PrefixCache  # noqa: F401
