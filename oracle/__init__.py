"""fp64 CPU oracle for paged decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke check in
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use
it.  It shares no code with the HIP library or its Python binding; both sides
read only the seeded inputs that ``paged_kv_cache_288_amd.workloads`` draws.

Everything here is plain numpy in float64, written for a reader to check by
eye against the pages it follows (cited per function).  Where the pages leave
a step open, the reading taken is stated at the function.
"""

from .paged_attention import (  # noqa: F401
    bf16_bits_to_f64,
    fp8_e4m3fn_table,
    decode_kv_bits,
    gather_sequence,
    paged_decode_attention,
    multi_token_decode_attention,
    mla_decode_attention,
    kv_append,
    partition_partials,
    merge_partials,
    kv_bytes_per_token,
)
