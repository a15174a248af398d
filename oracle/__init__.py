"""Plain, slow, fp64 CPU oracle for the paged KV-cache decode path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package may import, call or
execute anything in this directory.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code,
headers, tables or helpers with the HIP path; the only thing both sides consume
is the seeded input generator, which contains none of the attention arithmetic.

Modules
  bf16             exact bf16 bit-pattern <-> float64 conversion
  paged_attention  block copy (copy-on-write), slot-mapped append,
                   block-table gather, textbook decode
                   attention, and the per-block / Equation-4 / split-K
                   formulations used to cross-check it

Parity status: every function here is pinned by ``tests/test_oracle.py``
against page-printed values, closed forms, invariants or a library routine
(torch's fp64 ``scaled_dot_product_attention``).  No function is
"parity unpinned".
"""

from .bf16 import bf16_bits_to_f64, f64_to_bf16_bits_rne
from .paged_attention import (
    copy_blocks,
    cache_append,
    gather_sequence,
    attention_textbook,
    paged_decode,
    contiguous_decode,
    multi_query_decode,
    paged_decode_online,
    paged_decode_eq4,
    split_partials,
    combine_partials,
)

__all__ = [
    "bf16_bits_to_f64",
    "f64_to_bf16_bits_rne",
    "copy_blocks",
    "cache_append",
    "gather_sequence",
    "attention_textbook",
    "paged_decode",
    "contiguous_decode",
    "multi_query_decode",
    "paged_decode_online",
    "paged_decode_eq4",
    "split_partials",
    "combine_partials",
]
