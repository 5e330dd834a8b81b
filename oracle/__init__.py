"""CPU oracle for paged-KV decode attention — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct reference of what the hot path computes:
fp64 numpy (and, for tiny cases, pure-Python loops).  Only the test-suite,
the smoke check of the package entry point and the benchmark's CPU-baseline
leg may import it.  The product library never calls it and shares no code
with it; the two meet only in the seeded input generators of `workloads`.

Modules
  formats     bf16 and OCP FP8 E4M3FN decoding/encoding from the formats' definitions
  paged       the pool layout, the slot scatter (kv_append), the copy-on-write block copy, the
              swap gather/scatter of whole blocks, gather-then-attend decode and causal prefill
  brute       a second, pure-Python decode for tiny cases (no max subtraction, fsum)
  alloc_model the fixed-block free-list allocator with refcounted shared blocks
  footprint   KV byte arithmetic and allocation-waste accounting

Parity status: every function here is pinned by tests under tests/ (see the
test modules named test_oracle_*); none is "parity unpinned".
"""
from .formats import (bf16_bits_to_f64, e4m3_decode_table, e4m3_decode, e4m3_encode,
                      E4M3_MAX)
from .paged import (pool_shapes, lanes_per_16b, ref_append, ref_decode, gather_sequence,
                    empty_pools, ref_copy_blocks, ref_gather_blocks,
                    ref_scatter_blocks, attended, ref_prefill)
from .brute import brute_decode, brute_prefill
from .alloc_model import AllocModel, Status
from .footprint import (bytes_per_token, request_bytes, memory_bill, kv_bytes_logical,
                        kv_bytes_unique, paged_waste, contiguous_waste)

__all__ = [
    "bf16_bits_to_f64", "e4m3_decode_table", "e4m3_decode", "e4m3_encode", "E4M3_MAX",
    "pool_shapes", "lanes_per_16b", "ref_append", "ref_decode", "gather_sequence", "empty_pools",
    "ref_copy_blocks", "ref_gather_blocks", "ref_scatter_blocks", "attended", "ref_prefill",
    "brute_decode", "brute_prefill", "AllocModel", "Status",
    "bytes_per_token", "request_bytes", "memory_bill", "kv_bytes_logical", "kv_bytes_unique",
    "paged_waste", "contiguous_waste",
]
