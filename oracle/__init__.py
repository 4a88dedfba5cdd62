"""CPU oracle for paged decode attention (test infrastructure).

This package is the slow, obviously correct reference that the HIP path is checked
against. It is test infrastructure: only the test suite, the smoke check in
__graft_entry__ and the bench's CPU-baseline leg import it. The library under
paged_kv_cache_367_amd/ never imports, links or calls anything here, and nothing here
imports the library.

Everything is plain numpy in float64:

  storage      decoding of the four KV encodings (fp32, fp16, bf16, OCP fp8 E4M3FN)
               to float64, each from its bit-level definition.
  attention    decode_ref: gather each sequence's blocks through its block table into
               a contiguous array, truncate to the context length, and apply textbook
               softmax attention per query head (GQA kv head = h // group).
  cache_ops    cache_write_ref (slot write of new tokens), block_copy_ref (copy-on-write
               block copy) and block_swap_ref (blocks between two pools), bit copies.
  block_manager  BlockManager: free list, reference counts, copy-on-write, prefix-cache
               key chain, LRU eviction and swapping to a host pool (host bookkeeping).
  prefill      prefill_ref: n new query tokens per sequence attending causally over
               the paged cache (chunked prefill, prefix-cache tail prefill).
  quantize     e4m3_encode and cache_write_fp8_ref: the slot write into an fp8 E4M3
               cache, quantising each new value by a per-tensor scale.
  formulas     the per-token KV size formula.

Every function is pinned by tests in tests/test_oracle_*.py against values the pages
print, closed forms, library routines and brute force.
"""
from .storage import decode_storage, e4m3_table, bf16_bits_to_f64
from .attention import decode_ref, attend, gather_sequence, head_scales, kv_head_of
from .cache_ops import cache_write_ref, block_copy_ref, block_swap_ref
from .quantize import e4m3_encode, quant_inputs, cache_write_fp8_ref
from .prefill import prefill_ref, query_positions
from .formulas import kv_bytes_per_token, kv_bytes_per_request

__all__ = [
    "decode_storage", "e4m3_table", "bf16_bits_to_f64",
    "decode_ref", "attend", "gather_sequence", "head_scales", "kv_head_of",
    "cache_write_ref", "block_copy_ref", "block_swap_ref",
    "e4m3_encode", "quant_inputs", "cache_write_fp8_ref",
    "prefill_ref", "query_positions",
    "kv_bytes_per_token", "kv_bytes_per_request",
]
