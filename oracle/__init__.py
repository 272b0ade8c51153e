"""Reference oracle for paged single-token decode attention.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, CPU implementation
(NumPy, float64 for the attention arithmetic) of what the paged decode path
computes.  It exists to check the HIP library, so only the test suite, the
smoke check in ``__graft_entry__.smoke`` and the CPU-baseline leg of
``bench.py`` may import it.  The library and its Python binding never import
it, and it imports nothing from them: the two implementations share no code,
no constants tables and no helpers.

Sources (the pages this follows; section names as printed on each page):

* "KV-Cache & PagedAttention" (parallelcs.dmj.one) -- "Core concepts to master",
  "Common mistakes".
* "KV cache and PagedAttention" (askaiml.pages.dev) -- §1 "The setup",
  §2 "Memory cost" (formula and worked examples), §3 "Naive implementation",
  §4 "PagedAttention", §6 "Prefix caching", §7 "KV cache quantisation",
  §8 "Sliding-window cache and attention sinks", §9 "The big picture".
* "KV Cache" glossary (inferensys.com) -- cache-size calculation, PagedAttention
  block management, GQA and MQA entries.
* "Memoizing Context via KV Caching" (blog.sanjeevnode.in) -- the attention
  step: query compared against all keys, weights, weighted sum of values.

Readings taken where the pages are silent are listed in each module's header.
"""

from .sizes import (kv_bytes_per_token, kv_total_bytes, kv_total_bytes_hidden,
                    sliding_window_bytes, blocks_for, wasted_slots)
from .allocator import RefAllocator, AllocError, NoBlocks, BadBlock
from .paging import (slot_for, slot_mapping, SharedBlockWrite, RefPool, SeqKV,
                     bf16_bits_to_f64, raw_to_f64)
from .fp8 import (E4M3_MAX, e4m3_decode, e4m3_encode, e4m3_value_table,
                  quantize_run)
from .attention import (attention_fp64, attention_bruteforce, partitioned_fp64,
                        partition_states, combine_partitions, decode_batch_fp64)
from .int8 import INT8_MAX, int8_encode, int8_decode, quantize_run_int8
from .prefix_cache import RefPrefixCache, reserve_cow
from .prefill import prefill_attention_fp64, prefill_flops
from .window import (window_positions, attention_window_fp64, dead_pages, window_cache_bytes,
                     window_release)

__all__ = [
    "kv_bytes_per_token", "kv_total_bytes", "kv_total_bytes_hidden",
    "sliding_window_bytes", "blocks_for", "wasted_slots",
    "RefAllocator", "AllocError", "NoBlocks", "BadBlock",
    "slot_for", "slot_mapping", "SharedBlockWrite", "RefPool", "SeqKV",
    "bf16_bits_to_f64", "raw_to_f64",
    "E4M3_MAX", "e4m3_decode", "e4m3_encode", "e4m3_value_table", "quantize_run",
    "attention_fp64", "attention_bruteforce", "partitioned_fp64",
    "partition_states", "combine_partitions", "decode_batch_fp64",
    "INT8_MAX", "int8_encode", "int8_decode", "quantize_run_int8",
    "RefPrefixCache", "reserve_cow", "prefill_attention_fp64", "prefill_flops",
    "window_positions", "attention_window_fp64", "dead_pages", "window_cache_bytes", "window_release",
]
