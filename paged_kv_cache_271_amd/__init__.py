"""MI355X-native paged KV cache: single-token GQA decode attention over a paged
cache, a slot-mapped append, and a refcounted O(1) block allocator, as a C-ABI
HIP library (libpagedkv.so) with a thin ctypes binding."""

from .binding import (  # noqa: F401
    KV_F32, KV_BF16, KV_FP8_E4M3, KV_INT8, BLOCK_SIZE, STATUS, SIGNATURES, KVError, KvPoolDesc, Pool,
    load_library, make_desc, kv_bytes_per_token, kv_blocks_for_tokens, kv_pool_buffer_bytes,
    kv_pool_create, kv_pool_destroy, kv_block_alloc, kv_block_retain, kv_block_release, kv_block_retain_n, kv_block_release_n,
    kv_block_refcount, kv_num_free_blocks, kv_num_shared_blocks, kv_slot_mapping, kv_batch_reserve, kv_append,
    paged_attention_workspace_bytes, paged_attention_workspace_init, new_workspace, paged_attention_decode,
    paged_attention_decode_append, paged_attention_decode_append_noalloc,
    kv_prefix_match, kv_prefix_insert, kv_prefix_evict, kv_prefix_num_entries, kv_batch_reserve_cow,
    kv_block_copy, paged_attention_decode_window, paged_attention_decode_window_append, kv_window_release, paged_attention_prefill, kv_probe_gather, kv_status_string,
    kv_last_error)
from .build import LIB_PATH, build as build_library  # noqa: F401
