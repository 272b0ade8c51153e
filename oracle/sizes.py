"""KV-cache memory arithmetic and block counts (oracle; test infrastructure).

Follows:
* "KV cache and PagedAttention" (askaiml.pages.dev), §2 "Memory cost": the
  per-token cost is two tensors (K and V) per layer, each holding one vector of
  h_kv * d_h elements of b bytes; the batch total multiplies by B * T.
* "KV Cache" glossary (inferensys.com), cache-size calculation: the same cost
  written with the model's hidden width in place of h_kv * d_h (the multi-head
  special case, where every query head has its own KV head).
* same askaiml page, §8 "Sliding-window cache": a window of W tokens costs W
  tokens' worth, independent of the sequence length.
* same askaiml page, §4 "PagedAttention": storage is handed out in fixed pages of
  block_size tokens, so a request of n tokens holds ceil(n / block_size) pages
  and wastes the unused tail of the last one.

All results are exact Python integers.
"""


def kv_bytes_per_token(num_layers, num_kv_heads, head_dim, dtype_bytes):
    """Bytes of K plus V one token occupies across all layers."""
    return 2 * num_layers * num_kv_heads * head_dim * dtype_bytes


def kv_total_bytes(batch, seq_len, num_layers, num_kv_heads, head_dim, dtype_bytes):
    """Bytes of K plus V for `batch` requests of `seq_len` tokens each."""
    return batch * seq_len * kv_bytes_per_token(num_layers, num_kv_heads,
                                                head_dim, dtype_bytes)


def kv_total_bytes_hidden(batch, seq_len, num_layers, hidden_dim, dtype_bytes):
    """The glossary's form, with the hidden width standing for h_kv * d_h."""
    return 2 * batch * seq_len * num_layers * hidden_dim * dtype_bytes


def sliding_window_bytes(window, num_layers, kv_width, dtype_bytes):
    """Per-request bytes of a cache that keeps only the last `window` tokens."""
    return 2 * window * num_layers * kv_width * dtype_bytes


def blocks_for(n_tokens, block_size):
    """Number of fixed-size pages needed to hold n_tokens (ceiling division)."""
    if n_tokens < 0 or block_size <= 0:
        raise ValueError("n_tokens must be >= 0 and block_size > 0")
    return (n_tokens + block_size - 1) // block_size


def wasted_slots(n_tokens, block_size):
    """Token slots reserved but unused in the last page of an n-token request."""
    return blocks_for(n_tokens, block_size) * block_size - n_tokens
