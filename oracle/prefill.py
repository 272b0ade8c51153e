"""Causal prefill attention over a request's cache (oracle; test infrastructure).

Follows "KV cache and PagedAttention" (askaiml.pages.dev), §1 "The setup":
the prompt is processed in one big forward pass that fills the cache, after
which decode reads it a token at a time; the "KV Cache" glossary
(inferensys.com), FlashAttention entry: the prompt's attention is exact
attention, computed in tiles so the full score matrix never sits in HBM.

Readings taken where the pages are silent:
* The new tokens are the last P positions of the request's n cached tokens
  (their K and V already appended, as for a decode step); earlier positions
  (a cached prefix, or earlier chunks of a chunked prefill) are read as they
  are.  Query i of the P new tokens sits at position n - P + i and attends to
  positions t <= n - P + i (causal), with the same scaled softmax and GQA
  grouping as the decode.
* With P = 1 this is exactly the decode step.
"""

import numpy as np

from .attention import attention_fp64


def prefill_attention_fp64(q, K, V, scale):
    """q: [P, h_q, d] queries of the last P positions; K, V: [n, h_kv, d] the
    request's whole cache (n >= P).  Returns [P, h_q, d]."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    P, n = q.shape[0], K.shape[0]
    if P > n:
        raise ValueError("more queries than cached positions")
    out = np.zeros(q.shape, dtype=np.float64)
    for i in range(P):
        pos = n - P + i
        out[i] = attention_fp64(q[i], K[:pos + 1], V[:pos + 1], scale)
    return out


def prefill_flops(n_ctx, n_q, h_q, head_dim):
    """Multiply-adds counted as 2 FLOP: per (query, key it reads) 2*d for the
    score and 2*d for the weighted sum of V."""
    total = 0
    for c, p in zip(n_ctx, n_q):
        keys = sum(c - p + i + 1 for i in range(p))
        total += keys * h_q * 4 * head_dim
    return total
