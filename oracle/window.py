"""Sliding-window decode with attention sinks (oracle; test infrastructure).

Follows "KV cache and PagedAttention" (askaiml.pages.dev), §8 "Sliding-window
cache and attention sinks": a model trained with sliding-window attention only
needs the last W tokens in its cache, so the cache stays the same size however
long the sequence grows (2 * W * L * d_kv * b bytes per request); with
attention sinks the first few tokens are kept as well as the last W.

Readings taken where the page is silent:
* For a request of n tokens (the new one included) the decode attends over
  positions T(n) = {t < S} U {n - W <= t < n}, with S sink tokens and a window
  of W >= 1 tokens; positions keep their original index (the cache holds keys
  as they were written).  When S + W >= n that is every position.
* The attention over T(n) is the ordinary one (`attention_fp64`) applied to the
  selected positions.
* A page can go back to the pool once none of its positions can be read again:
  the window only moves forward as the request grows, so page p (positions
  16p .. 16p + 15) is dead for a request of n tokens when all its positions
  are at or past S and before n - W.  `window_release` drops the request's
  reference on each dead page, request by request and page by page, and marks
  the table entry -1 (a free page is never read again by that request).
"""

import numpy as np

from .attention import attention_fp64


def window_positions(n, sink, window):
    """Sorted positions T(n) the decode reads."""
    if window < 1 or sink < 0:
        raise ValueError("window must be >= 1 and sink >= 0")
    return [t for t in range(n) if t < sink or t >= n - window]


def attention_window_fp64(q, K, V, scale, sink, window):
    """Decode attention of one request over T(n), n = len(K)."""
    idx = window_positions(len(K), sink, window)
    K = np.asarray(K)[idx]
    V = np.asarray(V)[idx]
    return attention_fp64(q, K, V, scale)


def dead_pages(n, sink, window, block_size=16):
    """Logical pages of an n-token request that no later decode reads."""
    if window < 1 or sink < 0:
        raise ValueError("window must be >= 1 and sink >= 0")
    out = []
    for p in range(-(-n // block_size)):
        lo, hi = p * block_size, (p + 1) * block_size
        if lo >= sink and hi <= n - window:
            out.append(p)
    return out


def window_cache_bytes(window, sink, num_layers, kv_width, dtype_bytes):
    """Bytes one request keeps in a window-plus-sinks cache (whole tokens,
    before rounding to pages): the page's formula 2 * W * L * d_kv * b with
    the sink tokens added to W."""
    return 2 * (window + sink) * num_layers * kv_width * dtype_bytes


def window_release(alloc, table, lens, sink, window, block_size=16):
    """Give back every dead page of each request (request order, then page
    order), marking its table entry -1; entries already -1 are skipped.
    table: per-request page lists (edited in place).  Returns the number
    released.  Nothing changes if a page is not allocated (BadBlock)."""
    from .allocator import BadBlock
    drops = {}
    for b, row in enumerate(table):
        for p in dead_pages(lens[b], sink, window, block_size):
            blk = row[p]
            if blk == -1:
                continue
            drops[blk] = drops.get(blk, 0) + 1
            if alloc.refcount(blk) < drops[blk]:
                raise BadBlock(blk)
    n = 0
    for b, row in enumerate(table):
        for p in dead_pages(lens[b], sink, window, block_size):
            if row[p] == -1:
                continue
            alloc.release(row[p])
            row[p] = -1
            n += 1
    return n
