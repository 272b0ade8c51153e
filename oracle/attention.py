"""Single-token decode attention over one request's cache (oracle; test
infrastructure).

Follows "Memoizing Context via KV Caching" (blog.sanjeevnode.in), first
section: the current token's query is compared against the keys of every
cached token to give attention weights, and the output is the weighted sum of
the value vectors.  "KV cache and PagedAttention" (askaiml.pages.dev), §1 "The
setup": the new token's own K and V are in the cache when attention reads it.
"KV Cache" glossary (inferensys.com), GQA and MQA entries: several query heads
share one KV head.

Readings taken where the pages are silent:
* The weights are the softmax of the scaled dot products
  s_t = scale * <q_h, k_t>, with `scale` supplied by the caller (1/sqrt(d_h) in
  every workload).
* GQA grouping is contiguous: query head h reads KV head h // G with
  G = h_q / h_kv.  G = 1 is ordinary multi-head attention, h_kv = 1 is MQA.
* A request with no cached tokens yields an all-zero output.

`partition_states` / `combine_partitions` restate the same result as a split
over token ranges: each range keeps (m, l, acc) = (max score, sum of
exp(s - m), sum of exp(s - m) * v), and the ranges merge by rescaling to the
common maximum.  In exact arithmetic it equals the unsplit softmax.
"""

import math

import numpy as np


def _check(q, K, V):
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    h_q, d = q.shape
    n, h_kv, dk = K.shape
    if V.shape != K.shape or dk != d or h_q % h_kv != 0:
        raise ValueError("shape mismatch")
    return q, K, V, h_q // h_kv


def attention_fp64(q, K, V, scale):
    """q: [h_q, d]; K, V: [n, h_kv, d] (float64 values).  Returns [h_q, d]."""
    q, K, V, G = _check(q, K, V)
    h_q, d = q.shape
    out = np.zeros((h_q, d), dtype=np.float64)
    if K.shape[0] == 0:
        return out
    for h in range(h_q):
        g = h // G
        s = scale * (K[:, g, :] @ q[h])          # [n]
        e = np.exp(s - s.max())
        p = e / e.sum()
        out[h] = p @ V[:, g, :]
    return out


def attention_bruteforce(q, K, V, scale):
    """The same definition with scalar math.exp / math.fsum loops (tiny inputs)."""
    q, K, V, G = _check(q, K, V)
    h_q, d = q.shape
    n = K.shape[0]
    out = [[0.0] * d for _ in range(h_q)]
    if n == 0:
        return np.array(out)
    for h in range(h_q):
        g = h // G
        s = [scale * math.fsum(q[h, i] * K[t, g, i] for i in range(d)) for t in range(n)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = math.fsum(e)
        for i in range(d):
            out[h][i] = math.fsum(e[t] / z * V[t, g, i] for t in range(n))
    return np.array(out)


def partition_states(q, K, V, scale, part):
    """Per-range (m, l, acc) for ranges [j*part, (j+1)*part).  Returns lists
    indexed by range j of arrays m [h_q], l [h_q], acc [h_q, d]."""
    q, K, V, G = _check(q, K, V)
    h_q, d = q.shape
    n = K.shape[0]
    states = []
    for start in range(0, n, part):
        Kj, Vj = K[start:start + part], V[start:start + part]
        m = np.empty(h_q)
        l = np.empty(h_q)
        acc = np.empty((h_q, d))
        for h in range(h_q):
            g = h // G
            s = scale * (Kj[:, g, :] @ q[h])
            m[h] = s.max()
            e = np.exp(s - m[h])
            l[h] = e.sum()
            acc[h] = e @ Vj[:, g, :]
        states.append((m, l, acc))
    return states


def combine_partitions(states, h_q, d):
    """Merge per-range states into the normalised output."""
    if not states:
        return np.zeros((h_q, d))
    M = np.max([m for m, _, _ in states], axis=0)
    L = np.zeros(h_q)
    A = np.zeros((h_q, d))
    for m, l, acc in states:
        w = np.exp(m - M)
        L += w * l
        A += w[:, None] * acc
    return A / L[:, None]


def partitioned_fp64(q, K, V, scale, part):
    q = np.asarray(q, dtype=np.float64)
    return combine_partitions(partition_states(q, K, V, scale, part), *q.shape)


def decode_batch_fp64(q_batch, seqs, scale):
    """Batch decode: q_batch [B, h_q, d] float64; seqs: list of (K, V) float64
    [n_b, h_kv, d].  Returns [B, h_q, d]."""
    q_batch = np.asarray(q_batch, dtype=np.float64)
    return np.stack([attention_fp64(q_batch[b], K, V, scale)
                     for b, (K, V) in enumerate(seqs)])
