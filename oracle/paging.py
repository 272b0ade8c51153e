"""Page tables, slot mapping, a byte-level model of the paged pool, and the
contiguous per-sequence cache (oracle; test infrastructure).

Follows:
* "KV cache and PagedAttention" (askaiml.pages.dev), §4 "PagedAttention": one
  big physical pool of pages, a per-request list of page indices, and an
  attention kernel that gathers K/V through that indirection.  A position p of
  a request lives in logical page p // block_size, at offset p % block_size.
* same page, §1 "The setup" and "Memoizing Context via KV Caching"
  (blog.sanjeevnode.in): each step appends the new token's K and V to the cache
  before attention reads the whole cache.
* same askaiml page, §3 "Naive implementation": one contiguous tensor per
  request, grown by concatenation along the token axis.  `SeqKV` is that model
  (per layer, per request), kept independent of the pool.
* "KV-Cache & PagedAttention" (parallelcs.dmj.one), "Common mistakes": a logical
  sequence may be physically scattered; only its logical content matters.

Readings taken where the pages are silent:
* Page size is 16 in every workload (the askaiml page's example size).
* Physical layout of one layer's pool (the library's documented layout, which
  `RefPool` models byte for byte):
      K: [num_blocks][num_kv_heads][block_size][head_dim]   (token-major tile)
      V: [num_blocks][num_kv_heads][head_dim][block_size]   (dim-major tile)
  so each (block, kv-head) tile of K and of V is one contiguous run of bytes.
  fp8 and int8 pools also hold one fp32 scale per (block, kv-head) for K and
  for V.
* Writing a token into a page mapped by more than one table is refused (the
  library answers KV_E_SHARED); the slot mapping raises SharedBlockWrite.
* A slot of -1 means "skip this token".
"""

import numpy as np

from .fp8 import e4m3_decode, quantize_run
from .int8 import int8_decode, quantize_run_int8
from .allocator import BadBlock


class SharedBlockWrite(Exception):
    """A token would be written into a page with reference count > 1."""


def bf16_bits_to_f64(bits):
    """uint16 bfloat16 bit patterns -> float64 (exact widening)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def raw_to_f64(raw, dtype):
    """Stored element representation -> float64.  fp8 needs scales, see RefPool."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(raw)
    raise ValueError(dtype)


def _raw_to_f32(raw, in_dtype):
    if in_dtype == "f32":
        return np.asarray(raw, dtype=np.float32)
    b = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def slot_for(table_row, pos, block_size):
    """Physical slot of logical position `pos` of one request."""
    return int(table_row[pos // block_size]) * block_size + pos % block_size


def slot_mapping(table_row, positions, block_size, refcount=None):
    """Slots for a list of positions of one request.

    With `refcount` (a callable block -> count), writing into an unallocated
    page raises BadBlock and into a shared page raises SharedBlockWrite.
    """
    out = []
    for p in positions:
        p = int(p)
        if p < 0 or p // block_size >= len(table_row):
            raise ValueError("position outside the table")
        blk = int(table_row[p // block_size])
        if refcount is not None:
            rc = refcount(blk)
            if rc == 0:
                raise BadBlock(blk)
            if rc > 1:
                raise SharedBlockWrite(blk)
        out.append(blk * block_size + p % block_size)
    return np.array(out, dtype=np.int64)


class SeqKV:
    """One request's cache for one layer as contiguous [n, h_kv, d_h] arrays,
    grown by concatenation.  Holds the raw stored representation of the
    *input* values (float32, or bf16 bit patterns)."""

    def __init__(self, num_kv_heads, head_dim, in_dtype):
        self.in_dtype = in_dtype
        np_t = np.float32 if in_dtype == "f32" else np.uint16
        self.K = np.zeros((0, num_kv_heads, head_dim), dtype=np_t)
        self.V = np.zeros((0, num_kv_heads, head_dim), dtype=np_t)

    def append(self, k_new, v_new):
        self.K = np.concatenate([self.K, np.asarray(k_new, dtype=self.K.dtype)], axis=0)
        self.V = np.concatenate([self.V, np.asarray(v_new, dtype=self.V.dtype)], axis=0)

    def __len__(self):
        return self.K.shape[0]

    def f64(self):
        return raw_to_f64(self.K, self.in_dtype), raw_to_f64(self.V, self.in_dtype)


class RefPool:
    """Byte-level model of the device pool (all layers).

    dtype: "f32" (inputs float32), "bf16" (inputs bf16 bits),
           "fp8" (inputs bf16 bits, stored as E4M3 codes plus scales),
           "int8" (inputs bf16 bits, stored as symmetric int8 codes plus scales).
    """

    def __init__(self, num_layers, num_blocks, num_kv_heads, head_dim,
                 block_size=16, dtype="bf16", k_init=None, v_init=None,
                 k_scale_init=None, v_scale_init=None):
        self.L, self.N, self.H, self.D, self.bs = (num_layers, num_blocks,
                                                   num_kv_heads, head_dim, block_size)
        self.dtype = dtype
        np_t = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8, "int8": np.int8}[dtype]
        kshape = (num_layers, num_blocks, num_kv_heads, block_size, head_dim)
        vshape = (num_layers, num_blocks, num_kv_heads, head_dim, block_size)
        self.K = np.zeros(kshape, np_t) if k_init is None else np.array(k_init, np_t).reshape(kshape)
        self.V = np.zeros(vshape, np_t) if v_init is None else np.array(v_init, np_t).reshape(vshape)
        if dtype in ("fp8", "int8"):
            sshape = (num_layers, num_blocks, num_kv_heads)
            self.Ks = np.zeros(sshape, np.float32) if k_scale_init is None \
                else np.array(k_scale_init, np.float32).reshape(sshape)
            self.Vs = np.zeros(sshape, np.float32) if v_scale_init is None \
                else np.array(v_scale_init, np.float32).reshape(sshape)
        self.in_dtype = "f32" if dtype == "f32" else "bf16"

    # -- write path ----------------------------------------------------------
    def append(self, layer, k_new, v_new, slots):
        """Write tokens t with slots[t] >= 0.  k_new, v_new: [T, H, D] raw
        inputs (float32 for f32 pools, bf16 bits otherwise)."""
        slots = [int(s) for s in slots]
        k_new = np.asarray(k_new)
        v_new = np.asarray(v_new)
        if self.dtype not in ("fp8", "int8"):
            for t, s in enumerate(slots):
                if s < 0:
                    continue
                blk, off = divmod(s, self.bs)
                self.K[layer, blk, :, off, :] = k_new[t]
                self.V[layer, blk, :, :, off] = v_new[t]
            return
        # fp8 / int8: group consecutive tokens that land in the same block into runs
        qrun = quantize_run if self.dtype == "fp8" else quantize_run_int8
        t = 0
        T = len(slots)
        while t < T:
            if slots[t] < 0:
                t += 1
                continue
            blk = slots[t] // self.bs
            u = t
            while u + 1 < T and slots[u + 1] >= 0 and slots[u + 1] // self.bs == blk:
                u += 1
            run = list(range(t, u + 1))
            offs = [slots[r] % self.bs for r in run]
            first = offs[0]
            kx = _raw_to_f32(k_new[run], "bf16")     # [n, H, D]
            vx = _raw_to_f32(v_new[run], "bf16")
            for g in range(self.H):
                # K tile [bs][D]
                codes, tile, s1 = qrun(kx[:, g, :], self.K[layer, blk, g],
                                               self.Ks[layer, blk, g], first)
                tile[offs] = codes
                self.K[layer, blk, g] = tile
                self.Ks[layer, blk, g] = s1
                # V tile is stored [D][bs]; quantise in [bs][D] view
                vt = self.V[layer, blk, g].T.copy()
                codes, vt, s1 = qrun(vx[:, g, :], vt, self.Vs[layer, blk, g], first)
                vt[offs] = codes
                self.V[layer, blk, g] = vt.T
                self.Vs[layer, blk, g] = s1
            t = u + 1

    # -- copy-on-write -------------------------------------------------------
    def copy_pages(self, src, dst):
        """Page dst[i] receives a copy of page src[i], in every layer, K and
        V (and both scales for 8-bit pools).  This is the private copy a
        request takes before writing into a page it shares ("KV Cache"
        glossary, PagedAttention entry: blocks shared by parallel samples or
        beams are copied when one of them writes).  Pairs with an id outside
        the pool, or src == dst, are skipped."""
        for s_, d_ in zip(src, dst):
            s_, d_ = int(s_), int(d_)
            if not (0 <= s_ < self.N and 0 <= d_ < self.N) or s_ == d_:
                continue
            self.K[:, d_] = self.K[:, s_]
            self.V[:, d_] = self.V[:, s_]
            if self.dtype in ("fp8", "int8"):
                self.Ks[:, d_] = self.Ks[:, s_]
                self.Vs[:, d_] = self.Vs[:, s_]

    # -- read path -----------------------------------------------------------
    def gather_raw(self, layer, table_row, n):
        """Raw stored K, V of the first n logical positions, [n, H, D]."""
        ks, vs = [], []
        for p in range(n):
            blk, off = int(table_row[p // self.bs]), p % self.bs
            ks.append(self.K[layer, blk, :, off, :])
            vs.append(self.V[layer, blk, :, :, off])
        np_t = self.K.dtype
        if n == 0:
            return (np.zeros((0, self.H, self.D), np_t), np.zeros((0, self.H, self.D), np_t))
        return np.stack(ks), np.stack(vs)

    def gather_f64(self, layer, table_row, n):
        """Values the attention reads for the first n positions, float64."""
        kr, vr = self.gather_raw(layer, table_row, n)
        if self.dtype not in ("fp8", "int8"):
            return raw_to_f64(kr, self.dtype), raw_to_f64(vr, self.dtype)
        ksc = np.array([self.Ks[layer, int(table_row[p // self.bs])] for p in range(n)],
                       dtype=np.float64).reshape(n, self.H, 1)
        vsc = np.array([self.Vs[layer, int(table_row[p // self.bs])] for p in range(n)],
                       dtype=np.float64).reshape(n, self.H, 1)
        dec = e4m3_decode if self.dtype == "fp8" else int8_decode
        return dec(kr) * ksc, dec(vr) * vsc
