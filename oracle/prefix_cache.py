"""Prefix cache over whole pages, and copy-on-write reservation (oracle; test
infrastructure).

Follows:
* "KV cache and PagedAttention" (askaiml.pages.dev), §6 "Prefix caching": when
  many requests start with the same long prompt, the engine hashes the prefix
  tokens, keeps the prefix's KV pages under that key, and a later request with
  the same prefix reuses those pages instead of computing them again.  Its
  list of pitfalls adds that the cache key must carry the user or tenant id,
  or different tenants' prompts leak into each other.
* same page, §4 "PagedAttention": several requests with a common prefix map
  the same physical pages.
* "KV Cache" glossary (inferensys.com), PagedAttention and prefix-caching
  entries: blocks are shared across sequences for parallel sampling and beam
  search; prefix caching reuses the KV of a shared prompt across requests.

Readings taken where the pages are silent (the library must give the same
page ids, counts and order):
* Granularity is one whole page of 16 tokens; a partly filled page is never
  cached.  A page's key is (tenant, key of the page before it, its 16 token
  ids): the KV of a token depends on every earlier token, so a page is reused
  only when the whole prefix up to and including it matches.  Keys compare
  exactly; a hash may locate them but never decides a match.
* The cache holds one reference on every cached page.  `match` walks the
  prompt's whole pages from the start and stops at the first miss; every
  matched page gets one more reference (the request's mapping).
* `insert` is called once the request's pages hold the prompt's KV: for each
  whole page of the prompt it keeps an existing entry with that key (the
  request's own page then stays private) or adds one for the request's page
  and retains it.  Every page of the row must be allocated, else nothing
  changes (BadBlock).
* Every touch (match or insert) stamps the entry with the next value of a
  counter.  `evict` frees pages least recently touched first, among entries
  that no request maps (page refcount 1: the cache's own reference) and that
  no other entry continues; removing an entry may make its parent evictable.
* Copy-on-write (askaiml §4 sharing; the glossary's parallel sampling and beam
  search): a request about to write into its partly filled last page while
  that page is shared gets a fresh page instead; the old page loses one
  reference and the pair (old, new) is returned so the caller copies the old
  contents first.  Per request the copy's page is allocated before any new
  pages, requests in order.  On any error every change is undone.
"""

import copy

from .allocator import BadBlock, NoBlocks


class RefPrefixCache:
    """Entries keyed by (tenant, parent key, tuple of 16 token ids)."""

    def __init__(self, alloc, block_size=16):
        self.alloc = alloc
        self.bs = block_size
        self.entries = {}   # key -> dict(block, tick, children)
        self.clock = 0

    def _keys(self, tenant, tokens):
        """Keys of the prompt's whole pages, in order."""
        keys, parent = [], None
        for i in range(len(tokens) // self.bs):
            k = (int(tenant), parent, tuple(int(t) for t in tokens[i * self.bs:(i + 1) * self.bs]))
            keys.append(k)
            parent = k
        return keys

    def _touch(self, e):
        self.clock += 1
        e["tick"] = self.clock

    def match(self, tenant, tokens):
        """Pages of the longest cached prefix of whole pages; each is retained."""
        out = []
        for k in self._keys(tenant, tokens):
            e = self.entries.get(k)
            if e is None:
                break
            self.alloc.retain(e["block"])
            self._touch(e)
            out.append(e["block"])
        return out

    def insert(self, tenant, tokens, table_row):
        """Cache the whole pages of `tokens`, held in table_row; returns how many
        entries were added."""
        keys = self._keys(tenant, tokens)
        if len(keys) > len(table_row):
            raise ValueError("table row shorter than the prompt's whole pages")
        for i in range(len(keys)):      # all or nothing: check before changing
            if self.alloc.refcount(int(table_row[i])) == 0:
                raise BadBlock(int(table_row[i]))
        added = 0
        for i, k in enumerate(keys):
            e = self.entries.get(k)
            if e is None:
                blk = int(table_row[i])
                self.alloc.retain(blk)      # BadBlock if not live
                e = {"block": blk, "tick": 0, "children": 0}
                self.entries[k] = e
                if k[1] is not None:
                    self.entries[k[1]]["children"] += 1
                added += 1
            self._touch(e)
        return added

    def evict(self, n):
        """Free up to n pages; returns them in eviction order."""
        freed = []
        while len(freed) < n:
            cands = [(e["tick"], k) for k, e in self.entries.items()
                     if e["children"] == 0 and self.alloc.refcount(e["block"]) == 1]
            if not cands:
                break
            _, k = min(cands)
            e = self.entries.pop(k)
            if k[1] is not None:
                self.entries[k[1]]["children"] -= 1
            self.alloc.release(e["block"])
            freed.append(e["block"])
        return freed

    def num_entries(self):
        return len(self.entries)


def reserve_cow(alloc, table, lens, n_new, block_size=16):
    """Batch reservation with copy-on-write.

    table: list of per-request page lists (extended and edited in place),
    lens: tokens held per request (advanced in place), n_new: tokens each
    request appends.  Returns (slots, copies): the slots of the new positions,
    request after request, and the (old page, new page) pairs to copy before
    the new tokens are written.  State is unchanged if an error is raised."""
    saved = (copy.deepcopy(alloc.__dict__), [list(r) for r in table], list(lens))
    bs = block_size
    slots, copies = [], []
    try:
        for b, add in enumerate(n_new):
            add = int(add)
            if add < 0 or lens[b] < 0:
                raise ValueError("negative length")
            if add == 0:
                continue
            row, n = table[b], lens[b]
            have = -(-n // bs)
            if n % bs:
                last = row[have - 1]
                if alloc.refcount(last) == 0:
                    raise BadBlock(last)
                if alloc.refcount(last) > 1:
                    new = alloc.alloc()
                    copies.append((last, new))
                    alloc.release(last)
                    row[have - 1] = new
            need = -(-(n + add) // bs)
            for _ in range(have, need):
                row.append(alloc.alloc())
            for pos in range(n, n + add):
                slots.append(row[pos // bs] * bs + pos % bs)
            lens[b] = n + add
    except (BadBlock, NoBlocks, ValueError):
        alloc.__dict__.update(saved[0])
        for r, old in zip(table, saved[1]):
            r[:] = old
        lens[:] = saved[2]
        raise
    return slots, copies
