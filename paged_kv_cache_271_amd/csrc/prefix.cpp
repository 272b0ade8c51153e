// Host half of prefix sharing: a cache of whole pages keyed by their prompt
// prefix, and a batch reservation that copies a shared page on write.
//
// "KV cache and PagedAttention" (askaiml.pages.dev), §6 "Prefix caching": the
// engine hashes the prefix tokens, keeps the prefix's KV pages under that key
// and lets a later request with the same prefix reuse them; its pitfalls say
// the key must carry the tenant.  §4 "PagedAttention": requests with a common
// prefix map the same pages.  "KV Cache" glossary (inferensys.com),
// PagedAttention entry: blocks are shared across sequences for parallel
// sampling and beam search, which is where copy-on-write comes in.
//
// A page's key is (tenant, entry of the page before it, its 16 tokens), so a
// page is reused only when everything before it matches as well.  Keys are
// compared exactly; an FNV-1a style hash over the key's 32-bit words only
// picks the hash bucket.  The cache holds one reference on each cached page; every match or
// insert touch stamps the entry with a counter, and eviction frees, least
// recently touched first, entries that no request maps (refcount 1) and that
// no other entry continues.

#include <algorithm>
#include <cstring>

#include "internal.h"

namespace pagedkv {

size_t PrefixKeyHash::operator()(const PrefixKey& k) const {
  // FNV-1a's xor-then-multiply step with its 64-bit offset basis and prime,
  // taken over 32-bit words instead of bytes (19 steps per key, not 76)
  uint64_t h = 0xcbf29ce484222325ull;
  auto step = [&h](uint32_t w) {
    h ^= w;
    h *= 0x100000001b3ull;
  };
  step(uint32_t(uint64_t(k.tenant)));
  step(uint32_t(uint64_t(k.tenant) >> 32));
  step(uint32_t(k.parent));
  for (const int32_t t : k.tokens) step(uint32_t(t));
  return size_t(h ^ (h >> 32));
}

namespace {

void touch(PrefixCache& c, int32_t e) {
  PrefixEntry& x = c.entries[e];
  if (x.children == 0) c.leaves.erase({x.tick, e});
  x.tick = ++c.clock;
  if (x.children == 0) c.leaves.insert({x.tick, e});
}

PrefixKey page_key(int64_t tenant, int32_t parent, const int32_t* tokens) {
  PrefixKey k;
  k.tenant = tenant;
  k.parent = parent;
  std::memcpy(k.tokens.data(), tokens, sizeof(int32_t) * kBlockSize);
  return k;
}

}  // namespace
}  // namespace pagedkv

using namespace pagedkv;

extern "C" {

int kv_prefix_match(kv_pool* p, int64_t tenant, const int32_t* tokens, int32_t n_tokens,
                    int32_t* blocks_out, int32_t max_blocks, int32_t* n_matched) {
  return nothrow_call([&]() -> int {
    if (!p || !n_matched) return fail(KV_E_INVALID, "NULL argument");
    if (n_tokens < 0 || max_blocks < 0) return fail(KV_E_INVALID, "negative size");
    const int32_t pages = std::min(n_tokens / kBlockSize, max_blocks);
    if (pages > 0 && (!tokens || !blocks_out)) return fail(KV_E_INVALID, "NULL array");
    PrefixCache& c = p->prefix;
    int32_t parent = -1, m = 0;
    for (; m < pages; ++m) {
      const auto it = c.index.find(page_key(tenant, parent, tokens + int64_t(m) * kBlockSize));
      if (it == c.index.end()) break;
      const int32_t e = it->second;
      ++p->rc[c.entries[e].block];  // live: the cache holds a reference
      touch(c, e);
      blocks_out[m] = c.entries[e].block;
      parent = e;
    }
    *n_matched = m;
    return ok();
  });
}

int kv_prefix_insert(kv_pool* p, int64_t tenant, const int32_t* tokens, int32_t n_tokens,
                     const int32_t* table_row, int32_t n_table, int32_t* n_added) {
  return nothrow_call([&]() -> int {
    if (!p || !n_added) return fail(KV_E_INVALID, "NULL argument");
    if (n_tokens < 0 || n_table < 0) return fail(KV_E_INVALID, "negative size");
    const int32_t pages = n_tokens / kBlockSize;
    if (pages > n_table)
      return fail(KV_E_INVALID, "%d whole pages of tokens but a table row of %d", pages, n_table);
    if (pages > 0 && (!tokens || !table_row)) return fail(KV_E_INVALID, "NULL array");
    for (int32_t i = 0; i < pages; ++i)  // all or nothing
      if (!block_live(p, table_row[i]))
        return fail(KV_E_BAD_BLOCK, "table entry %d (block %d) is out of range or free", i, table_row[i]);
    PrefixCache& c = p->prefix;
    int32_t parent = -1, added = 0;
    for (int32_t i = 0; i < pages; ++i) {
      const PrefixKey k = page_key(tenant, parent, tokens + int64_t(i) * kBlockSize);
      const auto it = c.index.find(k);
      int32_t e;
      if (it != c.index.end()) {
        e = it->second;
      } else {
        if (c.free_entries.empty()) {
          e = int32_t(c.entries.size());
          c.entries.push_back({});
        } else {
          e = c.free_entries.back();
          c.free_entries.pop_back();
        }
        PrefixEntry& x = c.entries[e];
        x.key = k;
        x.block = table_row[i];
        x.tick = 0;
        x.children = 0;
        ++p->rc[x.block];
        c.index.emplace(k, e);
        c.leaves.insert({0, e});
        if (parent >= 0) {
          PrefixEntry& par = c.entries[parent];
          if (par.children++ == 0) c.leaves.erase({par.tick, parent});
        }
        ++added;
      }
      touch(c, e);
      parent = e;
    }
    *n_added = added;
    return ok();
  });
}

int kv_prefix_evict(kv_pool* p, int32_t n_wanted, int32_t* blocks_freed, int32_t* n_freed) {
  return nothrow_call([&]() -> int {
    if (!p || !n_freed) return fail(KV_E_INVALID, "NULL argument");
    if (n_wanted < 0) return fail(KV_E_INVALID, "negative count");
    PrefixCache& c = p->prefix;
    int32_t freed = 0;
    while (freed < n_wanted) {
      int32_t e = -1;
      for (const auto& te : c.leaves) {  // oldest touch first
        if (p->rc[c.entries[te.second].block] == 1) {
          e = te.second;
          break;
        }
      }
      if (e < 0) break;
      PrefixEntry& x = c.entries[e];
      c.leaves.erase({x.tick, e});
      c.index.erase(x.key);
      if (x.key.parent >= 0) {
        PrefixEntry& par = c.entries[x.key.parent];
        if (--par.children == 0) c.leaves.insert({par.tick, x.key.parent});
      }
      const int32_t b = x.block;
      if (--p->rc[b] == 0) p->stack.push_back(b);
      c.free_entries.push_back(e);
      if (blocks_freed) blocks_freed[freed] = b;
      ++freed;
    }
    *n_freed = freed;
    return ok();
  });
}

int kv_prefix_num_entries(const kv_pool* p, int32_t* n) {
  if (!p || !n) return fail(KV_E_INVALID, "NULL argument");
  *n = int32_t(p->prefix.index.size());
  return ok();
}

int kv_batch_reserve_cow(kv_pool* p, int32_t B, int32_t* table, int32_t max_blocks, int32_t* lens,
                         const int32_t* n_new, int32_t* slots_out, int32_t* copy_src, int32_t* copy_dst,
                         int32_t* n_copies) {
  return nothrow_call([&]() -> int {
    if (!p || !n_copies) return fail(KV_E_INVALID, "NULL argument");
    if (B < 0 || max_blocks < 0) return fail(KV_E_INVALID, "negative size");
    *n_copies = 0;
    if (B == 0) return ok();
    if (!table || !lens || !n_new || !slots_out || !copy_src || !copy_dst)
      return fail(KV_E_INVALID, "NULL array");
    const int32_t bs = p->desc.block_size;
    // undo log: an allocation (table index, previous value, block) or, with
    // at = -1, the release of the shared page `prev` that was copied
    struct Undo {
      int64_t at;
      int32_t prev, blk;
    };
    std::vector<Undo> undo;
    // room for every allocation and release this call can log, before anything changes
    undo.reserve(reserve_bound(B, lens, n_new, bs, p->stack.size()) + size_t(B));
    auto take = [&](int64_t at, int32_t* slot_in_table) -> bool {
      if (p->stack.empty()) return false;
      const int32_t nb = p->stack.back();
      p->stack.pop_back();
      p->rc[nb] = 1;
      undo.push_back({at, *slot_in_table, nb});
      *slot_in_table = nb;
      return true;
    };
    int status = KV_OK;
    int64_t o = 0;
    int32_t nc = 0;
    for (int32_t b = 0; b < B && status == KV_OK; ++b) {
      const int32_t len = lens[b], add = n_new[b];
      if (len < 0 || add < 0) {
        status = fail(KV_E_INVALID, "request %d: negative length", b);
        break;
      }
      const int64_t end = int64_t(len) + add;
      if (end > INT32_MAX || kv_blocks_for_tokens(int32_t(end), bs) > max_blocks) {
        status = fail(KV_E_INVALID, "request %d grows to %lld tokens, beyond %d blocks", b, (long long)end,
                      max_blocks);
        break;
      }
      if (add == 0) continue;
      int32_t* row = table + int64_t(b) * max_blocks;
      const int32_t have = kv_blocks_for_tokens(len, bs);
      if (len % bs != 0) {  // the partly filled last page is written
        const int32_t last = row[have - 1];
        if (!block_live(p, last)) {
          status = fail(KV_E_BAD_BLOCK, "request %d: last block %d out of range or free", b, last);
          break;
        }
        if (p->rc[last] > 1) {  // shared: write into a private copy
          if (!take(int64_t(b) * max_blocks + have - 1, &row[have - 1])) {
            status = fail(KV_E_NO_BLOCKS, "request %d: no free block to copy shared block %d", b, last);
            break;
          }
          --p->rc[last];  // was > 1: still mapped elsewhere
          undo.push_back({-1, last, -1});
          copy_src[nc] = last;
          copy_dst[nc] = row[have - 1];
          ++nc;
        }
      }
      const int32_t need = kv_blocks_for_tokens(int32_t(end), bs);
      for (int32_t j = have; j < need; ++j) {
        if (!take(int64_t(b) * max_blocks + j, &row[j])) {
          status = fail(KV_E_NO_BLOCKS, "request %d: no free block for logical block %d", b, j);
          break;
        }
      }
      if (status != KV_OK) break;
      for (int32_t i = 0; i < add; ++i) {
        const int32_t pos = len + i;
        slots_out[o++] = row[pos / bs] * bs + pos % bs;
      }
    }
    if (status != KV_OK) {
      for (size_t i = undo.size(); i-- > 0;) {  // reverse order: stack as before
        const Undo& u = undo[i];
        if (u.at < 0) {
          ++p->rc[u.prev];
        } else {
          p->rc[u.blk] = 0;
          p->stack.push_back(u.blk);
          table[u.at] = u.prev;
        }
      }
      return status;
    }
    for (int32_t i = 0; i < B; ++i) lens[i] += n_new[i];
    *n_copies = nc;
    return ok();
  });
}

int kv_block_copy(kv_pool* p, const int32_t* src, const int32_t* dst, int32_t n, void* stream) {
  if (!p) return fail(KV_E_INVALID, "NULL pool");
  if (n < 0) return fail(KV_E_INVALID, "negative count");
  if (n == 0) return ok();
  if (!src || !dst) return fail(KV_E_INVALID, "NULL device array");
  return launch_block_copy(p, src, dst, n, static_cast<hipStream_t>(stream));
}

}  // extern "C"
