// Host half of libpagedkv: pool descriptor checks, the O(1) LIFO block
// allocator with reference counts, slot mapping, the batched per-step
// reservation, argument checks of the device entry points, and error strings.
//
// The allocator follows "KV cache and PagedAttention" (askaiml.pages.dev),
// §4 "PagedAttention": uniform pages make allocation O(1) and let requests
// with a common prefix share pages; the slot of position p of a request is
// table[p / block_size] * block_size + p % block_size.

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <memory>

#include "internal.h"

namespace {
thread_local char g_last_error[512];

bool desc_valid(const kv_pool_desc* d) {
  return d && d->num_layers >= 1 && d->num_blocks >= 1 && d->block_size >= 1 &&
         d->num_kv_heads >= 1 && d->head_dim >= 1 && d->cache_dtype >= KV_F32 &&
         d->cache_dtype <= KV_INT8;
}
}  // namespace

namespace pagedkv {

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return status;
}

int ok() { return KV_OK; }

}  // namespace pagedkv

using namespace pagedkv;

extern "C" {

int64_t kv_bytes_per_token(const kv_pool_desc* d) {
  if (!desc_valid(d)) return -1;
  return 2 * int64_t(d->num_layers) * d->num_kv_heads * d->head_dim * elem_bytes(d->cache_dtype);
}

int32_t kv_blocks_for_tokens(int32_t n, int32_t block_size) {
  if (n < 0 || block_size <= 0) return -1;
  return int32_t((int64_t(n) + block_size - 1) / block_size);
}

int kv_pool_buffer_bytes(const kv_pool_desc* d, int64_t* cache_bytes, int64_t* scale_bytes) {
  if (!desc_valid(d)) return fail(KV_E_INVALID, "invalid pool descriptor");
  const int64_t cb = int64_t(d->num_layers) * layer_elems(*d) * elem_bytes(d->cache_dtype);
  const int64_t sb = scaled_dtype(d->cache_dtype)
                         ? int64_t(d->num_layers) * d->num_blocks * d->num_kv_heads * 4
                         : 0;
  if (cache_bytes) *cache_bytes = cb;
  if (scale_bytes) *scale_bytes = sb;
  return ok();
}

int kv_pool_create(const kv_pool_desc* d, void* k_cache, void* v_cache, float* k_scale,
                   float* v_scale, const int32_t* order, kv_pool** out) {
  return nothrow_call([&]() -> int {
    if (!out) return fail(KV_E_INVALID, "out is NULL");
    *out = nullptr;
    if (!desc_valid(d)) return fail(KV_E_INVALID, "invalid pool descriptor");
    if (d->block_size != kBlockSize)
      return fail(KV_E_UNSUPPORTED, "block_size %d not supported (16 only)", d->block_size);
    if (d->head_dim != 64 && d->head_dim != 128)
      return fail(KV_E_UNSUPPORTED, "head_dim %d not supported (64 or 128)", d->head_dim);
    if (!k_cache || !v_cache) return fail(KV_E_INVALID, "k_cache and v_cache are required");
    const bool scaled = scaled_dtype(d->cache_dtype);
    if (scaled && (!k_scale || !v_scale))
      return fail(KV_E_INVALID, "fp8 and int8 pools need k_scale and v_scale");
    if (!scaled && (k_scale || v_scale))
      return fail(KV_E_INVALID, "scale arrays are only for fp8 and int8 pools");
    const int32_t n = d->num_blocks;
    std::vector<int32_t> seen(n, 0);
    std::unique_ptr<kv_pool> owned(new kv_pool());
    kv_pool* p = owned.get();
    p->desc = *d;
    p->k_cache = k_cache;
    p->v_cache = v_cache;
    p->k_scale = k_scale;
    p->v_scale = v_scale;
    p->rc.assign(n, 0);
    p->stack.resize(n);
    for (int32_t i = 0; i < n; ++i) {
      const int32_t b = order ? order[i] : i;
      if (b < 0 || b >= n || seen[b])
        return fail(KV_E_INVALID, "initial_free_order is not a permutation (entry %d = %d)", i, b);
      seen[b] = 1;
      p->stack[n - 1 - i] = b;  // order[0] ends on top
    }
    *out = owned.release();
    return ok();
  });
}

int kv_pool_destroy(kv_pool* p) {
  delete p;
  return ok();
}

int kv_block_alloc(kv_pool* p, int32_t* block) {
  if (!p || !block) return fail(KV_E_INVALID, "NULL argument");
  if (p->stack.empty()) return fail(KV_E_NO_BLOCKS, "no free block (pool of %d)", p->desc.num_blocks);
  const int32_t b = p->stack.back();
  p->stack.pop_back();
  p->rc[b] = 1;
  *block = b;
  return ok();
}

int kv_block_retain(kv_pool* p, int32_t b) {
  if (!p) return fail(KV_E_INVALID, "NULL pool");
  if (!block_live(p, b)) return fail(KV_E_BAD_BLOCK, "retain of block %d that is out of range or free", b);
  ++p->rc[b];
  return ok();
}

int kv_block_release(kv_pool* p, int32_t b) {
  if (!p) return fail(KV_E_INVALID, "NULL pool");
  if (!block_live(p, b)) return fail(KV_E_BAD_BLOCK, "release of block %d that is out of range or free", b);
  if (--p->rc[b] == 0) p->stack.push_back(b);
  return ok();
}

int kv_block_retain_n(kv_pool* p, const int32_t* blocks, int32_t n) {
  if (!p || n < 0 || (n > 0 && !blocks)) return fail(KV_E_INVALID, "invalid arguments");
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = blocks[i];
    if (!block_live(p, b)) {
      for (int32_t j = i; j-- > 0;) --p->rc[blocks[j]];  // counts were >= 2, none freed
      return fail(KV_E_BAD_BLOCK, "retain of block %d (entry %d) that is out of range or free", b, i);
    }
    ++p->rc[b];
  }
  return ok();
}

int kv_block_release_n(kv_pool* p, const int32_t* blocks, int32_t n) {
  if (!p || n < 0 || (n > 0 && !blocks)) return fail(KV_E_INVALID, "invalid arguments");
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = blocks[i];
    if (!block_live(p, b)) {
      for (int32_t j = i; j-- > 0;) {  // undo in reverse: a freed block is on top
        const int32_t u = blocks[j];
        if (p->rc[u] == 0) p->stack.pop_back();
        ++p->rc[u];
      }
      return fail(KV_E_BAD_BLOCK, "release of block %d (entry %d) that is out of range or free", b, i);
    }
    if (--p->rc[b] == 0) p->stack.push_back(b);
  }
  return ok();
}

int kv_num_shared_blocks(const kv_pool* p, int32_t* n) {
  if (!p || !n) return fail(KV_E_INVALID, "NULL argument");
  *n = p->rc.shared();
  return ok();
}

int kv_block_refcount(const kv_pool* p, int32_t b, int32_t* rc) {
  if (!p || !rc) return fail(KV_E_INVALID, "NULL argument");
  if (b < 0 || b >= p->desc.num_blocks) return fail(KV_E_BAD_BLOCK, "block %d out of range", b);
  *rc = p->rc[b];
  return ok();
}

int kv_num_free_blocks(const kv_pool* p, int32_t* n) {
  if (!p || !n) return fail(KV_E_INVALID, "NULL argument");
  *n = int32_t(p->stack.size());
  return ok();
}

int kv_slot_mapping(const kv_pool* p, const int32_t* table_row, int32_t n_table,
                    const int32_t* positions, int32_t n, int32_t* slots_out) {
  if (!p) return fail(KV_E_INVALID, "NULL pool");
  if (n < 0 || n_table < 0) return fail(KV_E_INVALID, "negative size");
  if (n > 0 && (!positions || !slots_out || (n_table > 0 && !table_row)))
    return fail(KV_E_INVALID, "NULL array");
  const int32_t bs = p->desc.block_size;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t pos = positions[i];
    if (pos < 0 || pos / bs >= n_table)
      return fail(KV_E_INVALID, "position %d (index %d) outside a table of %d blocks", pos, i, n_table);
    const int32_t b = table_row[pos / bs];
    if (!block_live(p, b)) return fail(KV_E_BAD_BLOCK, "position %d maps to block %d that is out of range or free", pos, b);
    if (p->rc[b] > 1) return fail(KV_E_SHARED, "position %d maps to block %d shared by %d tables", pos, b,
                                  int32_t(p->rc[b]));
    slots_out[i] = b * bs + pos % bs;
  }
  return ok();
}

int kv_batch_reserve(kv_pool* p, int32_t B, int32_t* table, int32_t max_blocks, int32_t* lens,
                     const int32_t* n_new, int32_t* slots_out) {
  return nothrow_call([&]() -> int {
    if (!p) return fail(KV_E_INVALID, "NULL pool");
    if (B < 0 || max_blocks < 0) return fail(KV_E_INVALID, "negative size");
    if (B == 0) return ok();
    if (!table || !lens || !n_new || !slots_out) return fail(KV_E_INVALID, "NULL array");
    const int32_t bs = p->desc.block_size;
    // (request, block index, previous table value) of every block taken here
    std::vector<int64_t> taken_at;
    std::vector<int32_t> taken_prev, taken_blk;
    {  // room for every block this call can take, before anything changes
      const size_t cap = reserve_bound(B, lens, n_new, bs, p->stack.size());
      taken_at.reserve(cap);
      taken_prev.reserve(cap);
      taken_blk.reserve(cap);
    }
    int status = KV_OK;
    int64_t o = 0;
    int32_t b = 0;
    for (; b < B && status == KV_OK; ++b) {
      const int32_t len = lens[b], add = n_new[b];
      if (len < 0 || add < 0) {
        status = fail(KV_E_INVALID, "request %d: negative length", b);
        break;
      }
      const int64_t end = int64_t(len) + add;
      if (kv_blocks_for_tokens(int32_t(end), bs) > max_blocks || end > INT32_MAX) {
        status = fail(KV_E_INVALID, "request %d grows to %lld tokens, beyond %d blocks", b,
                      (long long)end, max_blocks);
        break;
      }
      if (add == 0) continue;
      int32_t* row = table + int64_t(b) * max_blocks;
      const int32_t have = kv_blocks_for_tokens(len, bs);
      if (len % bs != 0) {  // the partially filled last block is written in place
        const int32_t last = row[have - 1];
        if (!block_live(p, last)) {
          status = fail(KV_E_BAD_BLOCK, "request %d: last block %d out of range or free", b, last);
          break;
        }
        if (p->rc[last] > 1) {
          status = fail(KV_E_SHARED, "request %d: last block %d is shared", b, last);
          break;
        }
      }
      const int32_t need = kv_blocks_for_tokens(int32_t(end), bs);
      for (int32_t j = have; j < need; ++j) {
        if (p->stack.empty()) {
          status = fail(KV_E_NO_BLOCKS, "request %d: no free block for logical block %d", b, j);
          break;
        }
        const int32_t nb = p->stack.back();
        p->stack.pop_back();
        p->rc[nb] = 1;
        taken_at.push_back(int64_t(b) * max_blocks + j);
        taken_prev.push_back(row[j]);
        taken_blk.push_back(nb);
        row[j] = nb;
      }
      if (status != KV_OK) break;
      for (int32_t i = 0; i < add; ++i) {
        const int32_t pos = len + i;
        slots_out[o++] = row[pos / bs] * bs + pos % bs;
      }
    }
    if (status != KV_OK) {
      for (size_t i = taken_blk.size(); i-- > 0;) {  // undo in reverse: stack as before
        p->rc[taken_blk[i]] = 0;
        p->stack.push_back(taken_blk[i]);
        table[taken_at[i]] = taken_prev[i];
      }
      return status;
    }
    for (int32_t i = 0; i < B; ++i) lens[i] += n_new[i];
    return ok();
  });
}

int kv_append(kv_pool* p, int32_t layer, const void* k_new, const void* v_new,
              const int32_t* slots, int32_t T, void* stream) {
  if (!p) return fail(KV_E_INVALID, "NULL pool");
  if (layer < 0 || layer >= p->desc.num_layers) return fail(KV_E_INVALID, "layer %d out of range", layer);
  if (T < 0) return fail(KV_E_INVALID, "negative token count");
  if (T == 0) return ok();
  if (!k_new || !v_new || !slots) return fail(KV_E_INVALID, "NULL device array");
  return launch_append(p, layer, k_new, v_new, slots, T, static_cast<hipStream_t>(stream));
}

int64_t paged_attention_workspace_bytes(const kv_pool* p, int32_t B, int32_t h_q, int32_t max_ctx,
                                        int32_t part) {
  if (!p || B < 0 || h_q <= 0 || max_ctx < 0 || part < 0) return -1;
  if (h_q % p->desc.num_kv_heads != 0) return -1;
  DecodeArgs plan{};
  const int64_t need = plan_decode(p->desc, B, h_q, max_ctx, part, &plan);
  return need < 0 ? -1 : need;
}

int paged_attention_workspace_init(const kv_pool* p, void* ws, int64_t ws_bytes, void* stream) {
  if (!p) return fail(KV_E_INVALID, "NULL pool");
  if (ws_bytes < 0) return fail(KV_E_INVALID, "negative workspace size");
  if (p->desc.cache_dtype == KV_F32 || ws_bytes == 0) return ok();  // no counters
  if (!ws) return fail(KV_E_INVALID, "NULL workspace");
  if (reinterpret_cast<uintptr_t>(ws) % 16 != 0) return fail(KV_E_INVALID, "workspace not 16-byte aligned");
  if (ws_bytes < kMergeCounterBytes)
    return fail(KV_E_WORKSPACE, "workspace of %lld bytes, below the %lld counter bytes", (long long)ws_bytes,
                (long long)kMergeCounterBytes);
  return launch_zero(ws, kMergeCounterBytes, static_cast<hipStream_t>(stream));
}

namespace {

// Checks shared by the decode entry points; fills the plan on success.
int prepare_decode(kv_pool* p, int32_t layer, void* out, const void* q, int32_t q_dtype,
                   const int32_t* tables, int32_t max_blocks, const int32_t* ctx, int32_t B, int32_t h_q,
                   int32_t max_ctx, float scale, int32_t part, void* ws, int64_t ws_bytes, DecodeArgs* a) {
  if (!p) return fail(KV_E_INVALID, "NULL pool");
  const kv_pool_desc& d = p->desc;
  if (layer < 0 || layer >= d.num_layers) return fail(KV_E_INVALID, "layer %d out of range", layer);
  if (B < 0) return fail(KV_E_INVALID, "negative batch");
  if (B == 0) return KV_OK;  // nothing to do; the caller returns before launching
  if (B > 65535) return fail(KV_E_UNSUPPORTED, "batch %d above 65535", B);
  if (!out || !q || !tables || !ctx) return fail(KV_E_INVALID, "NULL device array");
  const int32_t want_q = d.cache_dtype == KV_F32 ? KV_F32 : KV_BF16;
  if (q_dtype != want_q)
    return fail(KV_E_UNSUPPORTED, "q dtype %d does not match the pool (needs %d)", q_dtype, want_q);
  if (h_q <= 0 || h_q % d.num_kv_heads != 0)
    return fail(KV_E_INVALID, "h_q %d is not a positive multiple of %d KV heads", h_q, d.num_kv_heads);
  if (max_blocks <= 0 || max_ctx < 0 || int64_t(max_ctx) > int64_t(max_blocks) * d.block_size)
    return fail(KV_E_INVALID, "max_ctx %d outside [0, %d blocks * %d]", max_ctx, max_blocks, d.block_size);
  if (part < 0 || part % d.block_size != 0)
    return fail(KV_E_INVALID, "partition_tokens %d is not a multiple of %d", part, d.block_size);
  const int64_t need = plan_decode(d, B, h_q, max_ctx, part, a);
  if (need < 0) return int(need);  // plan_decode recorded the message
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(KV_E_WORKSPACE, "workspace of %lld bytes, %lld needed", (long long)ws_bytes, (long long)need);
  if (need > 0 && reinterpret_cast<uintptr_t>(ws) % 16 != 0)
    return fail(KV_E_INVALID, "workspace not 16-byte aligned");
  a->pool = p;
  a->layer = layer;
  a->out = out;
  a->q = q;
  a->tables = tables;
  a->max_blocks = max_blocks;
  a->ctx = ctx;
  a->B = B;
  a->h_q = h_q;
  a->max_ctx = max_ctx;
  a->scale = scale;
  if (need > 0) {
    // bf16 / fp8 / int8: the merge counters come first
    char* base = static_cast<char*>(ws);
    if (d.cache_dtype != KV_F32) {
      a->ws_cnt = reinterpret_cast<int32_t*>(base);
      base += kMergeCounterBytes;
    }
    a->ws_ml = reinterpret_cast<float*>(base);
    a->ws_acc = a->ws_ml + a->slots * 2;
    a->ws_pref = reinterpret_cast<int32_t*>(a->ws_acc + a->slots * d.head_dim);
  }
  return KV_OK;
}

}  // namespace

int paged_attention_decode(kv_pool* p, int32_t layer, void* out, const void* q, int32_t q_dtype,
                           const int32_t* tables, int32_t max_blocks, const int32_t* ctx, int32_t B,
                           int32_t h_q, int32_t max_ctx, float scale, int32_t part, void* ws,
                           int64_t ws_bytes, void* stream) {
  DecodeArgs a{};
  const int st = prepare_decode(p, layer, out, q, q_dtype, tables, max_blocks, ctx, B, h_q, max_ctx, scale,
                                part, ws, ws_bytes, &a);
  if (st != KV_OK) return st;
  if (B == 0) return ok();
  return launch_decode(a, static_cast<hipStream_t>(stream));
}

int paged_attention_decode_append(kv_pool* p, int32_t layer, void* out, const void* q, int32_t q_dtype,
                                  const void* k_new, const void* v_new, const int32_t* slot_mapping,
                                  const int32_t* tables, int32_t max_blocks, const int32_t* ctx, int32_t B,
                                  int32_t h_q, int32_t max_ctx, float scale, int32_t part, void* ws,
                                  int64_t ws_bytes, void* stream) {
  DecodeArgs a{};
  const int st = prepare_decode(p, layer, out, q, q_dtype, tables, max_blocks, ctx, B, h_q, max_ctx, scale,
                                part, ws, ws_bytes, &a);
  if (st != KV_OK) return st;
  if (B == 0) return ok();
  if (!k_new || !v_new || !slot_mapping) return fail(KV_E_INVALID, "NULL device array");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // one kernel for bf16 pools, and for fp8 / int8 pools whose kv heads have
  // at most 16 query heads (one wave owns each tile it appends to); f32 and
  // the other 8-bit shapes run the append kernel, then the decode
  const bool q8 = scaled_dtype(p->desc.cache_dtype);
  if (p->desc.cache_dtype != KV_BF16 && !(q8 && h_q / p->desc.num_kv_heads <= 16)) {
    const int e = launch_append(p, layer, k_new, v_new, slot_mapping, B, s);
    if (e != KV_OK) return e;
    return launch_decode(a, s);
  }
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_slots = slot_mapping;
  return launch_decode(a, s);
}

int paged_attention_decode_window(kv_pool* p, int32_t layer, void* out, const void* q, int32_t q_dtype,
                                  const int32_t* tables, int32_t max_blocks, const int32_t* ctx, int32_t B,
                                  int32_t h_q, int32_t max_ctx, float scale, int32_t sink, int32_t window,
                                  int32_t part, void* ws, int64_t ws_bytes, void* stream) {
  if (p && p->desc.cache_dtype == KV_F32)
    return fail(KV_E_UNSUPPORTED, "sliding-window decode is built for bf16 and fp8 pools");
  if (sink < 0 || window < 1)
    return fail(KV_E_INVALID, "sink %d must be >= 0 and window %d >= 1", sink, window);
  DecodeArgs a{};
  const int st = prepare_decode(p, layer, out, q, q_dtype, tables, max_blocks, ctx, B, h_q, max_ctx, scale,
                                part, ws, ws_bytes, &a);
  if (st != KV_OK) return st;
  if (B == 0) return ok();
  a.sink = sink;
  a.window = window;
  return launch_decode(a, static_cast<hipStream_t>(stream));
}

int paged_attention_decode_window_append(kv_pool* p, int32_t layer, void* out, const void* q, int32_t q_dtype,
                                         const void* k_new, const void* v_new, const int32_t* slot_mapping,
                                         const int32_t* tables, int32_t max_blocks, const int32_t* ctx, int32_t B,
                                         int32_t h_q, int32_t max_ctx, float scale, int32_t sink, int32_t window,
                                         int32_t part, void* ws, int64_t ws_bytes, void* stream) {
  if (p && p->desc.cache_dtype == KV_F32)
    return fail(KV_E_UNSUPPORTED, "sliding-window decode is built for bf16 and fp8 pools");
  if (sink < 0 || window < 1)
    return fail(KV_E_INVALID, "sink %d must be >= 0 and window %d >= 1", sink, window);
  DecodeArgs a{};
  const int st = prepare_decode(p, layer, out, q, q_dtype, tables, max_blocks, ctx, B, h_q, max_ctx, scale,
                                part, ws, ws_bytes, &a);
  if (st != KV_OK) return st;
  if (B == 0) return ok();
  if (!k_new || !v_new || !slot_mapping) return fail(KV_E_INVALID, "NULL device array");
  a.sink = sink;
  a.window = window;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (p->desc.cache_dtype != KV_BF16) {  // the append kernel, then the windowed decode
    const int e = launch_append(p, layer, k_new, v_new, slot_mapping, B, s);
    if (e != KV_OK) return e;
    return launch_decode(a, s);
  }
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_slots = slot_mapping;
  return launch_decode(a, s);
}

int paged_attention_prefill(kv_pool* p, int32_t layer, void* out, const void* q, int32_t q_dtype,
                            const int32_t* tables, int32_t max_blocks, const int32_t* ctx,
                            const int32_t* query_start, int32_t B, int32_t h_q, int32_t max_q_len,
                            int32_t max_ctx, float scale, void* stream) {
  if (!p) return fail(KV_E_INVALID, "NULL pool");
  const kv_pool_desc& d = p->desc;
  if (layer < 0 || layer >= d.num_layers) return fail(KV_E_INVALID, "layer %d out of range", layer);
  if (B < 0 || max_q_len < 0) return fail(KV_E_INVALID, "negative size");
  if (B == 0 || max_q_len == 0) return ok();
  if (B > 65535) return fail(KV_E_UNSUPPORTED, "batch %d above 65535", B);
  if (d.cache_dtype != KV_BF16) return fail(KV_E_UNSUPPORTED, "prefill attention is built for bf16 pools");
  if (q_dtype != KV_BF16) return fail(KV_E_UNSUPPORTED, "q dtype %d: bf16 queries only", q_dtype);
  if (!out || !q || !tables || !ctx || !query_start) return fail(KV_E_INVALID, "NULL device array");
  if (h_q <= 0 || h_q % d.num_kv_heads != 0)
    return fail(KV_E_INVALID, "h_q %d is not a positive multiple of %d KV heads", h_q, d.num_kv_heads);
  if (h_q / d.num_kv_heads > 128)
    return fail(KV_E_UNSUPPORTED, "%d query heads per KV head (at most 128)", h_q / d.num_kv_heads);
  if (max_blocks <= 0 || max_ctx < 0 || int64_t(max_ctx) > int64_t(max_blocks) * d.block_size)
    return fail(KV_E_INVALID, "max_ctx %d outside [0, %d blocks * %d]", max_ctx, max_blocks, d.block_size);
  const int64_t tpt = 128 / (h_q / d.num_kv_heads);  // tokens per 128-row query tile
  const int64_t tiles = (int64_t(max_q_len) + tpt - 1) / tpt;
  if (tiles * B > INT32_MAX) return fail(KV_E_UNSUPPORTED, "too many query tiles");
  return launch_prefill(p, layer, out, q, tables, max_blocks, ctx, query_start, B, h_q, max_q_len, max_ctx, scale,
                        static_cast<hipStream_t>(stream));
}

int kv_window_release(kv_pool* p, int32_t B, int32_t* table, int32_t max_blocks, const int32_t* lens,
                      int32_t sink, int32_t window, int32_t* n_released) {
  return nothrow_call([&]() -> int {
    if (!p || !n_released) return fail(KV_E_INVALID, "NULL argument");
    if (B < 0 || max_blocks < 0) return fail(KV_E_INVALID, "negative size");
    if (sink < 0 || window < 1)
      return fail(KV_E_INVALID, "sink %d must be >= 0 and window %d >= 1", sink, window);
    *n_released = 0;
    if (B == 0) return ok();
    if (!table || !lens) return fail(KV_E_INVALID, "NULL array");
    const int32_t bs = p->desc.block_size;
    // check everything first (a block may be dropped by several tables, at most
    // as often as it is mapped): nothing changes on an error
    std::unordered_map<int32_t, int32_t> drops;
    for (int32_t b = 0; b < B; ++b) {
      const int32_t n = lens[b];
      if (n < 0 || kv_blocks_for_tokens(n, bs) > max_blocks)
        return fail(KV_E_INVALID, "request %d: length %d outside a table of %d blocks", b, n, max_blocks);
      const int32_t* row = table + int64_t(b) * max_blocks;
      for (int32_t j = 0; int64_t(j + 1) * bs <= int64_t(n) - window; ++j) {
        if (int64_t(j) * bs < sink || row[j] == -1) continue;
        if (!block_live(p, row[j]) || ++drops[row[j]] > p->rc[row[j]])
          return fail(KV_E_BAD_BLOCK, "request %d: block %d (page %d) out of range, free or over-released", b,
                      row[j], j);
      }
    }
    int32_t released = 0;
    for (int32_t b = 0; b < B; ++b) {
      int32_t* row = table + int64_t(b) * max_blocks;
      // dead pages: every position at or past the sinks and before n - window
      for (int32_t j = 0; int64_t(j + 1) * bs <= int64_t(lens[b]) - window; ++j) {
        if (int64_t(j) * bs < sink || row[j] == -1) continue;
        const int32_t blk = row[j];
        if (--p->rc[blk] == 0) p->stack.push_back(blk);
        row[j] = -1;
        ++released;
      }
    }
    *n_released = released;
    return ok();
  });
}

const char* kv_status_string(int s) {
  switch (s) {
    case KV_OK: return "KV_OK";
    case KV_E_INVALID: return "KV_E_INVALID";
    case KV_E_UNSUPPORTED: return "KV_E_UNSUPPORTED";
    case KV_E_NO_BLOCKS: return "KV_E_NO_BLOCKS";
    case KV_E_BAD_BLOCK: return "KV_E_BAD_BLOCK";
    case KV_E_SHARED: return "KV_E_SHARED";
    case KV_E_WORKSPACE: return "KV_E_WORKSPACE";
    case KV_E_HIP: return "KV_E_HIP";
    default: return "KV_E_UNKNOWN";
  }
}

const char* kv_last_error(void) { return g_last_error; }

}  // extern "C"
