// Internal declarations shared by the host and device translation units of
// libpagedkv.  Not part of the ABI.
#pragma once

#include <array>
#include <cstdint>
#include <exception>
#include <set>
#include <string>
#include <unordered_map>
#include <utility>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "pagedkv.h"

namespace pagedkv {

// Prefix-cache key of one whole page: tenant, the entry of the page before it
// (-1 for the first page) and its 16 token ids.  Compared exactly; the hash
// only locates it.
struct PrefixKey {
  int64_t tenant;
  int32_t parent;
  std::array<int32_t, 16> tokens;
  bool operator==(const PrefixKey& o) const {
    return tenant == o.tenant && parent == o.parent && tokens == o.tokens;
  }
};

struct PrefixKeyHash {
  size_t operator()(const PrefixKey& k) const;
};

struct PrefixEntry {
  PrefixKey key;
  int32_t block;
  int64_t tick;      // last touch
  int32_t children;  // entries whose parent this is
};

struct PrefixCache {
  std::unordered_map<PrefixKey, int32_t, PrefixKeyHash> index;  // key -> entry
  std::vector<PrefixEntry> entries;
  std::vector<int32_t> free_entries;                // reusable entry slots
  std::set<std::pair<int64_t, int32_t>> leaves;     // (tick, entry) with no children
  int64_t clock = 0;
};

// Reference counts of the pool's blocks (0 = free), which also keep the
// number of blocks counted at least twice: blocks that several tables, or a
// table and the prefix cache, map.  Every change goes through an element
// reference, so the number stays exact whichever entry point changed a count.
class RefCounts {
 public:
  class Ref {
   public:
    Ref(int32_t& v, int32_t& shared) : v_(v), shared_(shared) {}
    operator int32_t() const { return v_; }
    Ref& operator=(int32_t x) {
      set(x);
      return *this;
    }
    int32_t operator++() {
      set(v_ + 1);
      return v_;
    }
    int32_t operator--() {
      set(v_ - 1);
      return v_;
    }

   private:
    void set(int32_t x) {
      shared_ += int32_t(x >= 2) - int32_t(v_ >= 2);
      v_ = x;
    }
    int32_t& v_;
    int32_t& shared_;
  };
  void assign(size_t n, int32_t x) {
    v_.assign(n, x);
    shared_ = x >= 2 ? int32_t(n) : 0;
  }
  Ref operator[](size_t i) { return Ref(v_[i], shared_); }
  int32_t operator[](size_t i) const { return v_[i]; }
  int32_t shared() const { return shared_; }

 private:
  std::vector<int32_t> v_;
  int32_t shared_ = 0;
};

}  // namespace pagedkv

struct kv_pool {
  kv_pool_desc desc;
  void* k_cache;
  void* v_cache;
  float* k_scale;
  float* v_scale;
  std::vector<int32_t> stack;  // free blocks; the back is the top
  pagedkv::RefCounts rc;      // reference count per block, 0 = free
  pagedkv::PrefixCache prefix;
};

namespace pagedkv {

constexpr int kBlockSize = 16;
constexpr int kDefaultPartition = 512;
// Balanced decode (bf16, fp8, int8 caches): its waves, 256 compute units x 4
// SIMDs x 3 resident waves, so one launch fills MI355X once; the largest
// batch (the block prefix of the batch is kept in LDS); rows whose estimated
// piece count is at most kNarrowPieces are merged inside the decode kernel,
// or one wave per row by the reduce kernel when the counters do not cover
// the batch.
constexpr int kStreamWorkers = 256 * 4 * 3;
constexpr int kMaxStreamB = 8192;
constexpr int64_t kNarrowPieces = 16;

// Records a message for kv_last_error() and returns `status` (never throws).
int fail(int status, const char* fmt, ...);
int ok();

// Runs the body of an entry point that allocates host memory, turning a
// failed allocation into an error status so that no C++ exception crosses
// the C interface.
template <class F>
int nothrow_call(F&& body) {
  try {
    return body();
  } catch (const std::exception& e) {
    return fail(KV_E_INVALID, "host memory: %s", e.what());
  }
}

// Upper bound on the blocks a batch reservation can take: the new blocks
// every request needs (requests with negative sizes count none; the
// reservation rejects them), and never more than the free list holds.
inline size_t reserve_bound(int32_t B, const int32_t* lens, const int32_t* n_new, int32_t bs, size_t n_free) {
  size_t total = 0;
  for (int32_t b = 0; b < B && total < n_free; ++b) {
    if (lens[b] < 0 || n_new[b] <= 0) continue;
    const int64_t have = (int64_t(lens[b]) + bs - 1) / bs;
    const int64_t need = (int64_t(lens[b]) + n_new[b] + bs - 1) / bs;
    total += size_t(need - have);
  }
  return total < n_free ? total : n_free;
}

inline int elem_bytes(int dtype) { return dtype == KV_F32 ? 4 : dtype == KV_BF16 ? 2 : 1; }

// Caches of 8-bit codes with one fp32 scale per (layer, block, kv-head).
inline bool scaled_dtype(int dtype) { return dtype == KV_FP8_E4M3 || dtype == KV_INT8; }

// Elements of one layer of the K (or V) array.
inline int64_t layer_elems(const kv_pool_desc& d) {
  return int64_t(d.num_blocks) * d.num_kv_heads * d.block_size * d.head_dim;
}

// Device launches (append.hip, decode.hip).  Arguments are already checked.
int launch_append(const kv_pool* pool, int32_t layer, const void* k_new, const void* v_new,
                  const int32_t* slots, int32_t T, hipStream_t stream);
int launch_block_copy(const kv_pool* pool, const int32_t* src, const int32_t* dst, int32_t n,
                      hipStream_t stream);
int launch_prefill(const kv_pool* pool, int32_t layer, void* out, const void* q, const int32_t* tables,
                   int32_t max_blocks, const int32_t* ctx, const int32_t* qstart, int32_t B, int32_t h_q,
                   int32_t max_q_len, int32_t max_ctx, float scale, hipStream_t stream);

// Host allocator primitives shared by pool.cpp and prefix.cpp.
inline bool block_live(const kv_pool* p, int32_t b) {
  return b >= 0 && b < p->desc.num_blocks && p->rc[b] > 0;
}

// Launch plan of one decode.  fp32 caches use fixed partitions of `part`
// tokens (num_part of them, states [B][h_q][num_part]); bf16 and fp8 caches
// use the balanced split (`workers` waves, chunks of `chunk` blocks or
// balanced when 0, states [2 * chunks][hs]).
struct DecodeArgs {
  const kv_pool* pool;
  int32_t layer;
  void* out;
  const void* q;
  const int32_t* tables;
  int32_t max_blocks;
  const int32_t* ctx;
  int32_t B, h_q, max_ctx;
  float scale;
  int32_t part;      // fp32: tokens per partition (multiple of 16)
  int32_t num_part;  // fp32: partitions covering max_ctx (>= 1)
  int32_t chunk;     // bf16/fp8: blocks per chunk, 0 = balanced
  int32_t workers;   // bf16/fp8: waves of the decode kernel
  int32_t hs;        // bf16/fp8: query heads per state (min(16, h_q / h_kv))
  int64_t slots;     // number of states the workspace holds
  int64_t pieces;    // bf16/fp8: estimated pieces per row (chooses the merge)
  bool merge_inline; // bf16/fp8: the decode kernel merges the pieces itself
  int32_t* ws_cnt;   // bf16/fp8: [kMergeCounterBytes / 4] arrival counters, zero between calls
  float* ws_ml;      // [slots][2]  (max in log2 units, sum)
  float* ws_acc;     // [slots][head_dim]
  int32_t* ws_pref;  // bf16/fp8: [B + 1] blocks before each request
  // bf16 decode with the step's append fused in (all null otherwise): one
  // token per request, [B][H][D] each, written at new_slots[b] (-1: none)
  const void* k_new;
  const void* v_new;
  const int32_t* new_slots;
  // bf16/fp8 sliding-window decode: positions [0, sink) and the last `window`
  // are read (window 0: every position)
  int32_t sink;
  int32_t window;
};

// Arrival counters of the in-kernel piece merge: the first bytes of every
// bf16 / fp8 / int8 decode workspace, one int32 per (request, kv-head group),
// zero before a workspace's first use and left zero by every call.
constexpr int64_t kMergeCounterBytes = 256 * 1024;
constexpr int64_t kv_merge_counter_slots() { return kMergeCounterBytes / 4; }

// Fills the plan for a decode of this shape (pointers excluded) and returns
// the workspace bytes it needs, or a negative kv_status.
int64_t plan_decode(const kv_pool_desc& d, int32_t B, int32_t h_q, int32_t max_ctx,
                    int32_t partition_tokens, DecodeArgs* plan);
int launch_decode(const DecodeArgs& a, hipStream_t stream);
// Zero `bytes` (a multiple of 16) of device memory with a fill kernel.
int launch_zero(void* p, int64_t bytes, hipStream_t stream);

}  // namespace pagedkv
