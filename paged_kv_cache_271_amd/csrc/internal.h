// Internal declarations shared by the host and device translation units of
// libpagedkv.  Not part of the ABI.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include <hip/hip_runtime.h>

#include "pagedkv.h"

struct kv_pool {
  kv_pool_desc desc;
  void* k_cache;
  void* v_cache;
  float* k_scale;
  float* v_scale;
  std::vector<int32_t> stack;  // free blocks; the back is the top
  std::vector<int32_t> rc;     // reference count per block, 0 = free
};

namespace pagedkv {

constexpr int kBlockSize = 16;
constexpr int kDefaultPartition = 512;

// Records a message for kv_last_error() and returns `status`.
int fail(int status, const char* fmt, ...);
int ok();

inline int elem_bytes(int dtype) { return dtype == KV_F32 ? 4 : dtype == KV_BF16 ? 2 : 1; }

// Elements of one layer of the K (or V) array.
inline int64_t layer_elems(const kv_pool_desc& d) {
  return int64_t(d.num_blocks) * d.num_kv_heads * d.block_size * d.head_dim;
}

// Device launches (append.hip, decode.hip).  Arguments are already checked.
int launch_append(const kv_pool* pool, int32_t layer, const void* k_new, const void* v_new,
                  const int32_t* slots, int32_t T, hipStream_t stream);

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
  float* ws_ml;      // [slots][2]  (max in log2 units, sum)
  float* ws_acc;     // [slots][head_dim]
  int32_t* ws_pref;  // bf16/fp8: [B + 1] blocks before each request
  // bf16 decode with the step's append fused in (all null otherwise): one
  // token per request, [B][H][D] each, written at new_slots[b] (-1: none)
  const void* k_new;
  const void* v_new;
  const int32_t* new_slots;
};

// Fills the plan for a decode of this shape (pointers excluded) and returns
// the workspace bytes it needs, or a negative kv_status.
int64_t plan_decode(const kv_pool_desc& d, int32_t B, int32_t h_q, int32_t max_ctx,
                    int32_t partition_tokens, DecodeArgs* plan);
int launch_decode(const DecodeArgs& a, hipStream_t stream);

}  // namespace pagedkv
