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
  int32_t part;      // tokens per partition (multiple of 16)
  int32_t num_part;  // partitions covering max_ctx (>= 1)
  float* ws_ml;      // [B][h_q][num_part][2]  (max in log2 units, sum)
  float* ws_acc;     // [B][h_q][num_part][head_dim]
};
int launch_decode(const DecodeArgs& a, hipStream_t stream);

int64_t workspace_bytes(int32_t B, int32_t h_q, int32_t head_dim, int32_t num_part);

}  // namespace pagedkv
