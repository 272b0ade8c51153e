// Launch plan of a decode: the work split, the workspace layout and how the
// split pieces are merged.  Host code only (shared by the library and its
// sanitizer build).

#include <algorithm>
#include <cstdint>

#include "internal.h"

namespace pagedkv {

int64_t plan_decode(const kv_pool_desc& d, int32_t B, int32_t h_q, int32_t max_ctx,
                    int32_t partition_tokens, DecodeArgs* a) {
  const int H = d.num_kv_heads;
  const int G = h_q / H;
  const int nhg = (G + 15) / 16;
  const int64_t hge = int64_t(H) * nhg;
  if (hge > 65535) return fail(KV_E_UNSUPPORTED, "too many heads");
  const int64_t fsz = int64_t(sizeof(float));
  if (d.cache_dtype == KV_F32) {
    const int32_t part = partition_tokens == 0 ? kDefaultPartition : partition_tokens;
    const int32_t np = max_ctx == 0 ? 1 : int32_t((int64_t(max_ctx) + part - 1) / part);
    if (hge * B * np > INT32_MAX) return fail(KV_E_UNSUPPORTED, "too many partitions");
    a->part = part;
    a->num_part = np;
    a->slots = np > 1 ? int64_t(B) * h_q * np : 0;
    return a->slots * (2 + d.head_dim) * fsz;
  }
  if (B > kMaxStreamB) return fail(KV_E_UNSUPPORTED, "batch %d above %d for bf16/fp8 caches", B, kMaxStreamB);
  const int32_t chunk = partition_tokens / kBlockSize;  // 0: balanced
  const int64_t umax = int64_t(B) * hge * ((int64_t(max_ctx) + kBlockSize - 1) / kBlockSize);
  // wave states per role: one per wave chunk (sets of four pairs: four per
  // workgroup chunk, kStreamWorkers / 4 of them when balanced)
  const bool coop = hge % 4 == 0;
  int64_t chunks = kStreamWorkers;
  if (chunk > 0)
    chunks = coop ? 4 * std::max<int64_t>(1, (umax / 4 + chunk - 1) / chunk)
                  : std::max<int64_t>(1, (umax + chunk - 1) / chunk);
  a->chunk = chunk;
  a->workers = kStreamWorkers;
  a->hs = std::min(16, G);
  a->slots = 2 * chunks * a->hs;
  // pieces per (request, set of kv-head groups): on average the chunks of
  // the balanced split over the batch's sets, at most the partitions of the
  // longest request with forced chunks
  const int64_t sets = coop ? hge / 4 : hge;
  const int64_t streams = coop ? kStreamWorkers / 4 : kStreamWorkers;
  a->pieces = chunk > 0 ? (int64_t(max_ctx) + kBlockSize - 1) / kBlockSize / chunk + 2
                        : streams / std::max<int64_t>(1, sets * B) + 1;
  // Rows with few pieces are merged inside the decode kernel by their last
  // piece (arrival counters at the start of the workspace); rows with many
  // pieces by a reduce kernel, which spreads a row's pieces over more lanes.
  const int64_t state_bytes = a->slots * (2 + d.head_dim) * fsz;
  a->merge_inline = a->pieces <= kNarrowPieces && int64_t(B) * hge <= kv_merge_counter_slots() &&
                    state_bytes < (int64_t(1) << 31);
  return kMergeCounterBytes + state_bytes + (int64_t(B) + 1) * int64_t(sizeof(int32_t));
}

}  // namespace pagedkv
