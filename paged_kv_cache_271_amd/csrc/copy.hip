// kv_block_copy: copy whole pages of the pool, every layer, K and V (and the
// fp8 scales), for copy-on-write of a shared page ("KV cache and
// PagedAttention", askaiml.pages.dev, §4: requests with a common prefix share
// pages; "KV Cache" glossary, inferensys.com, PagedAttention entry: blocks are
// shared across sequences for parallel sampling and beam search, so a
// sequence that writes into a shared block first takes a copy of it).
//
// A page of one layer is contiguous in K and in V (all kv heads' tiles), so
// each workgroup streams one (pair, layer, K or V) run with 16-byte loads and
// stores.  HBM-bound: 2 x page bytes moved per (pair, layer, K or V).  Loads
// and stores carry the non-temporal hint: the copy is read next by a later
// decode step of its layer, long after the caches have turned over (same box,
// the 256-fork step took 212.6 us with plain loads and stores, 200.2 with
// non-temporal stores, 186.5 with both).

#include <cstdint>

#include <hip/hip_runtime.h>

#include "internal.h"

namespace pagedkv {
namespace {

typedef uint32_t u32x4 __attribute__((__vector_size__(16)));

// grid (n pairs, layers, 2); 256 threads.  Pairs with an id out of range, or
// src == dst, are skipped (device ids are a caller contract; this keeps a bad
// id from reaching memory).
__global__ void __launch_bounds__(256) block_copy_kernel(uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                                                         float* __restrict__ ks, float* __restrict__ vs,
                                                         const int32_t* __restrict__ src,
                                                         const int32_t* __restrict__ dst, int32_t N, int H,
                                                         int64_t page_bytes) {
  const int i = blockIdx.x, l = blockIdx.y, which = blockIdx.z;
  const int32_t s = src[i], d = dst[i];
  if (s < 0 || s >= N || d < 0 || d >= N || s == d) return;
  uint8_t* base = (which ? vc : kc) + int64_t(l) * N * page_bytes;
  const uint4* from = reinterpret_cast<const uint4*>(base + int64_t(s) * page_bytes);
  uint4* to = reinterpret_cast<uint4*>(base + int64_t(d) * page_bytes);
  const int64_t n16 = page_bytes / 16;
  for (int64_t k = threadIdx.x; k < n16; k += 4 * 256) {  // four 16-byte loads in flight
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (k + u * 256 < n16)
        v[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(from + k + u * 256)));
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (k + u * 256 < n16)
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v[u]), reinterpret_cast<u32x4*>(to + k + u * 256));
  }
  if (ks && threadIdx.x < H) {
    float* sc = (which ? vs : ks) + int64_t(l) * N * H;
    sc[int64_t(d) * H + threadIdx.x] = sc[int64_t(s) * H + threadIdx.x];
  }
}

}  // namespace

int launch_block_copy(const kv_pool* p, const int32_t* src, const int32_t* dst, int32_t n,
                      hipStream_t stream) {
  const kv_pool_desc& d = p->desc;
  const int64_t page_bytes = int64_t(d.num_kv_heads) * d.block_size * d.head_dim * elem_bytes(d.cache_dtype);
  const dim3 grid(n, d.num_layers, 2);
  block_copy_kernel<<<grid, 256, 0, stream>>>(static_cast<uint8_t*>(p->k_cache), static_cast<uint8_t*>(p->v_cache),
                                              p->k_scale, p->v_scale, src, dst, d.num_blocks, d.num_kv_heads,
                                              page_bytes);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KV_E_HIP, "kv_block_copy launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace pagedkv
