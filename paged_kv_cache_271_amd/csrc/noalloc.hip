// paged_attention_decode_append_noalloc: the fused decode step for callers
// that cannot allocate device memory (code under graph capture, tight serving
// loops, harnesses that forbid allocation).  It runs exactly the kernels of
// paged_attention_decode_append, with a fixed scratch array of this file in
// place of the caller's workspace.

#include <atomic>
#include <cstdint>
#include <mutex>

#include <hip/hip_runtime.h>

#include "internal.h"

namespace pagedkv {

constexpr int64_t kScratchBytes = 24ll << 20;  // 24 MiB per device

// The workspace of the no-allocation entry point, one copy per device (module
// globals are per device), zero-filled when the code object is loaded.  The
// decode's merge counters at its start are therefore zero before the first
// call, and every call leaves them zero.  In host code this name is only a
// stand-in for the device object: its device address comes from
// hipGetSymbolAddress, kept per device in g_scratch.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on `dev`, looked up once with that device
// current; nullptr (and the error recorded) when the lookup fails.
void* scratch_on(int dev) {
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (p) return p;
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) {
    fail(KV_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) {
    fail(KV_E_HIP, "hipSetDevice(%d): %s", dev, hipGetErrorString(e));
    return nullptr;
  }
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess || !p) {
    fail(KV_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    return nullptr;
  }
  g_scratch[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace
}  // namespace pagedkv

using namespace pagedkv;

extern "C" int paged_attention_decode_append_noalloc(kv_pool* p, int32_t layer, void* out, const void* q,
                                                     int32_t q_dtype, const void* k_new, const void* v_new,
                                                     const int32_t* slot_mapping, const int32_t* tables,
                                                     int32_t max_blocks, const int32_t* ctx, int32_t B, int32_t h_q,
                                                     int32_t max_ctx, float scale, int32_t part, void* stream) {
  if (!p) return fail(KV_E_INVALID, "NULL pool");
  const int64_t need = paged_attention_workspace_bytes(p, B, h_q, max_ctx, part);
  if (need < 0) return fail(KV_E_INVALID, "invalid batch shape (B %d, h_q %d, max_ctx %d, partition %d)", B, h_q,
                            max_ctx, part);
  if (need > kScratchBytes)
    return fail(KV_E_WORKSPACE, "this batch needs %lld bytes of scratch; the no-allocation entry point's static "
                "scratch holds %lld", (long long)need, (long long)kScratchBytes);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = 0;
  const hipError_t e = hipStreamGetDevice(s, &dev);
  if (e != hipSuccess) return fail(KV_E_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(KV_E_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  void* ws = scratch_on(dev);
  if (!ws) return KV_E_HIP;  // scratch_on recorded the message
  return paged_attention_decode_append(p, layer, out, q, q_dtype, k_new, v_new, slot_mapping, tables, max_blocks,
                                       ctx, B, h_q, max_ctx, scale, part, ws, kScratchBytes, stream);
}
