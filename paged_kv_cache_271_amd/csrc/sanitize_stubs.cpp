// Device entry points of the host-only sanitizer build of libpagedkv
// (pool.cpp, prefix.cpp and plan.cpp built with g++ and AddressSanitizer /
// UndefinedBehaviorSanitizer).  That build has no device code: every launch
// reports KV_E_HIP, so only the host half (allocator, slot mapping,
// reservations, prefix cache, window release and every argument check made
// before a launch) runs under the sanitizers.

#include <cstdint>

#include "internal.h"
#include "pagedkv_probe.h"

namespace pagedkv {

namespace {
int no_device() { return fail(KV_E_HIP, "host-only sanitizer build: no device code"); }
}  // namespace

int launch_append(const kv_pool*, int32_t, const void*, const void*, const int32_t*, int32_t, hipStream_t) {
  return no_device();
}
int launch_block_copy(const kv_pool*, const int32_t*, const int32_t*, int32_t, hipStream_t) { return no_device(); }
int launch_prefill(const kv_pool*, int32_t, void*, const void*, const int32_t*, int32_t, const int32_t*,
                   const int32_t*, int32_t, int32_t, int32_t, int32_t, float, hipStream_t) {
  return no_device();
}
int launch_decode(const DecodeArgs&, hipStream_t) { return no_device(); }
int launch_zero(void*, int64_t, hipStream_t) { return no_device(); }

}  // namespace pagedkv

extern "C" int paged_attention_decode_append_noalloc(kv_pool*, int32_t, void*, const void*, int32_t, const void*,
                                                     const void*, const int32_t*, const int32_t*, int32_t,
                                                     const int32_t*, int32_t, int32_t, int32_t, float, int32_t,
                                                     void*) {
  return pagedkv::no_device();
}

extern "C" int kv_probe_gather(const void*, const void*, const int64_t*, const int64_t*, int32_t, int32_t,
                               uint32_t*, int32_t, void*) {
  return pagedkv::no_device();
}
