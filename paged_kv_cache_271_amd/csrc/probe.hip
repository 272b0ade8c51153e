// kv_probe_gather: a measurement aid beside the attention path.  It reads a
// list of equal-length byte runs from two base addresses (the K and the V run
// of each unit) with 16-byte loads, splitting the units over a persistent grid
// in balanced chunks as the decode does, and keeps only an XOR of the words
// read.  Given the runs a decode step reads, its time is the cost of that
// gather alone on this GPU, with no arithmetic, no table lookups and no
// second kernel: the practical ceiling for the decode's HBM-bound stream.

#include <cstdint>

#include <hip/hip_runtime.h>

#include "internal.h"
#include "pagedkv_probe.h"

namespace pagedkv {
namespace {

typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));

// The runs are read with the non-temporal hint, as the decode reads K/V.
__device__ inline u32x4 ldnt(const u32x4* p) { return __builtin_nontemporal_load(p); }

// grid = workgroups, 256 threads; unit u reads run16 16-byte pieces at
// kb + k_off[u] and at vb + v_off[u]; workgroup c takes units
// [c n / W, (c + 1) n / W) and writes the XOR of its words to sink[c].  The
// offsets come through LDS 64 units at a time, and two units are read
// together: 16 loads of 16 bytes in flight per thread for 16 KiB runs, 64 KiB
// per workgroup, as in the decode.
constexpr int kProbeBatch = 64;

__global__ void __launch_bounds__(256) gather_probe_kernel(const uint8_t* __restrict__ kb,
                                                           const uint8_t* __restrict__ vb,
                                                           const int64_t* __restrict__ k_off,
                                                           const int64_t* __restrict__ v_off, int32_t n,
                                                           int32_t run16, uint32_t* __restrict__ sink) {
  __shared__ int64_t s_k[kProbeBatch], s_v[kProbeBatch];
  __shared__ uint32_t s_x[4];
  const int64_t W = gridDim.x, c = blockIdx.x;
  const int64_t u0 = c * n / W, u1 = (c + 1) * n / W;
  const int tid = threadIdx.x;
  u32x4 x = {0, 0, 0, 0};
  for (int64_t ub = u0; ub < u1; ub += kProbeBatch) {
    const int nb = int(u1 - ub < kProbeBatch ? u1 - ub : kProbeBatch);
    __syncthreads();  // the previous batch's offsets are no longer read
    if (tid < nb) {
      s_k[tid] = k_off[ub + tid];
      s_v[tid] = v_off[ub + tid];
    }
    __syncthreads();
    int q = 0;
    for (; q + 1 < nb; q += 2) {
      const u32x4* k0 = reinterpret_cast<const u32x4*>(kb + s_k[q]);
      const u32x4* v0 = reinterpret_cast<const u32x4*>(vb + s_v[q]);
      const u32x4* k1 = reinterpret_cast<const u32x4*>(kb + s_k[q + 1]);
      const u32x4* v1 = reinterpret_cast<const u32x4*>(vb + s_v[q + 1]);
#pragma unroll 4
      for (int i = tid; i < run16; i += 256) x ^= ldnt(k0 + i) ^ ldnt(v0 + i) ^ ldnt(k1 + i) ^ ldnt(v1 + i);
    }
    if (q < nb) {
      const u32x4* k0 = reinterpret_cast<const u32x4*>(kb + s_k[q]);
      const u32x4* v0 = reinterpret_cast<const u32x4*>(vb + s_v[q]);
#pragma unroll 4
      for (int i = tid; i < run16; i += 256) x ^= ldnt(k0 + i) ^ ldnt(v0 + i);
    }
  }
  uint32_t w = x[0] ^ x[1] ^ x[2] ^ x[3];
  for (int o = 32; o > 0; o >>= 1) w ^= __shfl_xor(w, o);
  if ((tid & 63) == 0) s_x[tid >> 6] = w;
  __syncthreads();
  if (tid == 0) sink[c] = s_x[0] ^ s_x[1] ^ s_x[2] ^ s_x[3];
}

}  // namespace
}  // namespace pagedkv

using namespace pagedkv;

extern "C" int kv_probe_gather(const void* k_base, const void* v_base, const int64_t* k_offsets,
                               const int64_t* v_offsets, int32_t n_runs, int32_t run_bytes, uint32_t* sink,
                               int32_t workgroups, void* hip_stream) {
  if (!k_base || !v_base || !sink) return fail(KV_E_INVALID, "NULL device pointer");
  if (n_runs < 0) return fail(KV_E_INVALID, "negative run count");
  if (run_bytes <= 0 || run_bytes % 16 != 0)
    return fail(KV_E_INVALID, "run_bytes %d is not a positive multiple of 16", run_bytes);
  if (workgroups < 1 || workgroups > 65535)
    return fail(KV_E_INVALID, "workgroups %d outside [1, 65535]", workgroups);
  if (n_runs > 0 && (!k_offsets || !v_offsets)) return fail(KV_E_INVALID, "NULL offsets");
  const auto* kb = static_cast<const uint8_t*>(k_base);
  const auto* vb = static_cast<const uint8_t*>(v_base);
  gather_probe_kernel<<<workgroups, 256, 0, static_cast<hipStream_t>(hip_stream)>>>(
      kb, vb, k_offsets, v_offsets, n_runs, run_bytes / 16, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KV_E_HIP, "kv_probe_gather launch: %s", hipGetErrorString(e));
  return ok();
}
