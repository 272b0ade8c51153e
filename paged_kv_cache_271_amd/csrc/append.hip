// kv_append: write each new token's K and V into its slot of the paged pool.
//
// "KV cache and PagedAttention" (askaiml.pages.dev), §1 "The setup": every
// decode step appends the new token's K and V to the cache; §4
// "PagedAttention": position p of a request lives in page table[p / 16] at
// offset p % 16 (the slot the caller computed).  §7 "KV cache quantisation":
// the cache may be held as fp8 E4M3 or as INT8.
//
// Layout per layer: K [block][kv_head][16][head_dim], V [block][kv_head][head_dim][16].
// f32 and bf16 pools copy bits.  fp8 and int8 pools quantise one (block,
// kv-head) tile per workgroup with one fp32 scale per tile; the rule is
// spelled out in pagedkv.h at kv_append.

#include <cstdint>
#include <type_traits>

#include <hip/hip_runtime.h>

#include "codec8.h"
#include "internal.h"

namespace pagedkv {
namespace {

constexpr int kBS = kBlockSize;


// ---------------------------------------------------------------- copy ----
// f32 and bf16 pools copy bits.  Two launch shapes: bulk calls (prefills,
// admitted prompts) take one workgroup per 16 tokens and move whole runs;
// short calls take one workgroup per token, which keeps their latency to one
// slot read and one data round trip.
constexpr int kAppendRangeMin = 1024;  // tokens per call from which ranges are used

// Bulk calls: one workgroup of 256 threads per (range of 16 tokens, kv-head
// g).  A run is a maximal sequence of tokens of the call whose slots are
// consecutive within one block (1 to 16 tokens).  The workgroup copies the K
// rows of its own tokens (a row is contiguous in the tile: 16-byte pieces)
// and writes V for the runs that start in its range, which may reach up to 15
// tokens past it: those tokens' V rows pass through LDS, and each thread
// writes one (run, dimension) pair's entries into the dim-major tile at a
// time, a whole 16-token row in 16-byte stores when the run fills the block.
// The slots of tokens t0 - 1 .. t0 + 31 are read in one round trip.
constexpr int kAppendRange = 16;

template <typename T, int D>
__global__ void __launch_bounds__(256)
append_copy_range_kernel(T* __restrict__ kc, T* __restrict__ vc, const T* __restrict__ k_new,
                         const T* __restrict__ v_new, const int32_t* __restrict__ slots, int n_tok, int H) {
  constexpr int RB = D * int(sizeof(T));  // bytes of one token row
  constexpr int PR = RB / 16;             // 16-byte pieces per row
  constexpr int R = kAppendRange;
  __shared__ int32_t s_slot[2 * R + 1];  // tokens t0 - 1 .. t0 + 2R - 1 (-1: none or beyond)
  __shared__ int32_t s_len[R];           // length of the run starting at t0 + i (0: none)
  __shared__ int32_t s_first[R + 1];     // range indices of the runs starting here; [R]: their count
  __shared__ __attribute__((aligned(16))) T s_v[2 * R][D];
  const int t0 = blockIdx.x * R;
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  if (tid <= 2 * R) {
    const int t = t0 - 1 + tid;
    s_slot[tid] = t >= 0 && t < n_tok ? slots[t] : -1;
  }
  __syncthreads();
  if (tid < R) {
    const int32_t sl = s_slot[tid + 1], sp = s_slot[tid];
    int len = 0;
    if (sl >= 0 && !(sp >= 0 && sp + 1 == sl && sl % kBS != 0)) {
      len = 1;  // then at most to the end of the block (index <= tid + 16)
      while (len < kBS - sl % kBS && s_slot[tid + 1 + len] == sl + len) ++len;
    }
    s_len[tid] = len;
  }
  // K rows of this range's tokens
  for (int p = tid; p < R * PR; p += 256) {
    const int r = p / PR, c = p - r * PR;
    const int32_t sl = s_slot[r + 1];
    if (t0 + r < n_tok && sl >= 0) {
      const int64_t tile = (int64_t(sl / kBS) * H + g) * kBS * D;  // elements
      *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(kc + tile) + (sl % kBS) * RB + 16 * c) =
          *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(k_new) +
                                          (int64_t(t0 + r) * H + g) * RB + 16 * c);
    }
  }
  __syncthreads();
  if (tid == 0) {
    int k = 0;
    for (int i = 0; i < R; ++i)
      if (s_len[i] > 0) s_first[k++] = i;
    s_first[R] = k;
  }
  // V rows of the tokens up to the end of the last run starting here (every
  // one of them exists: a run only holds tokens whose slot was read)
  int rows = 0;
#pragma unroll
  for (int i = 0; i < R; ++i) rows = s_len[i] > 0 ? i + s_len[i] : rows;
  for (int p = tid; p < rows * PR; p += 256) {
    const int r = p / PR, c = p - r * PR;
    *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(&s_v[r][0]) + 16 * c) =
        *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(v_new) +
                                        (int64_t(t0 + r) * H + g) * RB + 16 * c);
  }
  __syncthreads();
  // one (run, dimension) pair per thread and pass
  for (int p = tid; p < s_first[R] * D; p += 256) {
    const int i = s_first[p / D], d = p % D;
    const int n = s_len[i];
    const int32_t sl = s_slot[i + 1];
    const int o0 = sl % kBS;
    T* row = vc + (int64_t(sl / kBS) * H + g) * kBS * D + int64_t(d) * kBS;  // dimension d
    if (n == kBS) {
      alignas(16) T e[kBS];
#pragma unroll
      for (int r = 0; r < kBS; ++r) e[r] = s_v[i + r][d];
#pragma unroll
      for (int w = 0; w < kBS * int(sizeof(T)) / 16; ++w)
        reinterpret_cast<uint4*>(row)[w] = reinterpret_cast<const uint4*>(e)[w];
    } else {
      for (int r = 0; r < n; ++r) row[o0 + r] = s_v[i + r][d];
    }
  }
}

// Calls of up to kAppendRangeMin tokens (a decode step's one token per
// request): one workgroup of 256 threads per (token t, kv-head g); only the
// first token of a run works, for the whole run.  A run is a maximal sequence of tokens
// of the call whose slots are consecutive within one block (1 to 16 tokens).
// The slots of tokens t - 1 .. t + 16 are read in one round trip by wave 0,
// and a ballot gives the run's length.  K rows go over in 16-byte pieces
// (a row is contiguous in the tile); V rows pass through LDS so that each
// thread writes its dimension's entries of the run into the dim-major tile,
// a whole 16-token row in 16-byte stores when the run fills the block.
template <typename T, int D>
__global__ void __launch_bounds__(256)
append_copy_run_kernel(T* __restrict__ kc, T* __restrict__ vc, const T* __restrict__ k_new,
                       const T* __restrict__ v_new, const int32_t* __restrict__ slots, int n_tok, int H) {
  constexpr int RB = D * int(sizeof(T));  // bytes of one token row
  constexpr int PR = RB / 16;             // 16-byte pieces per row
  __shared__ __attribute__((aligned(16))) T s_v[kBS][D];
  __shared__ int32_t s_run[2];  // first slot, run length (0: not a run start)
  const int t = blockIdx.x;
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int i = tid - 1;  // lane 1 + i reads the slot of token t + i
    int32_t sl = -1;
    if (tid <= kBS && t + i >= 0 && t + i < n_tok) sl = slots[t + i];
    const int32_t s0 = __shfl(sl, 1);
    const int32_t sp = __shfl(sl, 0);
    const bool start = s0 >= 0 && !(sp >= 0 && sp + 1 == s0 && s0 % kBS != 0);
    const bool ok = tid >= 1 && tid <= kBS && s0 >= 0 && sl == s0 + i && s0 % kBS + i < kBS;
    // leading lanes 1.. that continue the run; lane 17 never does
    const uint64_t broken = ~(uint64_t(__ballot(ok)) >> 1);
    if (tid == 0) {
      s_run[0] = s0;
      s_run[1] = start ? __builtin_ctzll(broken) : 0;
    }
  }
  __syncthreads();
  const int n = s_run[1];
  if (n == 0) return;
  const int32_t s0 = s_run[0];
  const int o0 = s0 % kBS;
  const int64_t tile = (int64_t(s0 / kBS) * H + g) * kBS * D;  // elements
  uint8_t* kt = reinterpret_cast<uint8_t*>(kc + tile);
  for (int p = tid; p < n * PR; p += 256) {
    const int r = p / PR, c = p - r * PR;
    const int64_t src = (int64_t(t + r) * H + g) * RB + 16 * c;
    *reinterpret_cast<uint4*>(kt + (o0 + r) * RB + 16 * c) =
        *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(k_new) + src);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(&s_v[r][0]) + 16 * c) =
        *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(v_new) + src);
  }
  __syncthreads();
  if (tid < D) {
    T* row = vc + tile + int64_t(tid) * kBS;  // the tile's row of dimension tid
    if (n == kBS) {
      alignas(16) T e[kBS];
#pragma unroll
      for (int r = 0; r < kBS; ++r) e[r] = s_v[r][tid];
#pragma unroll
      for (int w = 0; w < kBS * int(sizeof(T)) / 16; ++w)
        reinterpret_cast<uint4*>(row)[w] = reinterpret_cast<const uint4*>(e)[w];
    } else {
      for (int r = 0; r < n; ++r) row[o0 + r] = s_v[r][tid];
    }
  }
}

__device__ inline float bf16_bits_to_float(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Max over the workgroup (one or two waves).
__device__ inline float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return blockDim.x > 64 ? fmaxf(red[0], red[1]) : red[0];
}

// fp8 E4M3 and int8 caches share the kernel; only the codec differs.
// One workgroup per (token t, kv-head g); only the first token of a run (the
// consecutive tokens of this call landing in one block) does the work, for
// the whole run.  Wave 0 reads the slots of tokens t - 1 .. t + 62 in one
// round trip and a ballot finds the run; the first token's inputs are loaded
// before its slot is known.  The run's K tile ([16][D] codes) and V tile
// ([D][16]) are staged in LDS with one 16-byte load per thread, re-encoded and
// written there, and the changed bytes go back with 16-byte stores.
// blockDim.x = D (64 or 128); thread d owns dimension d.
template <int D, bool INT8>
__global__ void __launch_bounds__(D) append_q8_kernel(uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                                                       float* __restrict__ ks, float* __restrict__ vs,
                                                       const uint16_t* __restrict__ k_new,
                                                       const uint16_t* __restrict__ v_new,
                                                       const int32_t* __restrict__ slots, int T, int H) {
  constexpr int TILE = kBS * D;        // bytes of one tile
  constexpr int CHUNKS = TILE / 16;    // 16-byte pieces of a tile (= D)
  constexpr int kWin = 63;              // run tokens whose slots wave 0 reads at once
  __shared__ __attribute__((aligned(16))) uint8_t s_tile[2][TILE];  // [0] K, [1] V
  __shared__ float red[2];
  __shared__ int32_t s_run[2];          // last token of the run (-1: not a run start), first slot
  __shared__ int32_t s_off[kWin];       // offsets of the run's tokens t .. t + kWin - 1
  const int t = blockIdx.x;
  const int g = blockIdx.y;
  const int d = threadIdx.x;
  // the first token's inputs need no slot: in flight from the start
  const float x0[2] = {bf16_bits_to_float(k_new[(int64_t(t) * H + g) * D + d]),
                       bf16_bits_to_float(v_new[(int64_t(t) * H + g) * D + d])};
  if (d < 64) {
    // wave 0: slots of tokens t - 1 .. t + 62 in one round trip; the run is
    // the leading lanes from 1 whose token lands in the first token's block
    const int i = d - 1;
    int32_t sl = -1;
    if (t + i >= 0 && t + i < T) sl = slots[t + i];
    const int32_t s0 = __shfl(sl, 1), sp = __shfl(sl, 0);
    const bool start = s0 >= 0 && !(sp >= 0 && sp / kBS == s0 / kBS);
    const bool ok = d >= 1 && s0 >= 0 && sl >= 0 && sl / kBS == s0 / kBS;
    const uint64_t broken = ~(uint64_t(__ballot(ok)) >> 1);  // bit 63 always set
    const int n = start ? __builtin_ctzll(broken) : 0;        // 0 .. kWin
    if (d >= 1 && i < n) s_off[i] = sl % kBS;
    if (d == 0) {
      s_run[0] = start ? t + n - 1 : -1;
      s_run[1] = s0;
    }
  }
  __syncthreads();
  int u = s_run[0];
  if (u < 0) return;
  const int32_t slot = s_run[1];
  const int32_t blk = slot / kBS;
  // a run past the window (only with repeated slots) continues serially
  if (u == t + kWin - 1)
    while (u + 1 < T && slots[u + 1] >= 0 && slots[u + 1] / kBS == blk) ++u;
  auto off_of = [&](int r) { return r - t < kWin ? s_off[r - t] : slots[r] % kBS; };
  const int first_off = slot % kBS;
  const int64_t tile = (int64_t(blk) * H + g) * TILE;
  const int64_t sidx = int64_t(blk) * H + g;

  // stage the tiles: V always (its 16-byte rows mix the run's slots with the
  // others and are written back whole), K only when rows below the run may be
  // re-encoded (the run's own K rows are rewritten whole)
  if (first_off > 0)
    *reinterpret_cast<uint4*>(&s_tile[0][16 * d]) = *reinterpret_cast<const uint4*>(kc + tile + 16 * d);
  *reinterpret_cast<uint4*>(&s_tile[1][16 * d]) = *reinterpret_cast<const uint4*>(vc + tile + 16 * d);
  const float sk0 = first_off == 0 ? 0.0f : ks[sidx];
  const float sv0 = first_off == 0 ? 0.0f : vs[sidx];
  __syncthreads();

  // byte position of (token offset o, dimension d) in each staged tile
  auto pos = [&](int which, int o) { return which == 0 ? o * D + d : d * kBS + o; };
  bool reenc[2];
  for (int which = 0; which < 2; ++which) {
    const uint16_t* src = which == 0 ? k_new : v_new;
    const float s0 = which == 0 ? sk0 : sv0;
    float amax = fabsf(x0[which]);
    for (int r = t + 1; r <= u; ++r)
      amax = fmaxf(amax, fabsf(bf16_bits_to_float(src[(int64_t(r) * H + g) * D + d])));
    amax = block_max(amax, red);
    const float s1 = fmaxf(s0, amax / Codec8<INT8>::kMax);
    reenc[which] = s1 != s0 && first_off > 0;
    uint8_t* st = s_tile[which];
    if (s1 == 0.0f) {
      for (int r = t; r <= u; ++r) st[pos(which, off_of(r))] = 0;
    } else {
      const float inv = 1.0f / s1;
      if (reenc[which])
        for (int o = 0; o < first_off; ++o) {
          const float x = Codec8<INT8>::decode(st[pos(which, o)]) * s0;
          st[pos(which, o)] = uint8_t(Codec8<INT8>::encode(x * inv));
        }
      for (int r = t; r <= u; ++r) {
        const float x = r == t ? x0[which] : bf16_bits_to_float(src[(int64_t(r) * H + g) * D + d]);
        st[pos(which, off_of(r))] = uint8_t(Codec8<INT8>::encode(x * inv));
      }
    }
    if (d == 0) (which == 0 ? ks : vs)[sidx] = s1;
  }
  __syncthreads();

  // write back: K rows of the run (and the re-encoded rows below it); V is
  // dim-major, so every 16-byte row changes
  const int last_off = off_of(u);
  for (int c = d; c < CHUNKS; c += D) {
    const int o = (16 * c) / D;  // token row of this K chunk
    if ((o >= first_off && o <= last_off) || (o < first_off && reenc[0]))
      *reinterpret_cast<uint4*>(kc + tile + 16 * c) = *reinterpret_cast<const uint4*>(&s_tile[0][16 * c]);
    *reinterpret_cast<uint4*>(vc + tile + 16 * c) = *reinterpret_cast<const uint4*>(&s_tile[1][16 * c]);
  }
}

}  // namespace

int launch_append(const kv_pool* p, int32_t layer, const void* k_new, const void* v_new,
                  const int32_t* slots, int32_t T, hipStream_t stream) {
  const kv_pool_desc& d = p->desc;
  const int64_t lo = int64_t(layer) * layer_elems(d);
  const dim3 grid(T, d.num_kv_heads);
  const int D = d.head_dim;
  if (d.cache_dtype == KV_F32 || d.cache_dtype == KV_BF16) {
    auto go = [&](auto elem, auto dim) {
      using E = decltype(elem);
      constexpr int DD = decltype(dim)::value;
      E* kcp = static_cast<E*>(p->k_cache) + lo;
      E* vcp = static_cast<E*>(p->v_cache) + lo;
      if (T > kAppendRangeMin) {
        const dim3 ranges((T + kAppendRange - 1) / kAppendRange, d.num_kv_heads);
        append_copy_range_kernel<E, DD><<<ranges, 256, 0, stream>>>(
            kcp, vcp, static_cast<const E*>(k_new), static_cast<const E*>(v_new), slots, T, d.num_kv_heads);
      } else {
        append_copy_run_kernel<E, DD><<<grid, 256, 0, stream>>>(
            kcp, vcp, static_cast<const E*>(k_new), static_cast<const E*>(v_new), slots, T, d.num_kv_heads);
      }
    };
    using D64 = std::integral_constant<int, 64>;
    using D128 = std::integral_constant<int, 128>;
    if (d.cache_dtype == KV_F32) {
      if (D == 128) go(float{}, D128{});
      else go(float{}, D64{});
    } else {
      if (D == 128) go(uint16_t{}, D128{});
      else go(uint16_t{}, D64{});
    }
  } else {
    const int64_t so = int64_t(layer) * d.num_blocks * d.num_kv_heads;
    auto* kc8 = static_cast<uint8_t*>(p->k_cache) + lo;
    auto* vc8 = static_cast<uint8_t*>(p->v_cache) + lo;
    auto* kn = static_cast<const uint16_t*>(k_new);
    auto* vn = static_cast<const uint16_t*>(v_new);
    float* ks = p->k_scale + so;
    float* vs = p->v_scale + so;
    const int H = d.num_kv_heads;
    if (d.cache_dtype == KV_FP8_E4M3) {
      if (D == 128) append_q8_kernel<128, false><<<grid, 128, 0, stream>>>(kc8, vc8, ks, vs, kn, vn, slots, T, H);
      else append_q8_kernel<64, false><<<grid, 64, 0, stream>>>(kc8, vc8, ks, vs, kn, vn, slots, T, H);
    } else {
      if (D == 128) append_q8_kernel<128, true><<<grid, 128, 0, stream>>>(kc8, vc8, ks, vs, kn, vn, slots, T, H);
      else append_q8_kernel<64, true><<<grid, 64, 0, stream>>>(kc8, vc8, ks, vs, kn, vn, slots, T, H);
    }
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KV_E_HIP, "kv_append launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace pagedkv
