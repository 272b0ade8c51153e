// paged_attention_decode: single-token GQA decode attention over the paged
// KV cache, for gfx950.
//
// What is computed ("Memoizing Context via KV Caching", blog.sanjeevnode.in;
// "KV cache and PagedAttention", askaiml.pages.dev, §1 and §4): the new
// token's query of every head is compared with the key of every cached token
// of its request, the weights are a softmax of the scaled scores, and the
// output is the weighted sum of the value vectors; K and V are gathered
// through the request's page table.  Query head h reads KV head
// h / (h_q / h_kv) ("KV Cache" glossary, inferensys.com, GQA entry).
//
// Every (request, kv-head) keeps, per query head, the running max m of the
// scores (log2 units), the sum l of 2^(s - m) and the weighted sum acc of V
// (the online softmax).  Pieces of one request's context are merged by
// rescaling to the common maximum.
//
// bf16 / fp8 caches: decode_stream_kernel splits the blocks of the whole
// batch evenly over its waves (details at the kernel) and uses MFMA
// (v_mfma_f32_16x16x32_bf16) for q.K^T and p.V; stream_reduce_kernel (or
// stream_reduce_rows_kernel, when rows have few pieces) merges the pieces.
// fp8 codes are widened to bf16 exactly (every E4M3 value is a bf16 value);
// the K scale multiplies the scores and the V scale multiplies p.
// Padding columns of the MFMA (query heads beyond the group) carry zero
// queries and are never stored.
//
// fp32 caches: decode_f32_kernel (VALU) over fixed partitions per (request,
// kv-head), reduce_kernel merges the partitions.

#include <algorithm>
#include <cstdint>
#include <type_traits>

#include <hip/hip_runtime.h>

#include "codec8.h"
#include "internal.h"

namespace pagedkv {
namespace {

constexpr int kBS = kBlockSize;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyLog2 = 8.0f;  // headroom of the decode's lazy running maximum (log2 units)

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef _Float16 f16x2 __attribute__((__vector_size__(2 * sizeof(_Float16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x2 __attribute__((__vector_size__(2 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

__device__ inline u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// K/V loads of the decode.  NT: the non-temporal hint (nt), so that the
// caches do not keep tiles that nothing reads again in the launch.  Used when
// no block of the pool is mapped twice; a shared page (a common prefix) is
// read by every request that maps it, and then the caches serve the repeats.
// Against plain loads, nt took the Llama-3-8B-shaped decode from 112.3 to
// 105.9 us and the 70B-shaped one from 232.6 to 208.4 us (same box), and the
// 32-layer prefix-sharing step from 6.3 to 10.7 ms.
template <bool NT>
__device__ inline u32x4 ld16_kv(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else return *reinterpret_cast<const u32x4*>(p);
}
template <bool NT>
__device__ inline u32x2 ld8_kv(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  else return *reinterpret_cast<const u32x2*>(p);
}
// One direct-to-LDS K/V copy of 16 bytes per lane (cache-policy bits: nt is 2).
template <bool NT>
__device__ __forceinline__ void copy16_kv(const uint8_t* src, uint8_t* dst) {
  if constexpr (NT) __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 2);
  else __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

__device__ inline uint32_t f2bf_bits(float x) {
  const __bf16 h = static_cast<__bf16>(x);  // round to nearest even
  return uint32_t(__builtin_bit_cast(uint16_t, h));
}

// Two floats -> two bf16 (round to nearest even) in one dword: one
// v_cvt_pk_bf16_f32.
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Four E4M3 codes (one dword) -> four bf16 (two dwords), exact.
__device__ inline u32x2 fp8x4_to_bf16x4(uint32_t w) {
  const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  u32x2 r;
  r[0] = __builtin_bit_cast(uint32_t, lo);
  r[1] = __builtin_bit_cast(uint32_t, hi);
  return r;
}

// Cache element types of the balanced decode.  bf16 and fp8 caches feed the
// MFMAs bf16 operands; int8 caches feed them fp16 operands, which hold every
// int8 code exactly and come from the codes in one permute and one packed
// subtract per pair (below), where bf16 would need a convert per code.
constexpr int kQBf16 = 0, kQFp8 = 1, kQInt8 = 2;

// Four symmetric int8 codes (one dword) -> four fp16 (two dwords), exact:
// with the sign bit flipped a code c is the byte u = c + 128, 0x6400 | u is
// the fp16 1024 + u, and subtracting 1152 leaves c.  Each pair's high bytes
// come from one v_perm_b32: selector bytes 0-3 take bytes of the second
// operand (u), 4-7 bytes of the first (0x64 everywhere).
__device__ inline u32x2 int8x4_to_f16x4(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);  // [u0, 64, u1, 64]
  const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);  // [u2, 64, u3, 64]
  const f16x2 bias = {static_cast<_Float16>(-1152.0f), static_cast<_Float16>(-1152.0f)};
  u32x2 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, lo) + bias);
  r[1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, hi) + bias);
  return r;
}

// Four 8-bit codes of cache type QT -> four MFMA operand elements.
template <int QT>
__device__ inline u32x2 q8x4_to_op(uint32_t w) {
  if constexpr (QT == kQFp8) return fp8x4_to_bf16x4(w);
  else return int8x4_to_f16x4(w);
}

// Two fp32 values -> one dword of two MFMA operand elements (bf16, or fp16
// for int8 caches), round to nearest even.
template <int QT>
__device__ inline uint32_t pack_op(float lo, float hi) {
  if constexpr (QT == kQInt8) {
    const f16x2 h = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
    return __builtin_bit_cast(uint32_t, h);
  } else {
    return pack_bf16(lo, hi);
  }
}

// c += a * b on one 16x16x32 MFMA tile of the cache type's operands.
template <int QT>
__device__ inline f32x4 mfma_op(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (QT == kQInt8)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}


// Context length of request b, clamped to [0, max_ctx] so that no kernel can
// index past the table row or the workspace sized from max_ctx.
__device__ inline int clamp_ctx(const int32_t* ctx_lens, int b, int max_ctx) {
  return min(max(ctx_lens[b], 0), max_ctx);
}

__device__ inline float wave_max16(float x) {  // over lanes r, r+16, r+32, r+48
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ inline float wave_sum16(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// ------------------------------------------------------------------------
// Device-coherent accesses for the in-kernel piece merge.  Each XCD has its
// own L2, which is not kept coherent with the others for ordinary accesses;
// loads and stores carrying the sc1 cache-policy bit (agent scope, as the
// compiler emits for agent-scope atomic loads and stores) bypass the
// non-coherent levels, so a state stored by a wave on one XCD is what a
// wave on another XCD loads after it has seen that store's arrival count.
constexpr int kCoherent = 16;  // sc1 bit of the buffer instructions' cache policy

__device__ inline __amdgpu_buffer_rsrc_t raw_rsrc(const void* base) {
  // raw buffer (stride 0), no bounds beyond the 32-bit offset range
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}
__device__ inline void store16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCoherent);
}
__device__ inline void store8_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kCoherent);
}
__device__ inline u32x4 load16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherent);
}
__device__ inline u32x2 load8_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCoherent);
}
// Wait until every memory access this wave issued has completed, between a
// workgroup-scope release and acquire: the wave's earlier stores are then
// visible to its own later loads (and device-coherent stores at agent
// scope); also a compiler barrier.
__device__ inline void wait_all_memory() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt left alone
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <typename OutT>
__device__ inline OutT to_out(float x);
template <>
__device__ inline float to_out<float>(float x) { return x; }
template <>
__device__ inline uint16_t to_out<uint16_t>(float x) { return uint16_t(f2bf_bits(x)); }

// ------------------------------------------------------------------------
// Balanced decode for bf16 and fp8 caches (queries and output bf16).
//
// The work of the whole batch is a list of units (request b, kv-head group gh,
// block j), ordered by b, then gh, then j; one kv-head group is a kv-head and
// up to 16 of its query heads.  The list is cut into chunks of consecutive
// units and every wave streams whole chunks: a chunk is a run of segments, each a
// range of blocks of one (b, gh).  A segment that covers all of its (b, gh)
// is finished in place and written to `out`; the others (at most the first
// and the last of a chunk) store their (m, l, acc) state in the workspace and
// a reduce kernel merges the pieces of each (b, gh) in chunk order.
// By default the units are cut into one chunk per worker (or per unit when
// there are fewer), sizes differing by at most one, so every wave gets the
// same number of blocks
// whatever the context lengths; a caller-chosen chunk length forces
// more pieces (each wave then takes every workers-th chunk).  When the number
// of kv-head groups is a multiple of four, a workgroup's four waves move
// together over four adjacent groups (see the kernel).  Waves lower their
// issue priority as their chunk completes (progress_prio), so the workgroups
// sharing a CU finish together.
//
// Inside a segment a wave takes NB = 2 blocks per step.  Lane group q (lanes
// 16q..16q+15) owns tokens 8(q&1)..8(q&1)+7 of block q>>1 of the step:
//   scores  S^T[token][head] = K[token][:] . Q^T[:][head]   (2 MFMA row groups
//           j = 0, 1; row 4q+i is token 8(q&1) + 4j + i of block q>>1)
//   output  O^T[dim][head] += V^T[dim][token] . P^T[token][head]
// The dim-major V tile gives a lane its 8 tokens of one dimension in one
// 16-byte load; those are exactly the 8 scores the lane holds, so p never
// crosses lanes.  Only the per-head max and sum are reduced across the four
// lane groups.
constexpr int kStreamNB = 2;

template <int D>
struct WaveState {
  float m = -INFINITY;  // running max, log2 units
  float l = 0.0f;       // running sum of 2^(s - m) (this lane group's tokens)
  f32x4 acc[D / 16];    // lane (r, q): head r, dims 16t + 4q + i
  // int8 caches: acc holds the weighted sum divided by vs, the largest V
  // tile scale the segment has read so far (0 before the first tile), so
  // that the fp16 weights p * v_scale / vs fed to the MFMA stay in [0, 1]
  // whatever the magnitude of V; the true sum is acc * vs
  float vs = 0.0f;
  float vs_inv = 0.0f;  // 1 / vs once vs > 0, recomputed only when vs grows
};

// The lane's share of the query row as MFMA operands (bf16 bits).  Returns
// the factor the scores must be multiplied by: 1, except for int8 caches,
// whose operands are fp16: there the group's queries are first multiplied by
// 2^k, the power of two that puts their largest magnitude in [2^14, 2^15)
// (exact, and every bf16 value within 2^-24 of that maximum stays an fp16
// normal, so the conversion is exact for all of them), and 2^-k is returned.
template <int QT, int D>
__device__ inline float load_q(u32x4 (&qv)[D / 32], const uint16_t* q, int64_t row0, int r, int grp, int nh) {
  float qscale_inv = 1.0f;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    const int dim0 = QT != kQBf16 ? (D / 4) * grp + 8 * kk : 32 * kk + 8 * grp;
    u32x4 v = {0, 0, 0, 0};
    if (r < nh) v = ld16(q + (row0 + r) * D + dim0);
    qv[kk] = v;
  }
  if constexpr (QT == kQInt8) {
    // largest |q| of the wave's heads (bf16: the top 16 bits of an fp32)
    uint32_t mx = 0;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
      for (int w = 0; w < 4; ++w) mx = max(mx, max(qv[kk][w] & 0x7FFFu, (qv[kk][w] >> 16) & 0x7FFFu));
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) mx = max(mx, uint32_t(__shfl_xor(int(mx), o)));
    // exponent of the maximum (bf16 exponent field), 0 for an all-zero group;
    // scale 2^k with k = 14 - (e - 127), clamped to fp32's normal range
    const int e = int(mx >> 7);
    const int k = e == 0 ? 0 : min(max(14 - (e - 127), -126), 127);
    const float sq = __uint_as_float(uint32_t(127 + k) << 23);
    qscale_inv = __uint_as_float(uint32_t(127 - k) << 23);
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t v = qv[kk][w];
        qv[kk][w] = pack_op<QT>(__uint_as_float(v << 16) * sq, __uint_as_float(v & 0xFFFF0000u) * sq);
      }
  }
  return qscale_inv;
}


// Wave issue priority from the progress of the wave's chunk: `done` of `total`
// units streamed.  Waves of the three workgroups that share a CU would
// otherwise issue oldest first, so the first-dispatched workgroup runs ahead
// and the last ones finish long after it with the CU half idle; lowering the
// priority as a chunk completes lets the lagging waves catch up.  Both values
// are wave-uniform (scalar branches); total = 0 leaves the priority alone.
__device__ inline int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(x)));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(x) >> 32));
  return int64_t((uint64_t(hi) << 32) | lo);
}

__device__ inline void progress_prio(int64_t done, int64_t total) {
  done = uniform64(done);
  total = uniform64(total);
  if (total <= 0) return;
  const int64_t x = done * 20;  // priority 3 below 50% done, 2 below 75%, 1 below 90%, then 0
  if (x < 10 * total) __builtin_amdgcn_s_setprio(3);
  else if (x < 15 * total) __builtin_amdgcn_s_setprio(2);
  else if (x < 18 * total) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// The arithmetic of one step of a segment over blocks cb, cb + 1 of the
// request (block cb + 1 counts only below j1), once its K operands and V
// slices are in registers: scores, the online-softmax update, the weighted
// sum of V.  Positions at or past ctx are masked; WIN: so are positions in
// [sink, win_lo).  8-bit caches: ksc / vsc are this lane's tile scales (int8
// loads them late, through late_scales(ksc, vsc), where registers allow).
template <int QT, int D, bool WIN, class LateScales>
__device__ __forceinline__ void stream_step(WaveState<D>& st, const u32x4 (&kop)[kStreamNB][D / 32],
                                            u32x4 (&vraw)[D / 16], const u32x4 (&qv)[D / 32], int cb, int j1,
                                            int ctx, float scale_log2, float ksc, float vsc, int grp, int sink,
                                            int win_lo, float qscale_inv, LateScales&& late_scales) {
  constexpr int NB = kStreamNB;
  constexpr int KK = D / 32;
  constexpr int T8 = D / 16;
  constexpr bool Q8 = QT != kQBf16;
  const int vb_rel = grp >> 1;  // block whose scores / V this lane owns
  const int vtok = 8 * (grp & 1);
  const int bV = cb + vb_rel;
  const bool vV = bV < j1;
  // ---- scores
  f32x4 S[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    S[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      S[j] = mfma_op<QT>(kop[j][kk], qv[kk], S[j]);
  }

  // ---- online softmax over the step's 32 tokens
  float kfac = scale_log2;
  float vfac = 1.0f;
  if constexpr (Q8) {
    if constexpr (QT == kQInt8) late_scales(ksc, vsc);
    kfac *= ksc;
    vfac = vV ? vsc : 0.0f;  // tiles past the segment: zero weights anyway
  }
  float vs_fold = 1.0f;  // int8: acc rescale for a larger V-scale reference
  bool vs_grew = false;
  if constexpr (QT == kQInt8) {
    kfac *= qscale_inv;
    // the step's two tiles: lane groups 0-1 hold one, 2-3 the other
    // (wave-uniform: both halves of the wave see both tiles' scales)
    const float vs_new = fmaxf(st.vs, fmaxf(vfac, __shfl_xor(vfac, 32)));
    vs_grew = vs_new != st.vs;
    if (vs_grew) {  // a larger reference: fold the old one into acc
      st.vs_inv = 1.0f / vs_new;
      vs_fold = st.vs * st.vs_inv;
      st.vs = vs_new;
    }
    vfac *= st.vs_inv;
  }
  // A step whose two blocks lie inside the segment and whose 32 positions
  // are all read (below ctx; WIN: all sinks or all inside the window)
  // needs no mask: the common case, one wave-uniform test.
  bool full = cb + 1 < j1 && (cb + NB) * kBS <= ctx;
  if constexpr (WIN) full = full && ((cb + NB) * kBS <= sink || cb * kBS >= win_lo);
  int valid = 8;      // valid among the lane's 8 tokens (not WIN)
  uint32_t keep = 0xFFu;  // WIN: bit e set when token vtok + e of block bV is read
  float mx = -INFINITY;
  if (full) {
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        S[j][i] *= kfac;
        mx = fmaxf(mx, S[j][i]);
      }
  } else {
    valid = vV ? min(kBS, ctx - bV * kBS) - vtok : 0;
    if constexpr (WIN) {
      keep = 0;
      const int p0 = bV * kBS + vtok;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int p = p0 + e;
        keep |= uint32_t(vV && p < ctx && (p < sink || p >= win_lo)) << e;
      }
    }
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = WIN ? ((keep >> (4 * j + i)) & 1u) != 0 : 4 * j + i < valid;
        const float sv = ok ? S[j][i] * kfac : -INFINITY;
        S[j][i] = sv;
        mx = fmaxf(mx, sv);
      }
  }
  mx = wave_max16(mx);
  // Lazy maximum: the running maximum moves (and the accumulators are
  // rescaled) only when a step's maximum exceeds it by more than 2^8 in a
  // lane of the wave; otherwise the weights are formed against the stale
  // maximum and stay below 2^8.  The state (m, l, acc) is the same softmax
  // for any m, which is all the finish and the piece merge assume.
  if (__builtin_amdgcn_ballot_w64(mx > st.m + kLazyLog2 || vs_grew) != 0) {
    const float m_new = fmaxf(st.m, mx);
    // a fused append: a row may have read no cached token yet (its segment
    // starts at the block that holds only the new token, or a window of one
    // whose only position is that token); its state stays empty
    const float m_ref = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_ref);
    st.l *= alpha;
    st.m = m_new;
    const float afac = QT == kQInt8 ? alpha * vs_fold : alpha;
#pragma unroll
    for (int t = 0; t < T8; ++t) st.acc[t] *= afac;
  }
  const float m_use = st.m == -INFINITY ? 0.0f : st.m;
  float psum = 0.0f;
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = __builtin_amdgcn_exp2f(S[j][i] - m_use);
      S[j][i] = e;
      psum += e;
    }
  st.l += psum;

  // ---- weighted sum of V: k-slot e is token vtok + e of block bV
  const f32x4 lo = S[0] * vfac, hi = S[1] * vfac;
  const u32x4 pop = {pack_op<QT>(lo[0], lo[1]), pack_op<QT>(lo[2], lo[3]), pack_op<QT>(hi[0], hi[1]),
                     pack_op<QT>(hi[2], hi[3])};
  auto v_op = [&](int t) -> u32x4 {  // this lane's V slice t as MFMA operand pairs
    if constexpr (Q8) {
      const u32x2 a = q8x4_to_op<QT>(vraw[t][0]);
      const u32x2 c2 = q8x4_to_op<QT>(vraw[t][1]);
      return u32x4{a[0], a[1], c2[0], c2[1]};
    } else {
      return vraw[t];
    }
  };
  // Stale or poisoned slots past the context (WIN: outside the window)
  // are zeroed before their weight-zero product: one mask for the step,
  // applied to the raw registers (8-bit codes: per byte, code 0 is +0);
  // a full step skips it.
  if (!full) {
    const int vh = min(max(valid, 0), 8);
    const uint32_t k8 = WIN ? keep : (1u << vh) - 1u;
    if constexpr (Q8) {
      uint32_t bm[2];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        bm[w] = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) bm[w] |= ((k8 >> (4 * w + e)) & 1u ? 0xFFu : 0u) << (8 * e);
      }
#pragma unroll
      for (int t = 0; t < T8; ++t) {
        vraw[t][0] &= bm[0];
        vraw[t][1] &= bm[1];
      }
    } else {
      u32x4 vm;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        vm[w] = ((k8 >> (2 * w)) & 1u ? 0x0000FFFFu : 0u) | ((k8 >> (2 * w + 1)) & 1u ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int t = 0; t < T8; ++t) vraw[t] &= vm;
    }
  }
#pragma unroll
  for (int t = 0; t < T8; ++t) st.acc[t] = mfma_op<QT>(v_op(t), pop, st.acc[t]);
}

// Stream blocks [j0, j1) of one (request, kv-head) into the wave state.
// Positions at or past ctx are masked.  WIN: so are positions in
// [sink, win_lo) (a sliding window with attention sinks).
// The new token's K row and this lane's part of its V row (dimensions
// 16 t + 4 grp .. + 3), for a fused append.
template <int D>
struct TokenRows {
  u32x4 k[D / 32];
  u32x2 v[D / 16];
};

// The fused append's V slot, written as whole rows: the step's V slices are
// in registers (lane (r, grp): dimension 16 t + r, key half grp & 1 of the
// step's block grp >> 1), so the lanes holding block `be` (the token's block)
// put the new token's value at offset o of their half rows and store them.
// Every row of the tile is rewritten with the bytes the step copied, which
// are the tile's current ones: no other wave of the launch reads or writes
// this tile.  val[t] is the token's value of dimension 16 t + r (bf16 bits).
template <int D>
__device__ __forceinline__ void patch_token_v(const u32x4 (&vraw)[D / 16], const uint32_t (&val)[D / 16],
                                              uint8_t* vtile, int be, int o, int r, int grp) {
  const int h = grp & 1;
  const int p = o & 7;
  const uint32_t sh = 16u * uint32_t(p & 1);
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    u32x4 row = vraw[t];
    if (h == (o >> 3)) {
#pragma unroll
      for (int wi = 0; wi < 4; ++wi)
        if (wi == (p >> 1)) row[wi] = (row[wi] & ~(0xFFFFu << sh)) | (val[t] << sh);
    }
    if ((grp >> 1) == be) *reinterpret_cast<u32x4*>(vtile + ((16 * t + r) * kBS + 8 * h) * 2) = row;
  }
}

// The same after the segment, for the register-streaming kernel (whose step
// has no registers to spare): the tile's V rows are loaded again (lanes of
// groups 0 and 1: dimension 16 t + r, half grp), the token's values with
// them, and the rows go back with the token in place.
template <int D>
__device__ __forceinline__ void reload_patch_token_v(uint8_t* vtile, const uint16_t* __restrict__ vn, int o, int r,
                                                     int grp) {
  if (grp >= 2) return;
  u32x4 rows[D / 16];
  uint32_t val[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    rows[t] = ld16(vtile + ((16 * t + r) * kBS + 8 * grp) * 2);
    val[t] = vn[16 * t + r];
  }
  patch_token_v<D>(rows, val, vtile, 0, o, r, grp);
}

// The values patch_token_v needs, from TokenRows: trw.v[t] holds dimensions
// 16 t + 4 grp .. + 3 in every lane of group grp, so dimension 16 t + r comes
// from lane r + 16 (r >> 2).  Every lane of the wave must take part.
template <int D>
__device__ __forceinline__ void token_v_values(uint32_t (&val)[D / 16], const TokenRows<D>& trw, int r) {
  const int src = r + 16 * (r >> 2);
  const int e = r & 3;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    const uint32_t w0 = __shfl(trw.v[t][0], src), w1 = __shfl(trw.v[t][1], src);
    val[t] = (((e >> 1) ? w1 : w0) >> (16 * (e & 1))) & 0xFFFFu;
  }
}

template <int QT, int D, bool NT, bool WIN = false>
__device__ __forceinline__ void run_segment(WaveState<D>& st, const uint8_t* __restrict__ kc,
                                   const uint8_t* __restrict__ vc, const float* __restrict__ kscale,
                                   const float* __restrict__ vscale, const int32_t* __restrict__ trow,
                                   int ctx, int H, int g, int j0, int j1, float scale_log2,
                                   const u32x4 (&qv)[D / 32], int r, int grp, int sink = 0,
                                   int win_lo = 0, int64_t done0 = 0, int64_t total = 0,
                                   float qscale_inv = 1.0f) {
  constexpr int NB = kStreamNB;
  constexpr int KK = D / 32;
  constexpr int T8 = D / 16;
  constexpr bool Q8 = QT != kQBf16;  // 8-bit codes with per-tile scales
  constexpr int EB = Q8 ? 1 : 2;
  const int64_t tile_bytes = int64_t(kBS) * D * EB;
  const int kb_rel = r >> 3;    // block (of the step) feeding this lane's K row
  const int vb_rel = grp >> 1;  // block whose scores / V this lane owns
  const int vtok = 8 * (grp & 1);
  const int jlast = j1 - 1;
  int32_t tK = trow[min(j0 + kb_rel, jlast)];
  int32_t tV = trow[min(j0 + vb_rel, jlast)];
  for (int cb = j0; cb < j1; cb += NB) {
    progress_prio(done0 + (cb - j0), total);
    const int64_t pK = tK;
    const int64_t pV = tV;
    // next step's table entries, in flight while this step computes
    tK = trow[min(cb + NB + kb_rel, jlast)];
    tV = trow[min(cb + NB + vb_rel, jlast)];
    const uint8_t* ktile = kc + (pK * H + g) * tile_bytes;
    const uint8_t* vtile = vc + (pV * H + g) * tile_bytes;
    // fp8: the tile scales go out before the K/V loads, so that waiting for
    // them (loads complete in order) never waits for V (same box, fp8 calls
    // 1% faster; int8, whose extra state makes registers tight, lost as much
    // and loads them after)
    float ksc = 1.0f, vsc = 1.0f;
    if constexpr (QT == kQFp8) {
      ksc = kscale[pV * H + g];
      vsc = vscale[pV * H + g];
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- loads: K rows for the score MFMAs, this lane's V slice.  A block
    // past the segment (an odd last step) is loaded from the clamped table
    // entry like any other: its scores are masked to -inf and its V zeroed
    // below, so its bytes never count, and no load needs a lane mask.
    u32x4 kop[NB][KK];
    u32x4 vraw[T8];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int ktok = 8 * ((r >> 2) & 1) + 4 * j + (r & 3);
      if constexpr (!Q8) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) kop[j][kk] = ld16_kv<NT>(ktile + (ktok * D + 32 * kk + 8 * grp) * 2);
      } else {
        constexpr int NSEG = D / 64;  // 16-byte pieces of a lane's D/4 codes
        u32x4 seg[NSEG];
#pragma unroll
        for (int s = 0; s < NSEG; ++s) seg[s] = ld16_kv<NT>(ktile + ktok * D + (D / 4) * grp + 16 * s);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const u32x4& sv = seg[kk / 2];
          const u32x2 a = q8x4_to_op<QT>(sv[(kk % 2) * 2 + 0]);
          const u32x2 bq = q8x4_to_op<QT>(sv[(kk % 2) * 2 + 1]);
          kop[j][kk] = u32x4{a[0], a[1], bq[0], bq[1]};
        }
      }
    }
#pragma unroll
    for (int t = 0; t < T8; ++t) {
      if constexpr (!Q8) {
        vraw[t] = ld16_kv<NT>(vtile + ((16 * t + r) * kBS + vtok) * 2);
      } else {
        const u32x2 v = ld8_kv<NT>(vtile + (16 * t + r) * kBS + vtok);
        vraw[t] = u32x4{v[0], v[1], 0, 0};
      }
    }

    stream_step<QT, D, WIN>(st, kop, vraw, qv, cb, j1, ctx, scale_log2, ksc, vsc, grp, sink, win_lo, qscale_inv,
                            [&](float& ks, float& vs) {
                              ks = kscale[pV * H + g];
                              vs = vscale[pV * H + g];
                            });
  }
}

// The step's append for an 8-bit cache, inside the decode: the wave that
// owns tile (block, kv head) `sidx` writes the new token at offset o of it
// ("KV cache and PagedAttention", askaiml §7: the cache holds codes with a
// scale).  The rule and the arithmetic are append_q8_kernel's for a run of
// one token: s1 = max(s0, max |x| / largest code) with s0 = 0 when o == 0;
// when the scale grows the tile's older codes are re-encoded from
// decode(code) * s0; the new codes are encode(x * (1 / s1)), 0 when s1 == 0.
// Plain loads and stores: only this wave touches the tile in this launch,
// and the workgroup-scope release / acquire that follows (wait_all_memory)
// orders them before the wave's reads of it.
// Not inlined: its fp8 codec is large, and inlined into the ring decode's
// step loop (where it runs once per request and kv head) the code grew the
// fused fp8 step from 210 to 251 us.
template <int D, bool INT8>
__device__ __attribute__((noinline)) void append8_token(uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                                              float* __restrict__ ksc, float* __restrict__ vsc, int64_t sidx, int o,
                                              const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
                                              int lane) {
  using C = Codec8<INT8>;
  constexpr int TILE = kBS * D;
  constexpr int KP = TILE / 16 / 64;  // K pieces per lane
  constexpr int VR = D / 64;          // V rows per lane
  auto bf = [](uint16_t b) { return __uint_as_float(uint32_t(b) << 16); };
  uint8_t* ktile = kc + sidx * TILE;
  uint8_t* vtile = vc + sidx * TILE;
  // everything the rule reads, in flight together: both old scales, the new
  // rows, the old K pieces below the token and the V rows
  const float sk0 = o == 0 ? 0.0f : ksc[sidx];
  const float sv0 = o == 0 ? 0.0f : vsc[sidx];
  float kx[VR], vx[VR];
#pragma unroll
  for (int i = 0; i < VR; ++i) {
    kx[i] = bf(kn[lane + 64 * i]);
    vx[i] = bf(vn[lane + 64 * i]);
  }
  u32x4 kp[KP], vr[VR];
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const int row = (lane + 64 * i) / (D / 16);
    kp[i] = row < o ? ld16(ktile + 16 * (lane + 64 * i)) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < VR; ++i) vr[i] = ld16(vtile + 16 * (lane + 64 * i));
  float ka = fabsf(kx[0]), va = fabsf(vx[0]);
#pragma unroll
  for (int i = 1; i < VR; ++i) {
    ka = fmaxf(ka, fabsf(kx[i]));
    va = fmaxf(va, fabsf(vx[i]));
  }
#pragma unroll
  for (int w = 32; w > 0; w >>= 1) {
    ka = fmaxf(ka, __shfl_xor(ka, w));
    va = fmaxf(va, __shfl_xor(va, w));
  }
  const float sk1 = fmaxf(sk0, ka / C::kMax), sv1 = fmaxf(sv0, va / C::kMax);
  const bool rek = sk1 != sk0 && o > 0, rev = sv1 != sv0 && o > 0;
  const float ik = sk1 == 0.0f ? 0.0f : 1.0f / sk1, iv = sv1 == 0.0f ? 0.0f : 1.0f / sv1;
  auto reenc = [](uint32_t c, float s0, float inv) -> uint32_t {
    const float x = C::decode(c) * s0;
    return C::encode(x * inv) & 0xFFu;
  };
  // K tile [16][D]: 16-byte pieces lane, lane + 64, ...; the new row's codes
  // come from the token's values, the rows below it are re-encoded
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const int pc = lane + 64 * i;
    const int row = pc / (D / 16), col0 = (pc % (D / 16)) * 16;
    if (row > o || (row < o && !rek)) continue;
    u32x4 w = {0, 0, 0, 0};
    if (row < o) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) w[k] |= reenc((kp[i][k] >> (8 * e)) & 0xFFu, sk0, ik) << (8 * e);
    } else if (sk1 != 0.0f) {
      const u32x4 a = ld16(kn + col0), b = ld16(kn + col0 + 8);  // the row's 16 values
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int idx = 4 * k + e;
          const u32x4& src = idx < 8 ? a : b;
          const uint32_t word = src[(idx & 7) >> 1];
          const float x = __uint_as_float((idx & 1) ? (word & 0xFFFF0000u) : (word << 16));
          w[k] |= (C::encode(x * ik) & 0xFFu) << (8 * e);
        }
    }
    *reinterpret_cast<u32x4*>(ktile + 16 * pc) = w;
  }
  // V tile [D][16]: dimension rows lane, lane + 64, ...; byte o is the new
  // token, the bytes below it are re-encoded, the ones above stay
#pragma unroll
  for (int i = 0; i < VR; ++i) {
    const uint32_t cnew = sv1 == 0.0f ? 0u : (C::encode(vx[i] * iv) & 0xFFu);
    u32x4 w = vr[i];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 4 * k + e;
        if (t > o) continue;
        const uint32_t c = (w[k] >> (8 * e)) & 0xFFu;
        const uint32_t v = t == o ? cnew : rev ? reenc(c, sv0, iv) : c;
        w[k] = (w[k] & ~(0xFFu << (8 * e))) | (v << (8 * e));
      }
    *reinterpret_cast<u32x4*>(vtile + 16 * (lane + 64 * i)) = w;
  }
  if (lane == 0) {
    ksc[sidx] = sk1;
    vsc[sidx] = sv1;
  }
}

// One token's K and V rows (head_dim values each, one kv head), this lane's
// share: K dims 32 kk + 8 grp .. + 7, V dims 16 t + 4 grp .. + 3.

template <int D>
__device__ inline void load_token(TokenRows<D>& t, const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
                                  int grp) {
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) t.k[kk] = ld16(kn + 32 * kk + 8 * grp);
#pragma unroll
  for (int i = 0; i < D / 16; ++i) t.v[i] = *reinterpret_cast<const u32x2*>(vn + 16 * i + 4 * grp);
}

// Fold one more token into the wave state: the score of head r is the dot
// product of the lane group's quarter of q and of the key, summed over the
// four lane groups; then the usual online-softmax update.  The weight is
// counted once in l (lane group 0) since l is summed over lane groups later.
template <int D>
__device__ inline void fold_token(WaveState<D>& st, const TokenRows<D>& tr, const u32x4 (&qv)[D / 32],
                                  float scale_log2, int grp) {
  float s = 0.0f;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    const bf16x8 kx = __builtin_bit_cast(bf16x8, tr.k[kk]);
    const bf16x8 qx = __builtin_bit_cast(bf16x8, qv[kk]);  // bf16 caches only
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(float(qx[e]), float(kx[e]), s);
  }
  s = wave_sum16(s) * scale_log2;
  const float m_new = fmaxf(st.m, s);
  const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
  const float p = __builtin_amdgcn_exp2f(s - m_new);
  st.l = st.l * alpha + (grp == 0 ? p : 0.0f);
  st.m = m_new;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    const u32x2 w = tr.v[t];
    const f32x4 v = {__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xFFFF0000u),
                     __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xFFFF0000u)};
    st.acc[t] = st.acc[t] * alpha + v * p;
  }
}

// Pages a decode reads for a request of n tokens: logical pages [0, a) and
// [c, nb), nb = ceil(n / 16).  Without a window a = c = nb.  With `sink`
// sink tokens and a window of `window` tokens, c is the page of position
// max(0, n - window) and a = min(pages holding the sinks, c) (a == c: the two
// ranges meet and every page is read).  Every page read holds at least one
// position that is read.
struct VisitedPages {
  int a, c, nb;
  __device__ int count() const { return a + nb - c; }
};

template <bool WIN>
__device__ inline VisitedPages visited_pages(int n, int sink, int window) {
  const int nb = (n + kBS - 1) / kBS;
  if constexpr (!WIN) {
    return {nb, nb, nb};
  } else {
    const int c = max(0, n - window) / kBS;
    const int a = min((min(sink, n) + kBS - 1) / kBS, c);
    return {a, c, nb};
  }
}

// Exclusive prefix sums of the pages each request reads into s_pref[0..B]
// (256 threads).
template <bool WIN>
__device__ inline void block_prefix_blocks(int32_t* s_pref, int32_t* s_tmp, const int32_t* ctx_lens, int B,
                                           int max_ctx, int sink, int window) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int32_t carry = 0;
  for (int base = 0; base < B; base += 256) {
    const int b = base + tid;
    const int32_t v = b < B ? visited_pages<WIN>(clamp_ctx(ctx_lens, b, max_ctx), sink, window).count() : 0;
    int32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) s_tmp[w] = x;
    __syncthreads();
    int32_t before = carry;
    for (int k = 0; k < w; ++k) before += s_tmp[k];
    if (b < B) s_pref[b + 1] = before + x;
    const int32_t total = s_tmp[0] + s_tmp[1] + s_tmp[2] + s_tmp[3];
    __syncthreads();
    carry += total;
  }
  if (tid == 0) s_pref[0] = 0;
  __syncthreads();
}

// The chunks of the unit list [0, U) for W workers (shared by the decode and
// reduce kernels).  Fixed: chunk c holds [c C, c C + C) and worker w takes
// chunks w, w + W, ...  Balanced: N = min(W, U) chunks, one per worker, chunk c
// holding [c U / N, (c + 1) U / N).  No chunk is empty and chunk ids follow
// the unit order, so the chunks holding one (b, gh) are consecutive.
struct StreamChunks {
  int64_t U, C, N;
  __device__ __forceinline__ StreamChunks(int64_t U_, int W, int chunk_fixed) : U(U_), C(chunk_fixed) {
    N = C > 0 ? (U + C - 1) / C : min<int64_t>(W, U);
  }
  __device__ __forceinline__ int64_t start(int64_t c) const { return C > 0 ? c * C : c * U / N; }
  __device__ __forceinline__ int64_t end(int64_t c) const { return C > 0 ? min(U, c * C + C) : (c + 1) * U / N; }
  // chunk holding unit x (0 <= x < U)
  __device__ __forceinline__ int64_t chunk_of(int64_t x) const { return C > 0 ? x / C : ((x + 1) * N - 1) / U; }
};

// Where piece k of a row lives: the row's pieces are the segments of chunks
// c0, c0 + 1, ... that cover it; the first may be the chunk's second segment
// (role 1), every later one is its chunk's first (role 0).  Two state sets
// per chunk, one per wave of a workgroup chunk (coop) and HS rows each.
__device__ inline int64_t piece_slot_base(int64_t c0, int first_role, int k, bool coop, int wv, int HS) {
  const int64_t cr = (c0 + k) * 2 + (k == 0 ? first_role : 0);
  return (coop ? cr * 4 + wv : cr) * HS;
}

// Merge the K pieces of one row set (request, kv-head group: nh query heads)
// in piece order and write its nh output rows, by one whole wave: every lane
// takes two (head, dimension quad) pairs per pass and folds the pieces with
// a running maximum, the loads of four pieces in flight together.  The
// states were stored with device-coherent stores and are loaded the same way.
template <int D>
__device__ __forceinline__ void merge_row_pieces(uint16_t* __restrict__ out, int64_t row0, int nh, int HS,
                                 __amdgpu_buffer_rsrc_t rml, __amdgpu_buffer_rsrc_t racc, int64_t c0,
                                 int first_role, int K, bool coop, int wv, int lane) {
  constexpr int DQ = D / 4;
  constexpr int PB = 4;
  const int quads = nh * DQ;
  for (int q0 = 0; q0 < quads; q0 += 128) {
    int qd[2], hh[2];
    bool on[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      qd[i] = q0 + lane + 64 * i;
      on[i] = qd[i] < quads;
      hh[i] = on[i] ? qd[i] / DQ : 0;
    }
    float M[2] = {-INFINITY, -INFINITY}, L[2] = {0.0f, 0.0f};
    f32x4 A[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    for (int k0 = 0; k0 < K; k0 += PB) {
      u32x2 ml[PB][2];
      u32x4 ac[PB][2];
#pragma unroll
      for (int p = 0; p < PB; ++p) {
        const int k = k0 + p;
        const int64_t sb = piece_slot_base(c0, first_role, k, coop, wv, HS);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          ml[p][i] = u32x2{0, 0};
          ac[p][i] = u32x4{0, 0, 0, 0};
          if (k < K && on[i]) {
            const int64_t s = sb + hh[i];
            ml[p][i] = load8_coherent(rml, uint32_t(s * 8));
            ac[p][i] = load16_coherent(racc, uint32_t((s * D + 4 * (qd[i] - hh[i] * DQ)) * 4));
          }
        }
      }
#pragma unroll
      for (int p = 0; p < PB; ++p) {
        if (k0 + p >= K) break;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float m = __uint_as_float(ml[p][i][0]), l = __uint_as_float(ml[p][i][1]);
          const float Mn = fmaxf(M[i], m);
          const float eo = __builtin_amdgcn_exp2f(M[i] - Mn), en = __builtin_amdgcn_exp2f(m - Mn);
          L[i] = L[i] * eo + l * en;
          A[i] = A[i] * eo + __builtin_bit_cast(f32x4, ac[p][i]) * en;
          M[i] = Mn;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (!on[i]) continue;
      const float inv = 1.0f / L[i];
      const u32x2 pk = {pack_bf16(A[i][0] * inv, A[i][1] * inv), pack_bf16(A[i][2] * inv, A[i][3] * inv)};
      *reinterpret_cast<u32x2*>(out + (row0 + hh[i]) * D + 4 * (qd[i] - hh[i] * DQ)) = pk;
    }
  }
}

// grid = workers / 4 workgroups of 256 threads; chunk_fixed = 0 for balanced chunks.
//
// APPEND (bf16 caches): request b also appends one token, k_new[b] / v_new[b]
// ([H][D] each), at new_slots[b] (-1: none), which is the slot of its
// position ctx - 1.  The attention then reads positions < ctx - 1 from the
// cache and takes the last one from k_new / v_new (fold_token, in the segment
// that ends the request).  The token goes into the cache in the same launch:
// threads store its K row while the block counts are summed (and its V slot
// when it starts a block, which no wave then reads), and the wave whose
// segment ends the request writes the V rows of the token's block whole,
// from the copy it read, with the token in place (patch_token_v).  The K
// slot's bytes may be loaded with the rest of its tile while the K stores
// land, unordered, but that lane is past the cached range and masked, so
// neither the old nor the new bytes reach the result.  8-bit caches: see the
// Q8 append branch.
//
// WIN: a sliding window of `window` tokens plus `sink` sink tokens; units
// run over the pages each request reads (visited_pages), so pages outside
// are never touched and may be free.  APPEND and WIN together: the window of
// the grown request, its new token taken from k_new / v_new.
template <int QT, int D, bool APPEND, bool WIN, bool NT>
__global__ void __launch_bounds__(256, 3)
decode_stream_kernel(void* __restrict__ kc_, void* __restrict__ vc_,
                     float* __restrict__ kscale, float* __restrict__ vscale,
                     const uint16_t* __restrict__ q, uint16_t* __restrict__ out,
                     const int32_t* __restrict__ tables, int max_blocks,
                     const int32_t* __restrict__ ctx_lens, int B, int max_ctx, int H, int h_q,
                     int G, int n_hgroups, int HS, float scale_log2, int chunk_fixed,
                     float* __restrict__ ws_ml, float* __restrict__ ws_acc,
                     int32_t* __restrict__ ws_pref, int32_t* __restrict__ ws_cnt,
                     const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
                     const int32_t* __restrict__ new_slots, int sink, int window) {
  constexpr int T8 = D / 16;
  __shared__ int32_t s_pref[kMaxStreamB + 1];
  __shared__ int32_t s_tmp[4];
  // APPEND: 16-byte pieces (8 dims) of the new rows; thread i of the grid
  // takes piece i (and i + grid, ... on big batches).  The first piece's
  // loads are issued before the block counts are summed, its stores after.
  constexpr bool APPEND16 = APPEND && QT == kQBf16;  // 8-bit caches append inside their segments
  const int pieces = APPEND16 ? B * H * (D / 8) : 0;
  const int gthreads = gridDim.x * 256;
  int piece = blockIdx.x * 256 + threadIdx.x;
  u32x4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
  int32_t pslot = -1;
  if (APPEND16 && piece < pieces) {
    pslot = new_slots[piece / (H * (D / 8))];
    kx = ld16(k_new + int64_t(piece) * 8);
    vx = ld16(v_new + int64_t(piece) * 8);
  }
  block_prefix_blocks<WIN>(s_pref, s_tmp, ctx_lens, B, max_ctx, sink, window);
  if constexpr (APPEND16) {
    uint16_t* kw = static_cast<uint16_t*>(kc_);
    uint16_t* vw = static_cast<uint16_t*>(vc_);
    while (piece < pieces) {
      if (pslot >= 0) {
        const int hd = piece % (H * (D / 8));  // kv head and dim piece within the request
        const int g = hd / (D / 8);
        const int d0 = 8 * (hd - g * (D / 8));
        const int64_t tile = (int64_t(pslot / kBS) * H + g) * kBS * D;
        const int off = pslot % kBS;
        *reinterpret_cast<u32x4*>(kw + tile + off * D + d0) = kx;
        // the V slot is 2 bytes in each 32-byte row: the wave that reads the
        // block writes its rows whole (patch_token_v); only a block holding
        // nothing but the token gets the scattered stores
        if (off == 0) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            vw[tile + int64_t(d0 + e) * kBS + off] = uint16_t(vx[e / 2] >> (16 * (e & 1)));
        }
      }
      piece += gthreads;
      if (piece < pieces) {
        pslot = new_slots[piece / (H * (D / 8))];
        kx = ld16(k_new + int64_t(piece) * 8);
        vx = ld16(v_new + int64_t(piece) * 8);
      }
    }
  }
  if (ws_cnt == nullptr) {
    if (blockIdx.x == 0)  // the block prefix of the reduce kernel
      for (int i = threadIdx.x; i <= B; i += 256) ws_pref[i] = s_pref[i];
  } else {
    // no reduce kernel follows: requests without pages get their zero rows here
    const int row8 = D / 4;  // 8-byte pieces of one output row (the alignment of every out store)
    for (int b = blockIdx.x; b < B; b += gridDim.x)
      if (s_pref[b + 1] == s_pref[b])
        for (int i = threadIdx.x; i < h_q * row8; i += 256)
          *reinterpret_cast<u32x2*>(out + (int64_t(b) * h_q * row8 + i) * 4) = u32x2{0, 0};
  }

  const int hge = H * n_hgroups;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index, uniform
  // When the (kv-head, head-group) pairs come in fours, a unit is (b, set of
  // four pairs, j) and a workgroup streams whole chunks, its wave wv taking
  // pair 4 * set + wv of every block: the four waves read adjacent tiles of
  // the same blocks (16 KiB runs for bf16, d 128) and share table entries and
  // fp8 scales in one L2.  Otherwise every wave streams chunks of its own.
  const bool coop = (hge & 3) == 0;
  const int hsets = coop ? hge >> 2 : hge;
  const int64_t U = uniform64(int64_t(hsets) * s_pref[B]);
  const int W = coop ? gridDim.x : gridDim.x * 4;
  const StreamChunks ch(U, W, chunk_fixed);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int grp = lane >> 4;
  const uint8_t* kc = static_cast<const uint8_t*>(kc_);
  const uint8_t* vc = static_cast<const uint8_t*>(vc_);
  const __amdgpu_buffer_rsrc_t rml = raw_rsrc(ws_ml), racc = raw_rsrc(ws_acc);

  for (int64_t c = coop ? int64_t(blockIdx.x) : int64_t(blockIdx.x) * 4 + wv; c < ch.N; c += W) {
    int64_t u = ch.start(c);
    const int64_t u_end = ch.end(c);
    const int64_t u0 = u;
    const int64_t ctot = chunk_fixed > 0 ? 0 : u_end - u0;  // progress priority on balanced chunks
    // request holding unit u: the last b with hsets * pref[b] <= u
    const int64_t x = u / hsets;
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] <= x) lo = mid;
      else hi = mid - 1;
    }
    int b = lo;
    int nb = s_pref[b + 1] - s_pref[b];
    int64_t rem = u - int64_t(hsets) * s_pref[b];
    int gs = int(rem / nb);
    int j = int(rem - int64_t(gs) * nb);
    int role = 0;
    while (true) {
      const int j1 = int(min<int64_t>(nb, j + (u_end - u)));
      const int gh = coop ? 4 * gs + wv : gs;
      const int g = gh / n_hgroups;
      const int hg = gh - g * n_hgroups;
      const int head0 = g * G + hg * 16;
      const int nh = min(16, G - hg * 16);
      const int64_t row0 = int64_t(b) * h_q + head0;
      u32x4 qv[D / 32];
      const float qsi = load_q<QT, D>(qv, q, row0, r, grp, nh);
      WaveState<D> st;
#pragma unroll
      for (int t = 0; t < T8; ++t) st.acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int ctx = clamp_ctx(ctx_lens, b, max_ctx);
      if constexpr (WIN) {
        // read positions [0, sink) and [ctx - window, ctx); visited pages
        // [j, j1) map to logical [0, a) then [c, nb).  APPEND: the cache
        // holds positions < ctx - 1, and the segment that ends the request
        // takes the last one from k_new / v_new
        const VisitedPages vp = visited_pages<true>(ctx, sink, window);
        const int win_lo = max(0, ctx - window);
        const bool app = APPEND && new_slots[b] >= 0;
        const int ctx_c = ctx - (app ? 1 : 0);
#pragma clang loop unroll(disable)
        for (int part = 0; part < 2; ++part) {
          const int lo = part == 0 ? j : max(j, vp.a);
          const int hi = part == 0 ? min(j1, vp.a) : j1;
          const int off = part == 0 ? 0 : vp.c - vp.a;
          if (lo < hi)
            run_segment<QT, D, NT, true>(st, kc, vc, kscale, vscale, tables + int64_t(b) * max_blocks, ctx_c, H, g,
                                      lo + off, hi + off, scale_log2, qv, r, grp, sink, win_lo, u - u0 + (lo - j),
                                      ctot, qsi);
        }
        // the segment that ends the request folds in the new token and, unless
        // it starts its block, writes that block's V rows (patch_token_v)
        if (app && j1 == nb) {
          const int64_t nrow = (int64_t(b) * H + g) * D;
          TokenRows<D> trw;
          load_token<D>(trw, k_new + nrow, v_new + nrow, grp);
          fold_token<D>(st, trw, qv, scale_log2, grp);
          const int o = (ctx - 1) & (kBS - 1);
          if (APPEND16 && o != 0)
            reload_patch_token_v<D>(static_cast<uint8_t*>(vc_) +
                                        (int64_t(tables[int64_t(b) * max_blocks + vp.nb - 1]) * H + g) * (kBS * D * 2),
                                    v_new + nrow, o, r, grp);
        }
      } else if constexpr (APPEND && QT != kQBf16) {
        // 8-bit cache: the wave whose segment ends the request writes the
        // new token into the request's last tile (re-encoding it when its
        // scale grows) before the segment's last step, then runs that step;
        // every position, the new one included,
        // comes from the cache, and the steps are those of the plain decode,
        // so the result is bit for bit that of kv_append followed by
        // paged_attention_decode.  Only this wave reads the tile (one kv-head
        // group per kv head).
        const int32_t slot = __builtin_amdgcn_readfirstlane(new_slots[b]);
        const int64_t trow_off = int64_t(b) * max_blocks;
        if (slot >= 0 && j1 == nb) {
          const int last = j + kStreamNB * ((nb - 1 - j) / kStreamNB);  // first block of the last step
          if (j < last)
            run_segment<QT, D, NT>(st, kc, vc, kscale, vscale, tables + trow_off, ctx, H, g, j, last, scale_log2,
                               qv, r, grp, 0, 0, u - u0, ctot, qsi);
          append8_token<D, QT == kQInt8>(static_cast<uint8_t*>(kc_), static_cast<uint8_t*>(vc_), kscale, vscale,
                                         int64_t(slot / kBS) * H + g, slot % kBS,
                                         k_new + (int64_t(b) * H + g) * D, v_new + (int64_t(b) * H + g) * D, lane);
          wait_all_memory();
          run_segment<QT, D, NT>(st, kc, vc, kscale, vscale, tables + trow_off, ctx, H, g, last, nb, scale_log2, qv, r,
                             grp, 0, 0, u - u0 + (last - j), ctot, qsi);
        } else {
          run_segment<QT, D, NT>(st, kc, vc, kscale, vscale, tables + trow_off, ctx, H, g, j, j1, scale_log2, qv, r,
                             grp, 0, 0, u - u0, ctot, qsi);
        }
      } else if constexpr (APPEND) {
        // the cache holds positions < ctx - 1; a segment cut down to nothing
        // is the request's last block holding only the new token
        const bool app = new_slots[b] >= 0;  // ctx > 0 here: b has blocks
        const int ctx_c = ctx - (app ? 1 : 0);
        const int jc1 = min(j1, (ctx_c + kBS - 1) / kBS);
        if (j < jc1)
          run_segment<QT, D, NT>(st, kc, vc, kscale, vscale, tables + int64_t(b) * max_blocks, ctx_c, H, g,
                              j, jc1, scale_log2, qv, r, grp, 0, 0, u - u0, ctot);
        // the segment that ends the request folds in the new token and, unless
        // it starts its block, writes that block's V rows (patch_token_v)
        if (app && j1 == nb) {
          const int64_t nrow = (int64_t(b) * H + g) * D;
          TokenRows<D> trw;
          load_token<D>(trw, k_new + nrow, v_new + nrow, grp);
          fold_token<D>(st, trw, qv, scale_log2, grp);
          const int o = (ctx - 1) & (kBS - 1);
          if (o != 0)
            reload_patch_token_v<D>(static_cast<uint8_t*>(vc_) +
                                        (int64_t(tables[int64_t(b) * max_blocks + nb - 1]) * H + g) * (kBS * D * 2),
                                    v_new + nrow, o, r, grp);
        }
      } else {
        run_segment<QT, D, NT>(st, kc, vc, kscale, vscale, tables + int64_t(b) * max_blocks, ctx, H, g, j, j1,
                            scale_log2, qv, r, grp, 0, 0, u - u0, ctot, qsi);
      }
      if constexpr (QT == kQInt8) {  // back to true units (acc was relative to st.vs)
#pragma unroll
        for (int t = 0; t < T8; ++t) st.acc[t] *= st.vs;
      }
      const float l = wave_sum16(st.l);
      if (j == 0 && j1 == nb) {  // the whole (b, gh): finish here
        if (r < nh) {
          const float inv = 1.0f / l;
#pragma unroll
          for (int t = 0; t < T8; ++t) {
            const f32x4 o = st.acc[t] * inv;
            const u32x2 pk = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
            *reinterpret_cast<u32x2*>(out + (row0 + r) * D + 16 * t + 4 * grp) = pk;
          }
        }
      } else {
        // a piece: its state goes to the workspace with device-coherent stores
        if (r < nh) {
          const int64_t slot = (coop ? (c * 2 + role) * 4 + wv : c * 2 + role) * HS + r;
          if (grp == 0) store8_coherent(rml, uint32_t(slot * 8), u32x2{__float_as_uint(st.m), __float_as_uint(l)});
#pragma unroll
          for (int t = 0; t < T8; ++t)
            store16_coherent(racc, uint32_t((slot * D + 16 * t + 4 * grp) * 4), __builtin_bit_cast(u32x4, st.acc[t]));
        }
        if (ws_cnt != nullptr) {
          // In-kernel merge: once its stores have completed, the wave counts
          // its piece in the row's arrival counter; the arrival that
          // completes the row's K pieces resets the counter to zero (every
          // call leaves the counters as it found them) and merges the pieces.
          const int64_t start = int64_t(hsets) * s_pref[b] + int64_t(gs) * nb;
          const int64_t c0 = ch.chunk_of(start);
          const int K = int(ch.chunk_of(start + nb - 1) - c0 + 1);
          const int first_role = start > ch.start(c0) ? 1 : 0;
          int32_t* cnt = ws_cnt + int64_t(b) * hge + gh;
          wait_all_memory();
          int old = 0;
          if (lane == 0) old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          old = __builtin_amdgcn_readfirstlane(old);
          if (old == K - 1) {
            if (lane == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            merge_row_pieces<D>(out, row0, nh, HS, rml, racc, c0, first_role, K, coop, wv, lane);
          }
        }
      }
      u += j1 - j;
      if (u >= u_end) break;
      role = 1;
      j = 0;
      if (++gs == hsets) {
        gs = 0;
        do {
          ++b;
        } while (s_pref[b + 1] == s_pref[b]);
        nb = s_pref[b + 1] - s_pref[b];
      }
    }
  }
}

// ------------------------------------------------------------------------
// Ring decode: head_dim 128, batches of up to kRingMaxB requests (bf16 caches,
// with or without a window; fp8 and int8 caches without one; the bf16 layout
// is described here, the 8-bit one below).  The same work split, state and
// piece merge as decode_stream_kernel,
// with its K/V loads taken off the waves' registers: each wave keeps a ring
// of two stages in LDS (a stage is one step's K and V tiles, 16 KiB) that it
// fills with direct-to-LDS copies (global_load_lds_dwordx4: no registers, no
// VALU per byte) one stage ahead of the step it computes, across segment
// boundaries, so its next stage is in flight all through the arithmetic.
// The ring takes 128 KiB of LDS, so one workgroup (four waves) runs per CU:
// one wave per SIMD, so no issue priorities either (same box, both decode
// batches about 0.5 us faster without them).
//
// Stage layout (bytes): K of the step's blocks 0 and 1 at 0 and 4096 (16
// token rows of 256 bytes each), V at 8192 and 12288 (128 dimension rows of
// 32 bytes).  16-byte granules are placed with XOR swizzles so that the 16
// lanes of every operand read fall in 16 different LDS bank quads (the bank
// of dword address a on gfx950 is a[5:0] with a[6] XORed into bit 5): K row R
// holds dimension granule c at slot c ^ f(R), f(R) = (R & 3) | ((R >> 3) & 3)
// << 2; V dimension d holds key half h at slot h ^ ((d >> 2) & 1).
constexpr int kRingStage = 16384;                 // bytes per stage
constexpr int kRingStages = 2;                    // stages per wave
constexpr int kRingLds = 4 * kRingStages * kRingStage;  // dynamic LDS of a workgroup
constexpr int kRingMaxB = 4096;                   // batch bound of the ring decode (its block prefix is in LDS)

// Per-lane offsets of the ring's copies and operand reads.
struct RingLane {
  uint32_t koff[2][2];  // K copy source offset in a tile: [block][copy pair]; copy i adds 1024 (i & 1)
  uint32_t voff;        // V copy source offset in a tile; copy i adds 1024 i
  uint32_t krd[4];      // LDS offset (in a stage) of the lane's K operand for dimension step kk; block j adds 1024
  uint32_t vrd;         // LDS offset of the lane's V slice; dimension tile t adds 512
};

__device__ inline RingLane ring_lane(int lane) {
  RingLane L;
  const int q = lane >> 4, slot = lane & 15;
  // copy i of block be writes rows 4i + q, slots 0-15 of LDS; the granule it
  // fetches for slot s of row R is s ^ f(R), f(R) = q | (2 be + (i >> 1)) << 2
#pragma unroll
  for (int be = 0; be < 2; ++be)
#pragma unroll
    for (int h = 0; h < 2; ++h) L.koff[be][h] = 2048 * h + 256 * q + 16 * (slot ^ (q | (((2 * be + h) & 3) << 2)));
  // copy i writes dimensions 32 i + (lane >> 1), half lane & 1 of LDS
  L.voff = 32 * (lane >> 1) + 16 * ((lane & 1) ^ ((lane >> 3) & 1));
  // operands: lane (r, grp) reads token row R0 + 4 j of the step (the row
  // decode_stream_kernel's lane loads) and V dimension 16 t + r, half grp & 1
  const int r = lane & 15, grp = lane >> 4;
  const int R0 = 16 * (r >> 3) + 8 * ((r >> 2) & 1) + (r & 3);
  const int f = (r & 3) | ((2 * (r >> 3) + ((r >> 2) & 1)) << 2);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) L.krd[kk] = 256 * R0 + 16 * ((4 * kk + grp) ^ f);
  L.vrd = 8192 + 4096 * (grp >> 1) + 16 * (2 * r + ((grp & 1) ^ ((r >> 2) & 1)));
  return L;
}

// Copy the K and V tiles of kv head g in physical pages p0, p1 into a stage:
// 16 copies of 1 KiB (64 lanes x 16 bytes).
template <bool NT>
__device__ __forceinline__ void ring_issue(uint8_t* stage, const uint8_t* kc, const uint8_t* vc, int32_t p0,
                                           int32_t p1, int H, int g, const RingLane& L) {
#pragma unroll
  for (int be = 0; be < 2; ++be) {
    const int64_t tile = (int64_t(be ? p1 : p0) * H + g) * (kBS * 128 * 2);
    const uint8_t* kt = kc + tile;
    const uint8_t* vt = vc + tile;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      copy16_kv<NT>(kt + L.koff[be][i >> 1] + 1024 * (i & 1), stage + 4096 * be + 1024 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      copy16_kv<NT>(vt + L.voff + 1024 * i, stage + 8192 + 4096 * be + 1024 * i);
  }
}

// This lane's K operands and V slices of a stage.  The reads are one asm
// block that waits for them before it ends: the compiler does not see them,
// so it cannot hold them back behind every copy in flight (it would wait for
// all direct-to-LDS copies, the next stage's included, before any LDS read
// of the ring); the caller has waited for the stage's own copies.
__device__ __forceinline__ void ring_read(u32x4 (&kop)[2][4], u32x4 (&vr)[8], const uint8_t* stage,
                                          const RingLane& L) {
  const uint32_t base = uint32_t(reinterpret_cast<uintptr_t>(stage));
  const uint32_t a0 = base + L.krd[0], a1 = base + L.krd[1], a2 = base + L.krd[2], a3 = base + L.krd[3];
  const uint32_t av = base + L.vrd;
  asm volatile(
      "ds_read_b128 %0, %16\n"
      "ds_read_b128 %1, %17\n"
      "ds_read_b128 %2, %18\n"
      "ds_read_b128 %3, %19\n"
      "ds_read_b128 %4, %16 offset:1024\n"
      "ds_read_b128 %5, %17 offset:1024\n"
      "ds_read_b128 %6, %18 offset:1024\n"
      "ds_read_b128 %7, %19 offset:1024\n"
      "ds_read_b128 %8, %20\n"
      "ds_read_b128 %9, %20 offset:512\n"
      "ds_read_b128 %10, %20 offset:1024\n"
      "ds_read_b128 %11, %20 offset:1536\n"
      "ds_read_b128 %12, %20 offset:2048\n"
      "ds_read_b128 %13, %20 offset:2560\n"
      "ds_read_b128 %14, %20 offset:3072\n"
      "ds_read_b128 %15, %20 offset:3584\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kop[0][0]), "=&v"(kop[0][1]), "=&v"(kop[0][2]), "=&v"(kop[0][3]), "=&v"(kop[1][0]), "=&v"(kop[1][1]),
        "=&v"(kop[1][2]), "=&v"(kop[1][3]), "=&v"(vr[0]), "=&v"(vr[1]), "=&v"(vr[2]), "=&v"(vr[3]), "=&v"(vr[4]),
        "=&v"(vr[5]), "=&v"(vr[6]), "=&v"(vr[7])
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(av));
}

// ---- 8-bit caches (fp8, int8) on the ring.  A tile is 2 KiB of K (16 token
// rows of 128 codes) and 2 KiB of V (128 dimension rows of 16 codes), so a
// step's two blocks fill 8 KiB and a wave keeps four stages (the bytes in
// flight of the bf16 ring's two).  Stage layout: K of block 0 and 1 at 0 and
// 2048, V at 4096 and 6144, then the two blocks' (K, V) scale pairs at 8192.
// K row R of block be holds code granule c (16 codes) at slot c ^ h(R, be),
// h = ((R >> 1) & 1) | ((R >> 3) & 1) << 1 | be << 2, so that the 16 lanes of
// each operand read (rows 8 ((r >> 2) & 1) + 4 j + (r & 3) of block r >> 3)
// fall in 16 different bank quads; V reads are conflict-free as laid out.
// Copies per stage: 4 of K and 4 of V (1 KiB each), 1 of the four scales.
constexpr int kRing8Stage = 8320;                 // bytes per stage (8 KiB + scales, 128-byte aligned)
constexpr int kRing8Stages = 4;                   // stages per wave
constexpr int kRing8Lds = 4 * kRing8Stages * kRing8Stage;
constexpr int kRing8Copies = 9;                   // copy instructions per stage

struct RingLane8 {
  uint32_t koff[2][2];  // K copy source offset in a tile: [block][copy]
  uint32_t krd[2][2];   // LDS offset of the lane's K granules: [j][s] (block r >> 3)
  uint32_t vrd;         // LDS offset of the lane's V half row of dimension r (t adds 256)
  uint32_t srd;         // LDS offset of the (K, V) scales of block grp >> 1
};

__device__ inline int ring8_h(int R, int be) { return ((R >> 1) & 1) | (((R >> 3) & 1) << 1) | (be << 2); }

__device__ inline RingLane8 ring_lane8(int lane) {
  RingLane8 L;
  // copy c of block be writes rows 8 c + (lane >> 3), slot lane & 7, linearly
#pragma unroll
  for (int be = 0; be < 2; ++be)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int R = 8 * c + (lane >> 3);
      L.koff[be][c] = 128 * R + 16 * ((lane & 7) ^ ring8_h(R, be));
    }
  const int r = lane & 15, grp = lane >> 4;
  const int be = r >> 3;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int R = 8 * ((r >> 2) & 1) + 4 * j + (r & 3);
#pragma unroll
    for (int s = 0; s < 2; ++s) L.krd[j][s] = 2048 * be + 128 * R + 16 * ((2 * grp + s) ^ ring8_h(R, be));
  }
  L.vrd = 4096 + 2048 * (grp >> 1) + 16 * r + 8 * (grp & 1);
  L.srd = 8192 + 8 * (grp >> 1);
  return L;
}

// One direct-to-LDS copy of 4 bytes per active lane.
template <bool NT>
__device__ __forceinline__ void copy4_kv(const float* src, uint8_t* dst) {
  if constexpr (NT) __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 2);
  else __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
}

// Copy the K and V tiles of kv head g in physical pages p0, p1 into a stage,
// and their scales (lanes 0-3: K and V of p0, then of p1).
template <bool NT>
__device__ __forceinline__ void ring_issue8(uint8_t* stage, const uint8_t* kc, const uint8_t* vc,
                                            const float* ksc, const float* vsc, int32_t p0, int32_t p1, int H,
                                            int g, int lane, const RingLane8& L) {
#pragma unroll
  for (int be = 0; be < 2; ++be) {
    const int64_t tile = (int64_t(be ? p1 : p0) * H + g) * (kBS * 128);
#pragma unroll
    for (int c = 0; c < 2; ++c) copy16_kv<NT>(kc + tile + L.koff[be][c], stage + 2048 * be + 1024 * c);
#pragma unroll
    for (int c = 0; c < 2; ++c) copy16_kv<NT>(vc + tile + 1024 * c + 16 * lane, stage + 4096 + 2048 * be + 1024 * c);
  }
  if (lane < 4) {
    const int64_t sidx = int64_t((lane >> 1) ? p1 : p0) * H + g;
    copy4_kv<NT>(((lane & 1) ? vsc : ksc) + sidx, stage + 8192);
  }
}

// This lane's K granules, V half rows and its block's scales from a stage, in
// one asm block that waits for them (see ring_read).
__device__ __forceinline__ void ring_read8(u32x4 (&kseg)[2][2], u32x2 (&vr)[8], u32x2& sc, const uint8_t* stage,
                                           const RingLane8& L) {
  const uint32_t base = uint32_t(reinterpret_cast<uintptr_t>(stage));
  const uint32_t a0 = base + L.krd[0][0], a1 = base + L.krd[0][1], a2 = base + L.krd[1][0],
                 a3 = base + L.krd[1][1];
  const uint32_t av = base + L.vrd, as = base + L.srd;
  asm volatile(
      "ds_read_b128 %0, %13\n"
      "ds_read_b128 %1, %14\n"
      "ds_read_b128 %2, %15\n"
      "ds_read_b128 %3, %16\n"
      "ds_read_b64 %4, %17\n"
      "ds_read_b64 %5, %17 offset:256\n"
      "ds_read_b64 %6, %17 offset:512\n"
      "ds_read_b64 %7, %17 offset:768\n"
      "ds_read_b64 %8, %17 offset:1024\n"
      "ds_read_b64 %9, %17 offset:1280\n"
      "ds_read_b64 %10, %17 offset:1536\n"
      "ds_read_b64 %11, %17 offset:1792\n"
      "ds_read_b64 %12, %18\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kseg[0][0]), "=&v"(kseg[0][1]), "=&v"(kseg[1][0]), "=&v"(kseg[1][1]), "=&v"(vr[0]), "=&v"(vr[1]),
        "=&v"(vr[2]), "=&v"(vr[3]), "=&v"(vr[4]), "=&v"(vr[5]), "=&v"(vr[6]), "=&v"(vr[7]), "=&v"(sc)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(av), "v"(as));
}

// A segment of a chunk: blocks [j, j1) of request b, kv-head set gs, of which
// [j, jr1) are read from the cache (APPEND: not the request's last block when
// it holds only the new token); u is the unit of block j.
// WIN: blocks count the pages the request visits (visited_pages); visited
// page v is logical page v below a and v + off from a on.  A step never
// spans the two ranges: each range is stepped from its start (ring_pend).
// Every block of the segment is read, the one holding a fused append's new
// token included (its slot is masked; the wave writes that block's V rows).
struct RingSeg {
  int b, gs, j, j1, nb, jr1;
  int a, off;
  int64_t u;
  bool live;
};

template <bool WIN>
__device__ __forceinline__ void ring_fill(RingSeg& s, const int32_t* ctx_lens, int max_ctx, int64_t u_end, int sink,
                                          int window) {
  s.j1 = int(min<int64_t>(s.nb, s.j + (u_end - s.u)));
  s.jr1 = s.j1;
  s.a = s.nb;
  s.off = 0;
  if constexpr (WIN) {
    const VisitedPages vp = visited_pages<true>(clamp_ctx(ctx_lens, s.b, max_ctx), sink, window);
    s.a = vp.a;
    s.off = vp.c - vp.a;
  }
}

// End (visited) of the range a step starting at visited page v lies in, the
// logical page of visited page v, and the next step's start.
__device__ __forceinline__ int ring_pend(const RingSeg& s, int v) { return v < s.a ? min(s.jr1, s.a) : s.jr1; }
__device__ __forceinline__ int ring_logical(const RingSeg& s, int v) { return v < s.a ? v : v + s.off; }
__device__ __forceinline__ int ring_step_next(const RingSeg& s, int v) { return min(v + 2, ring_pend(s, v)); }

// The chunk's next segment (live false past its end).
__device__ __forceinline__ void ring_next(RingSeg& s, const int32_t* s_pref, int hsets, int64_t u_end) {
  s.u += s.j1 - s.j;
  if (s.u >= u_end) {
    s.live = false;
    return;
  }
  s.j = 0;
  if (++s.gs == hsets) {
    s.gs = 0;
    do {
      ++s.b;
    } while (s_pref[s.b + 1] == s_pref[s.b]);
    s.nb = s_pref[s.b + 1] - s_pref[s.b];
  }
}

// grid: one workgroup per CU (at most kStreamWorkers / 4), 256 threads,
// kRingLds (bf16) or kRing8Lds (fp8, int8) bytes of dynamic LDS;
// B <= kRingMaxB.  Arguments and results as decode_stream_kernel<QT, 128,
// APPEND, WIN, NT> (windows and fused appends on bf16 caches; an 8-bit fused
// append needs one kv-head group per kv head).
template <int QT, bool APPEND, bool WIN, bool NT>
__global__ void __launch_bounds__(256, 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_ring_kernel(void* __restrict__ kc_, void* __restrict__ vc_, float* __restrict__ kscale,
                   float* __restrict__ vscale, const uint16_t* __restrict__ q,
                   uint16_t* __restrict__ out, const int32_t* __restrict__ tables, int max_blocks,
                   const int32_t* __restrict__ ctx_lens, int B, int max_ctx, int H, int h_q, int G, int n_hgroups,
                   int HS, float scale_log2, int chunk_fixed, float* __restrict__ ws_ml, float* __restrict__ ws_acc,
                   int32_t* __restrict__ ws_pref, int32_t* __restrict__ ws_cnt, const uint16_t* __restrict__ k_new,
                   const uint16_t* __restrict__ v_new, const int32_t* __restrict__ new_slots, int sink,
                   int window) {
  constexpr int D = 128;
  constexpr int T8 = D / 16;
  constexpr bool Q8 = QT != kQBf16;
  // bf16: two stages of 16 KiB per wave (16 copies each); 8-bit: four of 8 KiB
  // and the scales (kRing8Copies each)
  constexpr int NST = Q8 ? kRing8Stages : kRingStages;
  constexpr int STB = Q8 ? kRing8Stage : kRingStage;
  // 8-bit with APPEND: the wave owning a request's last tile applies the
  // append's tile rule there (append8_token) before copying it, so every
  // position, the new one included, is read from the cache
  constexpr bool APPEND16 = APPEND && !Q8;
  extern __shared__ __attribute__((aligned(16))) uint8_t s_ring[];  // NST * STB bytes per wave
  __shared__ int32_t s_pref[kRingMaxB + 1];
  __shared__ int32_t s_tmp[4];
  // APPEND (bf16): the new tokens' K rows go into the cache while the block
  // counts are summed; their V slots are written with the V rows of the
  // token's block by the wave that reads it
  const int pieces = APPEND16 ? B * H * (D / 8) : 0;
  const int gthreads = gridDim.x * 256;
  int piece = blockIdx.x * 256 + threadIdx.x;
  u32x4 kx = {0, 0, 0, 0};
  int32_t pslot = -1;
  if (APPEND16 && piece < pieces) {
    pslot = new_slots[piece / (H * (D / 8))];
    kx = ld16(k_new + int64_t(piece) * 8);
  }
  block_prefix_blocks<WIN>(s_pref, s_tmp, ctx_lens, B, max_ctx, sink, window);
  if constexpr (APPEND16) {
    uint16_t* kw = static_cast<uint16_t*>(kc_);
    while (piece < pieces) {
      if (pslot >= 0) {
        const int hd = piece % (H * (D / 8));
        const int g = hd / (D / 8);
        const int d0 = 8 * (hd - g * (D / 8));
        const int64_t tile = (int64_t(pslot / kBS) * H + g) * kBS * D;
        const int off = pslot % kBS;
        *reinterpret_cast<u32x4*>(kw + tile + off * D + d0) = kx;
        // V is dimension-major, so the slot is 2 bytes in each 32-byte row:
        // such scattered partial writes cost 6 us per Llama-3-8B call.  The
        // wave that reads the request's last block writes its V rows whole
        // instead (patch_token_v, below).
      }
      piece += gthreads;
      if (piece < pieces) {
        pslot = new_slots[piece / (H * (D / 8))];
        kx = ld16(k_new + int64_t(piece) * 8);
      }
    }
  }
  if (ws_cnt == nullptr) {
    if (blockIdx.x == 0)  // the block prefix of the reduce kernel
      for (int i = threadIdx.x; i <= B; i += 256) ws_pref[i] = s_pref[i];
  } else {
    const int row8 = D / 4;
    for (int b = blockIdx.x; b < B; b += gridDim.x)
      if (s_pref[b + 1] == s_pref[b])
        for (int i = threadIdx.x; i < h_q * row8; i += 256)
          *reinterpret_cast<u32x2*>(out + (int64_t(b) * h_q * row8 + i) * 4) = u32x2{0, 0};
  }

  const int hge = H * n_hgroups;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool coop = (hge & 3) == 0;
  const int hsets = coop ? hge >> 2 : hge;
  const int64_t U = uniform64(int64_t(hsets) * s_pref[B]);
  const int W = coop ? gridDim.x : gridDim.x * 4;
  const StreamChunks ch(U, W, chunk_fixed);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int grp = lane >> 4;
  const uint8_t* kc = static_cast<const uint8_t*>(kc_);
  const uint8_t* vc = static_cast<const uint8_t*>(vc_);
  const __amdgpu_buffer_rsrc_t rml = raw_rsrc(ws_ml), racc = raw_rsrc(ws_acc);
  const RingLane Lr = ring_lane(lane);
  const RingLane8 L8 = ring_lane8(lane);
  uint8_t* ring = s_ring + wv * NST * STB;
  auto noscale = [](float&, float&) {};

  for (int64_t c = coop ? int64_t(blockIdx.x) : int64_t(blockIdx.x) * 4 + wv; c < ch.N; c += W) {
    const int64_t u0 = ch.start(c);
    const int64_t u_end = ch.end(c);
    // request holding unit u0: the last b with hsets * pref[b] <= u0
    const int64_t x = u0 / hsets;
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] <= x) lo = mid;
      else hi = mid - 1;
    }
    RingSeg cs;
    cs.b = lo;
    cs.nb = s_pref[cs.b + 1] - s_pref[cs.b];
    const int64_t rem = u0 - int64_t(hsets) * s_pref[cs.b];
    cs.gs = int(rem / cs.nb);
    cs.j = int(rem - int64_t(cs.gs) * cs.nb);
    cs.u = u0;
    cs.live = true;
    ring_fill<WIN>(cs, ctx_lens, max_ctx, u_end, sink, window);

    // The copy issuer walks the same stages as the steps below, one stage
    // ahead: a stage is blocks (icb, icb + 1) of segment `is` (the second
    // clamped to the segment's last read block, masked by the step).
    RingSeg is = cs;
    int icb = is.j;
    auto iss_skip = [&]() {  // on to the next segment with a block to read
      while (is.live && icb >= is.jr1) {
        ring_next(is, s_pref, hsets, u_end);
        if (is.live) {
          ring_fill<WIN>(is, ctx_lens, max_ctx, u_end, sink, window);
          icb = is.j;
        }
      }
    };
    iss_skip();
    int issued = 0;
    auto issue_next = [&](uint8_t* stage) {
      if (!is.live) return;
      const int32_t* trow = tables + int64_t(is.b) * max_blocks;
      const int gh = coop ? 4 * is.gs + wv : is.gs;
      const int g = gh / n_hgroups;
      const int ipe = ring_pend(is, icb);
      const int32_t p0 = trow[ring_logical(is, icb)], p1 = trow[ring_logical(is, min(icb + 1, ipe - 1))];
      if constexpr (Q8) {
        if constexpr (APPEND) {
          // the stage holding a request's last block, whose tile takes the
          // new token: apply the append's rule to the tile first (only this
          // wave reads it: one kv-head group per kv head), and let its stores
          // land before the copy reads the tile
          const int tb = is.nb - 1;
          const int32_t slot = __builtin_amdgcn_readfirstlane(new_slots[is.b]);
          if (__builtin_expect(is.j1 == is.nb && slot >= 0 && unsigned(tb - icb) < 2u, 0)) {  // rare: keep it out of line
            append8_token<D, QT == kQInt8>(static_cast<uint8_t*>(kc_), static_cast<uint8_t*>(vc_), kscale, vscale,
                                           int64_t(slot / kBS) * H + g, slot % kBS,
                                           k_new + (int64_t(is.b) * H + g) * D, v_new + (int64_t(is.b) * H + g) * D,
                                           lane);
            wait_all_memory();
          }
        }
        ring_issue8<NT>(stage, kc, vc, kscale, vscale, p0, p1, H, g, lane, L8);
      } else {
        ring_issue<NT>(stage, kc, vc, p0, p1, H, g, Lr);
      }
      ++issued;
      icb = min(icb + 2, ipe);
      iss_skip();
    };
    // one copy of issue_next's code for the first stages (its 8-bit append
    // is large, and code size costs the one-workgroup-per-CU kernel)
#pragma unroll 1
    for (int n = 0; n < NST; ++n) issue_next(ring + n * STB);

    int consumed = 0;
    int role = 0;
    while (cs.live) {
      const int b = cs.b;
      const int gh = coop ? 4 * cs.gs + wv : cs.gs;
      const int g = gh / n_hgroups;
      const int hg = gh - g * n_hgroups;
      const int head0 = g * G + hg * 16;
      const int nh = min(16, G - hg * 16);
      const int64_t row0 = int64_t(b) * h_q + head0;
      u32x4 qv[D / 32];
      const float qsi = load_q<QT, D>(qv, q, row0, r, grp, nh);
      WaveState<D> st;
#pragma unroll
      for (int t = 0; t < T8; ++t) st.acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int ctx = clamp_ctx(ctx_lens, b, max_ctx);
      const bool app = APPEND16 && new_slots[b] >= 0;
      const int ctx_c = ctx - (app ? 1 : 0);
      // the segment that ends the request adds the new token: its rows are
      // loaded now, so that the copies in flight are not waited for at the end
      const bool tok = app && cs.j1 == cs.nb;
      TokenRows<D> trw;
      if (tok) {
        const int64_t nrow = (int64_t(b) * H + g) * D;
        load_token<D>(trw, k_new + nrow, v_new + nrow, grp);
      }
      // ... and this wave writes that block's V rows with the token's values
      // in place (patch_token_v)
      const int tb = (ctx + kBS - 1) / kBS - 1;  // the request's last (logical) block
      const bool vpatch = tok;
      uint8_t* vtile = nullptr;
      if (vpatch)
        vtile = static_cast<uint8_t*>(vc_) + (int64_t(tables[int64_t(b) * max_blocks + tb]) * H + g) * (kBS * D * 2);
      const int win_lo = WIN ? max(0, ctx - window) : 0;
      for (int cbv = cs.j; cbv < cs.jr1; cbv = ring_step_next(cs, cbv), ++consumed) {
        // the step's first block and the end of its range, as logical pages
        const int cb = ring_logical(cs, cbv);
        const int pe = ring_logical(cs, ring_pend(cs, cbv) - 1) + 1;
        uint8_t* stage = ring + (consumed % NST) * STB;
        u32x4 kop[kStreamNB][D / 32];
        u32x4 vraw[T8];
        float ksc = 1.0f, vsc = 1.0f;
        if constexpr (Q8) {
          // this stage's copies have landed once at most the later stages'
          // copies are in flight (copies complete in order)
          const int later = issued - consumed - 1;
          if (later >= 3) __builtin_amdgcn_s_waitcnt(0x4F7B);       // vmcnt(27)
          else if (later == 2) __builtin_amdgcn_s_waitcnt(0x4F72);  // vmcnt(18)
          else if (later == 1) __builtin_amdgcn_s_waitcnt(0x0F79);  // vmcnt(9)
          else __builtin_amdgcn_s_waitcnt(0x0F70);                  // vmcnt(0)
          u32x4 kseg[2][2];
          u32x2 v8[T8];
          u32x2 sc;
          ring_read8(kseg, v8, sc, stage, L8);
#pragma unroll
          for (int j = 0; j < kStreamNB; ++j)
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
              const u32x4& sv = kseg[j][kk / 2];
              const u32x2 a = q8x4_to_op<QT>(sv[(kk % 2) * 2 + 0]);
              const u32x2 bq = q8x4_to_op<QT>(sv[(kk % 2) * 2 + 1]);
              kop[j][kk] = u32x4{a[0], a[1], bq[0], bq[1]};
            }
#pragma unroll
          for (int t = 0; t < T8; ++t) vraw[t] = u32x4{v8[t][0], v8[t][1], 0, 0};
          ksc = __uint_as_float(sc[0]);
          vsc = __uint_as_float(sc[1]);
        } else {
          // this stage's 16 copies have landed once at most the next stage's
          // 16 are in flight (copies complete in order)
          if (issued > consumed + 1) __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16)
          else __builtin_amdgcn_s_waitcnt(0x0F70);                       // vmcnt(0)
          ring_read(kop, vraw, stage, Lr);
        }
        issue_next(stage);  // the stage is read: the copies two stages on refill it
        if constexpr (APPEND16) {
          if (vpatch && unsigned(tb - cb) < 2u) {
            uint32_t val[T8];
            token_v_values<D>(val, trw, r);
            patch_token_v<D>(vraw, val, vtile, tb - cb, (ctx - 1) & (kBS - 1), r, grp);
          }
        }
        if constexpr (Q8)
          stream_step<QT, D, WIN>(st, kop, vraw, qv, cb, pe, ctx, scale_log2, ksc, vsc, grp, sink, win_lo, qsi,
                                    [&](float& ks, float& vs) {
                                      ks = ksc;
                                      vs = vsc;
                                    });
        else
          stream_step<kQBf16, D, WIN>(st, kop, vraw, qv, cb, pe, ctx_c, scale_log2, 1.0f, 1.0f, grp, sink, win_lo,
                                      1.0f, noscale);
      }
      if constexpr (QT == kQInt8) {  // back to true units (acc was relative to st.vs)
#pragma unroll
        for (int t = 0; t < T8; ++t) st.acc[t] *= st.vs;
      }
      if (tok) fold_token<D>(st, trw, qv, scale_log2, grp);
      const float l = wave_sum16(st.l);
      if (cs.j == 0 && cs.j1 == cs.nb) {  // the whole (b, gh): finish here
        if (r < nh) {
          const float inv = 1.0f / l;
#pragma unroll
          for (int t = 0; t < T8; ++t) {
            const f32x4 o = st.acc[t] * inv;
            const u32x2 pk = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
            *reinterpret_cast<u32x2*>(out + (row0 + r) * D + 16 * t + 4 * grp) = pk;
          }
        }
      } else {  // a piece, merged as in decode_stream_kernel
        if (r < nh) {
          const int64_t slot = (coop ? (c * 2 + role) * 4 + wv : c * 2 + role) * HS + r;
          if (grp == 0) store8_coherent(rml, uint32_t(slot * 8), u32x2{__float_as_uint(st.m), __float_as_uint(l)});
#pragma unroll
          for (int t = 0; t < T8; ++t)
            store16_coherent(racc, uint32_t((slot * D + 16 * t + 4 * grp) * 4), __builtin_bit_cast(u32x4, st.acc[t]));
        }
        if (ws_cnt != nullptr) {
          const int64_t start = int64_t(hsets) * s_pref[b] + int64_t(cs.gs) * cs.nb;
          const int64_t c0 = ch.chunk_of(start);
          const int K = int(ch.chunk_of(start + cs.nb - 1) - c0 + 1);
          const int first_role = start > ch.start(c0) ? 1 : 0;
          int32_t* cnt = ws_cnt + int64_t(b) * hge + gh;
          wait_all_memory();
          int old = 0;
          if (lane == 0) old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          old = __builtin_amdgcn_readfirstlane(old);
          if (old == K - 1) {
            if (lane == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            merge_row_pieces<D>(out, row0, nh, HS, rml, racc, c0, first_role, K, coop, wv, lane);
          }
        }
      }
      ring_next(cs, s_pref, hsets, u_end);
      if (cs.live) ring_fill<WIN>(cs, ctx_lens, max_ctx, u_end, sink, window);
      role = 1;
    }
  }
}

// Merge the pieces of one (request, query head) left by decode_stream_kernel.
// grid (h_q, B), 256 threads = (256 / (D/4)) piece lanes x D/4 dimension quads.
template <int D, bool WIN>
__global__ void __launch_bounds__(256)
stream_reduce_kernel(uint16_t* __restrict__ out, const float* __restrict__ ws_ml,
                     const float* __restrict__ ws_acc, const int32_t* __restrict__ ws_pref,
                     const int32_t* __restrict__ ctx_lens, int B, int max_ctx, int h_q, int G,
                     int n_hgroups, int H, int HS, int workers, int chunk_fixed, int sink, int window) {
  constexpr int DQ = D / 4;
  constexpr int PL = 256 / DQ;
  __shared__ float s_m[PL], s_l[PL];
  __shared__ __attribute__((aligned(16))) float s_a[PL][D];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int64_t row = int64_t(b) * h_q + h;
  // the decode kernel's block prefix holds each request's visited block count
  const int nb = ws_pref[b + 1] - ws_pref[b];
  if (nb == 0) {
    if (tid < D) out[row * D + tid] = 0;
    return;
  }
  // the decode kernel's split: units (b, set, j), sets of four pairs when
  // they divide evenly (one chunk stream per workgroup), else one pair
  const int hge = H * n_hgroups;
  const bool coop = (hge & 3) == 0;
  const int hsets = coop ? hge >> 2 : hge;
  const int streams = coop ? workers / 4 : workers;
  const int64_t U = int64_t(hsets) * ws_pref[B];
  const int g = h / G;
  const int hg = (h - g * G) / 16;
  const int hh = (h - g * G) % 16;
  const int gh = g * n_hgroups + hg;
  const int gs = coop ? gh >> 2 : gh;
  const int wv = coop ? gh & 3 : 0;
  const int64_t start = int64_t(hsets) * ws_pref[b] + int64_t(gs) * nb;
  const StreamChunks ch(U, streams, chunk_fixed);
  const int64_t c0 = ch.chunk_of(start);
  const int64_t c1 = ch.chunk_of(start + nb - 1);
  if (c0 == c1) return;  // finished inside one chunk by the decode kernel
  const int K = int(c1 - c0 + 1);
  const int first_role = start > ch.start(c0) ? 1 : 0;
  auto slot = [&](int k) -> int64_t {
    const int64_t cr = (c0 + k) * 2 + (k == 0 ? first_role : 0);
    return (coop ? cr * 4 + wv : cr) * HS + hh;
  };

  // each thread merges the pieces k = pl, pl + PL, ... in one pass, keeping a
  // running maximum and rescaling its sums when it grows; four pieces' loads
  // are in flight at a time
  const int pl = tid / DQ, dq = tid - pl * DQ;
  float M = -INFINITY, L = 0.0f;
  f32x4 A = {0.f, 0.f, 0.f, 0.f};
  int k = pl;
  for (; k + 3 * PL < K; k += 4 * PL) {
    float m4[4], l4[4];
    f32x4 a4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t s = slot(k + u * PL);
      m4[u] = ws_ml[s * 2];
      l4[u] = ws_ml[s * 2 + 1];
      a4[u] = *reinterpret_cast<const f32x4*>(ws_acc + s * D + 4 * dq);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float Mn = fmaxf(M, m4[u]);
      const float eo = __builtin_amdgcn_exp2f(M - Mn), en = __builtin_amdgcn_exp2f(m4[u] - Mn);
      L = L * eo + l4[u] * en;
      A = A * eo + a4[u] * en;
      M = Mn;
    }
  }
  for (; k < K; k += PL) {
    const int64_t s = slot(k);
    const float mp = ws_ml[s * 2];
    const float Mn = fmaxf(M, mp);
    const float eo = __builtin_amdgcn_exp2f(M - Mn), en = __builtin_amdgcn_exp2f(mp - Mn);
    L = L * eo + ws_ml[s * 2 + 1] * en;
    A = A * eo + *reinterpret_cast<const f32x4*>(ws_acc + s * D + 4 * dq) * en;
    M = Mn;
  }
  // merge the PL lanes of each dimension quad (lanes without pieces hold M = -inf)
  if (dq == 0) {  // M and L are the same for every dq of a lane
    s_m[pl] = M;
    s_l[pl] = L;
  }
  *reinterpret_cast<f32x4*>(&s_a[pl][4 * dq]) = A;
  __syncthreads();
  if (tid < D) {
    float Mx = -INFINITY;
    for (int p = 0; p < PL; ++p) Mx = fmaxf(Mx, s_m[p]);
    float a = 0.0f, l = 0.0f;
    for (int p = 0; p < PL; ++p) {
      const float e = s_m[p] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s_m[p] - Mx);
      a += e * s_a[p][tid];
      l += e * s_l[p];
    }
    out[row * D + tid] = uint16_t(f2bf_bits(a / l));
  }
}

// The same merge for batches whose rows have few pieces (the host's estimate
// is at most kNarrowPieces per row): one wave per (request, query head),
// four rows per workgroup, lane = (piece lane, dimension quad); each lane
// merges its pieces in one pass with a running maximum, then the piece lanes
// merge by shuffles.  A quarter of the workgroups and no LDS stage; with many
// pieces per row its two (D = 128) piece lanes make long chains, where the
// kernel above spreads them over eight.
template <int D, bool WIN>
__global__ void __launch_bounds__(256)
stream_reduce_rows_kernel(uint16_t* __restrict__ out, const float* __restrict__ ws_ml,
                     const float* __restrict__ ws_acc, const int32_t* __restrict__ ws_pref,
                     const int32_t* __restrict__ ctx_lens, int B, int max_ctx, int h_q, int G,
                     int n_hgroups, int H, int HS, int workers, int chunk_fixed, int sink, int window) {
  constexpr int DQ = D / 4;
  constexpr int PL = 64 / DQ;
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= int64_t(B) * h_q) return;
  const int b = int(row / h_q), h = int(row - int64_t(b) * h_q);
  const int nb = ws_pref[b + 1] - ws_pref[b];
  if (nb == 0) {
    if (lane < D / 2) reinterpret_cast<uint32_t*>(out + row * D)[lane] = 0u;  // D / 2 dwords
    return;
  }
  const int hge = H * n_hgroups;
  const bool coop = (hge & 3) == 0;
  const int hsets = coop ? hge >> 2 : hge;
  const int streams = coop ? workers / 4 : workers;
  const int64_t U = int64_t(hsets) * ws_pref[B];
  const int g = h / G;
  const int hg = (h - g * G) / 16;
  const int hh = (h - g * G) % 16;
  const int gh = g * n_hgroups + hg;
  const int gs = coop ? gh >> 2 : gh;
  const int wv = coop ? gh & 3 : 0;
  const int64_t start = int64_t(hsets) * ws_pref[b] + int64_t(gs) * nb;
  const StreamChunks ch(U, streams, chunk_fixed);
  const int64_t c0 = ch.chunk_of(start);
  const int64_t c1 = ch.chunk_of(start + nb - 1);
  if (c0 == c1) return;  // finished inside one chunk by the decode kernel
  const int K = int(c1 - c0 + 1);
  const int first_role = start > ch.start(c0) ? 1 : 0;
  auto slot = [&](int k) -> int64_t {
    const int64_t cr = (c0 + k) * 2 + (k == 0 ? first_role : 0);
    return (coop ? cr * 4 + wv : cr) * HS + hh;
  };
  const int pl = lane / DQ, dq = lane - pl * DQ;
  float M = -INFINITY, L = 0.0f;
  f32x4 A = {0.f, 0.f, 0.f, 0.f};
  int k = pl;
  for (; k + 3 * PL < K; k += 4 * PL) {
    float m4[4], l4[4];
    f32x4 a4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t s = slot(k + u * PL);
      m4[u] = ws_ml[s * 2];
      l4[u] = ws_ml[s * 2 + 1];
      a4[u] = *reinterpret_cast<const f32x4*>(ws_acc + s * D + 4 * dq);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float Mn = fmaxf(M, m4[u]);
      const float eo = __builtin_amdgcn_exp2f(M - Mn), en = __builtin_amdgcn_exp2f(m4[u] - Mn);
      L = L * eo + l4[u] * en;
      A = A * eo + a4[u] * en;
      M = Mn;
    }
  }
  for (; k < K; k += PL) {
    const int64_t s = slot(k);
    const float mp = ws_ml[s * 2];
    const float Mn = fmaxf(M, mp);
    const float eo = __builtin_amdgcn_exp2f(M - Mn), en = __builtin_amdgcn_exp2f(mp - Mn);
    L = L * eo + ws_ml[s * 2 + 1] * en;
    A = A * eo + *reinterpret_cast<const f32x4*>(ws_acc + s * D + 4 * dq) * en;
    M = Mn;
  }
  // merge the piece lanes of each dimension quad (a lane without pieces holds M = -inf)
#pragma unroll
  for (int o = DQ; o < 64; o <<= 1) {
    const float Mo = __shfl_xor(M, o), Lo = __shfl_xor(L, o);
    f32x4 Ao;
#pragma unroll
    for (int i = 0; i < 4; ++i) Ao[i] = __shfl_xor(A[i], o);
    const float Mn = fmaxf(M, Mo);
    const float e1 = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
    const float e2 = Mo == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(Mo - Mn);
    L = L * e1 + Lo * e2;
    A = A * e1 + Ao * e2;
    M = Mn;
  }
  if (pl == 0) {
    const float inv = 1.0f / L;
    const u32x2 pk = {pack_bf16(A[0] * inv, A[1] * inv), pack_bf16(A[2] * inv, A[3] * inv)};
    *reinterpret_cast<u32x2*>(out + row * D + 4 * dq) = pk;
  }
}

// ------------------------------------------------------------------------
// fp32 partition kernel (VALU).  grid (num_part, H * n_hgroups, B), 256
// threads; up to 16 query heads per workgroup; tokens in chunks of 256 with
// the same (m, l, acc) state kept in LDS.
template <int D>
__global__ void __launch_bounds__(256)
decode_f32_kernel(const float* __restrict__ kc, const float* __restrict__ vc,
                  const float* __restrict__ q, float* __restrict__ out,
                  const int32_t* __restrict__ tables, int max_blocks,
                  const int32_t* __restrict__ ctx_lens, int max_ctx, int H, int h_q, int G,
                  int n_hgroups, float scale_log2, int part_blocks, int num_part,
                  float* __restrict__ ws_ml, float* __restrict__ ws_acc) {
  constexpr int CH = 256;
  __shared__ float s_q[16][D];
  __shared__ float s_s[16][CH];
  __shared__ float s_acc[16][D];
  __shared__ float s_m[16], s_l[16], s_alpha[16];
  __shared__ int32_t s_phys[CH];

  const int p = blockIdx.x;
  const int g = blockIdx.y / n_hgroups;
  const int hg = blockIdx.y - g * n_hgroups;
  const int b = blockIdx.z;
  const int head0 = g * G + hg * 16;
  const int nh = min(16, G - hg * 16);
  const int ctx = clamp_ctx(ctx_lens, b, max_ctx);
  const int tok_begin = p * part_blocks * kBS;
  if (tok_begin >= ctx) {
    if (num_part == 1 && ctx == 0)
      for (int i = threadIdx.x; i < nh * D; i += 256)
        out[(int64_t(b) * h_q + head0 + i / D) * D + i % D] = 0.0f;
    return;
  }
  const int tok_end = min(ctx, tok_begin + part_blocks * kBS);
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int32_t* trow = tables + int64_t(b) * max_blocks;

  for (int i = tid; i < nh * D; i += 256) {
    s_q[i / D][i % D] = q[(int64_t(b) * h_q + head0 + i / D) * D + i % D];
    s_acc[i / D][i % D] = 0.0f;
  }
  if (tid < 16) {
    s_m[tid] = -INFINITY;
    s_l[tid] = 0.0f;
  }
  __syncthreads();

  for (int c0 = tok_begin; c0 < tok_end; c0 += CH) {
    const int n = min(CH, tok_end - c0);
    // scores of token c0 + tid for every head
    if (tid < n) {
      const int pos = c0 + tid;
      const int32_t phys = trow[pos / kBS];
      s_phys[tid] = phys;
      const float* krow = kc + ((int64_t(phys) * H + g) * kBS + pos % kBS) * D;
      for (int hh = 0; hh < nh; ++hh) {
        float s = 0.0f;
        for (int d = 0; d < D; ++d) s = fmaf(s_q[hh][d], krow[d], s);
        s_s[hh][tid] = s * scale_log2;
      }
    }
    __syncthreads();
    // per-head max, weights and running sum; wave w takes heads w, w+4, ...
    for (int hh = w; hh < nh; hh += 4) {
      float mx = -INFINITY;
      for (int t = lane; t < n; t += 64) mx = fmaxf(mx, s_s[hh][t]);
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      const float m_new = fmaxf(s_m[hh], mx);
      float sum = 0.0f;
      for (int t = lane; t < n; t += 64) {
        const float e = __builtin_amdgcn_exp2f(s_s[hh][t] - m_new);
        s_s[hh][t] = e;
        sum += e;
      }
      for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
      if (lane == 0) {
        const float alpha = __builtin_amdgcn_exp2f(s_m[hh] - m_new);
        s_alpha[hh] = alpha;
        s_l[hh] = s_l[hh] * alpha + sum;
        s_m[hh] = m_new;
      }
    }
    __syncthreads();
    // acc[h][d] = acc * alpha + sum_t p[h][t] V[t][d]
    for (int i = tid; i < nh * D; i += 256) {
      const int hh = i / D, d = i - hh * D;
      float a = s_acc[hh][d] * s_alpha[hh];
      for (int t = 0; t < n; ++t) {
        const int pos = c0 + t;
        a = fmaf(s_s[hh][t], vc[((int64_t(s_phys[t]) * H + g) * D + d) * kBS + pos % kBS], a);
      }
      s_acc[hh][d] = a;
    }
    __syncthreads();
  }

  for (int i = tid; i < nh * D; i += 256) {
    const int hh = i / D, d = i - hh * D;
    const int64_t row = int64_t(b) * h_q + head0 + hh;
    if (num_part == 1) {
      out[row * D + d] = s_acc[hh][d] / s_l[hh];
    } else {
      const int64_t st = row * num_part + p;
      ws_acc[st * D + d] = s_acc[hh][d];
      if (d == 0) {
        ws_ml[st * 2] = s_m[hh];
        ws_ml[st * 2 + 1] = s_l[hh];
      }
    }
  }
}

// ------------------------------------------------------------------------
// Merge the partitions of one (request, kv-head group): for each query head,
// a single pass over the partition states in index order keeps a running
// maximum M and rescales the running sums when it grows, giving
// out = sum_p acc_p 2^(m_p - M) / sum_p l_p 2^(m_p - M).
// grid (H * n_hgroups, B), 256 threads; thread i owns (head i / D, dim i % D).
template <typename OutT, int D>
__global__ void __launch_bounds__(256)
reduce_kernel(OutT* __restrict__ out, const float* __restrict__ ws_ml,
              const float* __restrict__ ws_acc, const int32_t* __restrict__ ctx_lens, int max_ctx,
              int h_q, int G, int n_hgroups, int part_tokens, int num_part) {
  const int g = blockIdx.x / n_hgroups;
  const int hg = blockIdx.x - g * n_hgroups;
  const int b = blockIdx.y;
  const int head0 = g * G + hg * 16;
  const int nh = min(16, G - hg * 16);
  const int ctx = clamp_ctx(ctx_lens, b, max_ctx);
  const int np = (ctx + part_tokens - 1) / part_tokens;
  for (int i = threadIdx.x; i < nh * D; i += 256) {
    const int hh = i / D, d = i - hh * D;
    const int64_t row = int64_t(b) * h_q + head0 + hh;
    if (np == 0) {
      out[row * D + d] = to_out<OutT>(0.0f);
      continue;
    }
    const float* ml = ws_ml + row * num_part * 2;
    const float* acc = ws_acc + row * num_part * D + d;
    float M = ml[0], L = ml[1], A = acc[0];
    int p = 1;
    for (; p + 4 <= np; p += 4) {  // four partitions' loads in flight
      float m4[4], l4[4], a4[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        m4[k] = ml[2 * (p + k)];
        l4[k] = ml[2 * (p + k) + 1];
        a4[k] = acc[int64_t(p + k) * D];
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float Mn = fmaxf(M, m4[k]);
        const float eo = __builtin_amdgcn_exp2f(M - Mn), en = __builtin_amdgcn_exp2f(m4[k] - Mn);
        L = L * eo + l4[k] * en;
        A = A * eo + a4[k] * en;
        M = Mn;
      }
    }
    for (; p < np; ++p) {
      const float mp = ml[2 * p];
      const float Mn = fmaxf(M, mp);
      const float eo = __builtin_amdgcn_exp2f(M - Mn), en = __builtin_amdgcn_exp2f(mp - Mn);
      L = L * eo + ml[2 * p + 1] * en;
      A = A * eo + acc[int64_t(p) * D] * en;
      M = Mn;
    }
    out[row * D + d] = to_out<OutT>(A / L);
  }
}


// Workgroups of the ring decode on the current device: one per compute unit
// (at most kStreamWorkers / 4, the waves the workspace is sized for); 0 when
// the device cannot be queried.
int ring_workgroups() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64 && cache[dev] > 0) return cache[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 0;
  cus = std::min(cus, kStreamWorkers / 4);
  if (dev >= 0 && dev < 64) cache[dev] = cus;
  return cus;
}

template <int D>
int launch_decode_d(const DecodeArgs& a, hipStream_t s) {
  const kv_pool_desc& d = a.pool->desc;
  const int H = d.num_kv_heads;
  const int G = a.h_q / H;
  const int nhg = (G + 15) / 16;
  const int64_t lo = int64_t(a.layer) * layer_elems(d);
  const float sl = a.scale * kLog2e;
  hipError_t e;
  if (d.cache_dtype == KV_F32) {
    const dim3 grid(a.num_part, H * nhg, a.B);
    decode_f32_kernel<D><<<grid, 256, 0, s>>>(
        static_cast<const float*>(a.pool->k_cache) + lo, static_cast<const float*>(a.pool->v_cache) + lo,
        static_cast<const float*>(a.q), static_cast<float*>(a.out), a.tables, a.max_blocks, a.ctx,
        a.max_ctx, H, a.h_q, G, nhg, sl, a.part / kBS, a.num_part, a.ws_ml, a.ws_acc);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(KV_E_HIP, "decode partition launch: %s", hipGetErrorString(e));
    if (a.num_part > 1) {
      reduce_kernel<float, D><<<dim3(H * nhg, a.B), 256, 0, s>>>(
          static_cast<float*>(a.out), a.ws_ml, a.ws_acc, a.ctx, a.max_ctx, a.h_q, G, nhg, a.part,
          a.num_part);
      e = hipGetLastError();
      if (e != hipSuccess) return fail(KV_E_HIP, "decode reduce launch: %s", hipGetErrorString(e));
    }
    return ok();
  }
  const int64_t lb = lo * elem_bytes(d.cache_dtype);
  uint8_t* kc = static_cast<uint8_t*>(a.pool->k_cache) + lb;
  uint8_t* vc = static_cast<uint8_t*>(a.pool->v_cache) + lb;
  const int64_t so = int64_t(a.layer) * d.num_blocks * H;
  // head_dim 128: the ring decode, one workgroup per CU (bf16, fp8 and int8
  // caches; windows on bf16 caches)
  const bool ring = D == 128 && a.B <= kRingMaxB && (!(a.window > 0) || d.cache_dtype == KV_BF16);
  int workers = a.workers;
  if (ring) {
    const int cus = ring_workgroups();
    if (cus <= 0) return fail(KV_E_HIP, "decode: cannot query the device's compute units");
    workers = 4 * cus;
  }
  const dim3 grid(workers / 4);
  auto* q = static_cast<const uint16_t*>(a.q);
  auto* out = static_cast<uint16_t*>(a.out);
  const bool q8 = d.cache_dtype == KV_FP8_E4M3 || d.cache_dtype == KV_INT8;
  float* ks = q8 ? a.pool->k_scale + so : nullptr;
  float* vs = q8 ? a.pool->v_scale + so : nullptr;
  const bool win = a.window > 0;
  // plain or non-temporal K/V loads (ld16_kv)
  const bool nt = a.pool->rc.shared() == 0;
  auto go = [&](auto qt, auto append, auto window) {
    constexpr int QT = decltype(qt)::value;
    constexpr bool AP = decltype(append)::value, WN = decltype(window)::value;
    if (nt)
      decode_stream_kernel<QT, D, AP, WN, true><<<grid, 256, 0, s>>>(
          kc, vc, ks, vs, q, out, a.tables, a.max_blocks, a.ctx, a.B, a.max_ctx, H, a.h_q, G, nhg, a.hs, sl,
          a.chunk, a.ws_ml, a.ws_acc, a.ws_pref, a.merge_inline ? a.ws_cnt : nullptr,
          static_cast<const uint16_t*>(a.k_new), static_cast<const uint16_t*>(a.v_new), a.new_slots, a.sink,
          a.window);
    else
      decode_stream_kernel<QT, D, AP, WN, false><<<grid, 256, 0, s>>>(
          kc, vc, ks, vs, q, out, a.tables, a.max_blocks, a.ctx, a.B, a.max_ctx, H, a.h_q, G, nhg, a.hs, sl,
          a.chunk, a.ws_ml, a.ws_acc, a.ws_pref, a.merge_inline ? a.ws_cnt : nullptr,
          static_cast<const uint16_t*>(a.k_new), static_cast<const uint16_t*>(a.v_new), a.new_slots, a.sink,
          a.window);
  };
  using F = std::false_type;
  using T = std::true_type;
  auto go_ring = [&](auto qt, auto append, auto window, auto ntc) -> int {
    constexpr int QT = decltype(qt)::value;
    constexpr bool AP = decltype(append)::value, WN = decltype(window)::value, NT = decltype(ntc)::value;
    constexpr int lds = QT == kQBf16 ? kRingLds : kRing8Lds;
    static bool lds_set = false;  // the ring's dynamic LDS is above the default bound
    if (!lds_set) {
      const hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_ring_kernel<QT, AP, WN, NT>),
                                                hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (ea != hipSuccess) return fail(KV_E_HIP, "decode: ring LDS attribute: %s", hipGetErrorString(ea));
      lds_set = true;
    }
    decode_ring_kernel<QT, AP, WN, NT><<<grid, 256, lds, s>>>(
        kc, vc, ks, vs, q, out, a.tables, a.max_blocks, a.ctx, a.B, a.max_ctx, H, a.h_q, G, nhg, a.hs, sl, a.chunk, a.ws_ml,
        a.ws_acc, a.ws_pref, a.merge_inline ? a.ws_cnt : nullptr, static_cast<const uint16_t*>(a.k_new),
        static_cast<const uint16_t*>(a.v_new), a.new_slots, a.sink, a.window);
    return ok();
  };
  using QB = std::integral_constant<int, kQBf16>;
  using QF = std::integral_constant<int, kQFp8>;
  using QI = std::integral_constant<int, kQInt8>;
  if (ring) {
    auto ring_qt = [&](auto qt, auto window) -> int {
      return a.new_slots ? (nt ? go_ring(qt, T{}, window, T{}) : go_ring(qt, T{}, window, F{}))
                         : (nt ? go_ring(qt, F{}, window, T{}) : go_ring(qt, F{}, window, F{}));
    };
    const int rc = d.cache_dtype == KV_BF16 ? (win ? ring_qt(QB{}, T{}) : ring_qt(QB{}, F{}))
                   : d.cache_dtype == KV_FP8_E4M3 ? ring_qt(QF{}, F{})
                                                  : ring_qt(QI{}, F{});
    if (rc != KV_OK) return rc;
  } else if (d.cache_dtype == KV_BF16) {
    if (a.new_slots) {  // fused append
      if (win) go(QB{}, T{}, T{});
      else go(QB{}, T{}, F{});
    } else if (win) {
      go(QB{}, F{}, T{});
    } else {
      go(QB{}, F{}, F{});
    }
  } else if (d.cache_dtype == KV_FP8_E4M3) {
    if (win) go(QF{}, F{}, T{});
    else if (a.new_slots) go(QF{}, T{}, F{});  // fused append
    else go(QF{}, F{}, F{});
  } else {
    if (win) go(QI{}, F{}, T{});
    else if (a.new_slots) go(QI{}, T{}, F{});  // fused append
    else go(QI{}, F{}, F{});
  }
  e = hipGetLastError();
  if (e != hipSuccess) return fail(KV_E_HIP, "decode launch: %s", hipGetErrorString(e));
  if (a.merge_inline) return ok();  // the decode kernel merged its pieces
  const int64_t pieces = a.pieces;
  const dim3 rows_grid(unsigned((int64_t(a.B) * a.h_q + 3) / 4));
  auto reduce = [&](auto window) {
    constexpr bool WN = decltype(window)::value;
    const int sk = WN ? a.sink : 0, wn = WN ? a.window : 0;
    if (pieces <= kNarrowPieces)
      stream_reduce_rows_kernel<D, WN><<<rows_grid, 256, 0, s>>>(out, a.ws_ml, a.ws_acc, a.ws_pref, a.ctx, a.B,
                                                                  a.max_ctx, a.h_q, G, nhg, H, a.hs, workers,
                                                                  a.chunk, sk, wn);
    else
      stream_reduce_kernel<D, WN><<<dim3(a.h_q, a.B), 256, 0, s>>>(out, a.ws_ml, a.ws_acc, a.ws_pref, a.ctx, a.B,
                                                                    a.max_ctx, a.h_q, G, nhg, H, a.hs, workers,
                                                                    a.chunk, sk, wn);
  };
  if (win) reduce(std::true_type{});
  else reduce(std::false_type{});
  e = hipGetLastError();
  if (e != hipSuccess) return fail(KV_E_HIP, "decode reduce launch: %s", hipGetErrorString(e));
  return ok();
}

// Zero n 16-byte words (the workspace's merge counters).
__global__ void __launch_bounds__(256) zero_words_kernel(u32x4* __restrict__ p, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256)
    p[i] = u32x4{0, 0, 0, 0};
}

}  // namespace

int launch_zero(void* p, int64_t bytes, hipStream_t s) {
  const int64_t n = bytes / 16;
  if (n <= 0) return ok();
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
  zero_words_kernel<<<unsigned(blocks), 256, 0, s>>>(static_cast<u32x4*>(p), n);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KV_E_HIP, "workspace init launch: %s", hipGetErrorString(e));
  return ok();
}

int launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.pool->desc.head_dim == 128) return launch_decode_d<128>(a, s);
  return launch_decode_d<64>(a, s);
}

}  // namespace pagedkv
