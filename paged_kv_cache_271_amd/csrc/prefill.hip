// paged_attention_prefill: causal attention of a request's new tokens over
// its paged cache, for gfx950.
//
// What is computed ("KV cache and PagedAttention", askaiml.pages.dev, §1 "The
// setup": the prompt is processed in one big forward pass that fills the
// cache, then decode reads it; "KV Cache" glossary, inferensys.com,
// FlashAttention entry: exact attention computed in tiles so the score matrix
// never reaches HBM).  Request b's n_q new tokens are the last n_q of its ctx
// cached positions (their K/V already appended); query i (position
// ctx - n_q + i) attends to positions <= its own, every query head h reading
// kv head h / G.
//
// Work split: one workgroup (4 waves) per (query tile, request, kv head).  A
// tile is 128 rows, each a (token, query head of the group) pair: 128 / G
// tokens times the G heads, so the G heads share every K/V load.  Each wave
// holds 32 rows as two 16-row MFMA tiles, so every K and V operand read from
// LDS feeds two v_mfma_f32_16x16x32_bf16:
//   scores  S^T[key][row] = K[key][:] . Q^T[:][row]
//   output  O^T[dim][row] += V^T[dim][key] . P^T[key][row]
// Lane group q of a 32-key block owns keys 8q..8q+7, which are exactly its 8
// scores of each row, so the softmax needs no data movement.
//
// Keys stream in chunks of 32 (two pages), three workgroups per CU (three
// waves per SIMD: 164 VGPRs, 40 KiB of LDS each).  Waves 0-1 copy the K
// pages of a chunk, waves 2-3 its V pages, from HBM straight into LDS
// (global_load_lds_dwordx4, no registers) while the workgroup computes on
// the current chunk: three K buffers (K staged two chunks ahead, its copy
// kept in flight across the barrier) and two V buffers (one ahead), one
// barrier per chunk.  The copies place 16-byte granules with an XOR swizzle
// so that the MFMA operand reads of every 16 lanes touch 16 different bank
// groups.  For head_dim 128 the operand reads and MFMAs of both products are
// asm blocks that keep two reads in flight.  Softmax per chunk: the running
// row maximum only moves when a chunk's maximum exceeds it by more than 2^8
// (then the accumulators are rescaled), otherwise the weights are formed
// against the stale maximum and stay below 256, which changes no result
// beyond rounding.  The causal mask
// is applied only on the chunks that reach a row's own position, and the V
// rows past the context are zeroed in LDS on the request's last chunk
// (unwritten slots may hold any bits).  Tiles with the most keys launch
// first; the tiles of one (request, kv head) share an XCD when B * H is a
// multiple of 8, so its K/V stays in that XCD's L2.

#include <cstdint>

#include <hip/hip_runtime.h>

#include "internal.h"

namespace pagedkv {
namespace {

constexpr int kBS = kBlockSize;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRT = 2;                 // 16-row MFMA tiles per wave
constexpr int kRows = 4 * 16 * kRT;    // query rows per workgroup
constexpr int kChunk = 32;             // keys per chunk: two pages; waves 0-1 copy K, 2-3 copy V
constexpr int kKB = kChunk / 32;       // 32-key MFMA blocks per chunk
constexpr float kSlack = 8.0f;         // log2 headroom of the running maximum
// s_waitcnt immediates (vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitAll = 0x0070;       // vmcnt(0) lgkmcnt(0)
constexpr int kWaitLds = 0xC07F;       // lgkmcnt(0)
template <int N>
constexpr int kWaitVm = 0x0070 | N;     // vmcnt(N) lgkmcnt(0), N < 16
constexpr int kXcds = 8;               // workgroup ids go round-robin over the XCDs
constexpr int kPairGroup = 4;          // (request, kv head) pairs an XCD streams at a time

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 (round to nearest even) in one dword: one
// v_cvt_pk_bf16_f32.
__device__ inline uint32_t pack2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Largest of the arguments, NaN-propagating (v_maximum3_f32; the scores it
// sees are finite or -inf).
__device__ inline float max4(float a, float b, float c, float d) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), __builtin_elementwise_maximum(c, d));
}

__device__ inline f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// Barrier with no memory fence: the waits before it are explicit, so copies
// into the other buffer stay in flight across it.
template <int kWait>
__device__ inline void barrier() {
  __builtin_amdgcn_s_waitcnt(kWait);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One 16-byte piece per lane from global memory straight into LDS: lane i
// writes bytes [16 i, 16 i + 16) after the wave-uniform address `dst`.
__device__ inline void copy_to_lds(const uint16_t* src, uint16_t* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// 16-byte granule swizzles.  K buffer: key row r, dim granule g at slot
// r * (D/8) + (g ^ kswz(r)).  V buffer: page p, dim d, key half h at slot
// p * 2D + 2d + (h ^ vswz(d)).
// A ds_read_b128 serves 16 consecutive lanes per LDS cycle over 64 banks of
// 4 bytes, and on gfx950 the bank of dword address a is a[5:0] with a[6]
// XORed into bit 5 (fitted to conflict counts of read patterns on MI355X).
// For 16-byte granule G that is the bank quad (G & 15) ^ (G[4] << 3).  With
// these swizzles the 16 lanes of every K and V operand read fall in 16
// different bank quads; copies write 64 consecutive granules.
template <int D>
__device__ inline int kswz(int r) {
  const int c = ((r >> 3) & 3) * 4 + (r & 3);
  return D == 128 ? c : ((c & 7) ^ (c >> 3));
}
__device__ inline int vswz(int d) { return (d >> 2) & 1; }

template <int D>
struct Tile {
  static constexpr int KK = D / 32;   // MFMA k-steps over the head dimension
  static constexpr int T8 = D / 16;   // 16-dim output tiles
  static constexpr int PG = 2 * D;    // 16-byte granules per page tile (16 keys x D x 2 B)
  static constexpr int NI = PG / 64;  // wave copies per page tile
  u32x4 qv[kRT][KK];
  f32x4 acc[kRT][T8];
  float m[kRT], l[kRT];
  int pos[kRT];
  uint32_t kaddr[KK], vaddr;  // LDS read offsets (elements) of this lane's operands
  uint32_t csrc[NI];  // element offsets within a page tile of this lane's copies (K for waves 0-1, V for 2-3)
};

// Copy the K (or V) tiles of chunk `ci` (keys 32 ci .. 32 ci + 31): a copying
// wave takes page 2 ci + pg (pg = w for K, w - 2 for V), clamped to the
// request's last page (keys past the context are masked and, for V, zeroed
// before use).
template <int D>
__device__ __forceinline__ void issue_tiles(uint16_t* buf, const uint16_t* cache, const uint32_t (&src)[Tile<D>::NI],
                                            int ci, int nb, const int32_t* trow, int H, int g, int pg) {
  constexpr int PG = Tile<D>::PG;
  const int page = min(ci * (kChunk / kBS) + pg, nb - 1);
  const int64_t tile = (int64_t(trow[page]) * H + g) * kBS * D;
#pragma unroll
  for (int m = 0; m < Tile<D>::NI; ++m) copy_to_lds(cache + tile + src[m], buf + (pg * PG + 64 * m) * 8);
}

// Zero the V entries of keys >= ctx in a chunk buffer.
template <int D>
__device__ __forceinline__ void zero_tail(uint16_t* vbuf, int k0, int ctx, int tid) {
#pragma unroll
  for (int u = 0; u < (kChunk / kBS) * 2 * D / 256; ++u) {
    const int s = tid + 256 * u;
    const int p = s / (2 * D), rem = s % (2 * D);
    const int d = rem >> 1, h = (rem & 1) ^ vswz(d);
    const int valid = ctx - (k0 + kBS * p + 8 * h);  // keys of the granule below ctx
    if (valid < 8) {
      u32x4* ptr = reinterpret_cast<u32x4*>(vbuf + 8 * s);
      u32x4 v = *ptr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (2 * e >= valid) v[e] = 0;
        else if (2 * e + 1 >= valid) v[e] &= 0xFFFFu;
      }
      *ptr = v;
    }
  }
}

// Raw scores of a chunk: S[rt][kb][j][i] is key 32 kb + 8 qg + 4 j + i of the
// chunk against row 16 (kRT w + rt) + c (A operand row c is key
// 8 (c / 4) + 4 j + c % 4 of the block, so lane group qg gets keys 8 qg ..).
template <int D>
__device__ __forceinline__ void chunk_scores(f32x4 (&S)[kRT][kKB][2], const uint16_t* kbuf, const Tile<D>& t) {
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int j = 0; j < 2; ++j) S[rt][kb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < Tile<D>::KK; ++kk)  // eight independent accumulators per k-step
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(kbuf + (32 * kb + 4 * j) * D + t.kaddr[kk]);
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) S[rt][kb][j] = mfma(kv, t.qv[rt][kk], S[rt][kb][j]);
      }
}

// The same two products for D = 128 as asm blocks that keep two LDS operand
// reads in flight ahead of the MFMAs using a third.  At three waves per SIMD
// the compiler, short of registers, reads each operand right before its two
// MFMAs and waits for it, so every read's latency lies in the wave's path.
// Here three 16-byte buffers rotate: read i + 2 is issued as soon as the
// MFMAs of read i - 1 have taken their buffer, and `lgkmcnt(2)` waits only
// for read i (LDS reads return in order; a scalar load still outstanding
// only makes the wait stricter).  Every read completes inside its block.
// The compiler does not see the MFMAs in the blocks, so each block starts
// with 5 wait states (VALU-written operands read by the first MFMA follow
// three reads and a wait anyway) and ends with 18, more than an 8-pass
// MFMA's result needs before a VALU instruction may read it.
#define PF_MFMA_TAIL "s_nop 7\n s_nop 7\n s_nop 1\n"

// Scores: read 2 kk + j is K operand (k-step kk, keys 4 j ..), at
// LDS byte address a_kk + 1024 j; it feeds S[rt][0][j] with qv[rt][kk].
__device__ __forceinline__ void chunk_scores128(f32x4 (&S)[kRT][kKB][2], const uint16_t* kbuf, const Tile<128>& t) {
  const uint32_t base = uint32_t(reinterpret_cast<uintptr_t>(kbuf));  // LDS offset of the buffer
  const uint32_t a0 = base + 2 * t.kaddr[0], a1 = base + 2 * t.kaddr[1], a2 = base + 2 * t.kaddr[2],
                 a3 = base + 2 * t.kaddr[3];
  u32x4 r0, r1, r2;
  // %0 %1 = S[0][0][0..1], %2 %3 = S[1][0][0..1]; %4-%6 read buffers;
  // %7-%10 = qv[0][0..3], %11-%14 = qv[1][0..3]; %15-%18 = a0-a3
  asm volatile(
      "s_nop 4\n"
      "ds_read_b128 %4, %15\n"
      "ds_read_b128 %5, %15 offset:1024\n"
      "ds_read_b128 %6, %16\n"
      "s_waitcnt lgkmcnt(2)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %4, %7, 0\n"
      "v_mfma_f32_16x16x32_bf16 %2, %4, %11, 0\n"
      "ds_read_b128 %4, %16 offset:1024\n"
      "s_waitcnt lgkmcnt(2)\n"
      "v_mfma_f32_16x16x32_bf16 %1, %5, %7, 0\n"
      "v_mfma_f32_16x16x32_bf16 %3, %5, %11, 0\n"
      "ds_read_b128 %5, %17\n"
      "s_waitcnt lgkmcnt(2)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %6, %8, %0\n"
      "v_mfma_f32_16x16x32_bf16 %2, %6, %12, %2\n"
      "ds_read_b128 %6, %17 offset:1024\n"
      "s_waitcnt lgkmcnt(2)\n"
      "v_mfma_f32_16x16x32_bf16 %1, %4, %8, %1\n"
      "v_mfma_f32_16x16x32_bf16 %3, %4, %12, %3\n"
      "ds_read_b128 %4, %18\n"
      "s_waitcnt lgkmcnt(2)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %5, %9, %0\n"
      "v_mfma_f32_16x16x32_bf16 %2, %5, %13, %2\n"
      "ds_read_b128 %5, %18 offset:1024\n"
      "s_waitcnt lgkmcnt(2)\n"
      "v_mfma_f32_16x16x32_bf16 %1, %6, %9, %1\n"
      "v_mfma_f32_16x16x32_bf16 %3, %6, %13, %3\n"
      "s_waitcnt lgkmcnt(1)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %4, %10, %0\n"
      "v_mfma_f32_16x16x32_bf16 %2, %4, %14, %2\n"
      "s_waitcnt lgkmcnt(0)\n"
      "v_mfma_f32_16x16x32_bf16 %1, %5, %10, %1\n"
      "v_mfma_f32_16x16x32_bf16 %3, %5, %14, %3\n"
      PF_MFMA_TAIL
      : "=&v"(S[0][0][0]), "=&v"(S[0][0][1]), "=&v"(S[1][0][0]), "=&v"(S[1][0][1]), "=&v"(r0), "=&v"(r1),
        "=&v"(r2)
      : "v"(t.qv[0][0]), "v"(t.qv[0][1]), "v"(t.qv[0][2]), "v"(t.qv[0][3]), "v"(t.qv[1][0]), "v"(t.qv[1][1]),
        "v"(t.qv[1][2]), "v"(t.qv[1][3]), "v"(a0), "v"(a1), "v"(a2), "v"(a3)
      : "memory");
}

// PV: read t8 is the V operand of output dims 16 t8 .. (LDS byte address
// av + 512 t8); it feeds acc[rt][t8] with pop[rt][0].
__device__ __forceinline__ void chunk_pv128(Tile<128>& t, const uint16_t* vbuf, const u32x4 (&pop)[kRT][kKB]) {
  const uint32_t av = uint32_t(reinterpret_cast<uintptr_t>(vbuf)) + 2 * t.vaddr;
  u32x4 r0, r1, r2;
  // %0-%7 = acc[0][0..7], %8-%15 = acc[1][0..7]; %16-%18 read buffers;
  // %19 %20 = pop[0][0], pop[1][0]; %21 = av
  asm volatile(
      "s_nop 4\n"
      "ds_read_b128 %16, %21\n"
      "ds_read_b128 %17, %21 offset:512\n"
      "ds_read_b128 %18, %21 offset:1024\n"
      "s_waitcnt lgkmcnt(2)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %16, %19, %0\n"
      "v_mfma_f32_16x16x32_bf16 %8, %16, %20, %8\n"
      "ds_read_b128 %16, %21 offset:1536\n"
      "s_waitcnt lgkmcnt(2)\n"
      "v_mfma_f32_16x16x32_bf16 %1, %17, %19, %1\n"
      "v_mfma_f32_16x16x32_bf16 %9, %17, %20, %9\n"
      "ds_read_b128 %17, %21 offset:2048\n"
      "s_waitcnt lgkmcnt(2)\n"
      "v_mfma_f32_16x16x32_bf16 %2, %18, %19, %2\n"
      "v_mfma_f32_16x16x32_bf16 %10, %18, %20, %10\n"
      "ds_read_b128 %18, %21 offset:2560\n"
      "s_waitcnt lgkmcnt(2)\n"
      "v_mfma_f32_16x16x32_bf16 %3, %16, %19, %3\n"
      "v_mfma_f32_16x16x32_bf16 %11, %16, %20, %11\n"
      "ds_read_b128 %16, %21 offset:3072\n"
      "s_waitcnt lgkmcnt(2)\n"
      "v_mfma_f32_16x16x32_bf16 %4, %17, %19, %4\n"
      "v_mfma_f32_16x16x32_bf16 %12, %17, %20, %12\n"
      "ds_read_b128 %17, %21 offset:3584\n"
      "s_waitcnt lgkmcnt(2)\n"
      "v_mfma_f32_16x16x32_bf16 %5, %18, %19, %5\n"
      "v_mfma_f32_16x16x32_bf16 %13, %18, %20, %13\n"
      "s_waitcnt lgkmcnt(1)\n"
      "v_mfma_f32_16x16x32_bf16 %6, %16, %19, %6\n"
      "v_mfma_f32_16x16x32_bf16 %14, %16, %20, %14\n"
      "s_waitcnt lgkmcnt(0)\n"
      "v_mfma_f32_16x16x32_bf16 %7, %17, %19, %7\n"
      "v_mfma_f32_16x16x32_bf16 %15, %17, %20, %15\n"
      PF_MFMA_TAIL
      : "+v"(t.acc[0][0]), "+v"(t.acc[0][1]), "+v"(t.acc[0][2]), "+v"(t.acc[0][3]), "+v"(t.acc[0][4]),
        "+v"(t.acc[0][5]), "+v"(t.acc[0][6]), "+v"(t.acc[0][7]), "+v"(t.acc[1][0]), "+v"(t.acc[1][1]),
        "+v"(t.acc[1][2]), "+v"(t.acc[1][3]), "+v"(t.acc[1][4]), "+v"(t.acc[1][5]), "+v"(t.acc[1][6]),
        "+v"(t.acc[1][7]), "=&v"(r0), "=&v"(r1), "=&v"(r2)
      : "v"(pop[0][0]), "v"(pop[1][0]), "v"(av)
      : "memory");
}

// Step ci of the pipeline.  K of chunk ci is in k_cur (copied two steps
// ago), V of chunk ci in v_cur (one step ago).  Waves 0-1 copy K pages and
// keep the copy of K(ci + 1) in flight across the barrier; waves 2-3 copy V
// pages.  After the barrier the buffers of K(ci - 1) and V(ci - 1) are read
// no more, and the step starts the copies of K(ci + 2) and V(ci + 1) into
// them, then computes chunk ci: scores, softmax, the weighted sum of V.
template <int D>
__device__ __forceinline__ void chunk_step(Tile<D>& t, const uint16_t* k_cur, uint16_t* k_free, uint16_t* v_cur,
                                           uint16_t* v_free, int ci, int nch, int nb, int ctx, int pos_min,
                                           const int32_t* trow, const uint16_t* kc, const uint16_t* vc, int H,
                                           int g, int w, int tid, int qg, float sl) {
  constexpr int T8 = Tile<D>::T8;
  constexpr int NI = Tile<D>::NI;
  if (w < 2 && ci + 1 < nch) barrier<kWaitVm<NI>>();  // K(ci) landed; K(ci + 1) stays in flight
  else barrier<kWaitAll>();                          // K(ci) or V(ci) landed
  if (w < 2) {
    if (ci + 2 < nch) issue_tiles<D>(k_free, kc, t.csrc, ci + 2, nb, trow, H, g, w);
  } else {
    if (ci + 1 < nch) issue_tiles<D>(v_free, vc, t.csrc, ci + 1, nb, trow, H, g, w - 2);
  }
  const int k0 = ci * kChunk;
  if (k0 + kChunk > ctx) {  // the request's last chunk: no V copy is in flight
    zero_tail<D>(v_cur, k0, ctx, tid);
    barrier<kWaitLds>();
  }
  f32x4 S[kRT][kKB][2];
  if constexpr (D == 128) chunk_scores128(S, k_cur, t);
  else chunk_scores<D>(S, k_cur, t);
  // raw scores; sl > 0 is folded into the exponent below
  if (k0 + kChunk - 1 > pos_min) {  // some key of the chunk lies after some row of this wave
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = k0 + 32 * kb + 8 * qg + 4 * j + i;
            S[rt][kb][j][i] = key <= t.pos[rt] ? S[rt][kb][j][i] : -INFINITY;
          }
  }

  float mloc[kRT];  // this lane group's largest scaled score per row (log2 units)
  bool grow = false;
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        mx = __builtin_elementwise_maximum(mx, max4(S[rt][kb][j][0], S[rt][kb][j][1], S[rt][kb][j][2],
                                                    S[rt][kb][j][3]));
    mloc[rt] = mx * sl;
    grow |= mloc[rt] > t.m[rt] + kSlack;
  }
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {  // move the running maxima (rare after the first chunk)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      float mx = mloc[rt];
      mx = __builtin_elementwise_maximum(mx, __shfl_xor(mx, 16));
      mx = __builtin_elementwise_maximum(mx, __shfl_xor(mx, 32));
      const float m_new = __builtin_elementwise_maximum(t.m[rt], mx);  // finite: key 0 is visible to every row
      const float alpha = __builtin_amdgcn_exp2f(t.m[rt] - m_new);
      t.m[rt] = m_new;
      t.l[rt] *= alpha;
#pragma unroll
      for (int t8 = 0; t8 < T8; ++t8) t.acc[rt][t8] *= alpha;
    }
  }

  u32x4 pop[kRT][kKB];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    float ps = 0.0f;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
      float e[2][4];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          e[j][i] = __builtin_amdgcn_exp2f(fmaf(S[rt][kb][j][i], sl, -t.m[rt]));
          ps += e[j][i];
        }
      pop[rt][kb] = u32x4{pack2(e[0][0], e[0][1]), pack2(e[0][2], e[0][3]), pack2(e[1][0], e[1][1]),
                          pack2(e[1][2], e[1][3])};
    }
    t.l[rt] += ps;
  }
  // PV: each V operand read feeds the kRT row tiles.
  if constexpr (D == 128) {
    chunk_pv128(t, v_cur, pop);
    return;
  }
#pragma unroll
  for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
    for (int t8 = 0; t8 < T8; ++t8) {
      const u32x4 vv = *reinterpret_cast<const u32x4*>(v_cur + t.vaddr + 8 * (4 * D * kb + 32 * t8));
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) t.acc[rt][t8] = mfma(vv, pop[rt][kb], t.acc[rt][t8]);
    }
}

// grid: tiles * B * H workgroups of 256 threads, latest tiles first.
template <int D>
__global__ void __launch_bounds__(256, 3) __attribute__((amdgpu_waves_per_eu(3, 3)))
prefill_kernel(const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc, const uint16_t* __restrict__ q,
               uint16_t* __restrict__ out, const int32_t* __restrict__ tables, int max_blocks,
               const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ qstart, int B, int tiles,
               int max_ctx, int H, int h_q, int G, int tpt, float scale_log2, uint32_t q_sign) {
  using T = Tile<D>;
  constexpr int KK = T::KK, T8 = T::T8, NI = T::NI, PG = T::PG;
  __shared__ __attribute__((aligned(16))) uint16_t k_a[kChunk * D];
  __shared__ __attribute__((aligned(16))) uint16_t v_a[kChunk * D];
  __shared__ __attribute__((aligned(16))) uint16_t k_b[kChunk * D];
  __shared__ __attribute__((aligned(16))) uint16_t v_b[kChunk * D];
  __shared__ __attribute__((aligned(16))) uint16_t k_c[kChunk * D];

  // Which tile: the XCD running this workgroup (id % 8) takes the (request,
  // kv head) pairs x, x + 8, ... in groups of kPairGroup, each group's tiles
  // longest first, so the tiles in flight on one XCD read few K/V streams
  // (4 MB for four 2048-token pairs) that its L2 keeps.  Shapes where the pairs
  // do not split evenly take all tiles longest first.
  const int bh = B * H;
  const int id = int(blockIdx.x);
  int tile, pair;
  if (bh % (kXcds * kPairGroup) == 0) {
    const int x = id % kXcds, s = id / kXcds;
    const int grp = s / (tiles * kPairGroup), r = s % (tiles * kPairGroup);
    tile = tiles - 1 - r / kPairGroup;
    pair = x + kXcds * (grp * kPairGroup + r % kPairGroup);
  } else {
    tile = tiles - 1 - id / bh;
    pair = id % bh;
  }
  const int b = pair / H, g = pair % H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, qg = lane >> 4;
  const int q0 = qstart[b];
  const int n_q = qstart[b + 1] - q0;
  const int ctx = min(max(ctx_lens[b], 0), max_ctx);
  const int tok0 = tile * tpt;
  if (tok0 >= n_q) return;
  const int tok_end = min(tok0 + tpt, n_q);

  T t;
  // row rt of this lane: q / out row (q0 + tok) * h_q + head, recomputed
  // where needed rather than held through the key loop
  auto row_of = [&](int rt, int c, bool& ok) -> int64_t {
    const int row = 16 * (kRT * w + rt) + c;
    const int tl = row / G;
    ok = tl < tpt && tok0 + tl < tok_end;
    const int tok = tok0 + (ok ? tl : 0);
    return int64_t(q0 + tok) * h_q + g * G + row % G;
  };
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    bool ok;
    const int64_t qr = row_of(rt, c, ok);
    const int row = 16 * (kRT * w + rt) + c;
    const int tok = tok0 + (ok ? row / G : 0);
    t.pos[rt] = max(ctx - n_q + tok, 0);  // last key this row reads
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 v = {0, 0, 0, 0};
      if (ok) v = *reinterpret_cast<const u32x4*>(q + qr * D + 32 * kk + 8 * qg);
      t.qv[rt][kk] = v ^ q_sign;  // negated for negative scales (exact)
    }
    t.m[rt] = -INFINITY;
    t.l[rt] = 0.0f;
#pragma unroll
    for (int t8 = 0; t8 < T8; ++t8) t.acc[rt][t8] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // smallest position among this wave's rows (rows past the tile take tok0's)
  const int tl_first = (16 * kRT * w) / G, tl_last = (16 * kRT * w + 16 * kRT - 1) / G;
  const bool all_valid = tl_last < tpt && tok0 + tl_last < tok_end;
  const int pos_min = max(ctx - n_q + tok0 + (all_valid ? tl_first : 0), 0);

  // per-lane LDS read offsets (elements) and copy source offsets within a page tile
  {
    const int r = 8 * (c >> 2) + (c & 3);
    const int sw = kswz<D>(r);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) t.kaddr[kk] = r * D + 8 * ((4 * kk + qg) ^ sw);
  }
  t.vaddr = 8 * ((qg >> 1) * PG + 2 * c + ((qg & 1) ^ vswz(c)));
#pragma unroll
  for (int m = 0; m < NI; ++m) {
    const int s = 64 * m + lane;  // granule of the page tile, in LDS order
    if (w < 2) {  // K page w of a chunk: key row rl, dimension granule slot
      const int rl = s / (D / 8), slot = s % (D / 8);
      t.csrc[m] = rl * D + 8 * (slot ^ kswz<D>(kBS * w + rl));
    } else {  // V page w - 2: dimension d, key half s & 1
      const int d = s >> 1;
      t.csrc[m] = d * kBS + 8 * ((s & 1) ^ vswz(d));
    }
  }

  const int n_keys = min(ctx, max(ctx - n_q + tok_end, 0));  // keys the tile reads
  const int nch = (n_keys + kChunk - 1) / kChunk;
  const int nb = (ctx + kBS - 1) / kBS;
  const int32_t* trow = tables + int64_t(b) * max_blocks;
  if (nch > 0) {
    // K(0), K(1) (waves 0-1) and V(0) (waves 2-3) first; then steps in
    // groups of six, the period of the three K and two V buffers
    if (w < 2) {
      issue_tiles<D>(k_a, kc, t.csrc, 0, nb, trow, H, g, w);
      if (nch > 1) issue_tiles<D>(k_b, kc, t.csrc, 1, nb, trow, H, g, w);
    } else {
      issue_tiles<D>(v_a, vc, t.csrc, 0, nb, trow, H, g, w - 2);
    }
    for (int c6 = 0; c6 < nch; c6 += 6) {
#define PF_STEP(u, kcur, kfree, vcur, vfree)                                                                 \
  if (c6 + u < nch)                                                                                          \
    chunk_step<D>(t, kcur, kfree, vcur, vfree, c6 + u, nch, nb, ctx, pos_min, trow, kc, vc, H, g, w, tid, qg, \
                  scale_log2);
      PF_STEP(0, k_a, k_c, v_a, v_b)
      PF_STEP(1, k_b, k_a, v_b, v_a)
      PF_STEP(2, k_c, k_b, v_a, v_b)
      PF_STEP(3, k_a, k_c, v_b, v_a)
      PF_STEP(4, k_b, k_a, v_a, v_b)
      PF_STEP(5, k_c, k_b, v_b, v_a)
#undef PF_STEP
    }
  }


#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    float lt = t.l[rt];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    bool ok;
    // the row's lane column again, from the lane count: the compiler would
    // otherwise keep the rows' 64-bit column terms through the key loop
    const int c_end = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) & 15;
    const int64_t qr = row_of(rt, c_end, ok);
    if (ok) {
      const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
#pragma unroll
      for (int t8 = 0; t8 < T8; ++t8) {
        const f32x4 o = t.acc[rt][t8] * inv;
        const u32x2 pk = {pack2(o[0], o[1]), pack2(o[2], o[3])};
        *reinterpret_cast<u32x2*>(out + qr * D + 16 * t8 + 4 * qg) = pk;
      }
    }
  }
}

}  // namespace

int launch_prefill(const kv_pool* p, int32_t layer, void* out, const void* q, const int32_t* tables,
                   int32_t max_blocks, const int32_t* ctx, const int32_t* qstart, int32_t B, int32_t h_q,
                   int32_t max_q_len, int32_t max_ctx, float scale, hipStream_t stream) {
  const kv_pool_desc& d = p->desc;
  const int H = d.num_kv_heads;
  const int G = h_q / H;
  const int tpt = kRows / G;
  const int tiles = (max_q_len + tpt - 1) / tpt;
  if (tiles == 0 || B == 0) return ok();
  const int64_t lo = int64_t(layer) * layer_elems(d);
  const auto* kc = static_cast<const uint16_t*>(p->k_cache) + lo;
  const auto* vc = static_cast<const uint16_t*>(p->v_cache) + lo;
  const dim3 grid(uint32_t(int64_t(tiles) * B * H));
  // The kernel wants a positive score scale (it folds the scale into the
  // exponent after taking maxima of the raw scores): a negative scale negates
  // q instead, and a zero scale becomes the smallest normal float, which
  // leaves every weight 2^0 as a zero scale does.
  float sl = scale * kLog2e;
  const uint32_t q_sign = sl < 0.0f ? 0x80008000u : 0u;
  sl = sl < 0.0f ? -sl : sl;
  if (sl == 0.0f) sl = 1.17549435e-38f;
  if (d.head_dim == 128)
    prefill_kernel<128><<<grid, 256, 0, stream>>>(kc, vc, static_cast<const uint16_t*>(q), static_cast<uint16_t*>(out),
                                                  tables, max_blocks, ctx, qstart, B, tiles, max_ctx, H, h_q, G, tpt,
                                                  sl, q_sign);
  else
    prefill_kernel<64><<<grid, 256, 0, stream>>>(kc, vc, static_cast<const uint16_t*>(q), static_cast<uint16_t*>(out),
                                                 tables, max_blocks, ctx, qstart, B, tiles, max_ctx, H, h_q, G, tpt,
                                                 sl, q_sign);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KV_E_HIP, "prefill launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace pagedkv
