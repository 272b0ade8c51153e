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
// Work split: one workgroup per (request, kv head, query tile).  A tile is
// 128 rows, each a (token, query head of the group) pair: 128 / G tokens times
// the G heads, so the G heads share every K/V load.  The keys stream in chunks
// of 64 (four pages) staged through LDS by the whole workgroup; each of the
// four waves runs 32 rows (two 16-row MFMA tiles, so every K and V operand
// read from LDS serves both) with v_mfma_f32_16x16x32_bf16:
//   scores  S^T[token][row] = K[token][:] . Q^T[:][row]
//   output  O^T[dim][row]  += V^T[dim][token] . P^T[token][row]
// with the same lane layout as the decode (lane group q of a 32-token block
// owns tokens 8q..8q+7, which are exactly its 8 scores), an online softmax
// per row, and the causal mask applied per (row, token).  Tiles are issued
// latest first, so the tiles with the most keys start earliest.

#include <cstdint>

#include "internal.h"

namespace pagedkv {
namespace {

constexpr int kBS = kBlockSize;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRT = 2;                 // 16-row MFMA tiles per wave
constexpr int kRows = 4 * 16 * kRT;    // query rows per workgroup
constexpr int kChunk = 64;     // keys per staged chunk (4 pages)

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

__device__ inline uint32_t bf_bits(float x) {
  return uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(x)));  // round to nearest even
}
__device__ inline uint32_t pack2(float lo, float hi) { return bf_bits(lo) | (bf_bits(hi) << 16); }

__device__ inline f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// grid (B * tiles, H); 256 threads.  tpt = tokens per tile = kRows / G.
template <int D>
__global__ void __launch_bounds__(256)
prefill_kernel(const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc, const uint16_t* __restrict__ q,
               uint16_t* __restrict__ out, const int32_t* __restrict__ tables, int max_blocks,
               const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ qstart, int B, int tiles,
               int max_ctx, int H, int h_q, int G, int tpt, float scale_log2) {
  constexpr int KK = D / 32;     // MFMA k-steps over the head dimension
  constexpr int T8 = D / 16;     // output dim tiles
  constexpr int KS = D + 8;      // LDS row stride of K (elements), padded
  constexpr int VS = kChunk + 8; // LDS row stride of V (elements), padded
  __shared__ __attribute__((aligned(16))) uint16_t s_k[kChunk * KS];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[D * VS];

  const int b = blockIdx.x % B;
  const int tile = tiles - 1 - blockIdx.x / B;  // latest tiles first
  const int g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, qg = lane >> 4;
  const int q0 = qstart[b];
  const int n_q = qstart[b + 1] - q0;
  const int ctx = min(max(ctx_lens[b], 0), max_ctx);
  const int tok0 = tile * tpt;
  if (tok0 >= n_q) return;
  const int tok_end = min(tok0 + tpt, n_q);

  // this lane's query rows (one per row tile): (token tok0 + row / G, head row % G)
  bool valid[kRT];
  int pos[kRT];
  int64_t qrow[kRT];
  u32x4 qv[kRT][KK];
  float m[kRT], l[kRT];
  f32x4 acc[kRT][T8];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int row = 16 * (kRT * w + rt) + c;
    const int tl = row / G;
    valid[rt] = tl < tpt && tok0 + tl < tok_end;
    const int tok = tok0 + (valid[rt] ? tl : 0);
    const int head = g * G + row % G;
    pos[rt] = max(ctx - n_q + tok, 0);  // last key this row reads
    qrow[rt] = int64_t(q0 + tok) * h_q + head;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 v = {0, 0, 0, 0};
      if (valid[rt]) v = *reinterpret_cast<const u32x4*>(q + qrow[rt] * D + 32 * kk + 8 * qg);
      qv[rt][kk] = v;
    }
    m[rt] = -INFINITY;
    l[rt] = 0.0f;
#pragma unroll
    for (int t = 0; t < T8; ++t) acc[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int n_keys = min(ctx, max(ctx - n_q + tok_end, 0));  // keys the tile reads
  const int32_t* trow = tables + int64_t(b) * max_blocks;
  for (int k0 = 0; k0 < n_keys; k0 += kChunk) {
    // ---- stage four pages of K (token-major) and V (dim-major) in LDS;
    // positions at or past ctx are zeroed so stale bytes never reach a sum
    __syncthreads();
    constexpr int PC = kBS * D / 8;  // 16-byte pieces per page tile
#pragma unroll
    for (int u = 0; u < 4 * PC / 256; ++u) {
      const int k = tid + 256 * u;
      const int pg = k / PC, in = k % PC;
      const int page = k0 / kBS + pg;
      const bool live = page * kBS < n_keys;
      const int64_t tile_off = live ? (int64_t(trow[page]) * H + g) * kBS * D : 0;
      // K piece: token in / (D/8), dims 8 * (in % (D/8))
      {
        const int r = in / (D / 8), c8 = in % (D / 8);
        u32x4 v = {0, 0, 0, 0};
        if (live && page * kBS + r < ctx) v = *reinterpret_cast<const u32x4*>(kc + tile_off + r * D + 8 * c8);
        *reinterpret_cast<u32x4*>(&s_k[(pg * kBS + r) * KS + 8 * c8]) = v;
      }
      // V piece: dim in / 2, tokens 8 * (in % 2) .. + 7 of the page
      {
        const int d = in / 2, h8 = in % 2;
        u32x4 v = {0, 0, 0, 0};
        if (live) {
          v = *reinterpret_cast<const u32x4*>(vc + tile_off + d * kBS + 8 * h8);
          const int valid_t = ctx - (page * kBS + 8 * h8);  // tokens of the 8 before ctx
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (2 * e >= valid_t) v[e] = 0;
            else if (2 * e + 1 >= valid_t) v[e] &= 0xFFFFu;
          }
        }
        *reinterpret_cast<u32x4*>(&s_v[d * VS + pg * kBS + 8 * h8]) = v;
      }
    }
    __syncthreads();

    // ---- two 32-token blocks of the chunk
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (k0 + 32 * kb >= n_keys) break;
      f32x4 S[kRT][2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // A operand row c is token 8 (c / 4) + 4 j + c % 4 of the block, so
        // lane group qg ends up holding tokens 8 qg .. 8 qg + 7
        const int ktok = 32 * kb + 8 * (c >> 2) + 4 * j + (c & 3);
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) S[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const u32x4 kv = *reinterpret_cast<const u32x4*>(&s_k[ktok * KS + 32 * kk + 8 * qg]);
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt) S[rt][j] = mfma(kv, qv[rt][kk], S[rt][j]);
        }
      }
      // causal mask and online softmax per row (column c of the tiles)
      const int base = k0 + 32 * kb + 8 * qg;  // position of this lane's first token
      u32x4 pop[kRT];
      float alpha[kRT];
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float s = base + 4 * j + i <= pos[rt] ? S[rt][j][i] * scale_log2 : -INFINITY;
            S[rt][j][i] = s;
            mx = fmaxf(mx, s);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m[rt], mx);  // finite from the first block on (key 0 <= pos)
        alpha[rt] = __builtin_amdgcn_exp2f(m[rt] - m_new);
        float ps = 0.0f;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float e = __builtin_amdgcn_exp2f(S[rt][j][i] - m_new);
            S[rt][j][i] = e;
            ps += e;
          }
        l[rt] = l[rt] * alpha[rt] + ps;
        m[rt] = m_new;
        pop[rt] = u32x4{pack2(S[rt][0][0], S[rt][0][1]), pack2(S[rt][0][2], S[rt][0][3]),
                        pack2(S[rt][1][0], S[rt][1][1]), pack2(S[rt][1][2], S[rt][1][3])};
      }
#pragma unroll
      for (int t = 0; t < T8; ++t) {
        const u32x4 vv = *reinterpret_cast<const u32x4*>(&s_v[(16 * t + c) * VS + 32 * kb + 8 * qg]);
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) acc[rt][t] = mfma(vv, pop[rt], acc[rt][t] * alpha[rt]);
      }
    }
  }

#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    float lt = l[rt];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    if (valid[rt]) {
      const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
#pragma unroll
      for (int t = 0; t < T8; ++t) {
        const f32x4 o = acc[rt][t] * inv;
        const u32x2 pk = {pack2(o[0], o[1]), pack2(o[2], o[3])};
        *reinterpret_cast<u32x2*>(out + qrow[rt] * D + 16 * t + 4 * qg) = pk;
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
  const dim3 grid(uint32_t(int64_t(B) * tiles), H);
  const float sl = scale * kLog2e;
  if (d.head_dim == 128)
    prefill_kernel<128><<<grid, 256, 0, stream>>>(kc, vc, static_cast<const uint16_t*>(q), static_cast<uint16_t*>(out),
                                                  tables, max_blocks, ctx, qstart, B, tiles, max_ctx, H, h_q, G, tpt,
                                                  sl);
  else
    prefill_kernel<64><<<grid, 256, 0, stream>>>(kc, vc, static_cast<const uint16_t*>(q), static_cast<uint16_t*>(out),
                                                 tables, max_blocks, ctx, qstart, B, tiles, max_ctx, H, h_q, G, tpt,
                                                 sl);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KV_E_HIP, "prefill launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace pagedkv
