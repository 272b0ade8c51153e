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
// Work split: the context of each request is cut into partitions of `part`
// tokens.  One workgroup handles one (partition, kv-head, request) and keeps,
// per query head, the running max m (in log2 units), the sum l of
// exp2(s - m) and the weighted sum acc of V.  With one partition the
// workgroup writes the output directly; otherwise it stores (m, l, acc) and
// `reduce_kernel` merges the partitions by rescaling to the common maximum.
//
// bf16 / fp8 caches use MFMA (v_mfma_f32_16x16x32_bf16).  A wave handles four
// 16-token blocks per step; lane group q = lane/16 owns block q of the four.
//   scores  S^T[token][head] = K[token][:] . Q^T[:][head]   (4 MFMA row groups
//           j = 0..3, row 4q+i <-> block q, token 4j+i; D/32 k-steps)
//   output  O^T[dim][head] += V^T[dim][token] . P^T[token][head]
//           (the dim-major V tile gives each lane 8 consecutive tokens of one
//           dimension in one 16-byte load; the k-slots of lane group q are
//           block q's tokens 8h..8h+7, exactly the scores that lane holds)
// so scores never cross lanes except for the per-head max and sum.  Padding
// columns (heads beyond the group) carry zero queries and are not stored.
// fp8 codes are widened to bf16 exactly (every E4M3 value is a bf16 value);
// the K scale multiplies the scores and the V scale multiplies p.

#include <cstdint>

#include "internal.h"

namespace pagedkv {
namespace {

constexpr int kBS = kBlockSize;
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

__device__ inline u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ inline uint32_t f2bf_bits(float x) {
  const __bf16 h = static_cast<__bf16>(x);  // round to nearest even
  return uint32_t(__builtin_bit_cast(uint16_t, h));
}

__device__ inline uint32_t pack_bf16(float lo, float hi) { return f2bf_bits(lo) | (f2bf_bits(hi) << 16); }

// Four E4M3 codes (one dword) -> four bf16 (two dwords), exact.
__device__ inline u32x2 fp8x4_to_bf16x4(uint32_t w) {
  const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  u32x2 r;
  r[0] = __builtin_bit_cast(uint32_t, lo);
  r[1] = __builtin_bit_cast(uint32_t, hi);
  return r;
}

// Zero the 16-bit elements e >= valid (0 <= valid <= 8) of an 8-element vector.
__device__ inline u32x4 mask_tail(u32x4 v, int valid) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (2 * w >= valid) v[w] = 0;
    else if (2 * w + 1 >= valid) v[w] &= 0xFFFFu;
  }
  return v;
}

__device__ inline float wave_max16(float x) {  // over lanes r, r+16, r+32, r+48
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ inline float wave_sum16(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

template <typename OutT>
__device__ inline OutT to_out(float x);
template <>
__device__ inline float to_out<float>(float x) { return x; }
template <>
__device__ inline uint16_t to_out<uint16_t>(float x) { return uint16_t(f2bf_bits(x)); }

// ------------------------------------------------------------------------
// MFMA partition kernel for bf16 and fp8 caches (queries and output bf16).
// grid (num_part, H * n_hgroups, B), 256 threads (4 waves).
template <bool FP8, int D>
__global__ void __launch_bounds__(256, 2)
decode_mfma_kernel(const void* __restrict__ kc_, const void* __restrict__ vc_,
                   const float* __restrict__ kscale, const float* __restrict__ vscale,
                   const uint16_t* __restrict__ q, uint16_t* __restrict__ out,
                   const int32_t* __restrict__ tables, int max_blocks,
                   const int32_t* __restrict__ ctx_lens, int H, int h_q, int G, int n_hgroups,
                   float scale_log2, int part_blocks, int num_part, float* __restrict__ ws_ml,
                   float* __restrict__ ws_acc) {
  constexpr int KK = D / 32;  // k-steps of the score MFMA
  constexpr int T8 = D / 16;  // 16-dim tiles of the output
  constexpr int EB = FP8 ? 1 : 2;
  constexpr int DP = D + 4;   // padded LDS row
  __shared__ float s_m[4][16], s_l[4][16];
  __shared__ __attribute__((aligned(16))) float s_acc[4][16][DP];

  const int p = blockIdx.x;
  const int g = blockIdx.y / n_hgroups;
  const int hg = blockIdx.y - g * n_hgroups;
  const int b = blockIdx.z;
  const int head0 = g * G + hg * 16;
  const int nh = min(16, G - hg * 16);
  const int ctx = ctx_lens[b];
  const int nblk = (ctx + kBS - 1) / kBS;
  const int blk_begin = p * part_blocks;
  if (blk_begin >= nblk) {
    if (num_part == 1 && ctx == 0)
      for (int i = threadIdx.x; i < nh * D; i += 256)
        out[(int64_t(b) * h_q + head0 + i / D) * D + i % D] = 0;
    return;
  }
  const int blk_end = min(nblk, blk_begin + part_blocks);

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int r = lane & 15;
  const int grp = lane >> 4;

  // query operand: column r = head head0 + r; k-slots of lane group grp
  bf16x8 qv[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const int dim0 = FP8 ? (D / 4) * grp + 8 * kk : 32 * kk + 8 * grp;
    u32x4 v = {0, 0, 0, 0};
    if (r < nh) v = ld16(q + (int64_t(b) * h_q + head0 + r) * D + dim0);
    qv[kk] = __builtin_bit_cast(bf16x8, v);
  }

  const uint8_t* kc = static_cast<const uint8_t*>(kc_);
  const uint8_t* vc = static_cast<const uint8_t*>(vc_);
  const int32_t* trow = tables + int64_t(b) * max_blocks;
  const int64_t tile_bytes = int64_t(kBS) * D * EB;

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 acc[T8];
#pragma unroll
  for (int t = 0; t < T8; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nb = blk_end - blk_begin;
  for (int c = w; c * 4 < nb; c += 4) {
    const int cb = blk_begin + c * 4;
    const int bK = cb + (r >> 2);  // block feeding this lane's K row
    const int bV = cb + grp;       // block whose scores / V this lane owns
    const bool vK = bK < blk_end;
    const bool vV = bV < blk_end;
    const int64_t pK = vK ? trow[bK] : 0;
    const int64_t pV = vV ? trow[bV] : 0;
    const uint8_t* ktile = kc + (pK * H + g) * tile_bytes;
    const uint8_t* vtile = vc + (pV * H + g) * tile_bytes;

    // ---- loads: K rows (token 4j + r%4 of block bK), V rows (dims of block bV)
    bf16x8 kop[4][KK];
    u32x4 vraw[T8][FP8 ? 1 : 2];
    if constexpr (!FP8) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          u32x4 v = {0, 0, 0, 0};
          if (vK) v = ld16(ktile + ((4 * j + (r & 3)) * D + 32 * kk + 8 * grp) * 2);
          kop[j][kk] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
      for (int t = 0; t < T8; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          u32x4 v = {0, 0, 0, 0};
          if (vV) v = ld16(vtile + ((16 * t + r) * kBS + 8 * h) * 2);
          vraw[t][h] = v;
        }
    } else {
      constexpr int NSEG = D / 64;  // 16-byte pieces of a lane's D/4 codes
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 seg[NSEG];
#pragma unroll
        for (int s = 0; s < NSEG; ++s) {
          seg[s] = u32x4{0, 0, 0, 0};
          if (vK) seg[s] = ld16(ktile + (4 * j + (r & 3)) * D + (D / 4) * grp + 16 * s);
        }
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const u32x4& sv = seg[kk / 2];
          const u32x2 a = fp8x4_to_bf16x4(sv[(kk % 2) * 2 + 0]);
          const u32x2 bq = fp8x4_to_bf16x4(sv[(kk % 2) * 2 + 1]);
          kop[j][kk] = __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], bq[0], bq[1]});
        }
      }
#pragma unroll
      for (int t = 0; t < T8; ++t) {
        u32x4 v = {0, 0, 0, 0};
        if (vV) v = ld16(vtile + (16 * t + r) * kBS);
        vraw[t][0] = v;
      }
    }

    // ---- scores
    f32x4 S[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      S[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        S[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[j][kk], qv[kk], S[j], 0, 0, 0);
    }

    // ---- online softmax over this step's 64 tokens
    float kfac = scale_log2;
    float vfac = 1.0f;
    if constexpr (FP8) {
      if (vV) {
        kfac *= kscale[pV * H + g];
        vfac = vscale[pV * H + g];
      }
    }
    const int tok0 = bV * kBS;
    const int valid = vV ? min(kBS, ctx - tok0) : 0;  // valid tokens of block bV
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s = (4 * j + i < valid) ? S[j][i] * kfac : -INFINITY;
        S[j][i] = s;
        mx = fmaxf(mx, s);
      }
    mx = wave_max16(mx);
    const float m_new = fmaxf(m_run, mx);  // finite: the step holds a valid token
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = __builtin_amdgcn_exp2f(S[j][i] - m_new);
        S[j][i] = e;
        psum += e;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < T8; ++t) acc[t] *= alpha;

    // ---- weighted sum of V
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 lo = S[2 * h] * vfac, hi = S[2 * h + 1] * vfac;
      const u32x4 pw = {pack_bf16(lo[0], lo[1]), pack_bf16(lo[2], lo[3]), pack_bf16(hi[0], hi[1]),
                        pack_bf16(hi[2], hi[3])};
      const bf16x8 pop = __builtin_bit_cast(bf16x8, pw);
      const int vh = min(max(valid - 8 * h, 0), 8);  // valid tokens among 8h..8h+7
#pragma unroll
      for (int t = 0; t < T8; ++t) {
        u32x4 v;
        if constexpr (FP8) {
          const u32x2 a = fp8x4_to_bf16x4(vraw[t][0][2 * h]);
          const u32x2 c2 = fp8x4_to_bf16x4(vraw[t][0][2 * h + 1]);
          v = u32x4{a[0], a[1], c2[0], c2[1]};
        } else {
          v = vraw[t][h];
        }
        if (vh < 8) v = mask_tail(v, vh);  // stale or poisoned slots past the context
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), pop, acc[t], 0, 0, 0);
      }
    }
  }

  // ---- merge the four waves of the workgroup
  l_run = wave_sum16(l_run);
  if (grp == 0) {
    s_m[w][r] = m_run;
    s_l[w][r] = l_run;
  }
#pragma unroll
  for (int t = 0; t < T8; ++t) *reinterpret_cast<f32x4*>(&s_acc[w][r][16 * t + 4 * grp]) = acc[t];
  __syncthreads();
  for (int i = threadIdx.x; i < nh * D; i += 256) {
    const int hh = i / D, d = i - hh * D;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < 4; ++k) M = fmaxf(M, s_m[k][hh]);
    float L = 0.0f, A = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float e = __builtin_amdgcn_exp2f(s_m[k][hh] - M);  // 0 for idle waves
      L += e * s_l[k][hh];
      A += e * s_acc[k][hh][d];
    }
    const int64_t row = int64_t(b) * h_q + head0 + hh;
    if (num_part == 1) {
      out[row * D + d] = uint16_t(f2bf_bits(A / L));
    } else {
      const int64_t st = row * num_part + p;
      ws_acc[st * D + d] = A;
      if (d == 0) {
        ws_ml[st * 2] = M;
        ws_ml[st * 2 + 1] = L;
      }
    }
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
                  const int32_t* __restrict__ ctx_lens, int H, int h_q, int G, int n_hgroups,
                  float scale_log2, int part_blocks, int num_part, float* __restrict__ ws_ml,
                  float* __restrict__ ws_acc) {
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
  const int ctx = ctx_lens[b];
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
// Merge the partitions of one (request, query head): M = max m_p,
// L = sum l_p 2^(m_p - M), out = sum acc_p 2^(m_p - M) / L.  grid (h_q, B),
// D threads, thread d owns output dimension d.
template <typename OutT, int D>
__global__ void __launch_bounds__(D)
reduce_kernel(OutT* __restrict__ out, const float* __restrict__ ws_ml,
              const float* __restrict__ ws_acc, const int32_t* __restrict__ ctx_lens, int h_q,
              int part_tokens, int num_part) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int ctx = ctx_lens[b];
  const int np = (ctx + part_tokens - 1) / part_tokens;
  const int64_t row = int64_t(b) * h_q + h;
  if (np == 0) {
    out[row * D + d] = to_out<OutT>(0.0f);
    return;
  }
  const float* ml = ws_ml + row * num_part * 2;
  const float* acc = ws_acc + row * num_part * D + d;
  float M = -INFINITY;
  for (int p = 0; p < np; ++p) M = fmaxf(M, ml[2 * p]);
  float L = 0.0f, A = 0.0f;
  for (int p = 0; p < np; ++p) {
    const float e = __builtin_amdgcn_exp2f(ml[2 * p] - M);
    L += e * ml[2 * p + 1];
    A += e * acc[int64_t(p) * D];
  }
  out[row * D + d] = to_out<OutT>(A / L);
}

template <int D>
int launch_decode_d(const DecodeArgs& a, hipStream_t s) {
  const kv_pool_desc& d = a.pool->desc;
  const int H = d.num_kv_heads;
  const int G = a.h_q / H;
  const int nhg = (G + 15) / 16;
  const int part_blocks = a.part / kBS;
  const int64_t lo = int64_t(a.layer) * layer_elems(d);
  const float sl = a.scale * kLog2e;
  const dim3 grid(a.num_part, H * nhg, a.B);
  if (d.cache_dtype == KV_F32) {
    decode_f32_kernel<D><<<grid, 256, 0, s>>>(
        static_cast<const float*>(a.pool->k_cache) + lo, static_cast<const float*>(a.pool->v_cache) + lo,
        static_cast<const float*>(a.q), static_cast<float*>(a.out), a.tables, a.max_blocks, a.ctx, H,
        a.h_q, G, nhg, sl, part_blocks, a.num_part, a.ws_ml, a.ws_acc);
  } else {
    const int64_t lb = lo * elem_bytes(d.cache_dtype);
    const uint8_t* kc = static_cast<const uint8_t*>(a.pool->k_cache) + lb;
    const uint8_t* vc = static_cast<const uint8_t*>(a.pool->v_cache) + lb;
    const int64_t so = int64_t(a.layer) * d.num_blocks * H;
    if (d.cache_dtype == KV_BF16)
      decode_mfma_kernel<false, D><<<grid, 256, 0, s>>>(
          kc, vc, nullptr, nullptr, static_cast<const uint16_t*>(a.q), static_cast<uint16_t*>(a.out),
          a.tables, a.max_blocks, a.ctx, H, a.h_q, G, nhg, sl, part_blocks, a.num_part, a.ws_ml,
          a.ws_acc);
    else
      decode_mfma_kernel<true, D><<<grid, 256, 0, s>>>(
          kc, vc, a.pool->k_scale + so, a.pool->v_scale + so, static_cast<const uint16_t*>(a.q),
          static_cast<uint16_t*>(a.out), a.tables, a.max_blocks, a.ctx, H, a.h_q, G, nhg, sl,
          part_blocks, a.num_part, a.ws_ml, a.ws_acc);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KV_E_HIP, "decode partition launch: %s", hipGetErrorString(e));
  if (a.num_part > 1) {
    const dim3 rg(a.h_q, a.B);
    if (d.cache_dtype == KV_F32)
      reduce_kernel<float, D><<<rg, D, 0, s>>>(static_cast<float*>(a.out), a.ws_ml, a.ws_acc, a.ctx,
                                               a.h_q, a.part, a.num_part);
    else
      reduce_kernel<uint16_t, D><<<rg, D, 0, s>>>(static_cast<uint16_t*>(a.out), a.ws_ml, a.ws_acc,
                                                  a.ctx, a.h_q, a.part, a.num_part);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(KV_E_HIP, "decode reduce launch: %s", hipGetErrorString(e));
  }
  return ok();
}

}  // namespace

int launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.pool->desc.head_dim == 128) return launch_decode_d<128>(a, s);
  return launch_decode_d<64>(a, s);
}

}  // namespace pagedkv
