// Device codecs of the 8-bit caches (fp8 E4M3 and symmetric int8), shared by
// the append kernels and the decode kernel's fused append so that both
// produce the same codes bit for bit.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace pagedkv {

typedef short s16x2 __attribute__((ext_vector_type(2)));

// ----------------------------------------------------------------- fp8 ----
// OCP E4M3: bias 7, subnormals m * 2^-9, S.1111.111 = NaN, max 448.
__device__ inline float e4m3_to_float(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 24;
  const uint32_t e = (c >> 3) & 0xFu;
  const uint32_t m = c & 0x7u;
  float v;
  if (e == 0xFu && m == 0x7u) {
    v = __uint_as_float(0x7FC00000u);
  } else if (e == 0) {
    v = float(m) * 0.001953125f;  // m * 2^-9, exact
  } else {
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  }
  return __uint_as_float(__float_as_uint(v) | s);
}

// Round to nearest even, saturate to +-448, NaN -> S.1111.111, sign kept.
// NaN is handled here; every other value is clamped to +-448 (the largest
// finite code, so saturation is explicit) and converted by
// v_cvt_scalef32_pk_fp8_f32, which rounds to nearest even.  Its codes equal
// the rule's for every bf16 value, for millions of sampled fp32 values from
// the subnormal range up to 460, and at every rounding midpoint and the fp32
// values one ulp either side of it.
__device__ inline uint32_t float_to_e4m3(float y) {
  if (__builtin_isnan(y)) return ((__float_as_uint(y) >> 24) & 0x80u) | 0x7Fu;
  const float c = fminf(fmaxf(y, -448.0f), 448.0f);
  const s16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2{0, 0}, c, 0.0f, 1.0f, false);
  return uint32_t(uint16_t(r[0])) & 0xFFu;
}

// Symmetric int8: round half to even, clamp to +-127 (never -128).
__device__ inline uint32_t float_to_int8(float y) {
  const float r = fminf(fmaxf(rintf(y), -127.0f), 127.0f);
  return uint32_t(int32_t(r)) & 0xFFu;
}
__device__ inline float int8_to_float(uint32_t c) { return float(int8_t(uint8_t(c))); }

// The 8-bit codec of a cache type: largest code magnitude, encode, decode.
template <bool INT8>
struct Codec8 {
  static constexpr float kMax = INT8 ? 127.0f : 448.0f;
  __device__ static uint32_t encode(float y) { return INT8 ? float_to_int8(y) : float_to_e4m3(y); }
  __device__ static float decode(uint32_t c) { return INT8 ? int8_to_float(c) : e4m3_to_float(c); }
};


}  // namespace pagedkv
