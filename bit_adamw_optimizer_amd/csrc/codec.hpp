// codec.hpp -- device-side FP8 (OCP E4M3 / E5M2) and FP16 conversions for
// gfx950, and the per-tensor scale rule.
//
// FP8 encodings: the two formats named in TransformerEngine issue #131
// ("FP8 questions"), used for the weight gradient and the first moment by the
// MS-AMP optimization-level table. On gfx950 the hardware converts implement
// the OCP variants (E4M3 with max 448 and no Inf; E5M2 with IEEE Inf/NaN).
//
// Encoding rule (shared by every kernel): round to nearest even with
// saturation. The value is clamped to [-max, max] with v_med3 first, so that
// finite overflow and +-Inf give +-max, then converted by the hardware
// (round to nearest even, subnormals kept). NaN inputs are patched to
// 0x7F | sign afterwards by the callers that can see NaN (the quantize
// kernel); the optimizer passes only see finite values.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msamp {

enum Fp8Fmt : int { kE4M3 = 0, kE5M2 = 1 };

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <int FMT>
struct Fp8Traits;
template <>
struct Fp8Traits<kE4M3> {
  static constexpr float kMax = 448.0f;
};
template <>
struct Fp8Traits<kE5M2> {
  static constexpr float kMax = 57344.0f;
};

// Decode the two FP8 codes of one 16-bit half of a 32-bit word (HI selects
// bytes 2..3) to binary32. Exact: every FP8 value is a binary32 value.
template <int FMT, bool HI>
__device__ __forceinline__ f32x2 dec_pair(uint32_t word) {
  if constexpr (FMT == kE4M3)
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)word, HI);
  else
    return __builtin_amdgcn_cvt_pk_f32_bf8((int)word, HI);
}

// Four codes (byte k of word -> f[k]).
template <int FMT>
__device__ __forceinline__ void dec4(uint32_t word, float* f) {
  f32x2 lo = dec_pair<FMT, false>(word);
  f32x2 hi = dec_pair<FMT, true>(word);
  f[0] = lo.x;
  f[1] = lo.y;
  f[2] = hi.x;
  f[3] = hi.y;
}

// Saturating clamp to the finite range of the format.
template <int FMT>
__device__ __forceinline__ float sat(float x) {
  return __builtin_amdgcn_fmed3f(x, -Fp8Traits<FMT>::kMax, Fp8Traits<FMT>::kMax);
}

// Convert two binary32 values to FP8 codes (round to nearest even) into
// the half of 'old' selected by HI (bytes 0..1 or 2..3).
template <int FMT, bool HI>
__device__ __forceinline__ int cvt_pk(float a, float b, int old) {
  if constexpr (FMT == kE4M3)
    return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
  else
    return __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, HI);
}

// Encode four finite binary32 values (byte k <- f[k]), saturating.
template <int FMT>
__device__ __forceinline__ uint32_t enc4(const float* f) {
  int w = cvt_pk<FMT, false>(sat<FMT>(f[0]), sat<FMT>(f[1]), 0);
  w = cvt_pk<FMT, true>(sat<FMT>(f[2]), sat<FMT>(f[3]), w);
  return (uint32_t)w;
}

// Encode one value, NaN-aware: NaN -> 0x7F | sign.
template <int FMT>
__device__ __forceinline__ uint32_t enc1_nan(float x) {
  uint32_t c = (uint32_t)cvt_pk<FMT, false>(sat<FMT>(x), 0.0f, 0) & 0xFFu;
  if (__builtin_isnan(x)) c = 0x7Fu | ((__float_as_uint(x) >> 24) & 0x80u);
  return c;
}

// Encode four values, NaN-aware (used where inputs are not known finite).
template <int FMT>
__device__ __forceinline__ uint32_t enc4_nan(const float* f) {
  uint32_t w = enc4<FMT>(f);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (__builtin_isnan(f[k])) {
      uint32_t c = 0x7Fu | ((__float_as_uint(f[k]) >> 24) & 0x80u);
      w = (w & ~(0xFFu << (8 * k))) | (c << (8 * k));
    }
  }
  return w;
}

// Materializes x as a binary32 register value. The compiler would otherwise
// fold "round an fma result to binary32, then to binary16" into one mixed-
// precision fma that rounds once to binary16 (v_fma_mix*_f16), which is a
// different result whenever the binary32 rounding lands on a binary16
// midpoint. Emits no instruction.
__device__ __forceinline__ float as_f32(float x) {
  asm("" : "+v"(x));
  return x;
}

// FP16 <-> binary32 (IEEE, round to nearest even, subnormals kept).
__device__ __forceinline__ f32x2 h2_to_f2(uint32_t word) {
  f16x2 h = __builtin_bit_cast(f16x2, word);
  f32x2 r;
  r.x = (float)h.x;
  r.y = (float)h.y;
  return r;
}

__device__ __forceinline__ uint32_t f2_to_h2(float a, float b) {
  f16x2 h;
  h.x = (_Float16)as_f32(a);
  h.y = (_Float16)as_f32(b);
  return __builtin_bit_cast(uint32_t, h);
}

// Per-tensor scale rule: fmax / amax, or 1 when amax is 0 / Inf / NaN or the
// quotient is not a finite positive binary32 (correctly rounded division).
__device__ __forceinline__ float scale_rule(float amax, float fmax) {
  if (!(amax > 0.0f) || !__builtin_isfinite(amax)) return 1.0f;
  float s = fmax / amax;
  if (!__builtin_isfinite(s) || !(s > 0.0f)) return 1.0f;
  return s;
}

}  // namespace msamp
