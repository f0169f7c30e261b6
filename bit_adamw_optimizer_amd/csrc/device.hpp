// device.hpp -- device-side helpers of the multi-tensor kernels
// (kernels.hip): global address-space loads and stores, workgroup max
// reductions, packed FP8/FP16 conversions of 8 elements, and the AdamW
// arithmetic of one element.
//
// The AdamW arithmetic is binary32 with exactly the operation order of the
// definition in msamp.h; files including this header are compiled with
// -ffp-contract=off so that only the explicit fmaf calls are fused.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "codec.hpp"
#include "kernels.hpp"

namespace msamp {

constexpr float kE4M3Max = 448.0f;
constexpr float kF16Max = 65504.0f;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Tensor pointers come from the descriptor table as generic pointers; they
// are global memory, and saying so lets the compiler use global (not flat)
// memory instructions.
#define GLOBAL __attribute__((address_space(1)))

template <typename T>
__device__ __forceinline__ GLOBAL T* global_ptr(void* p) {
  return (GLOBAL T*)p;
}
template <typename T>
__device__ __forceinline__ const GLOBAL T* global_ptr(const void* p) {
  return (const GLOBAL T*)p;
}

// Non-temporal loads: for streams that need not stay in any cache until
// they are read again (read once, or read again only after far more data has
// gone through the caches), so that they do not evict data that is about to
// be read again.
template <typename T>
__device__ __forceinline__ T load_stream(const GLOBAL void* p) {
  return __builtin_nontemporal_load((const GLOBAL T*)p);
}
template <typename T>
__device__ __forceinline__ T load(const GLOBAL void* p) {
  return *(const GLOBAL T*)p;
}
template <typename T>
__device__ __forceinline__ void store(GLOBAL void* p, T v) {
  *(GLOBAL T*)p = v;
}
// Non-temporal stores: for output streams nothing reads back soon.
template <typename T>
__device__ __forceinline__ void store_stream(GLOBAL void* p, T v) {
  __builtin_nontemporal_store(v, (GLOBAL T*)p);
}

__device__ __forceinline__ uint32_t abs_bits(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = umax(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// Folds m into *dst with one atomic max. The destination starts at 0 and only
// grows, so the atomic is skipped when the value already there is at least as
// large: every workgroup of a tensor targets the same word, and without this
// check ~10^5 same-address atomics per launch serialize at one L2 channel.
__device__ __forceinline__ void atomic_max_if_larger(uint32_t m, uint32_t* dst) {
  if (m != 0u && m > __hip_atomic_load(dst, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
    atomicMax(dst, m);
}

// The same, returning only once the word is known to be at least m: the
// atomic's returned value is waited for (or the coherent load already saw a
// value at least m), so a later atomic of this thread is performed after it.
__device__ __forceinline__ void atomic_max_if_larger_wait(uint32_t m, uint32_t* dst) {
  uint32_t seen = __hip_atomic_load(dst, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (m != 0u && m > seen) seen = atomicMax(dst, m);
  asm volatile("" ::"v"(seen));
}

// Largest value over a workgroup of BS threads, returned to every thread.
// The closing barrier keeps a later reduction from overwriting the LDS
// partials before every thread has read them.
template <int BS>
__device__ __forceinline__ uint32_t block_max(uint32_t v) {
  __shared__ uint32_t partial[BS / 64];
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) partial[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t m = partial[0];
#pragma unroll
  for (int k = 1; k < BS / 64; ++k) m = umax(m, partial[k]);
  __syncthreads();
  return m;
}

// One FP8 code to binary32 (exact).
template <int FMT>
__device__ __forceinline__ float dec1(uint8_t code) {
  return dec_pair<FMT, false>((uint32_t)code).x;
}

// Eight FP8 codes (two words) to binary32.
template <int FMT>
__device__ __forceinline__ void dec8(const u32x2& q, float* f) {
  dec4<FMT>(q.x, f);
  dec4<FMT>(q.y, f + 4);
}

// Eight binary32 values to FP8 codes (finite inputs, saturating).
template <int FMT>
__device__ __forceinline__ u32x2 enc8(const float* f) {
  u32x2 r;
  r.x = enc4<FMT>(f);
  r.y = enc4<FMT>(f + 4);
  return r;
}

// One finite binary32 value to an E4M3 code (saturating).
__device__ __forceinline__ uint8_t enc1_e4m3(float x) {
  float mm[4] = {x, 0.0f, 0.0f, 0.0f};
  return (uint8_t)(enc4<kE4M3>(mm) & 0xFFu);
}

__device__ __forceinline__ void h8_to_f8(const u32x4& h, float* f) {
  f32x2 a = h2_to_f2(h.x), b = h2_to_f2(h.y), c = h2_to_f2(h.z), d = h2_to_f2(h.w);
  f[0] = a.x; f[1] = a.y; f[2] = b.x; f[3] = b.y;
  f[4] = c.x; f[5] = c.y; f[6] = d.x; f[7] = d.y;
}

__device__ __forceinline__ u32x4 f8_to_h8(const float* f) {
  u32x4 r;
  r.x = f2_to_h2(f[0], f[1]);
  r.y = f2_to_h2(f[2], f[3]);
  r.z = f2_to_h2(f[4], f[5]);
  r.w = f2_to_h2(f[6], f[7]);
  return r;
}

__device__ __forceinline__ float h_to_f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ uint16_t f_to_h(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)as_f32(f));
}

// Largest FP16 magnitude of eight packed FP16 values (their bits), as the
// FP16 bit pattern of the magnitude.
__device__ __forceinline__ uint32_t h8_absmax_bits(const u32x4& h) {
  const uint32_t ws[4] = {h.x, h.y, h.z, h.w};
  uint32_t m = 0u;
#pragma unroll
  for (int k = 0; k < 4; ++k) m = umax(m, umax(ws[k] & 0x7FFFu, (ws[k] >> 16) & 0x7FFFu));
  return m;
}

// ----------------------------------------------------- AdamW arithmetic ---

// m1 = beta1*m0 + (1-beta1)*g with one fused multiply-add.
__device__ __forceinline__ float first_moment(const StepConsts& k, float g, float m0) {
  return __builtin_fmaf(k.b1, m0, k.ob1 * g);
}

// The gradient the moments see: g for AdamW; g + wd*w0 (one fused
// multiply-add) for Adam's coupled L2 term.
template <bool COUPLED>
__device__ __forceinline__ float effective_grad(const StepConsts& k, float g, float w0) {
  return COUPLED ? __builtin_fmaf(k.wd, w0, g) : g;
}

// v1, den and w1 (see the AdamW definition in msamp.h).
__device__ __forceinline__ void second_moment_and_weight(const StepConsts& k, float g, float m1,
                                                         float v0, float w0, float& v1,
                                                         float& w1) {
  v1 = __builtin_fmaf(k.b2, v0, k.ob2 * (g * g));
  const float den = __builtin_fmaf(__builtin_sqrtf(v1), k.ibs, k.eps);
  w1 = __builtin_fmaf(-k.ss, m1 / den, w0 * k.dec);
}

}  // namespace msamp
