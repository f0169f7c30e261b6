// kernels.hip -- HIP kernels for gfx950 (MI355X): per-tensor amax, FP8
// quantize / dequantize, and the two- and three-pass low-precision AdamW step
// of the MS-AMP O2 and O3 layouts ("Optimization Level" page, sections O2 and
// O3 and the optimization-level table).
//
// All kernels are multi-tensor-apply launches: workgroup b takes ChunkRef b
// (tensor t, chunk j) and covers elements [j*kChunk, min(numel, (j+1)*kChunk))
// of tensor t through the 64-byte TensorDesc of t. Inside a chunk every
// thread owns kVec = 16 consecutive elements per tile, so the FP8 streams are
// moved with one 16-byte access per thread, the FP16 streams with two and
// the FP32 streams with four; a ragged end of a tensor is handled element by
// element. The work is bound by HBM bandwidth: no matrix cores are involved.
//
// Arithmetic is binary32 with the operation order of the AdamW definition in
// msamp.h; the file is compiled with -ffp-contract=off so that only the
// explicit fmaf calls are fused.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "codec.hpp"
#include "kernels.hpp"

namespace msamp {
namespace {

constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ uint32_t abs_bits(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Largest value of the workgroup, folded into *dst with one atomic max (only
// when it is nonzero: the destination starts at 0).
__device__ __forceinline__ void block_max_into(uint32_t v, uint32_t* dst) {
  __shared__ uint32_t partial[kBlock / 64];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = umax(v, (uint32_t)__shfl_xor((int)v, off, 64));
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (lane == 0) partial[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = partial[0];
#pragma unroll
    for (int k = 1; k < kBlock / 64; ++k) m = umax(m, partial[k]);
    if (m != 0u) atomicMax(dst, m);
  }
}

// One FP8 code to binary32 (exact).
template <int FMT>
__device__ __forceinline__ float dec1(uint8_t code) {
  return dec_pair<FMT, false>((uint32_t)code).x;
}

template <int FMT>
__device__ __forceinline__ void dec16(const uint4& q, float* f) {
  dec4<FMT>(q.x, f);
  dec4<FMT>(q.y, f + 4);
  dec4<FMT>(q.z, f + 8);
  dec4<FMT>(q.w, f + 12);
}

__device__ __forceinline__ void h8_to_f8(const uint4& h, float* f) {
  f32x2 a = h2_to_f2(h.x), b = h2_to_f2(h.y), c = h2_to_f2(h.z), d = h2_to_f2(h.w);
  f[0] = a.x; f[1] = a.y; f[2] = b.x; f[3] = b.y;
  f[4] = c.x; f[5] = c.y; f[6] = d.x; f[7] = d.y;
}

__device__ __forceinline__ uint4 f8_to_h8(const float* f) {
  uint4 r;
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

struct ChunkRange {
  int t;
  int64_t begin, end;
};

__device__ __forceinline__ ChunkRange chunk_range(const ChunkRef* chunks, const TensorDesc* desc) {
  const ChunkRef c = chunks[blockIdx.x];
  ChunkRange r;
  r.t = c.tensor;
  r.begin = (int64_t)c.chunk * kChunk;
  const int64_t n = desc[c.tensor].numel;
  r.end = r.begin + kChunk < n ? r.begin + kChunk : n;
  return r;
}

// ---------------------------------------------------------------- amax ---

__global__ __launch_bounds__(kBlock) void k_amax(const TensorDesc* __restrict__ desc,
                                                 const ChunkRef* __restrict__ chunks,
                                                 uint32_t* __restrict__ scratch) {
  const ChunkRange r = chunk_range(chunks, desc);
  const float* __restrict__ x = (const float*)desc[r.t].p0;
  uint32_t m = 0u;
  for (int64_t i = r.begin + (int64_t)threadIdx.x * kVec; i < r.end; i += kTile) {
    if (i + kVec <= r.end) {
      const uint4* p = (const uint4*)(x + i);
      uint4 a = p[0], b = p[1], c = p[2], d = p[3];
      uint32_t u[16] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w,
                        c.x, c.y, c.z, c.w, d.x, d.y, d.z, d.w};
#pragma unroll
      for (int k = 0; k < 16; ++k) m = umax(m, u[k] & 0x7FFFFFFFu);
    } else {
      for (int64_t e = i; e < r.end; ++e) m = umax(m, abs_bits(x[e]));
    }
  }
  block_max_into(m, &scratch[r.t]);
}

__global__ __launch_bounds__(kBlock) void k_amax_finalize(int32_t n, uint32_t* __restrict__ scratch,
                                                          msamp_meta* __restrict__ meta) {
  const int32_t t = blockIdx.x * kBlock + threadIdx.x;
  if (t >= n) return;
  meta[t].amax = __uint_as_float(scratch[t]);
  scratch[t] = 0u;
}

// ------------------------------------------------------------ quantize ---

template <int FMT>
__global__ __launch_bounds__(kBlock) void k_quantize(const TensorDesc* __restrict__ desc,
                                                     const ChunkRef* __restrict__ chunks,
                                                     msamp_meta* __restrict__ meta) {
  const ChunkRange r = chunk_range(chunks, desc);
  const float s = scale_rule(meta[r.t].amax, Fp8Traits<FMT>::kMax);
  if (chunks[blockIdx.x].chunk == 0 && threadIdx.x == 0) {
    meta[r.t].scale = s;
    meta[r.t].scale_inv = 1.0f / s;
    meta[r.t].reserved = 0.0f;
  }
  const float* __restrict__ x = (const float*)desc[r.t].p0;
  uint8_t* __restrict__ q = (uint8_t*)desc[r.t].p1;
  for (int64_t i = r.begin + (int64_t)threadIdx.x * kVec; i < r.end; i += kTile) {
    if (i + kVec <= r.end) {
      const float4* p = (const float4*)(x + i);
      float4 a = p[0], b = p[1], c = p[2], d = p[3];
      float f[16] = {a.x * s, a.y * s, a.z * s, a.w * s, b.x * s, b.y * s, b.z * s, b.w * s,
                     c.x * s, c.y * s, c.z * s, c.w * s, d.x * s, d.y * s, d.z * s, d.w * s};
      uint4 o;
      o.x = enc4_nan<FMT>(f);
      o.y = enc4_nan<FMT>(f + 4);
      o.z = enc4_nan<FMT>(f + 8);
      o.w = enc4_nan<FMT>(f + 12);
      *(uint4*)(q + i) = o;
    } else {
      for (int64_t e = i; e < r.end; ++e) q[e] = (uint8_t)enc1_nan<FMT>(x[e] * s);
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(kBlock) void k_dequantize(const TensorDesc* __restrict__ desc,
                                                       const ChunkRef* __restrict__ chunks,
                                                       const msamp_meta* __restrict__ meta) {
  const ChunkRange r = chunk_range(chunks, desc);
  const float si = meta[r.t].scale_inv;
  const uint8_t* __restrict__ q = (const uint8_t*)desc[r.t].p0;
  float* __restrict__ out = (float*)desc[r.t].p1;
  for (int64_t i = r.begin + (int64_t)threadIdx.x * kVec; i < r.end; i += kTile) {
    if (i + kVec <= r.end) {
      float f[16];
      dec16<FMT>(*(const uint4*)(q + i), f);
      float4* o = (float4*)(out + i);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        o[k] = make_float4(f[4 * k] * si, f[4 * k + 1] * si, f[4 * k + 2] * si, f[4 * k + 3] * si);
    } else {
      for (int64_t e = i; e < r.end; ++e) out[e] = dec1<FMT>(q[e]) * si;
    }
  }
}

// -------------------------------------------------------- AdamW passes ---

// m1 = beta1*m0 + (1-beta1)*g with one fused multiply-add.
__device__ __forceinline__ float first_moment(const StepConsts& k, float g, float m0) {
  return __builtin_fmaf(k.b1, m0, k.ob1 * g);
}

// v1, den and w1 (see the AdamW definition in msamp.h).
__device__ __forceinline__ void second_moment_and_weight(const StepConsts& k, float g, float m1,
                                                         float v0, float w0, float& v1,
                                                         float& w1) {
  v1 = __builtin_fmaf(k.b2, v0, k.ob2 * (g * g));
  const float den = __builtin_fmaf(__builtin_sqrtf(v1), k.ibs, k.eps);
  w1 = __builtin_fmaf(-k.ss, m1 / den, w0 * k.dec);
}

// Pass 1 (O2 and O3): new first moment and its per-tensor amax.
template <int GF>
__global__ __launch_bounds__(kBlock) void k_step_pass1(const TensorDesc* __restrict__ desc,
                                                       const ChunkRef* __restrict__ chunks,
                                                       const msamp_meta* __restrict__ gmeta,
                                                       const msamp_meta* __restrict__ mmeta,
                                                       uint32_t* __restrict__ amax_m,
                                                       StepConsts k) {
  const ChunkRange r = chunk_range(chunks, desc);
  const float gsi = gmeta[r.t].scale_inv;
  const float msi = mmeta[r.t].scale_inv;
  const uint8_t* __restrict__ gq = (const uint8_t*)desc[r.t].p0;
  const uint8_t* __restrict__ mq = (const uint8_t*)desc[r.t].p1;
  uint32_t mx = 0u;
  for (int64_t i = r.begin + (int64_t)threadIdx.x * kVec; i < r.end; i += kTile) {
    if (i + kVec <= r.end) {
      float g[16], m[16];
      dec16<GF>(*(const uint4*)(gq + i), g);
      dec16<kE4M3>(*(const uint4*)(mq + i), m);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float m1 = first_moment(k, g[e] * gsi, m[e] * msi);
        mx = umax(mx, abs_bits(m1));
      }
    } else {
      for (int64_t e = i; e < r.end; ++e) {
        const float m1 = first_moment(k, dec1<GF>(gq[e]) * gsi, dec1<kE4M3>(mq[e]) * msi);
        mx = umax(mx, abs_bits(m1));
      }
    }
  }
  block_max_into(mx, &amax_m[r.t]);
}

// Pass 2: recompute m1 exactly as in pass 1, then v1, w1; store m (E4M3 with
// the new scale), v and w (FP16). In the O3 layout the weight is the master
// and the amax of the stored master is reduced into amax_w.
template <int GF, bool O3>
__global__ __launch_bounds__(kBlock) void k_step_pass2(const TensorDesc* __restrict__ desc,
                                                       const ChunkRef* __restrict__ chunks,
                                                       const msamp_meta* __restrict__ gmeta,
                                                       const msamp_meta* __restrict__ mmeta,
                                                       const uint32_t* __restrict__ amax_m,
                                                       uint32_t* __restrict__ amax_w,
                                                       StepConsts k) {
  const ChunkRange r = chunk_range(chunks, desc);
  const float gsi = gmeta[r.t].scale_inv;
  const float msi = mmeta[r.t].scale_inv;
  const float s_m = scale_rule(__uint_as_float(amax_m[r.t]), kE4M3Max);
  const uint8_t* __restrict__ gq = (const uint8_t*)desc[r.t].p0;
  uint8_t* __restrict__ mq = (uint8_t*)desc[r.t].p1;
  uint16_t* __restrict__ vh = (uint16_t*)desc[r.t].p2;
  uint16_t* __restrict__ wh = (uint16_t*)desc[r.t].p3;
  uint32_t wmax = 0u;  // FP16 magnitude bits of the new weight (O3)
  for (int64_t i = r.begin + (int64_t)threadIdx.x * kVec; i < r.end; i += kTile) {
    if (i + kVec <= r.end) {
      const uint4 G = *(const uint4*)(gq + i);
      const uint4 M = *(const uint4*)(mq + i);
      const uint4 V0 = *(const uint4*)(vh + i);
      const uint4 V1 = *(const uint4*)(vh + i + 8);
      const uint4 W0 = *(const uint4*)(wh + i);
      const uint4 W1 = *(const uint4*)(wh + i + 8);
      float g[16], m[16], v[16], w[16];
      dec16<GF>(G, g);
      dec16<kE4M3>(M, m);
      h8_to_f8(V0, v);
      h8_to_f8(V1, v + 8);
      h8_to_f8(W0, w);
      h8_to_f8(W1, w + 8);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float ge = g[e] * gsi;
        const float m1 = first_moment(k, ge, m[e] * msi);
        float v1, w1;
        second_moment_and_weight(k, ge, m1, v[e], w[e], v1, w1);
        m[e] = m1 * s_m;
        v[e] = v1;
        w[e] = w1;
      }
      uint4 Mo;
      Mo.x = enc4<kE4M3>(m);
      Mo.y = enc4<kE4M3>(m + 4);
      Mo.z = enc4<kE4M3>(m + 8);
      Mo.w = enc4<kE4M3>(m + 12);
      const uint4 Vo0 = f8_to_h8(v), Vo1 = f8_to_h8(v + 8);
      const uint4 Wo0 = f8_to_h8(w), Wo1 = f8_to_h8(w + 8);
      *(uint4*)(mq + i) = Mo;
      *(uint4*)(vh + i) = Vo0;
      *(uint4*)(vh + i + 8) = Vo1;
      *(uint4*)(wh + i) = Wo0;
      *(uint4*)(wh + i + 8) = Wo1;
      if (O3) {
        const uint32_t ws[8] = {Wo0.x, Wo0.y, Wo0.z, Wo0.w, Wo1.x, Wo1.y, Wo1.z, Wo1.w};
#pragma unroll
        for (int k2 = 0; k2 < 8; ++k2)
          wmax = umax(wmax, umax(ws[k2] & 0x7FFFu, (ws[k2] >> 16) & 0x7FFFu));
      }
    } else {
      for (int64_t e = i; e < r.end; ++e) {
        const float ge = dec1<GF>(gq[e]) * gsi;
        const float m1 = first_moment(k, ge, dec1<kE4M3>(mq[e]) * msi);
        float v1, w1;
        second_moment_and_weight(k, ge, m1, h_to_f(vh[e]), h_to_f(wh[e]), v1, w1);
        float mm[4] = {m1 * s_m, 0.0f, 0.0f, 0.0f};
        mq[e] = (uint8_t)(enc4<kE4M3>(mm) & 0xFFu);
        vh[e] = f_to_h(v1);
        const uint16_t wn = f_to_h(w1);
        wh[e] = wn;
        if (O3) wmax = umax(wmax, (uint32_t)(wn & 0x7FFFu));
      }
    }
  }
  if (O3) {
    // magnitude of the largest stored master value as binary32 bits; the
    // binary16 -> binary32 widening is exact and preserves the order
    const uint32_t bits = abs_bits(h_to_f((uint16_t)wmax));
    block_max_into(bits, &amax_w[r.t]);
  }
}

// Pass 3 (O3): FP8 E4M3 copy of the stored master with its own scale.
__global__ __launch_bounds__(kBlock) void k_o3_pass3(const TensorDesc* __restrict__ desc,
                                                     const ChunkRef* __restrict__ chunks,
                                                     const uint32_t* __restrict__ amax_w) {
  const ChunkRange r = chunk_range(chunks, desc);
  const float s_w = scale_rule(__uint_as_float(amax_w[r.t]), kE4M3Max);
  const uint16_t* __restrict__ wh = (const uint16_t*)desc[r.t].p3;
  uint8_t* __restrict__ w8 = (uint8_t*)desc[r.t].p4;
  for (int64_t i = r.begin + (int64_t)threadIdx.x * kVec; i < r.end; i += kTile) {
    if (i + kVec <= r.end) {
      float w[16];
      h8_to_f8(*(const uint4*)(wh + i), w);
      h8_to_f8(*(const uint4*)(wh + i + 8), w + 8);
#pragma unroll
      for (int e = 0; e < 16; ++e) w[e] = w[e] * s_w;
      uint4 o;
      o.x = enc4<kE4M3>(w);
      o.y = enc4<kE4M3>(w + 4);
      o.z = enc4<kE4M3>(w + 8);
      o.w = enc4<kE4M3>(w + 12);
      *(uint4*)(w8 + i) = o;
    } else {
      for (int64_t e = i; e < r.end; ++e) {
        float ww[4] = {h_to_f(wh[e]) * s_w, 0.0f, 0.0f, 0.0f};
        w8[e] = (uint8_t)(enc4<kE4M3>(ww) & 0xFFu);
      }
    }
  }
}

__global__ __launch_bounds__(kBlock) void k_step_finalize(int32_t n, uint32_t* __restrict__ amax_a,
                                                          msamp_meta* __restrict__ meta_a,
                                                          uint32_t* __restrict__ amax_b,
                                                          msamp_meta* __restrict__ meta_b) {
  const int32_t t = blockIdx.x * kBlock + threadIdx.x;
  if (t >= n) return;
  {
    const float a = __uint_as_float(amax_a[t]);
    const float s = scale_rule(a, kE4M3Max);
    msamp_meta m;
    m.amax = a;
    m.scale = s;
    m.scale_inv = 1.0f / s;
    m.reserved = 0.0f;
    meta_a[t] = m;
    amax_a[t] = 0u;
  }
  if (meta_b != nullptr) {
    const float a = __uint_as_float(amax_b[t]);
    const float s = scale_rule(a, kE4M3Max);
    msamp_meta m;
    m.amax = a;
    m.scale = s;
    m.scale_inv = 1.0f / s;
    m.reserved = 0.0f;
    meta_b[t] = m;
    amax_b[t] = 0u;
  }
}

// --------------------------------------------------------- codec probe ---

__global__ __launch_bounds__(kBlock) void k_codec_probe(int op, const void* __restrict__ in,
                                                        void* __restrict__ out, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kBlock) {
    switch (op) {
      case MSAMP_PROBE_F32_TO_E4M3:
        ((uint8_t*)out)[i] = (uint8_t)enc1_nan<kE4M3>(((const float*)in)[i]);
        break;
      case MSAMP_PROBE_F32_TO_E5M2:
        ((uint8_t*)out)[i] = (uint8_t)enc1_nan<kE5M2>(((const float*)in)[i]);
        break;
      case MSAMP_PROBE_E4M3_TO_F32:
        ((float*)out)[i] = dec1<kE4M3>(((const uint8_t*)in)[i]);
        break;
      case MSAMP_PROBE_E5M2_TO_F32:
        ((float*)out)[i] = dec1<kE5M2>(((const uint8_t*)in)[i]);
        break;
      case MSAMP_PROBE_F32_TO_F16: {
        // through the packed converter of the update passes: element i is
        // converted together with its neighbour i^1 (itself at the end)
        const float* x = (const float*)in;
        const int64_t j = (i ^ 1) < n ? (i ^ 1) : i;
        const uint32_t pair = (i & 1) ? f2_to_h2(x[j], x[i]) : f2_to_h2(x[i], x[j]);
        ((uint16_t*)out)[i] = (uint16_t)((i & 1) ? (pair >> 16) : (pair & 0xFFFFu));
        break;
      }
      case MSAMP_PROBE_F16_TO_F32:
        ((float*)out)[i] = h_to_f(((const uint16_t*)in)[i]);
        break;
      default:
        break;
    }
  }
}

inline unsigned grid_of(int64_t nchunks) { return (unsigned)nchunks; }

}  // namespace

// ------------------------------------------------------------ launchers ---

hipError_t launch_amax(const TensorDesc* desc, const ChunkRef* chunks, int64_t nchunks,
                       uint32_t* scratch, hipStream_t stream) {
  if (nchunks <= 0) return hipSuccess;
  k_amax<<<grid_of(nchunks), kBlock, 0, stream>>>(desc, chunks, scratch);
  return hipGetLastError();
}

hipError_t launch_amax_finalize(int32_t n, uint32_t* scratch, msamp_meta* meta,
                                hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  k_amax_finalize<<<(unsigned)((n + kBlock - 1) / kBlock), kBlock, 0, stream>>>(n, scratch, meta);
  return hipGetLastError();
}

hipError_t launch_quantize(int fmt, const TensorDesc* desc, const ChunkRef* chunks,
                           int64_t nchunks, msamp_meta* meta, hipStream_t stream) {
  if (nchunks <= 0) return hipSuccess;
  if (fmt == kE4M3)
    k_quantize<kE4M3><<<grid_of(nchunks), kBlock, 0, stream>>>(desc, chunks, meta);
  else
    k_quantize<kE5M2><<<grid_of(nchunks), kBlock, 0, stream>>>(desc, chunks, meta);
  return hipGetLastError();
}

hipError_t launch_dequantize(int fmt, const TensorDesc* desc, const ChunkRef* chunks,
                             int64_t nchunks, const msamp_meta* meta, hipStream_t stream) {
  if (nchunks <= 0) return hipSuccess;
  if (fmt == kE4M3)
    k_dequantize<kE4M3><<<grid_of(nchunks), kBlock, 0, stream>>>(desc, chunks, meta);
  else
    k_dequantize<kE5M2><<<grid_of(nchunks), kBlock, 0, stream>>>(desc, chunks, meta);
  return hipGetLastError();
}

hipError_t launch_step_pass1(int gfmt, const TensorDesc* desc, const ChunkRef* chunks,
                             int64_t nchunks, const msamp_meta* gmeta, const msamp_meta* mmeta,
                             uint32_t* amax_m, const StepConsts& k, hipStream_t stream) {
  if (nchunks <= 0) return hipSuccess;
  if (gfmt == kE4M3)
    k_step_pass1<kE4M3><<<grid_of(nchunks), kBlock, 0, stream>>>(desc, chunks, gmeta, mmeta, amax_m, k);
  else
    k_step_pass1<kE5M2><<<grid_of(nchunks), kBlock, 0, stream>>>(desc, chunks, gmeta, mmeta, amax_m, k);
  return hipGetLastError();
}

hipError_t launch_step_pass2(int gfmt, bool o3, const TensorDesc* desc, const ChunkRef* chunks,
                             int64_t nchunks, const msamp_meta* gmeta, const msamp_meta* mmeta,
                             const uint32_t* amax_m, uint32_t* amax_w, const StepConsts& k,
                             hipStream_t stream) {
  if (nchunks <= 0) return hipSuccess;
  const unsigned g = grid_of(nchunks);
  if (gfmt == kE4M3) {
    if (o3)
      k_step_pass2<kE4M3, true><<<g, kBlock, 0, stream>>>(desc, chunks, gmeta, mmeta, amax_m, amax_w, k);
    else
      k_step_pass2<kE4M3, false><<<g, kBlock, 0, stream>>>(desc, chunks, gmeta, mmeta, amax_m, amax_w, k);
  } else {
    if (o3)
      k_step_pass2<kE5M2, true><<<g, kBlock, 0, stream>>>(desc, chunks, gmeta, mmeta, amax_m, amax_w, k);
    else
      k_step_pass2<kE5M2, false><<<g, kBlock, 0, stream>>>(desc, chunks, gmeta, mmeta, amax_m, amax_w, k);
  }
  return hipGetLastError();
}

hipError_t launch_o3_pass3(const TensorDesc* desc, const ChunkRef* chunks, int64_t nchunks,
                           const uint32_t* amax_w, hipStream_t stream) {
  if (nchunks <= 0) return hipSuccess;
  k_o3_pass3<<<grid_of(nchunks), kBlock, 0, stream>>>(desc, chunks, amax_w);
  return hipGetLastError();
}

hipError_t launch_step_finalize(int32_t n, uint32_t* amax_a, msamp_meta* meta_a,
                                uint32_t* amax_b, msamp_meta* meta_b, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  k_step_finalize<<<(unsigned)((n + kBlock - 1) / kBlock), kBlock, 0, stream>>>(n, amax_a, meta_a,
                                                                               amax_b, meta_b);
  return hipGetLastError();
}

hipError_t launch_codec_probe(int op, const void* in, void* out, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + kBlock - 1) / kBlock;
  if (blocks > 65536) blocks = 65536;
  k_codec_probe<<<(unsigned)blocks, kBlock, 0, stream>>>(op, in, out, n);
  return hipGetLastError();
}

}  // namespace msamp
