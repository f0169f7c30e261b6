// kernels.hip -- HIP kernels for gfx950 (MI355X): per-tensor amax, FP8
// quantize / dequantize, and the two- and three-pass low-precision AdamW step
// of the MS-AMP O2 and O3 layouts ("Optimization Level" page, sections O2 and
// O3 and the optimization-level table).
//
// All kernels are multi-tensor-apply launches: workgroup b takes ChunkRef b
// (tensor t, chunk j) and covers elements [j*c, min(numel, (j+1)*c)) of
// tensor t (c: the list's chunk size, in its TensorDesc) in tiles of 16
// elements per thread: 4,096 elements (4 waves x 1024), or 8,192 (8 waves,
// one tile per chunk) for the step passes of a large list. The update pass
// and the O3 copy may split every chunk evenly over several workgroups
// (workgroup b then takes part b % split of ChunkRef b / split). Inside a
// wave's 1024 elements the lanes are laid out so that every load and store
// instruction of the wave covers one contiguous span of memory:
//   FP8 / FP16 streams: lane l owns the 8-element groups at l*8 and
//     512 + l*8 (one 8-byte FP8 access or one 16-byte FP16 access per group)
//   FP32 streams: lane l owns the 4-element groups at k*256 + l*4, k = 0..3
//     (one 16-byte access per group)
//   AdamW pass 1 (FP8 streams only): lane l owns the 16 codes at l*16 (one
//     16-byte access per stream)
// A ragged end of a tensor is handled element by element. The work is bound
// by HBM bandwidth; no matrix cores are involved.
//
// Arithmetic is binary32 with the operation order of the AdamW definition in
// msamp.h; the file is compiled with -ffp-contract=off so that only the
// explicit fmaf calls are fused.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "codec.hpp"
#include "device.hpp"
#include "kernels.hpp"

namespace msamp {
namespace {

// Largest value of the workgroup, folded into *dst. The closing barrier
// keeps a later reduction of the same workgroup from overwriting the LDS
// partials before thread 0 has read them.
// WAIT: thread 0 waits until its update has been performed (the folded
// meta write of the same launch counts this workgroup only after that).
// LAST: no later use of these LDS partials in the kernel, so the closing
// barrier is left out and the other waves retire while thread 0 finishes
// (one-tile workgroups of the fused pass on the 7B list: 6.77 -> 6.62 ms).
template <bool WAIT = false, int BS = kBlock, bool LAST = false>
__device__ __forceinline__ void block_max_into(uint32_t v, uint32_t* dst) {
  __shared__ uint32_t partial[BS / 64];
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) partial[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = partial[0];
#pragma unroll
    for (int k = 1; k < BS / 64; ++k) m = umax(m, partial[k]);
    if (WAIT)
      atomic_max_if_larger_wait(m, dst);
    else
      atomic_max_if_larger(m, dst);
  }
  if (!LAST) __syncthreads();
}

// Two independent maxima of the workgroup in one reduction (separate LDS
// slots for each), folded into *dst_a and *dst_b.
__device__ __forceinline__ void block_max2_into(uint32_t a, uint32_t* dst_a, uint32_t b,
                                                uint32_t* dst_b) {
  __shared__ uint32_t partial[2][kBlock / 64];
  a = wave_max(a);
  b = wave_max(b);
  if ((threadIdx.x & 63) == 0) {
    partial[0][threadIdx.x >> 6] = a;
    partial[1][threadIdx.x >> 6] = b;
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    uint32_t m = partial[threadIdx.x][0];
#pragma unroll
    for (int k = 1; k < kBlock / 64; ++k) m = umax(m, partial[threadIdx.x][k]);
    atomic_max_if_larger(m, threadIdx.x == 0 ? dst_a : dst_b);
  }
  __syncthreads();
}

struct ChunkRange {
  int t;
  int64_t begin, end;
  bool head;  // the tensor's first workgroup
};

// The part of its chunk that this workgroup walks when every chunk is split
// over 'split' workgroups (blockIdx.x / split is the chunk); the chunk size
// is a multiple of 'split' tiles, and a part past the tensor's end is empty.
__device__ __forceinline__ ChunkRange part_range(const ChunkRef* chunks, const TensorDesc* desc, uint32_t split) {
  const ChunkRef c = chunks[blockIdx.x / split];
  const uint32_t part = blockIdx.x % split;
  ChunkRange r;
  r.t = c.tensor;
  const int64_t span = desc[c.tensor].chunk / split;
  r.begin = (int64_t)c.chunk * desc[c.tensor].chunk + (int64_t)part * span;
  const int64_t n = desc[c.tensor].numel;
  r.end = r.begin + span < n ? r.begin + span : n;
  r.head = c.chunk == 0 && part == 0;
  return r;
}

__device__ __forceinline__ ChunkRange chunk_range(const ChunkRef* chunks, const TensorDesc* desc) {
  return part_range(chunks, desc, 1u);
}

// Chunks of a tensor in a plan that folds the meta writes (at least one).
__device__ __forceinline__ uint32_t chunks_of(const TensorDesc& d) {
  return d.numel == 0 ? 1u : (uint32_t)((d.numel + d.chunk - 1) / d.chunk);
}

__device__ __forceinline__ void put_meta(msamp_meta* meta, float amax, float fmax) {
  const float s = scale_rule(amax, fmax);
  msamp_meta m;
  m.amax = amax;
  m.scale = s;
  m.scale_inv = 1.0f / s;
  m.reserved = 0.0f;
  *meta = m;
}

__device__ __forceinline__ uint32_t take_word(uint32_t* p) {
  const uint32_t v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(p, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v;
}

// Called by all threads of every workgroup after its last use of tensor t's
// data and amax words; the workgroup whose count completes the tensor
// writes the meta records: the full record {amax, scale, 1/scale} (E4M3
// range, for meta_a and meta_b), or only the amax field of meta_a when
// AMAX_ONLY. The amax and count words are only touched with device-scope
// atomics, which are performed at one coherence point; no fence is used (on
// gfx950 a device-scope fence writes back the whole L2 of the XCD).
// When the same launch raised the amax word (AMAX_ONLY: the amax kernel),
// thread 0 issued that atomic and waited for it (block_max_into<true>), so
// its update has been performed before its chunk is counted. Every other
// read of the words happened before the workgroup's count (the reads fed
// the work done since).
template <bool AMAX_ONLY>
__device__ __forceinline__ void fold_meta(const MetaFold& f, const TensorDesc* desc, int t, uint32_t parts = 1) {
  if (f.done == nullptr) return;
  __syncthreads();
  if (threadIdx.x != 0) return;
  const uint32_t before = __hip_atomic_fetch_add(&f.done[t], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (before + 1u != chunks_of(desc[t]) * parts) return;
  const float a = __uint_as_float(take_word(&f.amax_a[t]));
  if (AMAX_ONLY)
    f.meta_a[t].amax = a;
  else
    put_meta(&f.meta_a[t], a, kE4M3Max);
  if (f.meta_b != nullptr) put_meta(&f.meta_b[t], __uint_as_float(take_word(&f.amax_b[t])), kE4M3Max);
  __hip_atomic_store(&f.done[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// First element of this lane's 8-element groups (FP8/FP16 layout) in the
// tile starting at 'tile': e0 and e0 + 512.
__device__ __forceinline__ int64_t group8_base(int64_t tile) {
  return tile + (threadIdx.x >> 6) * 1024 + (threadIdx.x & 63) * 8;
}

// First element of this lane's 16-element group (FP8-only layout: one
// 16-byte access per stream, 1 KB per wave instruction).
__device__ __forceinline__ int64_t group16_base(int64_t tile) {
  return tile + (threadIdx.x >> 6) * 1024 + (threadIdx.x & 63) * 16;
}

// First element of this lane's 4-element group k (FP32 layout).
__device__ __forceinline__ int64_t group4_base(int64_t tile, int k) {
  return tile + (threadIdx.x >> 6) * 1024 + k * 256 + (threadIdx.x & 63) * 4;
}

// ---------------------------------------------------------------- amax ---

__global__ __launch_bounds__(kBlock) void k_amax(const TensorDesc* __restrict__ desc,
                                                 const ChunkRef* __restrict__ chunks,
                                                 uint32_t* __restrict__ scratch, MetaFold fold) {
  const ChunkRange r = chunk_range(chunks, desc);
  const GLOBAL float* __restrict__ x = global_ptr<float>(desc[r.t].p0);
  uint32_t m = 0u;
  for (int64_t tile = r.begin; tile < r.end; tile += kTile) {
    if (group4_base(tile, 3) + 4 <= r.end) {
      u32x4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = load_stream<u32x4>(x + group4_base(tile, k));
#pragma unroll
      for (int k = 0; k < 4; ++k)
        m = umax(m, umax(umax(v[k].x & 0x7FFFFFFFu, v[k].y & 0x7FFFFFFFu),
                         umax(v[k].z & 0x7FFFFFFFu, v[k].w & 0x7FFFFFFFu)));
    } else {
      // partial tile: whole 4-element groups as one 16-byte access, the
      // group holding the tensor's end element by element
      for (int k = 0; k < 4; ++k) {
        const int64_t e = group4_base(tile, k);
        if (e + 4 <= r.end) {
          const u32x4 v = load_stream<u32x4>(x + e);
          m = umax(m, umax(umax(v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu), umax(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu)));
        } else {
          for (int64_t i = e; i < r.end; ++i) m = umax(m, abs_bits(x[i]));
        }
      }
    }
  }
  if (fold.done != nullptr)
    block_max_into<true, kBlock, true>(m, &scratch[r.t]);
  else
    block_max_into<false, kBlock, true>(m, &scratch[r.t]);
  fold_meta<true>(fold, desc, r.t);
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
                                                     msamp_meta* __restrict__ meta, float world) {
  const ChunkRange r = chunk_range(chunks, desc);
  const float s = scale_rule(meta[r.t].amax * world, Fp8Traits<FMT>::kMax);
  if (r.head && threadIdx.x == 0) {
    meta[r.t].scale = s;
    meta[r.t].scale_inv = 1.0f / s;
    meta[r.t].reserved = 0.0f;
  }
  const GLOBAL float* __restrict__ x = global_ptr<float>(desc[r.t].p0);
  GLOBAL uint8_t* __restrict__ q = global_ptr<uint8_t>(desc[r.t].p1);
  for (int64_t tile = r.begin; tile < r.end; tile += kTile) {
    if (group4_base(tile, 3) + 4 <= r.end) {
      u32x4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = load_stream<u32x4>(x + group4_base(tile, k));
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float f[4] = {__uint_as_float(v[k].x) * s, __uint_as_float(v[k].y) * s,
                      __uint_as_float(v[k].z) * s, __uint_as_float(v[k].w) * s};
        store_stream<uint32_t>(q + group4_base(tile, k), enc4_nan<FMT>(f));
      }
    } else {
      for (int k = 0; k < 4; ++k) {
        const int64_t e = group4_base(tile, k);
        if (e + 4 <= r.end) {
          const u32x4 v = load_stream<u32x4>(x + e);
          float f[4] = {__uint_as_float(v.x) * s, __uint_as_float(v.y) * s, __uint_as_float(v.z) * s,
                        __uint_as_float(v.w) * s};
          store_stream<uint32_t>(q + e, enc4_nan<FMT>(f));
        } else {
          for (int64_t i = e; i < r.end; ++i) q[i] = (uint8_t)enc1_nan<FMT>(x[i] * s);
        }
      }
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(kBlock) void k_dequantize(const TensorDesc* __restrict__ desc,
                                                       const ChunkRef* __restrict__ chunks,
                                                       const msamp_meta* __restrict__ meta) {
  const ChunkRange r = chunk_range(chunks, desc);
  const float si = meta[r.t].scale_inv;
  const GLOBAL uint8_t* __restrict__ q = global_ptr<uint8_t>(desc[r.t].p0);
  GLOBAL float* __restrict__ out = global_ptr<float>(desc[r.t].p1);
  for (int64_t tile = r.begin; tile < r.end; tile += kTile) {
    if (group4_base(tile, 3) + 4 <= r.end) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t e = group4_base(tile, k);
        float f[4];
        dec4<FMT>(load<uint32_t>(q + e), f);
        u32x4 o;
        o.x = __float_as_uint(f[0] * si);
        o.y = __float_as_uint(f[1] * si);
        o.z = __float_as_uint(f[2] * si);
        o.w = __float_as_uint(f[3] * si);
        store<u32x4>(out + e, o);
      }
    } else {
      for (int k = 0; k < 4; ++k) {
        const int64_t e = group4_base(tile, k);
        if (e + 4 <= r.end) {
          float f[4];
          dec4<FMT>(load<uint32_t>(q + e), f);
          u32x4 o;
          o.x = __float_as_uint(f[0] * si);
          o.y = __float_as_uint(f[1] * si);
          o.z = __float_as_uint(f[2] * si);
          o.w = __float_as_uint(f[3] * si);
          store<u32x4>(out + e, o);
        } else {
          for (int64_t i = e; i < r.end; ++i) out[i] = dec1<FMT>(q[i]) * si;
        }
      }
    }
  }
}

// -------------------------------------------------------- AdamW passes ---

// Pass 1 (O2 and O3): new first moment and its per-tensor amax. Adam
// (COUPLED) also reads the weight for its L2 term. The step constants come
// by value (kv), or from device memory when kdev is not null (so that a
// captured launch can be replayed for later steps).
template <int GF, bool COUPLED, int BS = kBlock>
__global__ __launch_bounds__(BS) void k_step_pass1(const TensorDesc* __restrict__ desc,
                                                       const ChunkRef* __restrict__ chunks,
                                                       const msamp_meta* __restrict__ gmeta,
                                                       const msamp_meta* __restrict__ mmeta,
                                                       uint32_t* __restrict__ amax_m,
                                                       StepConsts kv,
                                                       const StepConsts* __restrict__ kdev) {
  const StepConsts k = kdev != nullptr ? *kdev : kv;
  const ChunkRange r = chunk_range(chunks, desc);
  const float gsi = gmeta[r.t].scale_inv;
  const float msi = mmeta[r.t].scale_inv;
  const GLOBAL uint8_t* __restrict__ gq = global_ptr<uint8_t>(desc[r.t].p0);
  const GLOBAL uint8_t* __restrict__ mq = global_ptr<uint8_t>(desc[r.t].p1);
  const GLOBAL uint16_t* __restrict__ wh = global_ptr<uint16_t>(desc[r.t].p3);
  uint32_t mx = 0u;
  for (int64_t tile = r.begin; tile < r.end; tile += (int64_t)BS * 16) {
    const int64_t e0 = group8_base(tile), e1 = e0 + 512;
    if (!COUPLED && group16_base(tile) + 16 <= r.end) {
      // only FP8 streams: 16 consecutive codes per lane, one 16-byte
      // non-temporal load per stream. Pass 2 reads these codes again, but
      // only after this pass has run over the whole list (13.5 GB of codes
      // for the 7B list), so no cache could keep them until then; the
      // non-temporal loads measured 7% faster than ordinary ones here.
      const int64_t e = group16_base(tile);
      const u32x4 G = load_stream<u32x4>(gq + e), Mq = load_stream<u32x4>(mq + e);
      float g[16], m[16];
      dec8<GF>(G.xy, g);
      dec8<GF>(G.zw, g + 8);
      dec8<kE4M3>(Mq.xy, m);
      dec8<kE4M3>(Mq.zw, m + 8);
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = umax(mx, abs_bits(first_moment(k, g[i] * gsi, m[i] * msi)));
    } else if (COUPLED && e1 + 8 <= r.end) {
      const u32x2 G0 = load<u32x2>(gq + e0), G1 = load<u32x2>(gq + e1);
      const u32x2 M0 = load<u32x2>(mq + e0), M1 = load<u32x2>(mq + e1);
      float g[16], m[16], w[16];
      h8_to_f8(load<u32x4>(wh + e0), w);
      h8_to_f8(load<u32x4>(wh + e1), w + 8);
      dec8<GF>(G0, g);
      dec8<GF>(G1, g + 8);
      dec8<kE4M3>(M0, m);
      dec8<kE4M3>(M1, m + 8);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float ge = effective_grad<COUPLED>(k, g[e] * gsi, w[e]);
        mx = umax(mx, abs_bits(first_moment(k, ge, m[e] * msi)));
      }
    } else {
      // partial tile: whole 8-element groups as vector accesses, the group
      // holding the tensor's end element by element
      for (int h = 0; h < 2; ++h) {
        const int64_t e = COUPLED ? (h ? e1 : e0) : group16_base(tile) + 8 * h;
        if (e + 8 <= r.end) {
          float g[8], m[8], w[8];
          dec8<GF>(load<u32x2>(gq + e), g);
          dec8<kE4M3>(load<u32x2>(mq + e), m);
          if (COUPLED) h8_to_f8(load<u32x4>(wh + e), w);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float ge = effective_grad<COUPLED>(k, g[i] * gsi, COUPLED ? w[i] : 0.0f);
            mx = umax(mx, abs_bits(first_moment(k, ge, m[i] * msi)));
          }
        } else {
          for (int64_t i = e; i < r.end; ++i) {
            const float ge = effective_grad<COUPLED>(k, dec1<GF>(gq[i]) * gsi, COUPLED ? h_to_f(wh[i]) : 0.0f);
            mx = umax(mx, abs_bits(first_moment(k, ge, dec1<kE4M3>(mq[i]) * msi)));
          }
        }
      }
    }
  }
  block_max_into<false, BS, true>(mx, &amax_m[r.t]);
}

// Gradient quantize fused with pass 1 (O2 and O3; AdamW, or Adam when
// COUPLED, which also reads the FP16 weight for its L2 term). The codes are
// computed exactly as k_quantize computes them (same scale, same NaN-aware
// saturating encode), stored, and decoded from registers for pass 1, so they
// are not read back from memory. Every stream uses the FP32 lane layout
// (4-element groups): 16-byte gradient loads, 4-byte code loads and stores,
// 8-byte weight loads. The step constants come by value (kv), or from device
// memory when kdev is not null (a captured launch replayed for later steps).
template <int GF, bool COUPLED>
__device__ __forceinline__ uint32_t qp1_group(const StepConsts& k, const u32x4& v, uint32_t mw, const u32x2& wv,
                                              float s, float gsi, float msi, uint32_t* code) {
  const float f[4] = {__uint_as_float(v.x) * s, __uint_as_float(v.y) * s, __uint_as_float(v.z) * s,
                      __uint_as_float(v.w) * s};
  const uint32_t c = enc4_nan<GF>(f);
  *code = c;
  float g[4], m[4], w[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  dec4<GF>(c, g);
  dec4<kE4M3>(mw, m);
  if (COUPLED) {
    const f32x2 a = h2_to_f2(wv.x), b = h2_to_f2(wv.y);
    w[0] = a.x;
    w[1] = a.y;
    w[2] = b.x;
    w[3] = b.y;
  }
  uint32_t mx = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    mx = umax(mx, abs_bits(first_moment(k, effective_grad<COUPLED>(k, g[i] * gsi, w[i]), m[i] * msi)));
  return mx;
}

template <int GF, bool COUPLED, int BS = kBlock>
__global__ __launch_bounds__(BS) void k_quantize_pass1(const TensorDesc* __restrict__ desc,
                                                           const ChunkRef* __restrict__ chunks,
                                                           msamp_meta* __restrict__ gmeta,
                                                           const msamp_meta* __restrict__ mmeta,
                                                           uint32_t* __restrict__ amax_m, StepConsts kv,
                                                           const StepConsts* __restrict__ kdev) {
  const StepConsts k = kdev != nullptr ? *kdev : kv;
  const ChunkRange r = chunk_range(chunks, desc);
  const float s = scale_rule(gmeta[r.t].amax, Fp8Traits<GF>::kMax);
  const float gsi = 1.0f / s;
  if (r.head && threadIdx.x == 0) {
    gmeta[r.t].scale = s;
    gmeta[r.t].scale_inv = gsi;
    gmeta[r.t].reserved = 0.0f;
  }
  const float msi = mmeta[r.t].scale_inv;
  const GLOBAL float* __restrict__ x = global_ptr<float>(desc[r.t].aux);
  // p0 is the step's (read-only) gradient role; this kernel produces it
  GLOBAL uint8_t* __restrict__ q = global_ptr<uint8_t>(const_cast<void*>(desc[r.t].p0));
  const GLOBAL uint8_t* __restrict__ mq = global_ptr<uint8_t>(desc[r.t].p1);
  // Adam's pass 1 reads the weight; pass 2 reads it again soon after
  const GLOBAL uint16_t* __restrict__ wh = global_ptr<uint16_t>(desc[r.t].p3);
  const u32x2 nowt = {0u, 0u};
  uint32_t mx = 0u;
  for (int64_t tile = r.begin; tile < r.end; tile += (int64_t)BS * 16) {
    if (group4_base(tile, 3) + 4 <= r.end) {
      u32x4 v[4];
      uint32_t mw[4];
      u32x2 wv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = load_stream<u32x4>(x + group4_base(tile, j));
        mw[j] = load_stream<uint32_t>(mq + group4_base(tile, j));
        wv[j] = COUPLED ? load<u32x2>(wh + group4_base(tile, j)) : nowt;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t c;
        mx = umax(mx, qp1_group<GF, COUPLED>(k, v[j], mw[j], wv[j], s, gsi, msi, &c));
        store_stream<uint32_t>(q + group4_base(tile, j), c);
      }
    } else {
      for (int j = 0; j < 4; ++j) {
        const int64_t e = group4_base(tile, j);
        if (e + 4 <= r.end) {
          uint32_t c;
          mx = umax(mx, qp1_group<GF, COUPLED>(k, load_stream<u32x4>(x + e), load_stream<uint32_t>(mq + e),
                                               COUPLED ? load<u32x2>(wh + e) : nowt, s, gsi, msi, &c));
          store_stream<uint32_t>(q + e, c);
        } else {
          for (int64_t i = e; i < r.end; ++i) {
            const uint32_t c = enc1_nan<GF>(x[i] * s);
            q[i] = (uint8_t)c;
            const float ge = effective_grad<COUPLED>(k, dec1<GF>((uint8_t)c) * gsi, COUPLED ? h_to_f(wh[i]) : 0.0f);
            mx = umax(mx, abs_bits(first_moment(k, ge, dec1<kE4M3>(mq[i]) * msi)));
          }
        }
      }
    }
  }
  block_max_into<false, BS, true>(mx, &amax_m[r.t]);
}

// Pass 2: recompute m1 exactly as in pass 1, then v1, w1; store m (E4M3 with
// the new scale), v and w (FP16). In the O3 layout the weight is the master
// and the amax of the stored master is reduced into amax_w.
//
// DELAYED (an ablation of the two-pass scheme, O2 only): the codes are
// encoded with the scale of the previous step's amax (mmeta.amax) and the
// amax of the new m1 is reduced into amax_w for the next step.
template <int GF, bool O3, bool COUPLED, bool DELAYED = false, int BS = kBlock>
__global__ __launch_bounds__(BS) void k_step_pass2(const TensorDesc* __restrict__ desc,
                                                       const ChunkRef* __restrict__ chunks,
                                                       const msamp_meta* __restrict__ gmeta,
                                                       const msamp_meta* __restrict__ mmeta,
                                                       const uint32_t* __restrict__ amax_m,
                                                       uint32_t* __restrict__ amax_w,
                                                       StepConsts kv,
                                                       const StepConsts* __restrict__ kdev,
                                                       MetaFold fold, uint32_t split) {
  static_assert(!(O3 && DELAYED), "the delayed-scaling ablation is O2 only");
  const StepConsts k = kdev != nullptr ? *kdev : kv;
  const ChunkRange r = part_range(chunks, desc, split);
  const float gsi = gmeta[r.t].scale_inv;
  const float msi = mmeta[r.t].scale_inv;
  const float s_m = DELAYED ? scale_rule(mmeta[r.t].amax, kE4M3Max)
                            : scale_rule(__uint_as_float(amax_m[r.t]), kE4M3Max);
  uint32_t mmax = 0u;  // DELAYED: magnitude bits of the new first moment
  const GLOBAL uint8_t* __restrict__ gq = global_ptr<uint8_t>(desc[r.t].p0);
  GLOBAL uint8_t* __restrict__ mq = global_ptr<uint8_t>(desc[r.t].p1);
  GLOBAL uint16_t* __restrict__ vh = global_ptr<uint16_t>(desc[r.t].p2);
  GLOBAL uint16_t* __restrict__ wh = global_ptr<uint16_t>(desc[r.t].p3);
  uint32_t wmax = 0u;  // FP16 magnitude bits of the new weight (O3)
  for (int64_t tile = r.begin; tile < r.end; tile += (int64_t)BS * 16) {
    const int64_t e0 = group8_base(tile), e1 = e0 + 512;
    if (e1 + 8 <= r.end) {
      const u32x2 G0 = load<u32x2>(gq + e0), G1 = load<u32x2>(gq + e1);
      const u32x2 M0 = load<u32x2>(mq + e0), M1 = load<u32x2>(mq + e1);
      const u32x4 V0 = load<u32x4>(vh + e0), V1 = load<u32x4>(vh + e1);
      const u32x4 W0 = load<u32x4>(wh + e0), W1 = load<u32x4>(wh + e1);
      // Loads issued: raise this wave's issue priority, so that waves with
      // their data in flight finish their arithmetic and stores ahead of
      // waves still issuing loads (update pass on the 7B list: 13.38 ->
      // 13.12 ms; the same in the fused pass made it slower).
      __builtin_amdgcn_s_setprio(3);
      float g[16], m[16], v[16], w[16];
      dec8<GF>(G0, g);
      dec8<GF>(G1, g + 8);
      dec8<kE4M3>(M0, m);
      dec8<kE4M3>(M1, m + 8);
      h8_to_f8(V0, v);
      h8_to_f8(V1, v + 8);
      h8_to_f8(W0, w);
      h8_to_f8(W1, w + 8);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float ge = effective_grad<COUPLED>(k, g[e] * gsi, w[e]);
        const float m1 = first_moment(k, ge, m[e] * msi);
        float v1, w1;
        second_moment_and_weight(k, ge, m1, v[e], w[e], v1, w1);
        if (DELAYED) mmax = umax(mmax, abs_bits(m1));
        m[e] = m1 * s_m;
        v[e] = v1;
        w[e] = w1;
      }
      const u32x4 Wo0 = f8_to_h8(w), Wo1 = f8_to_h8(w + 8);
      store<u32x2>(mq + e0, enc8<kE4M3>(m));
      store<u32x2>(mq + e1, enc8<kE4M3>(m + 8));
      store<u32x4>(vh + e0, f8_to_h8(v));
      store<u32x4>(vh + e1, f8_to_h8(v + 8));
      store<u32x4>(wh + e0, Wo0);
      store<u32x4>(wh + e1, Wo1);
      if (O3) {
        const uint32_t ws[8] = {Wo0.x, Wo0.y, Wo0.z, Wo0.w, Wo1.x, Wo1.y, Wo1.z, Wo1.w};
#pragma unroll
        for (int k2 = 0; k2 < 8; ++k2)
          wmax = umax(wmax, umax(ws[k2] & 0x7FFFu, (ws[k2] >> 16) & 0x7FFFu));
      }
    } else {
      for (int h = 0; h < 2; ++h) {
        const int64_t e = h ? e1 : e0;
        for (int64_t i = e; i < e + 8 && i < r.end; ++i) {
          const float w0 = h_to_f(wh[i]);
          const float ge = effective_grad<COUPLED>(k, dec1<GF>(gq[i]) * gsi, w0);
          const float m1 = first_moment(k, ge, dec1<kE4M3>(mq[i]) * msi);
          float v1, w1;
          second_moment_and_weight(k, ge, m1, h_to_f(vh[i]), w0, v1, w1);
          if (DELAYED) mmax = umax(mmax, abs_bits(m1));
          float mm[4] = {m1 * s_m, 0.0f, 0.0f, 0.0f};
          mq[i] = (uint8_t)(enc4<kE4M3>(mm) & 0xFFu);
          vh[i] = f_to_h(v1);
          const uint16_t wn = f_to_h(w1);
          wh[i] = wn;
          if (O3) wmax = umax(wmax, (uint32_t)(wn & 0x7FFFu));
        }
      }
    }
  }
  if (O3) {
    // magnitude of the largest stored master value as binary32 bits; the
    // binary16 -> binary32 widening is exact and preserves the order
    const uint32_t bits = abs_bits(h_to_f((uint16_t)wmax));
    block_max_into<false, BS, true>(bits, &amax_w[r.t]);
  }
  if (DELAYED) block_max_into<false, BS, true>(mmax, &amax_w[r.t]);
  if (!O3 && !DELAYED) fold_meta<false>(fold, desc, r.t, split);  // O3: the fold is in pass 3
}

// Pass 3 (O3): FP8 E4M3 copy of the stored master with its own scale.
template <int BS = kBlock>
__global__ __launch_bounds__(BS) void k_o3_pass3(const TensorDesc* __restrict__ desc,
                                                     const ChunkRef* __restrict__ chunks,
                                                     const uint32_t* __restrict__ amax_w, MetaFold fold,
                                                     uint32_t split) {
  const ChunkRange r = part_range(chunks, desc, split);
  const float s_w = scale_rule(__uint_as_float(amax_w[r.t]), kE4M3Max);
  const GLOBAL uint16_t* __restrict__ wh = global_ptr<uint16_t>(desc[r.t].p3);
  GLOBAL uint8_t* __restrict__ w8 = global_ptr<uint8_t>(desc[r.t].p4);
  for (int64_t tile = r.begin; tile < r.end; tile += (int64_t)BS * 16) {
    const int64_t e0 = group8_base(tile), e1 = e0 + 512;
    if (e1 + 8 <= r.end) {
      float w[16];
      h8_to_f8(load_stream<u32x4>(wh + e0), w);
      h8_to_f8(load_stream<u32x4>(wh + e1), w + 8);
#pragma unroll
      for (int e = 0; e < 16; ++e) w[e] = w[e] * s_w;
      store_stream<u32x2>(w8 + e0, enc8<kE4M3>(w));
      store_stream<u32x2>(w8 + e1, enc8<kE4M3>(w + 8));
    } else {
      for (int h = 0; h < 2; ++h) {
        const int64_t e = h ? e1 : e0;
        if (e + 8 <= r.end) {
          float w[8];
          h8_to_f8(load_stream<u32x4>(wh + e), w);
#pragma unroll
          for (int i = 0; i < 8; ++i) w[i] = w[i] * s_w;
          store_stream<u32x2>(w8 + e, enc8<kE4M3>(w));
        } else {
          for (int64_t i = e; i < r.end; ++i) {
            float ww[4] = {h_to_f(wh[i]) * s_w, 0.0f, 0.0f, 0.0f};
            w8[i] = (uint8_t)(enc4<kE4M3>(ww) & 0xFFu);
          }
        }
      }
    }
  }
  fold_meta<false>(fold, desc, r.t, split);
}

__global__ __launch_bounds__(kBlock) void k_step_finalize(int32_t n, uint32_t* __restrict__ amax_a,
                                                          msamp_meta* __restrict__ meta_a,
                                                          uint32_t* __restrict__ amax_b,
                                                          msamp_meta* __restrict__ meta_b,
                                                          float fmax_b) {
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
    const float s = scale_rule(a, fmax_b);
    msamp_meta m;
    m.amax = a;
    m.scale = s;
    m.scale_inv = 1.0f / s;
    m.reserved = 0.0f;
    meta_b[t] = m;
    amax_b[t] = 0u;
  }
}

// -------------------------------------------------- split-phase steps ---

// out[t] <- amax[t] (binary32 bits), then amax[t] <- 0: hands a tensor's
// amax from the scratch to the caller (who combines the ranks' values).
__global__ __launch_bounds__(kBlock) void k_export_amax(int32_t n, uint32_t* __restrict__ amax,
                                                        float* __restrict__ out) {
  const int32_t t = blockIdx.x * kBlock + threadIdx.x;
  if (t >= n) return;
  out[t] = __uint_as_float(amax[t]);
  amax[t] = 0u;
}

// meta[t] <- {a, scale(a, fmax), 1/scale, 0} with a = amax[t] (caller's).
__global__ __launch_bounds__(kBlock) void k_meta_from_amax(int32_t n, const float* __restrict__ amax,
                                                           msamp_meta* __restrict__ meta, float fmax) {
  const int32_t t = blockIdx.x * kBlock + threadIdx.x;
  if (t >= n) return;
  const float a = amax[t];
  const float s = scale_rule(a, fmax);
  msamp_meta m;
  m.amax = a;
  m.scale = s;
  m.scale_inv = 1.0f / s;
  m.reserved = 0.0f;
  meta[t] = m;
}

// ----------------------------------------- scaled-FP16-v ablation (O2) ---

// Pass 1 of the scaled-v ablation: new first and second moments and both
// per-tensor amaxes (v0 = f32(code) * old 1/s_v).
template <int GF>
__global__ __launch_bounds__(kBlock) void k_scaled_v_pass1(const TensorDesc* __restrict__ desc,
                                                           const ChunkRef* __restrict__ chunks,
                                                           const msamp_meta* __restrict__ gmeta,
                                                           const msamp_meta* __restrict__ mmeta,
                                                           const msamp_meta* __restrict__ vmeta,
                                                           uint32_t* __restrict__ amax_m,
                                                           uint32_t* __restrict__ amax_v,
                                                           StepConsts k) {
  const ChunkRange r = chunk_range(chunks, desc);
  const float gsi = gmeta[r.t].scale_inv, msi = mmeta[r.t].scale_inv, vsi = vmeta[r.t].scale_inv;
  const GLOBAL uint8_t* __restrict__ gq = global_ptr<uint8_t>(desc[r.t].p0);
  const GLOBAL uint8_t* __restrict__ mq = global_ptr<uint8_t>(desc[r.t].p1);
  const GLOBAL uint16_t* __restrict__ vh = global_ptr<uint16_t>(desc[r.t].p2);
  uint32_t mx = 0u, vx = 0u;
  for (int64_t tile = r.begin; tile < r.end; tile += kTile) {
    const int64_t e0 = group8_base(tile), e1 = e0 + 512;
    if (e1 + 8 <= r.end) {
      float g[16], m[16], v[16];
      dec8<GF>(load<u32x2>(gq + e0), g);
      dec8<GF>(load<u32x2>(gq + e1), g + 8);
      dec8<kE4M3>(load<u32x2>(mq + e0), m);
      dec8<kE4M3>(load<u32x2>(mq + e1), m + 8);
      h8_to_f8(load<u32x4>(vh + e0), v);
      h8_to_f8(load<u32x4>(vh + e1), v + 8);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float ge = g[e] * gsi;
        mx = umax(mx, abs_bits(first_moment(k, ge, m[e] * msi)));
        vx = umax(vx, abs_bits(__builtin_fmaf(k.b2, v[e] * vsi, k.ob2 * (ge * ge))));
      }
    } else {
      for (int h = 0; h < 2; ++h) {
        const int64_t e = h ? e1 : e0;
        for (int64_t i = e; i < e + 8 && i < r.end; ++i) {
          const float ge = dec1<GF>(gq[i]) * gsi;
          mx = umax(mx, abs_bits(first_moment(k, ge, dec1<kE4M3>(mq[i]) * msi)));
          vx = umax(vx, abs_bits(__builtin_fmaf(k.b2, h_to_f(vh[i]) * vsi, k.ob2 * (ge * ge))));
        }
      }
    }
  }
  block_max2_into(mx, &amax_m[r.t], vx, &amax_v[r.t]);
}

// Pass 2 of the scaled-v ablation: recompute m1, v1 identically; store m
// (E4M3, new scale), v = fp16(v1 * s_v) and w.
template <int GF>
__global__ __launch_bounds__(kBlock) void k_scaled_v_pass2(const TensorDesc* __restrict__ desc,
                                                           const ChunkRef* __restrict__ chunks,
                                                           const msamp_meta* __restrict__ gmeta,
                                                           const msamp_meta* __restrict__ mmeta,
                                                           const msamp_meta* __restrict__ vmeta,
                                                           const uint32_t* __restrict__ amax_m,
                                                           const uint32_t* __restrict__ amax_v,
                                                           StepConsts k) {
  const ChunkRange r = chunk_range(chunks, desc);
  const float gsi = gmeta[r.t].scale_inv, msi = mmeta[r.t].scale_inv, vsi = vmeta[r.t].scale_inv;
  const float s_m = scale_rule(__uint_as_float(amax_m[r.t]), kE4M3Max);
  const float s_v = scale_rule(__uint_as_float(amax_v[r.t]), kF16Max);
  const GLOBAL uint8_t* __restrict__ gq = global_ptr<uint8_t>(desc[r.t].p0);
  GLOBAL uint8_t* __restrict__ mq = global_ptr<uint8_t>(desc[r.t].p1);
  GLOBAL uint16_t* __restrict__ vh = global_ptr<uint16_t>(desc[r.t].p2);
  GLOBAL uint16_t* __restrict__ wh = global_ptr<uint16_t>(desc[r.t].p3);
  for (int64_t tile = r.begin; tile < r.end; tile += kTile) {
    const int64_t e0 = group8_base(tile), e1 = e0 + 512;
    if (e1 + 8 <= r.end) {
      float g[16], m[16], v[16], w[16];
      dec8<GF>(load<u32x2>(gq + e0), g);
      dec8<GF>(load<u32x2>(gq + e1), g + 8);
      dec8<kE4M3>(load<u32x2>(mq + e0), m);
      dec8<kE4M3>(load<u32x2>(mq + e1), m + 8);
      h8_to_f8(load<u32x4>(vh + e0), v);
      h8_to_f8(load<u32x4>(vh + e1), v + 8);
      h8_to_f8(load<u32x4>(wh + e0), w);
      h8_to_f8(load<u32x4>(wh + e1), w + 8);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float ge = g[e] * gsi;
        const float m1 = first_moment(k, ge, m[e] * msi);
        float v1, w1;
        second_moment_and_weight(k, ge, m1, v[e] * vsi, w[e], v1, w1);
        m[e] = m1 * s_m;
        v[e] = v1 * s_v;
        w[e] = w1;
      }
      store<u32x2>(mq + e0, enc8<kE4M3>(m));
      store<u32x2>(mq + e1, enc8<kE4M3>(m + 8));
      store<u32x4>(vh + e0, f8_to_h8(v));
      store<u32x4>(vh + e1, f8_to_h8(v + 8));
      store<u32x4>(wh + e0, f8_to_h8(w));
      store<u32x4>(wh + e1, f8_to_h8(w + 8));
    } else {
      for (int h = 0; h < 2; ++h) {
        const int64_t e = h ? e1 : e0;
        for (int64_t i = e; i < e + 8 && i < r.end; ++i) {
          const float ge = dec1<GF>(gq[i]) * gsi;
          const float m1 = first_moment(k, ge, dec1<kE4M3>(mq[i]) * msi);
          float v1, w1;
          second_moment_and_weight(k, ge, m1, h_to_f(vh[i]) * vsi, h_to_f(wh[i]), v1, w1);
          float mm[4] = {m1 * s_m, 0.0f, 0.0f, 0.0f};
          mq[i] = (uint8_t)(enc4<kE4M3>(mm) & 0xFFu);
          vh[i] = f_to_h(v1 * s_v);
          wh[i] = f_to_h(w1);
        }
      }
    }
  }
}

__global__ __launch_bounds__(kBlock) void k_delayed_finalize(int32_t n, uint32_t* __restrict__ amax_new,
                                                             msamp_meta* __restrict__ meta) {
  const int32_t t = blockIdx.x * kBlock + threadIdx.x;
  if (t >= n) return;
  const float s = scale_rule(meta[t].amax, kE4M3Max);  // the scale the step encoded with
  msamp_meta m;
  m.amax = __uint_as_float(amax_new[t]);
  m.scale = s;
  m.scale_inv = 1.0f / s;
  m.reserved = 0.0f;
  meta[t] = m;
  amax_new[t] = 0u;
}

// --------------------------------------------------------- codec probe ---

// The memory traffic of the update pass without its arithmetic: read g, m,
// v, w and write m, v, w back unchanged (the empty asm keeps the compiler
// from treating the stores of just-loaded values as removable). It measures
// what the memory system gives this traffic on the very same buffers.
template <int BS = kBlock>
__global__ __launch_bounds__(BS) void k_rmw_probe(const TensorDesc* __restrict__ desc,
                                                      const ChunkRef* __restrict__ chunks, uint32_t split) {
  const ChunkRange r = part_range(chunks, desc, split);
  const GLOBAL uint8_t* __restrict__ gq = global_ptr<uint8_t>(desc[r.t].p0);
  GLOBAL uint8_t* __restrict__ mq = global_ptr<uint8_t>(desc[r.t].p1);
  GLOBAL uint16_t* __restrict__ vh = global_ptr<uint16_t>(desc[r.t].p2);
  GLOBAL uint16_t* __restrict__ wh = global_ptr<uint16_t>(desc[r.t].p3);
  for (int64_t tile = r.begin; tile < r.end; tile += (int64_t)BS * 16) {
    const int64_t e0 = group8_base(tile), e1 = e0 + 512;
    if (e1 + 8 <= r.end) {
      u32x2 G0 = load<u32x2>(gq + e0), G1 = load<u32x2>(gq + e1);
      u32x2 M0 = load<u32x2>(mq + e0), M1 = load<u32x2>(mq + e1);
      u32x4 V0 = load<u32x4>(vh + e0), V1 = load<u32x4>(vh + e1);
      u32x4 W0 = load<u32x4>(wh + e0), W1 = load<u32x4>(wh + e1);
      asm volatile("" : "+v"(M0), "+v"(M1), "+v"(V0), "+v"(V1), "+v"(W0), "+v"(W1)
                   : "v"(G0), "v"(G1));
      store<u32x2>(mq + e0, M0);
      store<u32x2>(mq + e1, M1);
      store<u32x4>(vh + e0, V0);
      store<u32x4>(vh + e1, V1);
      store<u32x4>(wh + e0, W0);
      store<u32x4>(wh + e1, W1);
    } else {
      for (int h = 0; h < 2; ++h) {
        const int64_t e = h ? e1 : e0;
        for (int64_t i = e; i < e + 8 && i < r.end; ++i) {
          uint32_t g = gq[i], m = mq[i], v = vh[i], w = wh[i];
          asm volatile("" : "+v"(m), "+v"(v), "+v"(w) : "v"(g));
          mq[i] = (uint8_t)m;
          vh[i] = (uint16_t)v;
          wh[i] = (uint16_t)w;
        }
      }
    }
  }
}

// The fused quantize + pass 1's loads and stores without its arithmetic
// (measurement aid): the same lanes, tiles and launch; reads the binary32
// gradient (aux) and the first-moment codes (p1) and writes an unspecified
// mix of them to the gradient codes (p0), 6 bytes per element.
template <int BS = kBlock>
__global__ __launch_bounds__(BS) void k_qp1_probe(const TensorDesc* __restrict__ desc,
                                                      const ChunkRef* __restrict__ chunks) {
  const ChunkRange r = chunk_range(chunks, desc);
  const GLOBAL float* __restrict__ x = global_ptr<float>(desc[r.t].aux);
  GLOBAL uint8_t* __restrict__ q = global_ptr<uint8_t>(const_cast<void*>(desc[r.t].p0));
  const GLOBAL uint8_t* __restrict__ mq = global_ptr<uint8_t>(desc[r.t].p1);
  for (int64_t tile = r.begin; tile < r.end; tile += (int64_t)BS * 16) {
    if (group4_base(tile, 3) + 4 <= r.end) {
      u32x4 v[4];
      uint32_t mw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = load_stream<u32x4>(x + group4_base(tile, j));
        mw[j] = load_stream<uint32_t>(mq + group4_base(tile, j));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t c = v[j].x ^ v[j].y ^ v[j].z ^ v[j].w ^ mw[j];
        asm volatile("" : "+v"(c));
        store_stream<uint32_t>(q + group4_base(tile, j), c);
      }
    } else {
      for (int j = 0; j < 4; ++j) {
        const int64_t e = group4_base(tile, j);
        for (int64_t i = e; i < e + 4 && i < r.end; ++i) {
          uint32_t c = __float_as_uint(x[i]) ^ mq[i];
          asm volatile("" : "+v"(c));
          q[i] = (uint8_t)c;
        }
      }
    }
  }
}

// Plain streams over one buffer in 16-byte units (measurement aid): the
// lanes of the amax kernel's FP32 layout (each wave instruction covers 1 KB
// of consecutive memory), one 16 KB tile per workgroup (a copy ran 7% faster
// that way than with 16 tiles per workgroup, a read 1-2%), non-temporal
// loads and stores. READ only loads (the empty asm keeps the loaded values
// live, so the loads are issued and waited for); COPY stores what it loads.
constexpr int64_t kProbeTileUnits = 1024, kProbeChunkUnits = kProbeTileUnits;

template <bool COPY>
__global__ __launch_bounds__(kBlock) void k_stream_probe(const u32x4* __restrict__ src_p,
                                                         u32x4* __restrict__ dst_p, int64_t units) {
  const GLOBAL u32x4* __restrict__ src = (const GLOBAL u32x4*)src_p;
  GLOBAL u32x4* __restrict__ dst = (GLOBAL u32x4*)dst_p;
  const int64_t begin = (int64_t)blockIdx.x * kProbeChunkUnits;
  const int64_t end = begin + kProbeChunkUnits < units ? begin + kProbeChunkUnits : units;
  const int64_t lane = (threadIdx.x >> 6) * 256 + (threadIdx.x & 63);
  for (int64_t tile = begin; tile < end; tile += kProbeTileUnits) {
    if (tile + kProbeTileUnits <= end) {
      u32x4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = load_stream<u32x4>(src + tile + lane + k * 64);
      if (COPY) {
#pragma unroll
        for (int k = 0; k < 4; ++k) store_stream<u32x4>(dst + tile + lane + k * 64, v[k]);
      } else {
        asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]));
      }
    } else {
      for (int k = 0; k < 4; ++k) {
        const int64_t i = tile + lane + k * 64;
        if (i < end) {
          u32x4 x = src[i];
          if (COPY)
            dst[i] = x;
          else
            asm volatile("" ::"v"(x));
        }
      }
    }
  }
}

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
                       uint32_t* scratch, hipStream_t stream, const MetaFold& fold) {
  if (nchunks <= 0) return hipSuccess;
  k_amax<<<grid_of(nchunks), kBlock, 0, stream>>>(desc, chunks, scratch, fold);
  return hipGetLastError();
}

hipError_t launch_amax_finalize(int32_t n, uint32_t* scratch, msamp_meta* meta,
                                hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  k_amax_finalize<<<(unsigned)((n + kBlock - 1) / kBlock), kBlock, 0, stream>>>(n, scratch, meta);
  return hipGetLastError();
}

hipError_t launch_quantize(int fmt, const TensorDesc* desc, const ChunkRef* chunks,
                           int64_t nchunks, msamp_meta* meta, int32_t world, hipStream_t stream) {
  if (nchunks <= 0) return hipSuccess;
  const float wf = (float)world;
  if (fmt == kE4M3)
    k_quantize<kE4M3><<<grid_of(nchunks), kBlock, 0, stream>>>(desc, chunks, meta, wf);
  else
    k_quantize<kE5M2><<<grid_of(nchunks), kBlock, 0, stream>>>(desc, chunks, meta, wf);
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

template <int GF, bool COUPLED, int BS>
static void pass1_launch(unsigned g, hipStream_t stream, const TensorDesc* desc, const ChunkRef* chunks,
                         const msamp_meta* gmeta, const msamp_meta* mmeta, uint32_t* amax_m,
                         const StepConsts& k, const StepConsts* kdev) {
  k_step_pass1<GF, COUPLED, BS><<<g, BS, 0, stream>>>(desc, chunks, gmeta, mmeta, amax_m, k, kdev);
}

template <int BS>
static void pass1_dispatch(int gfmt, bool coupled, unsigned g, hipStream_t stream, const TensorDesc* desc,
                           const ChunkRef* chunks, const msamp_meta* gmeta, const msamp_meta* mmeta,
                           uint32_t* amax_m, const StepConsts& k, const StepConsts* kdev) {
  if (gfmt == kE4M3) {
    if (coupled) pass1_launch<kE4M3, true, BS>(g, stream, desc, chunks, gmeta, mmeta, amax_m, k, kdev);
    else pass1_launch<kE4M3, false, BS>(g, stream, desc, chunks, gmeta, mmeta, amax_m, k, kdev);
  } else {
    if (coupled) pass1_launch<kE5M2, true, BS>(g, stream, desc, chunks, gmeta, mmeta, amax_m, k, kdev);
    else pass1_launch<kE5M2, false, BS>(g, stream, desc, chunks, gmeta, mmeta, amax_m, k, kdev);
  }
}

template <int BS>
static void qp1_dispatch(int gfmt, bool coupled, unsigned g, hipStream_t stream, const TensorDesc* desc,
                         const ChunkRef* chunks, msamp_meta* gmeta, const msamp_meta* mmeta, uint32_t* amax_m,
                         const StepConsts& k, const StepConsts* kdev) {
  if (gfmt == kE4M3) {
    if (coupled)
      k_quantize_pass1<kE4M3, true, BS><<<g, BS, 0, stream>>>(desc, chunks, gmeta, mmeta, amax_m, k, kdev);
    else
      k_quantize_pass1<kE4M3, false, BS><<<g, BS, 0, stream>>>(desc, chunks, gmeta, mmeta, amax_m, k, kdev);
  } else {
    if (coupled)
      k_quantize_pass1<kE5M2, true, BS><<<g, BS, 0, stream>>>(desc, chunks, gmeta, mmeta, amax_m, k, kdev);
    else
      k_quantize_pass1<kE5M2, false, BS><<<g, BS, 0, stream>>>(desc, chunks, gmeta, mmeta, amax_m, k, kdev);
  }
}

hipError_t launch_quantize_pass1(int gfmt, bool coupled, const TensorDesc* desc, const ChunkRef* chunks,
                                 int64_t nchunks, msamp_meta* gmeta, const msamp_meta* mmeta, uint32_t* amax_m,
                                 const StepConsts& k, hipStream_t stream, const StepConsts* kdev, bool wide) {
  if (nchunks <= 0) return hipSuccess;
  const unsigned g = grid_of(nchunks);
  if (wide)
    qp1_dispatch<kWideBlock>(gfmt, coupled, g, stream, desc, chunks, gmeta, mmeta, amax_m, k, kdev);
  else
    qp1_dispatch<kBlock>(gfmt, coupled, g, stream, desc, chunks, gmeta, mmeta, amax_m, k, kdev);
  return hipGetLastError();
}

hipError_t launch_step_pass1(int gfmt, bool coupled, const TensorDesc* desc, const ChunkRef* chunks,
                             int64_t nchunks, const msamp_meta* gmeta, const msamp_meta* mmeta,
                             uint32_t* amax_m, const StepConsts& k, hipStream_t stream,
                             const StepConsts* kdev, bool wide) {
  if (nchunks <= 0) return hipSuccess;
  const unsigned g = grid_of(nchunks);
  if (wide)
    pass1_dispatch<kWideBlock>(gfmt, coupled, g, stream, desc, chunks, gmeta, mmeta, amax_m, k, kdev);
  else
    pass1_dispatch<kBlock>(gfmt, coupled, g, stream, desc, chunks, gmeta, mmeta, amax_m, k, kdev);
  return hipGetLastError();
}

template <int GF, bool O3, bool COUPLED, int BS>
static void pass2_launch(unsigned g, hipStream_t stream, const TensorDesc* desc, const ChunkRef* chunks,
                         const msamp_meta* gmeta, const msamp_meta* mmeta, const uint32_t* amax_m,
                         uint32_t* amax_w, const StepConsts& k, const StepConsts* kdev, const MetaFold& fold,
                         uint32_t split) {
  k_step_pass2<GF, O3, COUPLED, false, BS><<<g, BS, 0, stream>>>(desc, chunks, gmeta, mmeta, amax_m, amax_w, k,
                                                                 kdev, fold, split);
}

template <int GF, int BS>
static void pass2_dispatch(bool o3, bool coupled, unsigned g, hipStream_t stream,
                           const TensorDesc* desc, const ChunkRef* chunks, const msamp_meta* gmeta,
                           const msamp_meta* mmeta, const uint32_t* amax_m, uint32_t* amax_w,
                           const StepConsts& k, const StepConsts* kdev, const MetaFold& f, uint32_t sp) {
  if (o3) {
    if (coupled) pass2_launch<GF, true, true, BS>(g, stream, desc, chunks, gmeta, mmeta, amax_m, amax_w, k, kdev, f, sp);
    else pass2_launch<GF, true, false, BS>(g, stream, desc, chunks, gmeta, mmeta, amax_m, amax_w, k, kdev, f, sp);
  } else {
    if (coupled) pass2_launch<GF, false, true, BS>(g, stream, desc, chunks, gmeta, mmeta, amax_m, amax_w, k, kdev, f, sp);
    else pass2_launch<GF, false, false, BS>(g, stream, desc, chunks, gmeta, mmeta, amax_m, amax_w, k, kdev, f, sp);
  }
}

hipError_t launch_step_pass2(int gfmt, bool o3, bool coupled, const TensorDesc* desc,
                             const ChunkRef* chunks, int64_t nchunks, const msamp_meta* gmeta,
                             const msamp_meta* mmeta, const uint32_t* amax_m, uint32_t* amax_w,
                             const StepConsts& k, hipStream_t stream, const StepConsts* kdev,
                             const MetaFold& fold, bool wide, uint32_t split) {
  if (nchunks <= 0) return hipSuccess;
  if (split < 1) return hipErrorInvalidValue;
  const unsigned g = grid_of(nchunks * split);
  if (gfmt == kE4M3) {
    if (wide)
      pass2_dispatch<kE4M3, kWideBlock>(o3, coupled, g, stream, desc, chunks, gmeta, mmeta, amax_m, amax_w, k, kdev, fold,
                                        split);
    else
      pass2_dispatch<kE4M3, kBlock>(o3, coupled, g, stream, desc, chunks, gmeta, mmeta, amax_m, amax_w, k, kdev, fold,
                                    split);
  } else {
    if (wide)
      pass2_dispatch<kE5M2, kWideBlock>(o3, coupled, g, stream, desc, chunks, gmeta, mmeta, amax_m, amax_w, k, kdev, fold,
                                        split);
    else
      pass2_dispatch<kE5M2, kBlock>(o3, coupled, g, stream, desc, chunks, gmeta, mmeta, amax_m, amax_w, k, kdev, fold,
                                    split);
  }
  return hipGetLastError();
}

hipError_t launch_step_delayed(int gfmt, bool coupled, const TensorDesc* desc, const ChunkRef* chunks,
                               int64_t nchunks, const msamp_meta* gmeta, const msamp_meta* mmeta,
                               uint32_t* amax_new, const StepConsts& k, hipStream_t stream) {
  if (nchunks <= 0) return hipSuccess;
  const unsigned g = grid_of(nchunks);
  if (gfmt == kE4M3) {
    if (coupled)
      k_step_pass2<kE4M3, false, true, true><<<g, kBlock, 0, stream>>>(desc, chunks, gmeta, mmeta, nullptr, amax_new, k, nullptr, MetaFold{}, 1u);
    else
      k_step_pass2<kE4M3, false, false, true><<<g, kBlock, 0, stream>>>(desc, chunks, gmeta, mmeta, nullptr, amax_new, k, nullptr, MetaFold{}, 1u);
  } else {
    if (coupled)
      k_step_pass2<kE5M2, false, true, true><<<g, kBlock, 0, stream>>>(desc, chunks, gmeta, mmeta, nullptr, amax_new, k, nullptr, MetaFold{}, 1u);
    else
      k_step_pass2<kE5M2, false, false, true><<<g, kBlock, 0, stream>>>(desc, chunks, gmeta, mmeta, nullptr, amax_new, k, nullptr, MetaFold{}, 1u);
  }
  return hipGetLastError();
}

hipError_t launch_scaled_v_pass1(int gfmt, const TensorDesc* desc, const ChunkRef* chunks,
                                 int64_t nchunks, const msamp_meta* gmeta, const msamp_meta* mmeta,
                                 const msamp_meta* vmeta, uint32_t* amax_m, uint32_t* amax_v,
                                 const StepConsts& k, hipStream_t stream) {
  if (nchunks <= 0) return hipSuccess;
  const unsigned g = grid_of(nchunks);
  if (gfmt == kE4M3)
    k_scaled_v_pass1<kE4M3><<<g, kBlock, 0, stream>>>(desc, chunks, gmeta, mmeta, vmeta, amax_m, amax_v, k);
  else
    k_scaled_v_pass1<kE5M2><<<g, kBlock, 0, stream>>>(desc, chunks, gmeta, mmeta, vmeta, amax_m, amax_v, k);
  return hipGetLastError();
}

hipError_t launch_scaled_v_pass2(int gfmt, const TensorDesc* desc, const ChunkRef* chunks,
                                 int64_t nchunks, const msamp_meta* gmeta, const msamp_meta* mmeta,
                                 const msamp_meta* vmeta, const uint32_t* amax_m,
                                 const uint32_t* amax_v, const StepConsts& k, hipStream_t stream) {
  if (nchunks <= 0) return hipSuccess;
  const unsigned g = grid_of(nchunks);
  if (gfmt == kE4M3)
    k_scaled_v_pass2<kE4M3><<<g, kBlock, 0, stream>>>(desc, chunks, gmeta, mmeta, vmeta, amax_m, amax_v, k);
  else
    k_scaled_v_pass2<kE5M2><<<g, kBlock, 0, stream>>>(desc, chunks, gmeta, mmeta, vmeta, amax_m, amax_v, k);
  return hipGetLastError();
}

hipError_t launch_delayed_finalize(int32_t n, uint32_t* amax_new, msamp_meta* meta,
                                   hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  k_delayed_finalize<<<(unsigned)((n + kBlock - 1) / kBlock), kBlock, 0, stream>>>(n, amax_new, meta);
  return hipGetLastError();
}

hipError_t launch_o3_pass3(const TensorDesc* desc, const ChunkRef* chunks, int64_t nchunks,
                           const uint32_t* amax_w, hipStream_t stream, const MetaFold& fold, bool wide,
                           uint32_t split) {
  if (nchunks <= 0) return hipSuccess;
  if (split < 1) return hipErrorInvalidValue;
  const unsigned g = grid_of(nchunks * split);
  if (wide)
    k_o3_pass3<kWideBlock><<<g, kWideBlock, 0, stream>>>(desc, chunks, amax_w, fold, split);
  else
    k_o3_pass3<kBlock><<<g, kBlock, 0, stream>>>(desc, chunks, amax_w, fold, split);
  return hipGetLastError();
}

hipError_t launch_step_finalize(int32_t n, uint32_t* amax_a, msamp_meta* meta_a,
                                uint32_t* amax_b, msamp_meta* meta_b, float fmax_b,
                                hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  k_step_finalize<<<(unsigned)((n + kBlock - 1) / kBlock), kBlock, 0, stream>>>(n, amax_a, meta_a,
                                                                               amax_b, meta_b, fmax_b);
  return hipGetLastError();
}

hipError_t launch_codec_probe(int op, const void* in, void* out, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + kBlock - 1) / kBlock;
  if (blocks > 65536) blocks = 65536;
  k_codec_probe<<<(unsigned)blocks, kBlock, 0, stream>>>(op, in, out, n);
  return hipGetLastError();
}

hipError_t launch_export_amax(int32_t n, uint32_t* amax, float* out, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  k_export_amax<<<(unsigned)((n + kBlock - 1) / kBlock), kBlock, 0, stream>>>(n, amax, out);
  return hipGetLastError();
}

hipError_t launch_meta_from_amax(int32_t n, const float* amax, msamp_meta* meta, float fmax,
                                 hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  k_meta_from_amax<<<(unsigned)((n + kBlock - 1) / kBlock), kBlock, 0, stream>>>(n, amax, meta, fmax);
  return hipGetLastError();
}

hipError_t launch_stream_probe(bool copy, const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  const int64_t units = bytes / 16;
  if (units <= 0) return hipSuccess;
  const unsigned g = (unsigned)((units + kProbeChunkUnits - 1) / kProbeChunkUnits);
  if (copy)
    k_stream_probe<true><<<g, kBlock, 0, stream>>>((const u32x4*)src, (u32x4*)dst, units);
  else
    k_stream_probe<false><<<g, kBlock, 0, stream>>>((const u32x4*)src, (u32x4*)dst, units);
  return hipGetLastError();
}

hipError_t launch_qp1_probe(const TensorDesc* desc, const ChunkRef* chunks, int64_t nchunks, hipStream_t stream,
                            bool wide) {
  if (nchunks <= 0) return hipSuccess;
  if (wide)
    k_qp1_probe<kWideBlock><<<grid_of(nchunks), kWideBlock, 0, stream>>>(desc, chunks);
  else
    k_qp1_probe<kBlock><<<grid_of(nchunks), kBlock, 0, stream>>>(desc, chunks);
  return hipGetLastError();
}

hipError_t launch_rmw_probe(const TensorDesc* desc, const ChunkRef* chunks, int64_t nchunks,
                            hipStream_t stream, bool wide, uint32_t split) {
  if (nchunks <= 0) return hipSuccess;
  if (split < 1) return hipErrorInvalidValue;
  const unsigned g = grid_of(nchunks * split);
  if (wide)
    k_rmw_probe<kWideBlock><<<g, kWideBlock, 0, stream>>>(desc, chunks, split);
  else
    k_rmw_probe<kBlock><<<g, kBlock, 0, stream>>>(desc, chunks, split);
  return hipGetLastError();
}

}  // namespace msamp
