// persistent.hip -- the O2/O3 AdamW step of the MS-AMP optimization levels
// ("Optimization Level" page, sections O2 and O3 and the table) as ONE
// persistent, cooperative launch: one workgroup of 512 threads per compute
// unit, all co-resident, walking the tensor list in order.
//
// Per tensor t (tiles of 8192 elements; tile k belongs to workgroup
// (start_t + k) mod G, start_t = tiles of the tensors before t):
//   pass 1  each workgroup reads the gradient and first-moment codes of its
//           tiles and reduces amax(m1); it folds that into the tensor's word
//           with a returning atomic max, then adds its tile count to the
//           tensor's pass-1 counter;
//   wait    until the counter reaches the tensor's tile count. Meanwhile the
//           workgroup runs its pass-1 tiles of the next tensor, so the wait
//           costs no memory time;
//   pass 2  the update of its tiles, walked in reverse so that the codes
//           read last in pass 1 are re-read first (still in L2 or the
//           memory-side cache, so they do not come from HBM again);
//   O3      the amax of the new master is reduced the same way, a second
//           wait, then pass 3 writes the FP8 copy of the tiles;
//   finish  the workgroup whose counter update completes the tensor writes
//           its meta records and returns the tensor's scratch words to zero
//           for the next call.
// A tensor of a single tile is done entirely by its workgroup, with no
// global atomics. The codes read in pass 1 are loaded normally (so they stay
// in the caches); the second moment and weight are read and every output is
// written non-temporally, so that traffic does not evict them.
//
// Waits are bounded: after kMaxSpins polls a wait gives up, counts itself in
// the error word and continues (the results are then undefined). Every
// workgroup therefore reaches the end of the kernel.
//
// Cross-workgroup order: the amax atomic returns before the counter atomic
// is issued, and agent-scope atomic loads read the coherent value, so a
// workgroup that has seen the full count reads the final amax.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "codec.hpp"
#include "device.hpp"
#include "kernels.hpp"

namespace msamp {
namespace {

constexpr int kPB = kPersistentBlock;  // threads per workgroup (8 waves)
constexpr uint32_t kMaxSpins = 1u << 17;

struct PArgs {
  const TensorDesc* desc;
  int32_t n;
  const msamp_meta* gmeta;
  msamp_meta* mmeta;
  msamp_meta* wmeta;  // O3: FP8 weight-copy meta
  uint32_t* scr;      // kPersistentScratchWords per tensor, zero between calls
  uint32_t* err;      // wait time-outs
  StepConsts kv;
  const StepConsts* kdev;
};

// Scratch words of one tensor.
enum : int { kAmaxM = 0, kAmaxW = 1, kCount1 = 2, kCount2 = 3, kCount3 = 4 };

__device__ __forceinline__ uint32_t tiles_of(const TensorDesc& d) { return (uint32_t)d.reserved[0]; }

// This workgroup's first tile of a tensor whose tiles start at global tile
// 'start' (>= the tensor's tile count: no tile of it is ours).
__device__ __forceinline__ uint32_t first_tile(const TensorDesc& d) {
  const uint32_t G = gridDim.x;
  return (blockIdx.x + G - (uint32_t)((uint64_t)d.reserved[1] % G)) % G;
}

// ----------------------------------------------------------- pass 1 -----

// Largest |m1| bits over this thread's 16 elements of a tile (lane layout:
// thread i owns the 16 consecutive elements at i*16).
template <int GF, bool COUPLED>
__device__ __forceinline__ uint32_t p1_tile(const TensorDesc& d, int64_t tile, float gsi, float msi,
                                            const StepConsts& k) {
  const GLOBAL uint8_t* gq = global_ptr<uint8_t>(d.p0);
  const GLOBAL uint8_t* mq = global_ptr<uint8_t>(d.p1);
  const GLOBAL uint16_t* wh = global_ptr<uint16_t>(d.p3);
  const int64_t e = tile + threadIdx.x * 16;
  uint32_t mx = 0u;
  if (e + 16 <= d.numel) {
    const u32x4 G = load<u32x4>(gq + e), Mq = load<u32x4>(mq + e);
    float g[16], m[16], w[16];
    dec8<GF>(G.xy, g);
    dec8<GF>(G.zw, g + 8);
    dec8<kE4M3>(Mq.xy, m);
    dec8<kE4M3>(Mq.zw, m + 8);
    if (COUPLED) {
      h8_to_f8(load<u32x4>(wh + e), w);
      h8_to_f8(load<u32x4>(wh + e + 8), w + 8);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float ge = effective_grad<COUPLED>(k, g[i] * gsi, COUPLED ? w[i] : 0.0f);
      mx = umax(mx, abs_bits(first_moment(k, ge, m[i] * msi)));
    }
  } else {
    for (int64_t i = e; i < d.numel; ++i) {
      const float ge = effective_grad<COUPLED>(k, dec1<GF>(gq[i]) * gsi, COUPLED ? h_to_f(wh[i]) : 0.0f);
      mx = umax(mx, abs_bits(first_moment(k, ge, dec1<kE4M3>(mq[i]) * msi)));
    }
  }
  return mx;
}

// ----------------------------------------------------------- pass 2 -----

// The update of one tile (lane layout: wave w, lane l own the 8-element
// groups at w*1024 + l*8 and w*1024 + 512 + l*8). Returns, for O3, the
// largest FP16 magnitude bits of the new master of this thread's elements.
template <int GF, bool O3, bool COUPLED>
__device__ __forceinline__ uint32_t p2_tile(const TensorDesc& d, int64_t tile, float gsi, float msi,
                                            float s_m, const StepConsts& k) {
  const GLOBAL uint8_t* gq = global_ptr<uint8_t>(d.p0);
  GLOBAL uint8_t* mq = global_ptr<uint8_t>(d.p1);
  GLOBAL uint16_t* vh = global_ptr<uint16_t>(d.p2);
  GLOBAL uint16_t* wh = global_ptr<uint16_t>(d.p3);
  const int64_t e0 = tile + (threadIdx.x >> 6) * 1024 + (threadIdx.x & 63) * 8, e1 = e0 + 512;
  uint32_t wmax = 0u;
  if (e1 + 8 <= d.numel) {
    const u32x2 G0 = load<u32x2>(gq + e0), G1 = load<u32x2>(gq + e1);
    const u32x2 M0 = load<u32x2>(mq + e0), M1 = load<u32x2>(mq + e1);
    const u32x4 V0 = load_stream<u32x4>(vh + e0), V1 = load_stream<u32x4>(vh + e1);
    // Adam's pass 1 read the weight too, so it may still be cached
    const u32x4 W0 = COUPLED ? load<u32x4>(wh + e0) : load_stream<u32x4>(wh + e0);
    const u32x4 W1 = COUPLED ? load<u32x4>(wh + e1) : load_stream<u32x4>(wh + e1);
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
      m[e] = m1 * s_m;
      v[e] = v1;
      w[e] = w1;
    }
    const u32x4 Wo0 = f8_to_h8(w), Wo1 = f8_to_h8(w + 8);
    store_stream<u32x2>(mq + e0, enc8<kE4M3>(m));
    store_stream<u32x2>(mq + e1, enc8<kE4M3>(m + 8));
    store_stream<u32x4>(vh + e0, f8_to_h8(v));
    store_stream<u32x4>(vh + e1, f8_to_h8(v + 8));
    if (O3) {
      // the master is read back by pass 3: keep it cached
      store<u32x4>(wh + e0, Wo0);
      store<u32x4>(wh + e1, Wo1);
      wmax = umax(h8_absmax_bits(Wo0), h8_absmax_bits(Wo1));
    } else {
      store_stream<u32x4>(wh + e0, Wo0);
      store_stream<u32x4>(wh + e1, Wo1);
    }
  } else {
    for (int h = 0; h < 2; ++h) {
      const int64_t e = h ? e1 : e0;
      for (int64_t i = e; i < e + 8 && i < d.numel; ++i) {
        const float w0 = h_to_f(wh[i]);
        const float ge = effective_grad<COUPLED>(k, dec1<GF>(gq[i]) * gsi, w0);
        const float m1 = first_moment(k, ge, dec1<kE4M3>(mq[i]) * msi);
        float v1, w1;
        second_moment_and_weight(k, ge, m1, h_to_f(vh[i]), w0, v1, w1);
        mq[i] = enc1_e4m3(m1 * s_m);
        vh[i] = f_to_h(v1);
        const uint16_t wn = f_to_h(w1);
        wh[i] = wn;
        if (O3) wmax = umax(wmax, (uint32_t)(wn & 0x7FFFu));
      }
    }
  }
  return wmax;
}

// ----------------------------------------------------------- pass 3 -----

// FP8 E4M3 copy of the stored master of one tile (same lanes as pass 2, so
// every thread reads back what it wrote).
__device__ __forceinline__ void p3_tile(const TensorDesc& d, int64_t tile, float s_w) {
  const GLOBAL uint16_t* wh = global_ptr<uint16_t>(d.p3);
  GLOBAL uint8_t* w8 = global_ptr<uint8_t>(d.p4);
  const int64_t e0 = tile + (threadIdx.x >> 6) * 1024 + (threadIdx.x & 63) * 8, e1 = e0 + 512;
  if (e1 + 8 <= d.numel) {
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
      for (int64_t i = e; i < e + 8 && i < d.numel; ++i) w8[i] = enc1_e4m3(h_to_f(wh[i]) * s_w);
    }
  }
}

// magnitude of the largest stored master value as binary32 bits (the
// binary16 -> binary32 widening is exact and preserves the order)
__device__ __forceinline__ uint32_t f16_mag_to_f32_bits(uint32_t h) {
  return abs_bits(h_to_f((uint16_t)h));
}

__device__ __forceinline__ void write_meta(msamp_meta* meta, float amax) {
  const float s = scale_rule(amax, kE4M3Max);
  msamp_meta r;
  r.amax = amax;
  r.scale = s;
  r.scale_inv = 1.0f / s;
  r.reserved = 0.0f;
  *meta = r;
}

// Pass-1 tiles of one tensor run ahead of time while waiting on another.
template <int GF, bool COUPLED>
struct Ahead {
  int32_t t = -1;  // tensor, or -1
  TensorDesc d;
  uint32_t next = 0, tiles = 0, mx = 0, done = 0;
  float gsi = 1.0f, msi = 1.0f;

  __device__ __forceinline__ bool can_run() const { return t >= 0 && next < tiles; }
  __device__ __forceinline__ void run_one(const StepConsts& k) {
    mx = umax(mx, p1_tile<GF, COUPLED>(d, (int64_t)next * kPersistentTile, gsi, msi, k));
    next += gridDim.x;
    ++done;
  }
};

// Waits until *ctr >= target (all threads of the workgroup leave together),
// running pass-1 tiles of the tensor in 'ahead' meanwhile.
template <int GF, bool COUPLED>
__device__ __forceinline__ void wait_count(const uint32_t* ctr, uint32_t target, Ahead<GF, COUPLED>& ahead,
                                           const StepConsts& k, uint32_t* err) {
  __shared__ uint32_t sh_done;
  uint32_t spins = 0;
  for (;;) {
    if (threadIdx.x == 0)
      sh_done = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target ? 1u : 0u;
    __syncthreads();
    const uint32_t done = sh_done;
    __syncthreads();
    if (done) return;
    if (ahead.can_run()) {
      ahead.run_one(k);
    } else {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kMaxSpins) {
        if (threadIdx.x == 0) atomicAdd(err, 1u);
        return;
      }
    }
  }
}

// Reads a scratch word coherently and hands it to every thread.
__device__ __forceinline__ uint32_t broadcast_load(const uint32_t* p) {
  __shared__ uint32_t sh_val;
  if (threadIdx.x == 0) sh_val = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const uint32_t v = sh_val;
  __syncthreads();
  return v;
}

// Folds this workgroup's maximum into the tensor's word, then adds its tile
// count to the counter (the maximum is in place before the count rises).
__device__ __forceinline__ void publish(uint32_t mx, uint32_t* amax_word, uint32_t* ctr, uint32_t mine) {
  if (threadIdx.x == 0) {
    const uint32_t old = atomicMax(amax_word, mx);
    asm volatile("" ::"v"(old));  // the returned value orders the two atomics
    atomicAdd(ctr, mine);
  }
}

// Adds this workgroup's tiles to a completion counter; true (in every
// thread) for the workgroup that completes the tensor.
__device__ __forceinline__ bool finish(uint32_t* ctr, uint32_t mine, uint32_t tiles) {
  __shared__ uint32_t sh_last;
  __syncthreads();  // every thread's stores of the tensor are issued
  if (threadIdx.x == 0) sh_last = (atomicAdd(ctr, mine) + mine == tiles) ? 1u : 0u;
  __syncthreads();
  return sh_last != 0u;
}

__device__ __forceinline__ void zero_word(uint32_t* p) {
  __hip_atomic_store(p, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int GF, bool O3, bool COUPLED>
__global__ __launch_bounds__(kPB) void k_step_persistent(PArgs a) {
  const StepConsts k = a.kdev != nullptr ? *a.kdev : a.kv;
  Ahead<GF, COUPLED> ahead;
  for (int32_t t = 0; t < a.n; ++t) {
    const TensorDesc d = a.desc[t];
    const uint32_t tiles = tiles_of(d);
    if (tiles == 0) {
      // empty tensor: initial-state meta records
      if (blockIdx.x == (uint32_t)t % gridDim.x && threadIdx.x == 0) {
        write_meta(&a.mmeta[t], 0.0f);
        if (O3) write_meta(&a.wmeta[t], 0.0f);
      }
      continue;
    }
    const uint32_t first = first_tile(d);
    if (first >= tiles) continue;  // no tile of this tensor is ours
    const float gsi = a.gmeta[t].scale_inv;
    const float msi = a.mmeta[t].scale_inv;
    uint32_t* scr = a.scr + (size_t)t * kPersistentScratchWords;

    if (tiles == 1) {
      // one tile: the whole tensor in this workgroup
      const uint32_t mx = block_max<kPB>(p1_tile<GF, COUPLED>(d, 0, gsi, msi, k));
      const float amax_m = __uint_as_float(mx);
      const float s_m = scale_rule(amax_m, kE4M3Max);
      const uint32_t wm = p2_tile<GF, O3, COUPLED>(d, 0, gsi, msi, s_m, k);
      float amax_w = 0.0f;
      if (O3) {
        amax_w = __uint_as_float(f16_mag_to_f32_bits(block_max<kPB>(wm)));
        p3_tile(d, 0, scale_rule(amax_w, kE4M3Max));
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        write_meta(&a.mmeta[t], amax_m);
        if (O3) write_meta(&a.wmeta[t], amax_w);
      }
      continue;
    }

    // pass 1 (continuing what ran ahead during the previous wait)
    uint32_t next = first, mx = 0u, mine = 0u;
    if (ahead.t == t) {
      next = ahead.next;
      mx = ahead.mx;
      mine = ahead.done;
    }
    ahead.t = -1;
    for (; next < tiles; next += gridDim.x, ++mine)
      mx = umax(mx, p1_tile<GF, COUPLED>(d, (int64_t)next * kPersistentTile, gsi, msi, k));
    mx = block_max<kPB>(mx);
    publish(mx, &scr[kAmaxM], &scr[kCount1], mine);

    // run ahead on the next tensor while the others finish pass 1
    if (t + 1 < a.n) {
      const TensorDesc dn = a.desc[t + 1];
      const uint32_t tn = tiles_of(dn), fn = first_tile(dn);
      if (tn > 1 && fn < tn) {
        ahead.t = t + 1;
        ahead.d = dn;
        ahead.next = fn;
        ahead.tiles = tn;
        ahead.mx = 0u;
        ahead.done = 0u;
        ahead.gsi = a.gmeta[t + 1].scale_inv;
        ahead.msi = a.mmeta[t + 1].scale_inv;
      }
    }
    wait_count<GF, COUPLED>(&scr[kCount1], tiles, ahead, k, a.err);
    const float amax_m = __uint_as_float(broadcast_load(&scr[kAmaxM]));
    const float s_m = scale_rule(amax_m, kE4M3Max);

    // pass 2, newest pass-1 tiles first
    uint32_t wm = 0u;
    for (uint32_t j = mine; j-- > 0;)
      wm = umax(wm, p2_tile<GF, O3, COUPLED>(d, (int64_t)(first + j * gridDim.x) * kPersistentTile, gsi,
                                             msi, s_m, k));
    if (!O3) {
      if (finish(&scr[kCount2], mine, tiles)) {
        if (threadIdx.x == 0) {
          write_meta(&a.mmeta[t], amax_m);
          zero_word(&scr[kAmaxM]);
          zero_word(&scr[kCount1]);
          zero_word(&scr[kCount2]);
        }
      }
      continue;
    }
    // O3: amax of the new master over the tensor, then its FP8 copy
    wm = f16_mag_to_f32_bits(block_max<kPB>(wm));
    publish(wm, &scr[kAmaxW], &scr[kCount2], mine);
    wait_count<GF, COUPLED>(&scr[kCount2], tiles, ahead, k, a.err);
    const float amax_w = __uint_as_float(broadcast_load(&scr[kAmaxW]));
    const float s_w = scale_rule(amax_w, kE4M3Max);
    for (uint32_t j = 0; j < mine; ++j) p3_tile(d, (int64_t)(first + j * gridDim.x) * kPersistentTile, s_w);
    if (finish(&scr[kCount3], mine, tiles)) {
      if (threadIdx.x == 0) {
        write_meta(&a.mmeta[t], amax_m);
        write_meta(&a.wmeta[t], amax_w);
        zero_word(&scr[kAmaxM]);
        zero_word(&scr[kAmaxW]);
        zero_word(&scr[kCount1]);
        zero_word(&scr[kCount2]);
        zero_word(&scr[kCount3]);
      }
    }
  }
}

template <int GF, bool O3, bool COUPLED>
hipError_t launch_p(unsigned grid, const PArgs& a, hipStream_t stream) {
  PArgs args = a;
  void* kargs[] = {(void*)&args};
  return hipLaunchCooperativeKernel((const void*)k_step_persistent<GF, O3, COUPLED>, dim3(grid), dim3(kPB),
                                    kargs, 0, stream);
}

template <int GF>
hipError_t dispatch_p(bool o3, bool coupled, unsigned grid, const PArgs& a, hipStream_t stream) {
  if (o3) return coupled ? launch_p<GF, true, true>(grid, a, stream) : launch_p<GF, true, false>(grid, a, stream);
  return coupled ? launch_p<GF, false, true>(grid, a, stream) : launch_p<GF, false, false>(grid, a, stream);
}

}  // namespace

hipError_t persistent_occupancy(int* blocks_per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu,
                                                      (const void*)k_step_persistent<kE4M3, true, true>, kPB, 0);
}

hipError_t launch_step_persistent(int gfmt, bool o3, bool coupled, unsigned grid, const TensorDesc* desc,
                                  int32_t n, const msamp_meta* gmeta, msamp_meta* mmeta, msamp_meta* wmeta,
                                  uint32_t* scr, uint32_t* err, const StepConsts& k, hipStream_t stream,
                                  const StepConsts* kdev) {
  if (n <= 0) return hipSuccess;
  PArgs a;
  a.desc = desc;
  a.n = n;
  a.gmeta = gmeta;
  a.mmeta = mmeta;
  a.wmeta = wmeta;
  a.scr = scr;
  a.err = err;
  a.kv = k;
  a.kdev = kdev;
  return gfmt == kE4M3 ? dispatch_p<kE4M3>(o3, coupled, grid, a, stream)
                       : dispatch_p<kE5M2>(o3, coupled, grid, a, stream);
}

}  // namespace msamp
