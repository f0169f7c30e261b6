// kernels.hpp -- internal interface between the C ABI (abi.hip) and the HIP
// kernels (kernels.hip). Not installed, not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msamp.h"

namespace msamp {

// Launch geometry. One workgroup of kBlock threads (4 waves) owns one chunk
// of consecutive elements of one tensor and walks it in tiles of kTile
// elements, 16 per thread and 1024 per wave. A chunk is kChunk elements
// (16 tiles), or fewer tiles for a list too small to give every compute
// unit several chunks of that size (chunk_tiles_for); the descriptor of
// each tensor carries the chunk size of its list.
constexpr int kBlock = 256;
// Large lists (at least kWideMinTiles tiles of kTile) run the step's passes
// (launchers' 'wide') with kWideBlock-thread workgroups, one 8,192-element
// tile each (chunks of kWideChunk elements). Workgroups that each stream one
// tile, dispatched in list order, keep the accesses in flight within a
// narrow window of every stream; on the 7B list this took the update pass
// from 14.5 to 12.8 ms and the fused pass from 7.4 to 6.8 ms against 16
// such tiles per workgroup (the amax, a pure read with a reduction per
// workgroup, ran slower that way and keeps kChunk chunks).
constexpr int kWideBlock = 512;
constexpr int64_t kWideChunk = 16 * (int64_t)kWideBlock;  // 8,192 elements: one tile
// Pass 1 of the two-call step (2 B/p read, an amax reduction in every
// workgroup) keeps 16 such tiles per workgroup: 1.95 against 2.91 ms on
// the 7B list.
constexpr int64_t kWideCoarseChunk = 16 * kWideChunk;  // 131,072 elements
constexpr int64_t kWideMinTiles = (int64_t)16384 * 16;
constexpr int64_t kTile = (int64_t)kBlock * 16;
constexpr int64_t kMaxChunkTiles = 16;
constexpr int64_t kChunk = kMaxChunkTiles * kTile;  // 65536 elements

// Tiles per chunk for a list of 'total_tiles' tiles: 16, unless that gives
// fewer than 4 chunks per compute unit of a 256-CU device; then
// total_tiles / 1024, at least 1.
inline int64_t chunk_tiles_for(int64_t total_tiles) {
  const int64_t t = total_tiles / (256 * 4);
  return t < 1 ? 1 : (t > kMaxChunkTiles ? kMaxChunkTiles : t);
}

// Multi-tensor-apply descriptor of one tensor (64 bytes). The roles of the
// pointers depend on the operation:
//                 p0 (read)     p1            p2           p3          p4
//   amax          x f32         -             -            -           -
//   quantize      x f32         q u8 (out)    -            -           -
//   dequantize    q u8          out f32       -            -           -
//   O2 step       grad u8       exp_avg u8    exp_avg_sq   weight      -
//   O3 step       grad u8       exp_avg u8    exp_avg_sq   master      weight_fp8
// The quantizing steps use the step roles with p0 written by the fused
// quantize + pass 1, and 'aux' holding the binary32 gradient it reads.
struct TensorDesc {
  const void* p0;
  void* p1;
  void* p2;
  void* p3;
  void* p4;
  int64_t numel;
  const void* aux;
  int64_t chunk;  // elements per chunk of this tensor's list (a multiple of kTile)
};
static_assert(sizeof(TensorDesc) == 64, "descriptor must stay 64 bytes");

// One workgroup's work item: chunk 'chunk' of tensor 'tensor'.
struct ChunkRef {
  int32_t tensor;
  int32_t chunk;
};

// AdamW / Adam constants of one step (binary64 expressions rounded once).
// dec is 1 - lr*wd for AdamW and exactly 1 for Adam; wd is the coupled L2
// coefficient used by Adam only.
// The step kernels take them by value, or read them from device memory
// (the graph-capturable entry points); the layout is msamp_step_constants.
struct StepConsts {
  float b1, ob1, b2, ob2, eps, ss, ibs, dec, wd;
};

// Meta records written by the workgroup that completes each tensor instead
// of by a separate finalize launch (used for small lists, where a launch
// costs more than the work). 'done' counts the finished chunks of each
// tensor (zero between calls; a plan that folds gives every tensor, also an
// empty one, at least one chunk). The completing workgroup writes meta_a
// from amax_a (and meta_b from amax_b when meta_b is set) and returns the
// amax and count words to zero.
struct MetaFold {
  uint32_t* done = nullptr;  // null: no folding, a finalize launch follows
  msamp_meta* meta_a = nullptr;
  uint32_t* amax_a = nullptr;
  msamp_meta* meta_b = nullptr;
  uint32_t* amax_b = nullptr;
};

// Every launcher enqueues one kernel on 'stream' and returns the launch
// status. 'nchunks' workgroups are launched (nothing when 0).
// With fold.done set, the completing workgroup of each tensor writes
// fold.meta_a[t].amax (only the amax field) from the scratch word.
hipError_t launch_amax(const TensorDesc* desc, const ChunkRef* chunks, int64_t nchunks,
                       uint32_t* scratch, hipStream_t stream, const MetaFold& fold = MetaFold{});
hipError_t launch_amax_finalize(int32_t n, uint32_t* scratch, msamp_meta* meta,
                                hipStream_t stream);
// scale = scale_rule(meta.amax * world) (world = 1: the plain per-tensor
// scale; world > 1: the pre-scale of an FP8 all-reduce over 'world' ranks).
hipError_t launch_quantize(int fmt, const TensorDesc* desc, const ChunkRef* chunks,
                           int64_t nchunks, msamp_meta* meta, int32_t world, hipStream_t stream);
hipError_t launch_dequantize(int fmt, const TensorDesc* desc, const ChunkRef* chunks,
                             int64_t nchunks, const msamp_meta* meta, hipStream_t stream);
// 'coupled' selects Adam (L2 term wd*w added to the gradient before the
// moments); otherwise AdamW.
// Fused gradient quantize + pass 1: q = enc(x * s) into p0 (s from
// gmeta.amax; chunk 0 writes gmeta.scale / .scale_inv) and the pass-1 amax of
// the new first moment from the codes in registers ('coupled': Adam, which
// also reads the weight p3). Constants by value, or from kdev when not null.
hipError_t launch_quantize_pass1(int gfmt, bool coupled, const TensorDesc* desc, const ChunkRef* chunks,
                                 int64_t nchunks, msamp_meta* gmeta, const msamp_meta* mmeta, uint32_t* amax_m,
                                 const StepConsts& k, hipStream_t stream, const StepConsts* kdev = nullptr,
                                 bool wide = false);
hipError_t launch_step_pass1(int gfmt, bool coupled, const TensorDesc* desc, const ChunkRef* chunks,
                             int64_t nchunks, const msamp_meta* gmeta, const msamp_meta* mmeta,
                             uint32_t* amax_m, const StepConsts& k, hipStream_t stream,
                             const StepConsts* kdev = nullptr, bool wide = false);
// Ablation with a per-tensor-scaled FP16 second moment (O2 AdamW): pass 1
// also reduces amax(v1) into amax_v; pass 2 stores fp16(v1 * s_v).
hipError_t launch_scaled_v_pass1(int gfmt, const TensorDesc* desc, const ChunkRef* chunks,
                                 int64_t nchunks, const msamp_meta* gmeta, const msamp_meta* mmeta,
                                 const msamp_meta* vmeta, uint32_t* amax_m, uint32_t* amax_v,
                                 const StepConsts& k, hipStream_t stream);
hipError_t launch_scaled_v_pass2(int gfmt, const TensorDesc* desc, const ChunkRef* chunks,
                                 int64_t nchunks, const msamp_meta* gmeta, const msamp_meta* mmeta,
                                 const msamp_meta* vmeta, const uint32_t* amax_m,
                                 const uint32_t* amax_v, const StepConsts& k, hipStream_t stream);
hipError_t launch_step_pass2(int gfmt, bool o3, bool coupled, const TensorDesc* desc,
                             const ChunkRef* chunks, int64_t nchunks, const msamp_meta* gmeta,
                             const msamp_meta* mmeta, const uint32_t* amax_m, uint32_t* amax_w,
                             const StepConsts& k, hipStream_t stream,
                             const StepConsts* kdev = nullptr, const MetaFold& fold = MetaFold{},
                             bool wide = false, uint32_t split = 1);
// Ablation: the O2 update in one pass with delayed scaling of the first
// moment (encode with scale(mmeta.amax) of the previous step; reduce the new
// amax into amax_new).
hipError_t launch_step_delayed(int gfmt, bool coupled, const TensorDesc* desc, const ChunkRef* chunks,
                               int64_t nchunks, const msamp_meta* gmeta, const msamp_meta* mmeta,
                               uint32_t* amax_new, const StepConsts& k, hipStream_t stream);
// meta[t] <- {amax_new[t], s, 1/s} with s = scale(meta[t].amax) (the scale
// the delayed step used), then amax_new[t] <- 0.
hipError_t launch_delayed_finalize(int32_t n, uint32_t* amax_new, msamp_meta* meta,
                                   hipStream_t stream);
hipError_t launch_o3_pass3(const TensorDesc* desc, const ChunkRef* chunks, int64_t nchunks,
                           const uint32_t* amax_w, hipStream_t stream, const MetaFold& fold = MetaFold{},
                           bool wide = false, uint32_t split = 1);
// meta_a[t] <- {a, scale(a, 448), 1/scale, 0} with a = amax_a[t], then
// amax_a[t] <- 0; the same for (amax_b, meta_b) when meta_b is not NULL,
// with the range fmax_b (448 for an E4M3 copy, 65504 for a scaled FP16 v).
hipError_t launch_step_finalize(int32_t n, uint32_t* amax_a, msamp_meta* meta_a,
                                uint32_t* amax_b, msamp_meta* meta_b, float fmax_b,
                                hipStream_t stream);
// The fused quantize + pass 1's traffic without arithmetic, over a
// quantizing-step plan (writes unspecified values to the gradient codes).
hipError_t launch_qp1_probe(const TensorDesc* desc, const ChunkRef* chunks, int64_t nchunks, hipStream_t stream,
                            bool wide = false);
// Measurement streams: read 'bytes' from src, or copy them to dst (bytes a
// multiple of 16, 16-byte aligned pointers).
hipError_t launch_stream_probe(bool copy, const void* src, void* dst, int64_t bytes, hipStream_t stream);
hipError_t launch_codec_probe(int op, const void* in, void* out, int64_t n, hipStream_t stream);
// Split-phase steps: out[t] <- amax[t] as binary32 and amax[t] <- 0; and
// meta[t] <- {a, scale(a, fmax), 1/scale, 0} from a caller's amax array.
hipError_t launch_export_amax(int32_t n, uint32_t* amax, float* out, hipStream_t stream);
hipError_t launch_meta_from_amax(int32_t n, const float* amax, msamp_meta* meta, float fmax,
                                 hipStream_t stream);
// Reads g, m, v, w (roles p0..p3) and writes m, v, w back unchanged, with
// the same lanes, tiles and launch shape as the O2/O3 update pass.
hipError_t launch_rmw_probe(const TensorDesc* desc, const ChunkRef* chunks, int64_t nchunks,
                            hipStream_t stream, bool wide = false, uint32_t split = 1);

}  // namespace msamp
