// abi.hip -- the C ABI declared in include/msamp.h: argument validation,
// the multi-tensor-apply plan cache (descriptor tables and chunk maps in
// device memory, keyed on the tensor lists), host-side AdamW constants, the
// kernel sequence of each entry point, and optional event timing.
//
// No C++ exception crosses the interface: every entry point catches and maps
// failures to a status code with a per-thread message.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cstddef>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "kernels.hpp"
#include "msamp.h"

namespace msamp {
namespace {

thread_local std::string g_last_error;

msamp_status fail(msamp_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

msamp_status fail_hip(hipError_t e, const char* what) {
  std::string msg = std::string(what) + ": " + hipGetErrorString(e);
  return fail(MSAMP_E_HIP, msg);
}

#define MSAMP_TRY(expr)                 \
  do {                                  \
    msamp_status st__ = (expr);         \
    if (st__ != MSAMP_OK) return st__;  \
  } while (0)

// ------------------------------------------------------------ profiler ---

// Events created when timing is switched on (two per timed launch).
constexpr size_t kProfilerReserve = 4096;
// Timing events need no system-scope fence (nothing on the host reads the
// memory the kernels write through them); without it a record costs less.
constexpr unsigned kProfilerEventFlags = hipEventDisableSystemFence;

struct Profiler {
  std::mutex mu;
  bool enabled = false;
  uint32_t mask = 0xFFFFFFFFu;  // kernel kinds that are timed (bit = kind)
  struct Rec {
    int kind;
    hipEvent_t a, b;
  };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;

  hipEvent_t get_event() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, kProfilerEventFlags) != hipSuccess) return nullptr;
    return e;
  }
  void recycle_all() {
    for (auto& r : recs) {
      pool.push_back(r.a);
      pool.push_back(r.b);
    }
    recs.clear();
  }
};

Profiler& profiler() {
  static Profiler* p = new Profiler();  // never destroyed: events may outlive static teardown
  return *p;
}

// Runs 'launch' (which enqueues one kernel and returns its launch status),
// bracketed by events when profiling is on.
template <typename F>
hipError_t timed(msamp_kernel_kind kind, hipStream_t s, F&& launch) {
  Profiler& p = profiler();
  hipEvent_t a = nullptr, b = nullptr;
  bool on;
  {
    std::lock_guard<std::mutex> lk(p.mu);
    on = p.enabled && ((p.mask >> (int)kind) & 1u);
    if (on) {
      a = p.get_event();
      b = p.get_event();
    }
  }
  if (on && a && b) (void)hipEventRecord(a, s);
  hipError_t e = launch();
  if (on && a && b) {
    (void)hipEventRecord(b, s);
    std::lock_guard<std::mutex> lk(p.mu);
    p.recs.push_back({(int)kind, a, b});
  }
  return e;
}

// ---------------------------------------------------------- plan cache ---

enum PlanKind : uint64_t {
  kPlanAmax = 1, kPlanQuantize, kPlanDequantize, kPlanO2, kPlanO3, kPlanQuantizeO2, kPlanQuantizeO3,
  kPlanKinds  // one past the last kind
};

// Device tables of one tensor list: amax scratch (two u32 per tensor, kept
// at zero between calls), the descriptors and the chunk map, in one
// allocation uploaded once from pinned host memory.
struct Plan {
  int device = -1;
  std::vector<uint64_t> key;
  void* dev = nullptr;
  void* host = nullptr;
  size_t bytes = 0;
  uint32_t* scratch_a = nullptr;
  uint32_t* scratch_b = nullptr;
  uint32_t* done = nullptr;  // finished chunks per tensor (folded meta writes), zero between calls
  TensorDesc* desc = nullptr;
  ChunkRef* chunks = nullptr;
  int64_t nchunks = 0;
  // A large list's step plan also holds tables of kWideCoarseChunk-element
  // chunks, for pass 1 and the scaled-v ablation's pass 1 (null otherwise:
  // those use desc and chunks).
  TensorDesc* desc_coarse = nullptr;
  ChunkRef* chunks_coarse = nullptr;
  int64_t nchunks_coarse = 0;
  bool wide = false;  // one-tile chunks of kWideChunk for kWideBlock-thread step passes
  // Workgroups per chunk of the update pass and of the O3 copy (each
  // chunk's tiles split evenly between them), and whether those split
  // launches run kWideBlock-thread workgroups.
  uint32_t split_update = 1, split_copy = 1;
  bool wide_update = false, wide_copy = false;
  uint64_t last_use = 0;
  // Used by a launch captured into a graph: its memory stays until
  // msamp_unpin_captured_tables(), since a replay reads and writes it.
  bool pinned = false;

  ~Plan() {
    if (dev) (void)hipFree(dev);
    if (host) (void)hipHostFree(host);
  }
};

struct PlanCache {
  std::mutex mu;
  std::unordered_map<uint64_t, std::vector<std::unique_ptr<Plan>>> map;
  size_t count = 0;
  size_t bytes = 0;
  uint64_t tick = 0;
  // The plans each kind used last, most recent first: an optimizer passes
  // the same few lists every step (two gradient buffers, say), so a call
  // first compares its arrays with these in place.
  static constexpr int kRecent = 4;
  Plan* recent[kPlanKinds][kRecent] = {};

  void forget(const Plan* p) {
    for (auto& row : recent)
      for (Plan*& r : row)
        if (r == p) r = nullptr;
  }
  void touch(uint64_t kind, Plan* p) {
    Plan** row = recent[kind];
    int i = 0;
    while (i < kRecent - 1 && row[i] != p) ++i;
    for (; i > 0; --i) row[i] = row[i - 1];
    row[0] = p;
  }
};

PlanCache& cache() {
  static PlanCache* c = new PlanCache();
  return *c;
}

constexpr size_t kMaxPlans = 64;
constexpr size_t kMaxPlanBytes = size_t(512) << 20;

uint64_t hash_words(const std::vector<uint64_t>& w) {
  uint64_t h = 0x9E3779B97F4A7C15ull ^ (uint64_t)w.size();
  for (uint64_t x : w) {
    h ^= x + 0x9E3779B97F4A7C15ull + (h << 6) + (h >> 2);
    h *= 0xBF58476D1CE4E5B9ull;
    h ^= h >> 31;
  }
  return h;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Evicts least recently used plans until the cache is within bounds, never
// the most recently used one (it is being returned to a caller) and never a
// pinned one. Waits for the device first: an evicted table may still be read
// by queued work.
void evict_locked(PlanCache& c) {
  while (c.count > kMaxPlans || c.bytes > kMaxPlanBytes) {
    uint64_t best_tick = UINT64_MAX, best_hash = 0;
    size_t best_idx = 0;
    for (auto& kv : c.map)
      for (size_t i = 0; i < kv.second.size(); ++i)
        if (kv.second[i]->last_use < best_tick && kv.second[i]->last_use != c.tick && !kv.second[i]->pinned) {
          best_tick = kv.second[i]->last_use;
          best_hash = kv.first;
          best_idx = i;
        }
    if (best_tick == UINT64_MAX) return;
    auto& vec = c.map[best_hash];
    int cur = -1;
    (void)hipGetDevice(&cur);
    (void)hipSetDevice(vec[best_idx]->device);
    (void)hipDeviceSynchronize();
    c.bytes -= vec[best_idx]->bytes;
    c.count -= 1;
    c.forget(vec[best_idx].get());
    vec.erase(vec.begin() + (ptrdiff_t)best_idx);
    if (vec.empty()) c.map.erase(best_hash);
    if (cur >= 0) (void)hipSetDevice(cur);
  }
}

int64_t list_tiles(int32_t n, const int64_t* numel) {
  int64_t tiles = 0;
  for (int32_t t = 0; t < n; ++t) tiles += (numel[t] + kTile - 1) / kTile;
  return tiles;
}

// Elements per chunk of a list: whole tiles, fewer per chunk for a small
// list so that its launches still spread over every compute unit.
int64_t list_chunk_elems(int32_t n, const int64_t* numel) { return chunk_tiles_for(list_tiles(n, numel)) * kTile; }

bool is_step_plan(uint64_t kind) {
  return kind == kPlanO2 || kind == kPlanO3 || kind == kPlanQuantizeO2 || kind == kPlanQuantizeO3;
}

// Lists of at most this many chunks write their meta records from the
// workgroup that completes each tensor (one launch fewer per pass that ends
// in meta: the launch costs more than the work there); larger lists keep a
// finalize launch, which avoids one counter atomic per workgroup.
constexpr int64_t kFoldMaxChunks = 8192;

// Workgroups per chunk of the update pass and of the O3 copy in a list of
// 16-tile chunks (a large list's step plan has one-tile chunks already), of
// kSplitBlock threads: one tile each, or, for a list that folds its meta
// writes (each workgroup then also counts itself), about kSplitTarget
// workgroups in all.
constexpr int kSplitBlock = kWideBlock;
constexpr int64_t kSplitTarget = 16384;

// Workgroups of a launch over 'ce'-element chunks split 's' ways that get no
// elements (the parts past each tensor's end).
int64_t empty_parts(int32_t n, const int64_t* numel, int64_t ce, uint32_t s) {
  const int64_t span = ce / s;
  int64_t empty = 0;
  for (int32_t t = 0; t < n; ++t) {
    const int64_t chunks = std::max<int64_t>(1, (numel[t] + ce - 1) / ce);
    empty += chunks * s - (numel[t] + span - 1) / span;
  }
  return empty;
}

// The largest power of two <= want that divides the chunk's tiles (of
// 'block' threads), keeps the launch within 2^32 - 1 threads and leaves at
// most an eighth of the workgroups without elements.
uint32_t fit_split(uint32_t want, int32_t n, const int64_t* numel, int64_t ce, int64_t nchunks, int block) {
  const int64_t tiles = ce / ((int64_t)block * 16);
  uint32_t s = 1;
  while (s * 2 <= want && tiles % (s * 2) == 0 && nchunks * (int64_t)(s * 2) * block <= (int64_t)UINT32_MAX &&
         empty_parts(n, numel, ce, s * 2) * 8 <= nchunks * (int64_t)(s * 2))
    s *= 2;
  return s;
}

// Measured on gfx950: smaller workgroups help the passes without a
// per-workgroup amax reduction (O2 update, O3 copy); the fused pass, pass 1
// and the O3 update, which reduce an amax in every workgroup, ran slower
// with one-tile workgroups on lists of this size.
void choose_splits(Plan* p, uint64_t kind, int32_t n, const int64_t* numel, int64_t ce) {
  if (!is_step_plan(kind) || p->wide || ce != kMaxChunkTiles * kTile) return;
  const uint32_t tiles = (uint32_t)(ce / ((int64_t)kSplitBlock * 16));
  const bool fold = p->nchunks <= kFoldMaxChunks;
  uint32_t want = tiles;
  if (fold) {
    want = 1;
    while (want < tiles && p->nchunks * (int64_t)want * 2 <= kSplitTarget) want *= 2;
  }
  const bool o3 = kind == kPlanO3 || kind == kPlanQuantizeO3;
  if (!o3) p->split_update = fit_split(want, n, numel, ce, p->nchunks, kSplitBlock);
  if (o3 && !fold) p->split_copy = fit_split(tiles, n, numel, ce, p->nchunks, kSplitBlock);
  p->wide_update = kSplitBlock == kWideBlock && p->split_update > 1;
  p->wide_copy = kSplitBlock == kWideBlock && p->split_copy > 1;
}

// True if 'p' was built for exactly these arrays: the same kind, tensor
// count, sizes and role pointers (compared in place, without a key).
bool same_list(const Plan* p, uint64_t kind, int32_t n, const int64_t* numel,
               const void* const* const* ptrs, int nroles) {
  static_assert(sizeof(void*) == sizeof(uint64_t) && sizeof(int64_t) == sizeof(uint64_t), "64-bit words");
  const std::vector<uint64_t>& k = p->key;
  const size_t nn = (size_t)n;
  if (k.size() != 3 + nn * (1 + (size_t)nroles) || k[0] != kind || k[2] != (uint64_t)n) return false;
  if (std::memcmp(&k[3], numel, nn * sizeof(uint64_t)) != 0) return false;
  for (int r = 0; r < nroles; ++r) {
    const uint64_t* seg = &k[3 + nn * (1 + (size_t)r)];
    if (ptrs[r] != nullptr) {
      if (std::memcmp(seg, ptrs[r], nn * sizeof(uint64_t)) != 0) return false;
    } else {
      for (size_t t = 0; t < nn; ++t)
        if (seg[t] != 0) return false;
    }
  }
  return true;
}

bool stream_capturing(hipStream_t stream) {
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &capture) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return capture != hipStreamCaptureStatusNone;
}

msamp_status check_list(int32_t n, const int64_t* numel, const void* const* ptrs, const char* role);
msamp_status check_sizes(int32_t n, const int64_t* numel);

// The chunk map of a list: (tensor, chunk) for every 'ce'-element chunk,
// and one (empty) chunk for an empty tensor when 'min_one_chunk'.
msamp_status build_chunk_map(int32_t n, const int64_t* numel, int64_t ce, bool min_one_chunk,
                             std::vector<ChunkRef>* out) {
  int64_t total = 0;
  for (int32_t t = 0; t < n; ++t) {
    int64_t k = (numel[t] + ce - 1) / ce;
    if (k == 0 && min_one_chunk) k = 1;
    if (k > INT32_MAX) return fail(MSAMP_E_INVALID_ARG, "tensor too large for the chunk map");
    total += k;
  }
  if (total > (int64_t)INT32_MAX) return fail(MSAMP_E_INVALID_ARG, "too many chunks for one launch");
  out->reserve((size_t)total);
  for (int32_t t = 0; t < n; ++t) {
    int64_t k = (numel[t] + ce - 1) / ce;
    if (k == 0 && min_one_chunk) k = 1;
    for (int64_t j = 0; j < k; ++j) out->push_back({t, (int32_t)j});
  }
  return MSAMP_OK;
}

// Returns the plan of a tensor list, building and uploading it (on 'stream')
// the first time. 'ptrs' holds 'nroles' pointer arrays (each of length n, or
// null for a role the operation does not have, whose name is then null too):
// roles 0..4 fill p0..p4 of the descriptors and role 5 fills aux;
// 'min_one_chunk' gives every tensor at least one (possibly empty) chunk.
// The per-tensor checks (sizes >= 0; pointers non-null where numel > 0 and
// 16-byte aligned) run here, before any device call, for a list other than
// those this kind used last: a list equal to a cached plan's passed them
// when that plan was built.
// On success '*lease' holds the cache lock: the caller keeps it until its
// launches are enqueued, so that no other thread can evict (and free) the
// plan in between.
msamp_status get_plan(uint64_t kind, int32_t n, const int64_t* numel,
                      const void* const* const* ptrs, const char* const* names, int nroles,
                      bool min_one_chunk, hipStream_t stream, Plan** out,
                      std::unique_lock<std::mutex>* lease) {
  PlanCache& c = cache();
  bool arrays_present = true;
  for (int r = 0; r < nroles; ++r)
    if (names[r] != nullptr && ptrs[r] == nullptr) arrays_present = false;
  if (arrays_present) {
    std::unique_lock<std::mutex> lk(c.mu);
    for (int i = 0; i < PlanCache::kRecent; ++i) {
      Plan* r = c.recent[kind][i];
      if (r == nullptr || !same_list(r, kind, n, numel, ptrs, nroles)) continue;
      int dev = 0;
      hipError_t e = hipGetDevice(&dev);
      if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
      if ((uint64_t)dev != r->key[1]) continue;
      if (stream_capturing(stream)) r->pinned = true;
      r->last_use = ++c.tick;
      c.touch(kind, r);
      *out = r;
      *lease = std::move(lk);
      return MSAMP_OK;
    }
  }
  MSAMP_TRY(check_sizes(n, numel));
  for (int r = 0; r < nroles; ++r)
    if (names[r] != nullptr) MSAMP_TRY(check_list(n, numel, ptrs[r], names[r]));

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");

  std::vector<uint64_t> key;
  key.reserve(3 + (size_t)n * (1 + nroles));
  key.push_back(kind);
  key.push_back((uint64_t)dev);
  key.push_back((uint64_t)n);
  for (int32_t t = 0; t < n; ++t) key.push_back((uint64_t)numel[t]);
  for (int r = 0; r < nroles; ++r)
    for (int32_t t = 0; t < n; ++t) key.push_back(ptrs[r] ? (uint64_t)(uintptr_t)ptrs[r][t] : 0u);
  const uint64_t h = hash_words(key);

  // A launch being captured into a graph keeps the plan's addresses: pin it.
  const bool capturing = stream_capturing(stream);

  std::unique_lock<std::mutex> lk(c.mu);
  auto it = c.map.find(h);
  if (it != c.map.end()) {
    for (auto& p : it->second)
      if (p->key == key) {
        p->last_use = ++c.tick;
        if (capturing) p->pinned = true;
        c.touch(kind, p.get());
        *out = p.get();
        *lease = std::move(lk);
        return MSAMP_OK;
      }
  }

  // Build the chunk map: chunks of list_chunk_elems elements; for a large
  // list, one tile per workgroup in the step passes (kWideChunk, wide
  // workgroups) and in the casts (kTile: quantize 6.25 -> 5.46 ms and
  // dequantize 6.65 -> 5.7 ms on the 7B list against 16-tile chunks).
  const bool large = list_tiles(n, numel) >= kWideMinTiles;
  const bool wide = is_step_plan(kind) && large;
  const bool casts = kind == kPlanQuantize || kind == kPlanDequantize;
  const int64_t ce = wide ? kWideChunk : (large && casts) ? kTile : list_chunk_elems(n, numel);
  std::vector<ChunkRef> chunks, coarse;
  MSAMP_TRY(build_chunk_map(n, numel, ce, min_one_chunk, &chunks));
  if (wide) MSAMP_TRY(build_chunk_map(n, numel, kWideCoarseChunk, min_one_chunk, &coarse));

  auto plan = std::make_unique<Plan>();
  plan->device = dev;
  plan->key = std::move(key);
  const size_t scratch_bytes = align_up(sizeof(uint32_t) * 3 * (size_t)std::max(n, 1), 256);
  const size_t desc_bytes = align_up(sizeof(TensorDesc) * (size_t)std::max(n, 1), 256);
  const size_t chunk_bytes = align_up(sizeof(ChunkRef) * std::max<size_t>(chunks.size(), 1), 256);
  const size_t coarse_bytes = wide ? desc_bytes + align_up(sizeof(ChunkRef) * std::max<size_t>(coarse.size(), 1), 256) : 0;
  plan->bytes = scratch_bytes + desc_bytes + chunk_bytes + coarse_bytes;

  e = hipMalloc(&plan->dev, plan->bytes);
  if (e != hipSuccess) {
    plan->dev = nullptr;
    (void)hipGetLastError();
    return fail(MSAMP_E_NO_MEMORY, "hipMalloc of the descriptor tables failed");
  }
  e = hipHostMalloc(&plan->host, plan->bytes, hipHostMallocDefault);
  if (e != hipSuccess) {
    plan->host = nullptr;
    (void)hipGetLastError();
    return fail(MSAMP_E_NO_MEMORY, "hipHostMalloc of the descriptor staging failed");
  }
  char* hb = (char*)plan->host;
  std::memset(hb, 0, plan->bytes);
  TensorDesc* hd = (TensorDesc*)(hb + scratch_bytes);
  for (int32_t t = 0; t < n; ++t) {
    TensorDesc d;
    std::memset(&d, 0, sizeof d);
    d.numel = numel[t];
    d.chunk = ce;
    const void* p[6] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
    for (int r = 0; r < nroles && r < 6; ++r) p[r] = ptrs[r] ? ptrs[r][t] : nullptr;
    d.p0 = p[0];
    d.p1 = const_cast<void*>(p[1]);
    d.p2 = const_cast<void*>(p[2]);
    d.p3 = const_cast<void*>(p[3]);
    d.p4 = const_cast<void*>(p[4]);
    d.aux = p[5];
    hd[t] = d;
  }
  if (!chunks.empty())
    std::memcpy(hb + scratch_bytes + desc_bytes, chunks.data(), chunks.size() * sizeof(ChunkRef));
  const size_t coarse_at = scratch_bytes + desc_bytes + chunk_bytes;
  if (wide) {
    TensorDesc* hc = (TensorDesc*)(hb + coarse_at);
    for (int32_t t = 0; t < n; ++t) {
      hc[t] = hd[t];
      hc[t].chunk = kWideCoarseChunk;
    }
    if (!coarse.empty())
      std::memcpy(hb + coarse_at + desc_bytes, coarse.data(), coarse.size() * sizeof(ChunkRef));
  }

  char* db = (char*)plan->dev;
  plan->scratch_a = (uint32_t*)db;
  plan->scratch_b = (uint32_t*)db + std::max(n, 1);
  plan->done = (uint32_t*)db + 2 * (size_t)std::max(n, 1);
  plan->desc = (TensorDesc*)(db + scratch_bytes);
  plan->chunks = (ChunkRef*)(db + scratch_bytes + desc_bytes);
  plan->nchunks = (int64_t)chunks.size();
  if (wide) {
    plan->desc_coarse = (TensorDesc*)(db + coarse_at);
    plan->chunks_coarse = (ChunkRef*)(db + coarse_at + desc_bytes);
    plan->nchunks_coarse = (int64_t)coarse.size();
  }
  plan->wide = wide;
  choose_splits(plan.get(), kind, n, numel, ce);

  e = hipMemcpyAsync(plan->dev, plan->host, plan->bytes, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return fail_hip(e, "upload of the descriptor tables");

  plan->last_use = ++c.tick;
  plan->pinned = capturing;
  c.touch(kind, plan.get());
  *out = plan.get();
  c.bytes += plan->bytes;
  c.count += 1;
  c.map[h].push_back(std::move(plan));
  // Never evict the plan just returned: it is the most recently used.
  evict_locked(c);
  *lease = std::move(lk);
  return MSAMP_OK;
}

// --------------------------------------------------------- validation ---

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

msamp_status check_list(int32_t n, const int64_t* numel, const void* const* ptrs,
                        const char* role) {
  if (ptrs == nullptr) return fail(MSAMP_E_INVALID_ARG, std::string(role) + " array is NULL");
  for (int32_t t = 0; t < n; ++t) {
    if (numel[t] == 0) continue;
    if (ptrs[t] == nullptr)
      return fail(MSAMP_E_INVALID_ARG,
                  std::string(role) + "[" + std::to_string(t) + "] is NULL with numel > 0");
    if (!aligned16(ptrs[t]))
      return fail(MSAMP_E_MISALIGNED,
                  std::string(role) + "[" + std::to_string(t) + "] is not 16-byte aligned");
  }
  return MSAMP_OK;
}

// The tensor count and the sizes array (the sizes themselves are checked by
// check_sizes, which get_plan runs for a list it has not just seen).
msamp_status check_count(int32_t n, const int64_t* numel) {
  if (n < 0) return fail(MSAMP_E_INVALID_ARG, "n < 0");
  if (n > 0 && numel == nullptr) return fail(MSAMP_E_INVALID_ARG, "numel array is NULL");
  return MSAMP_OK;
}

msamp_status check_sizes(int32_t n, const int64_t* numel) {
  for (int32_t t = 0; t < n; ++t)
    if (numel[t] < 0) return fail(MSAMP_E_INVALID_ARG, "numel[" + std::to_string(t) + "] < 0");
  return MSAMP_OK;
}

msamp_status check_common(int32_t n, const int64_t* numel) {
  MSAMP_TRY(check_count(n, numel));
  return check_sizes(n, numel);
}

msamp_status check_fmt(int fmt) {
  if (fmt != MSAMP_FP8_E4M3 && fmt != MSAMP_FP8_E5M2)
    return fail(MSAMP_E_INVALID_ARG, "unknown FP8 format");
  return MSAMP_OK;
}

msamp_status check_meta(int32_t n, const void* meta, const char* role) {
  if (n > 0 && meta == nullptr) return fail(MSAMP_E_INVALID_ARG, std::string(role) + " is NULL");
  if (n > 0 && !aligned16(meta))
    return fail(MSAMP_E_MISALIGNED, std::string(role) + " is not 16-byte aligned");
  return MSAMP_OK;
}

msamp_status check_hparams(const msamp_adamw_hparams* hp, int64_t step) {
  if (hp == nullptr) return fail(MSAMP_E_INVALID_ARG, "hparams is NULL");
  if (step < 1) return fail(MSAMP_E_INVALID_ARG, "step must be >= 1");
  auto fin = [](double x) { return std::isfinite(x); };
  if (!fin(hp->lr) || hp->lr < 0.0) return fail(MSAMP_E_INVALID_ARG, "lr must be finite and >= 0");
  if (!fin(hp->beta1) || hp->beta1 < 0.0 || hp->beta1 >= 1.0)
    return fail(MSAMP_E_INVALID_ARG, "beta1 must be in [0, 1)");
  if (!fin(hp->beta2) || hp->beta2 < 0.0 || hp->beta2 >= 1.0)
    return fail(MSAMP_E_INVALID_ARG, "beta2 must be in [0, 1)");
  if (!fin(hp->eps) || !(hp->eps > 0.0)) return fail(MSAMP_E_INVALID_ARG, "eps must be > 0");
  if (!fin(hp->weight_decay) || hp->weight_decay < 0.0)
    return fail(MSAMP_E_INVALID_ARG, "weight_decay must be finite and >= 0");
  return MSAMP_OK;
}

// AdamW / Adam constants: binary64 expressions, each rounded once to
// binary32. Adam (coupled L2) has no decoupled decay: dec is exactly 1.
StepConsts make_consts(const msamp_adamw_hparams* hp, int64_t step, bool coupled) {
  const double t = (double)step;
  const double bc1 = 1.0 - std::pow(hp->beta1, t);
  const double bc2 = 1.0 - std::pow(hp->beta2, t);
  StepConsts k;
  k.b1 = (float)hp->beta1;
  k.ob1 = (float)(1.0 - hp->beta1);
  k.b2 = (float)hp->beta2;
  k.ob2 = (float)(1.0 - hp->beta2);
  k.eps = (float)hp->eps;
  k.ss = (float)(hp->lr / bc1);
  k.ibs = (float)(1.0 / std::sqrt(bc2));
  k.dec = coupled ? 1.0f : (float)(1.0 - hp->lr * hp->weight_decay);
  k.wd = (float)hp->weight_decay;
  return k;
}

#define MSAMP_LAUNCH(kind, stream, call)                                   \
  do {                                                                     \
    hipError_t e__ = timed((kind), (stream), [&]() { return (call); });   \
    if (e__ != hipSuccess) return fail_hip(e__, msamp_kernel_name(kind));  \
  } while (0)

bool wide_launch(const Plan* p) { return p->wide; }
bool wide_update(const Plan* p) { return p->wide || p->wide_update; }
bool wide_copy(const Plan* p) { return p->wide || p->wide_copy; }

// Tables for pass 1: workgroups of 16 wide tiles on a large list (pass 1
// reads 2 B/p and reduces an amax in every workgroup; one-tile workgroups
// made it slower), the plan's own tables otherwise.
struct Tables {
  const TensorDesc* desc;
  const ChunkRef* chunks;
  int64_t nchunks;
};
Tables pass1_tables(const Plan* p) {
  if (p->desc_coarse != nullptr) return {p->desc_coarse, p->chunks_coarse, p->nchunks_coarse};
  return {p->desc, p->chunks, p->nchunks};
}

// The meta writes of a step folded into its last pass (pass 2 for O2,
// pass 3 for O3), or none for a large list.
MetaFold step_fold(const Plan* p, bool o3, msamp_meta* exp_avg_meta, msamp_meta* weight_fp8_meta) {
  MetaFold f;
  if (p->nchunks > kFoldMaxChunks) return f;
  f.done = p->done;
  f.meta_a = exp_avg_meta;
  f.amax_a = p->scratch_a;
  if (o3) {
    f.meta_b = weight_fp8_meta;
    f.amax_b = p->scratch_b;
  }
  return f;
}

// The tensor lists and meta arrays of an O2 (o3 = false) or O3 step.
msamp_status check_step_lists(bool o3, int32_t n, const int64_t* numel, const uint8_t* const* grad,
                              const msamp_meta* grad_meta, uint8_t* const* exp_avg,
                              const msamp_meta* exp_avg_meta, uint16_t* const* exp_avg_sq,
                              uint16_t* const* weight, uint8_t* const* weight_fp8,
                              const msamp_meta* weight_fp8_meta) {
  MSAMP_TRY(check_list(n, numel, (const void* const*)grad, "grad"));
  MSAMP_TRY(check_list(n, numel, (const void* const*)exp_avg, "exp_avg"));
  MSAMP_TRY(check_list(n, numel, (const void* const*)exp_avg_sq, "exp_avg_sq"));
  MSAMP_TRY(check_list(n, numel, (const void* const*)weight, o3 ? "master" : "weight"));
  MSAMP_TRY(check_meta(n, grad_meta, "grad_meta"));
  MSAMP_TRY(check_meta(n, exp_avg_meta, "exp_avg_meta"));
  if (o3) {
    MSAMP_TRY(check_list(n, numel, (const void* const*)weight_fp8, "weight_fp8"));
    MSAMP_TRY(check_meta(n, weight_fp8_meta, "weight_fp8_meta"));
  }
  return MSAMP_OK;
}

// The meta arrays of an O2 (o3 = false) or O3 step (get_plan checks the
// tensor lists).
msamp_status check_step_meta(bool o3, int32_t n, const msamp_meta* grad_meta, const msamp_meta* exp_avg_meta,
                             const msamp_meta* weight_fp8_meta) {
  MSAMP_TRY(check_meta(n, grad_meta, "grad_meta"));
  MSAMP_TRY(check_meta(n, exp_avg_meta, "exp_avg_meta"));
  if (o3) MSAMP_TRY(check_meta(n, weight_fp8_meta, "weight_fp8_meta"));
  return MSAMP_OK;
}

// The cached tables of a step's tensor lists (the same plan for every
// entry point that takes these lists).
msamp_status step_plan(bool o3, int32_t n, const int64_t* numel, const uint8_t* const* grad,
                       uint8_t* const* exp_avg, uint16_t* const* exp_avg_sq, uint16_t* const* weight,
                       uint8_t* const* weight_fp8, hipStream_t s, Plan** p,
                       std::unique_lock<std::mutex>* lease) {
  const void* const* roles[5] = {(const void* const*)grad, (const void* const*)exp_avg,
                                 (const void* const*)exp_avg_sq, (const void* const*)weight,
                                 (const void* const*)weight_fp8};
  const char* names[5] = {"grad", "exp_avg", "exp_avg_sq", o3 ? "master" : "weight", "weight_fp8"};
  return get_plan(o3 ? kPlanO3 : kPlanO2, n, numel, roles, names, o3 ? 5 : 4, true, s, p, lease);
}

msamp_status check_amax_array(int32_t n, const float* a, const char* role) {
  if (n > 0 && a == nullptr) return fail(MSAMP_E_INVALID_ARG, std::string(role) + " is NULL");
  if (((uintptr_t)a & 3u) != 0) return fail(MSAMP_E_MISALIGNED, std::string(role) + " is not 4-byte aligned");
  return MSAMP_OK;
}

msamp_status step_impl(bool o3, bool coupled, int32_t n, const int64_t* numel, const uint8_t* const* grad,
                       int grad_fmt, const msamp_meta* grad_meta, uint8_t* const* exp_avg,
                       msamp_meta* exp_avg_meta, uint16_t* const* exp_avg_sq,
                       uint16_t* const* weight, uint8_t* const* weight_fp8,
                       msamp_meta* weight_fp8_meta, const msamp_adamw_hparams* hp, int64_t step,
                       void* stream_ptr, const StepConsts* kdev = nullptr) {
  g_last_error.clear();
  MSAMP_TRY(check_count(n, numel));
  if (n == 0) return MSAMP_OK;
  MSAMP_TRY(check_fmt(grad_fmt));
  if (kdev == nullptr) {
    MSAMP_TRY(check_hparams(hp, step));
  } else if (((uintptr_t)kdev & 3u) != 0) {
    return fail(MSAMP_E_MISALIGNED, "consts is not 4-byte aligned");
  }
  MSAMP_TRY(check_step_meta(o3, n, grad_meta, exp_avg_meta, weight_fp8_meta));
  hipStream_t s = (hipStream_t)stream_ptr;
  Plan* p = nullptr;
  std::unique_lock<std::mutex> lease;  // held until the launches are enqueued
  MSAMP_TRY(step_plan(o3, n, numel, grad, exp_avg, exp_avg_sq, weight, weight_fp8, s, &p, &lease));
  const StepConsts k = kdev == nullptr ? make_consts(hp, step, coupled) : StepConsts{};

  const Tables t1 = pass1_tables(p);
  MSAMP_LAUNCH(MSAMP_KERNEL_STEP_PASS1, s,
               launch_step_pass1(grad_fmt, coupled, t1.desc, t1.chunks, t1.nchunks, grad_meta,
                                 exp_avg_meta, p->scratch_a, k, s, kdev, wide_launch(p)));
  const MetaFold fold = step_fold(p, o3, exp_avg_meta, weight_fp8_meta);
  MSAMP_LAUNCH(o3 ? MSAMP_KERNEL_O3_PASS2 : MSAMP_KERNEL_O2_PASS2, s,
               launch_step_pass2(grad_fmt, o3, coupled, p->desc, p->chunks, p->nchunks, grad_meta,
                                 exp_avg_meta, p->scratch_a, p->scratch_b, k, s, kdev, o3 ? MetaFold{} : fold,
                                 wide_update(p), p->split_update));
  if (o3)
    MSAMP_LAUNCH(MSAMP_KERNEL_O3_PASS3, s,
                 launch_o3_pass3(p->desc, p->chunks, p->nchunks, p->scratch_b, s, fold, wide_copy(p),
                                 p->split_copy));
  if (fold.done == nullptr)
    MSAMP_LAUNCH(MSAMP_KERNEL_FINALIZE, s,
                 launch_step_finalize(n, p->scratch_a, exp_avg_meta, o3 ? p->scratch_b : nullptr,
                                      o3 ? weight_fp8_meta : nullptr, 448.0f, s));
  return MSAMP_OK;
}

// Gradient quantize + AdamW step (O2 or O3) with the quantize fused into
// pass 1; the rest is the step's sequence.
msamp_status quantize_step_impl(bool o3, bool coupled, int32_t n, const int64_t* numel,
                                const float* const* grad_f32, int grad_fmt, msamp_meta* grad_meta,
                                uint8_t* const* grad, uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                uint16_t* const* exp_avg_sq, uint16_t* const* weight,
                                uint8_t* const* weight_fp8, msamp_meta* weight_fp8_meta,
                                const msamp_adamw_hparams* hp, int64_t step, void* stream_ptr,
                                const StepConsts* kdev = nullptr) {
  g_last_error.clear();
  MSAMP_TRY(check_count(n, numel));
  if (n == 0) return MSAMP_OK;
  MSAMP_TRY(check_fmt(grad_fmt));
  if (kdev == nullptr) {
    MSAMP_TRY(check_hparams(hp, step));
  } else if (((uintptr_t)kdev & 3u) != 0) {
    return fail(MSAMP_E_MISALIGNED, "consts is not 4-byte aligned");
  }
  MSAMP_TRY(check_step_meta(o3, n, grad_meta, exp_avg_meta, weight_fp8_meta));
  hipStream_t s = (hipStream_t)stream_ptr;
  const void* const* roles[6] = {(const void* const*)grad,       (const void* const*)exp_avg,
                                 (const void* const*)exp_avg_sq, (const void* const*)weight,
                                 (const void* const*)weight_fp8, (const void* const*)grad_f32};
  const char* names[6] = {"grad", "exp_avg", "exp_avg_sq", o3 ? "master" : "weight", "weight_fp8", "grad_f32"};
  if (!o3) {
    roles[4] = nullptr;
    names[4] = nullptr;
  }
  Plan* p = nullptr;
  std::unique_lock<std::mutex> lease;  // held until the launches are enqueued
  MSAMP_TRY(get_plan(o3 ? kPlanQuantizeO3 : kPlanQuantizeO2, n, numel, roles, names, 6, true, s, &p, &lease));
  const StepConsts k = kdev == nullptr ? make_consts(hp, step, coupled) : StepConsts{};
  MSAMP_LAUNCH(MSAMP_KERNEL_QUANTIZE_PASS1, s,
               launch_quantize_pass1(grad_fmt, coupled, p->desc, p->chunks, p->nchunks, grad_meta, exp_avg_meta,
                                     p->scratch_a, k, s, kdev, wide_launch(p)));
  const MetaFold fold = step_fold(p, o3, exp_avg_meta, weight_fp8_meta);
  MSAMP_LAUNCH(o3 ? MSAMP_KERNEL_O3_PASS2 : MSAMP_KERNEL_O2_PASS2, s,
               launch_step_pass2(grad_fmt, o3, coupled, p->desc, p->chunks, p->nchunks, grad_meta,
                                 exp_avg_meta, p->scratch_a, p->scratch_b, k, s, kdev,
                                 o3 ? MetaFold{} : fold, wide_update(p), p->split_update));
  if (o3)
    MSAMP_LAUNCH(MSAMP_KERNEL_O3_PASS3, s,
                 launch_o3_pass3(p->desc, p->chunks, p->nchunks, p->scratch_b, s, fold, wide_copy(p),
                                 p->split_copy));
  if (fold.done == nullptr)
    MSAMP_LAUNCH(MSAMP_KERNEL_FINALIZE, s,
                 launch_step_finalize(n, p->scratch_a, exp_avg_meta, o3 ? p->scratch_b : nullptr,
                                      o3 ? weight_fp8_meta : nullptr, 448.0f, s));
  return MSAMP_OK;
}

// Ablation: O2 AdamW step with a per-tensor-scaled FP16 second moment.
msamp_status step_scaled_v_impl(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                int grad_fmt, const msamp_meta* grad_meta, uint8_t* const* exp_avg,
                                msamp_meta* exp_avg_meta, uint16_t* const* exp_avg_sq,
                                msamp_meta* exp_avg_sq_meta, uint16_t* const* weight,
                                const msamp_adamw_hparams* hp, int64_t step, void* stream_ptr) {
  g_last_error.clear();
  MSAMP_TRY(check_count(n, numel));
  if (n == 0) return MSAMP_OK;
  MSAMP_TRY(check_fmt(grad_fmt));
  MSAMP_TRY(check_hparams(hp, step));
  MSAMP_TRY(check_meta(n, grad_meta, "grad_meta"));
  MSAMP_TRY(check_meta(n, exp_avg_meta, "exp_avg_meta"));
  MSAMP_TRY(check_meta(n, exp_avg_sq_meta, "exp_avg_sq_meta"));
  hipStream_t s = (hipStream_t)stream_ptr;
  const void* const* roles[4] = {(const void* const*)grad, (const void* const*)exp_avg,
                                 (const void* const*)exp_avg_sq, (const void* const*)weight};
  Plan* p = nullptr;
  std::unique_lock<std::mutex> lease;  // held until the launches are enqueued
  const char* names[4] = {"grad", "exp_avg", "exp_avg_sq", "weight"};
  MSAMP_TRY(get_plan(kPlanO2, n, numel, roles, names, 4, true, s, &p, &lease));
  const StepConsts k = make_consts(hp, step, false);
  const Tables t1 = pass1_tables(p);
  MSAMP_LAUNCH(MSAMP_KERNEL_STEP_PASS1, s,
               launch_scaled_v_pass1(grad_fmt, t1.desc, t1.chunks, t1.nchunks, grad_meta,
                                     exp_avg_meta, exp_avg_sq_meta, p->scratch_a, p->scratch_b, k, s));
  MSAMP_LAUNCH(MSAMP_KERNEL_O2_PASS2, s,
               launch_scaled_v_pass2(grad_fmt, p->desc, p->chunks, p->nchunks, grad_meta,
                                     exp_avg_meta, exp_avg_sq_meta, p->scratch_a, p->scratch_b, k, s));
  MSAMP_LAUNCH(MSAMP_KERNEL_FINALIZE, s,
               launch_step_finalize(n, p->scratch_a, exp_avg_meta, p->scratch_b, exp_avg_sq_meta,
                                    65504.0f, s));
  return MSAMP_OK;
}

// Ablation: one-pass O2 step with delayed scaling of the first moment.
msamp_status step_delayed_impl(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                               int grad_fmt, const msamp_meta* grad_meta, uint8_t* const* exp_avg,
                               msamp_meta* exp_avg_meta, uint16_t* const* exp_avg_sq,
                               uint16_t* const* weight, const msamp_adamw_hparams* hp,
                               int64_t step, void* stream_ptr) {
  g_last_error.clear();
  MSAMP_TRY(check_count(n, numel));
  if (n == 0) return MSAMP_OK;
  MSAMP_TRY(check_fmt(grad_fmt));
  MSAMP_TRY(check_hparams(hp, step));
  MSAMP_TRY(check_meta(n, grad_meta, "grad_meta"));
  MSAMP_TRY(check_meta(n, exp_avg_meta, "exp_avg_meta"));
  hipStream_t s = (hipStream_t)stream_ptr;
  const void* const* roles[4] = {(const void* const*)grad, (const void* const*)exp_avg,
                                 (const void* const*)exp_avg_sq, (const void* const*)weight};
  Plan* p = nullptr;
  std::unique_lock<std::mutex> lease;  // held until the launches are enqueued
  const char* names[4] = {"grad", "exp_avg", "exp_avg_sq", "weight"};
  MSAMP_TRY(get_plan(kPlanO2, n, numel, roles, names, 4, true, s, &p, &lease));
  const StepConsts k = make_consts(hp, step, false);
  MSAMP_LAUNCH(MSAMP_KERNEL_O2_DELAYED, s,
               launch_step_delayed(grad_fmt, false, p->desc, p->chunks, p->nchunks, grad_meta,
                                   exp_avg_meta, p->scratch_a, k, s));
  MSAMP_LAUNCH(MSAMP_KERNEL_FINALIZE, s, launch_delayed_finalize(n, p->scratch_a, exp_avg_meta, s));
  return MSAMP_OK;
}

template <typename F>
msamp_status guarded(F&& f) {
  try {
    return f();
  } catch (const std::bad_alloc&) {
    return fail(MSAMP_E_NO_MEMORY, "host allocation failed");
  } catch (const std::exception& ex) {
    return fail(MSAMP_E_INVALID_ARG, std::string("internal error: ") + ex.what());
  } catch (...) {
    return fail(MSAMP_E_INVALID_ARG, "internal error");
  }
}

// Split-phase step for a flat intra-tensor partition (each rank holds a
// slice of every tensor): phase 1 exports the local amax of the new first
// moment; phase 2 takes the ranks' MAX of it (O3: and exports the local
// amax of the new master); phase 3 (O3) takes the MAX of that.
msamp_status phase_impl(int phase, bool o3, bool coupled, int32_t n, const int64_t* numel,
                        const uint8_t* const* grad, int grad_fmt, const msamp_meta* grad_meta,
                        uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                        uint16_t* const* exp_avg_sq, uint16_t* const* weight,
                        uint8_t* const* weight_fp8, msamp_meta* weight_fp8_meta,
                        const msamp_adamw_hparams* hp, int64_t step, float* amax_out,
                        const float* amax_in, void* stream_ptr) {
  g_last_error.clear();
  MSAMP_TRY(check_count(n, numel));
  if (n == 0) return MSAMP_OK;
  MSAMP_TRY(check_fmt(grad_fmt));
  if (phase != 3) MSAMP_TRY(check_hparams(hp, step));
  MSAMP_TRY(check_step_meta(o3, n, grad_meta, exp_avg_meta, weight_fp8_meta));
  if (phase == 1 || (phase == 2 && o3)) MSAMP_TRY(check_amax_array(n, amax_out, "amax output"));
  if (phase >= 2) MSAMP_TRY(check_amax_array(n, amax_in, "amax input"));
  hipStream_t s = (hipStream_t)stream_ptr;
  Plan* p = nullptr;
  std::unique_lock<std::mutex> lease;  // held until the launches are enqueued
  MSAMP_TRY(step_plan(o3, n, numel, grad, exp_avg, exp_avg_sq, weight, weight_fp8, s, &p, &lease));
  if (phase == 1) {
    const StepConsts k = make_consts(hp, step, coupled);
    const Tables t1 = pass1_tables(p);
    MSAMP_LAUNCH(MSAMP_KERNEL_STEP_PASS1, s,
                 launch_step_pass1(grad_fmt, coupled, t1.desc, t1.chunks, t1.nchunks, grad_meta,
                                   exp_avg_meta, p->scratch_a, k, s, nullptr, wide_launch(p)));
    MSAMP_LAUNCH(MSAMP_KERNEL_FINALIZE, s, launch_export_amax(n, p->scratch_a, amax_out, s));
  } else if (phase == 2) {
    const StepConsts k = make_consts(hp, step, coupled);
    // binary32 amax values are non-negative: their bits order like the
    // unsigned integers the update pass reads
    MSAMP_LAUNCH(o3 ? MSAMP_KERNEL_O3_PASS2 : MSAMP_KERNEL_O2_PASS2, s,
                 launch_step_pass2(grad_fmt, o3, coupled, p->desc, p->chunks, p->nchunks, grad_meta,
                                   exp_avg_meta, (const uint32_t*)amax_in, p->scratch_b, k, s, nullptr,
                                   MetaFold{}, wide_update(p), p->split_update));
    if (o3) MSAMP_LAUNCH(MSAMP_KERNEL_FINALIZE, s, launch_export_amax(n, p->scratch_b, amax_out, s));
    MSAMP_LAUNCH(MSAMP_KERNEL_FINALIZE, s, launch_meta_from_amax(n, amax_in, exp_avg_meta, 448.0f, s));
  } else {
    MSAMP_LAUNCH(MSAMP_KERNEL_O3_PASS3, s,
                 launch_o3_pass3(p->desc, p->chunks, p->nchunks, (const uint32_t*)amax_in, s, MetaFold{},
                                 wide_copy(p), p->split_copy));
    MSAMP_LAUNCH(MSAMP_KERNEL_FINALIZE, s,
                 launch_meta_from_amax(n, amax_in, weight_fp8_meta, 448.0f, s));
  }
  return MSAMP_OK;
}


// ------------------------------------------------- allocation-free step ---

// Size of the static device array of msamp_adamw_o2_step_noalloc: enough
// for the tables of 13.1e9 parameters in 291 tensors or 4.3e9 in 20,064.
constexpr size_t kNoAllocScratchBytes = MSAMP_NOALLOC_SCRATCH_BYTES;
// Devices whose scratch address the library keeps.
constexpr int kNoAllocMaxDevices = 64;

// Tables of msamp_adamw_o2_step_noalloc, rebuilt on every call in the
// library's static device array (see 'scratch' below): two u32 amax words
// per tensor (zero when the kernels start), the descriptor table and the
// chunk map, each section 256-byte aligned.
struct NoAllocLayout {
  size_t scratch_bytes = 0, desc_bytes = 0, chunk_bytes = 0, total = 0;
  int64_t nchunks = 0, chunk_elems = kChunk;
};

msamp_status noalloc_layout(int32_t n, const int64_t* numel, NoAllocLayout* l) {
  l->chunk_elems = list_chunk_elems(n, numel);
  int64_t chunks = 0;
  for (int32_t t = 0; t < n; ++t) chunks += (numel[t] + l->chunk_elems - 1) / l->chunk_elems;
  l->nchunks = chunks;
  l->scratch_bytes = align_up(sizeof(uint32_t) * 2 * (size_t)n, 256);
  l->desc_bytes = align_up(sizeof(TensorDesc) * (size_t)n, 256);
  l->chunk_bytes = sizeof(ChunkRef) * (size_t)chunks;
  l->total = l->scratch_bytes + l->desc_bytes + l->chunk_bytes;
  if (l->total > kNoAllocScratchBytes)
    return fail(MSAMP_E_INVALID_ARG,
                "the tensor list needs " + std::to_string(l->total) + " bytes of tables (" +
                    std::to_string(n) + " tensors, " + std::to_string(chunks) + " chunks of " +
                    std::to_string(l->chunk_elems) + " elements); msamp_adamw_o2_step_noalloc holds at most " +
                    std::to_string(kNoAllocScratchBytes));
  return MSAMP_OK;
}

// Host image of the tables, one for the whole process: the call holds
// 'mu' from building it until the synchronous copy has read it.
struct NoAllocHost {
  std::mutex mu;
  alignas(256) char image[kNoAllocScratchBytes];
};

NoAllocHost& noalloc_host() {
  static NoAllocHost h;  // static storage: nothing is allocated at run time
  return h;
}

}  // namespace
}  // namespace msamp

using namespace msamp;

// The static device array of the allocation-free O2 step. In host code
// 'scratch' names a host-side stand-in, not device memory: its device
// address is taken once per device with hipGetSymbolAddress (each device has
// its own copy) and only that address is passed to kernels and copies.
static __device__ __align__(256) uint8_t scratch[msamp::kNoAllocScratchBytes];

namespace {

struct NoAllocDevices {
  std::mutex mu;
  void* ptr[kNoAllocMaxDevices] = {};  // device address of 'scratch', per device (null = not yet taken)
};

NoAllocDevices& noalloc_devices() {
  static NoAllocDevices d;
  return d;
}

// The device address of 'scratch' on device 'dev' (the current device).
msamp_status noalloc_scratch(int dev, uint8_t** out) {
  if (dev < 0 || dev >= kNoAllocMaxDevices)
    return fail(MSAMP_E_INVALID_ARG, "msamp_adamw_o2_step_noalloc supports devices 0..63");
  NoAllocDevices& d = noalloc_devices();
  std::lock_guard<std::mutex> lk(d.mu);
  if (d.ptr[dev] != nullptr) {
    *out = (uint8_t*)d.ptr[dev];
    return MSAMP_OK;
  }
  void* ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress of the step's static scratch");
  if (ptr == nullptr) return fail(MSAMP_E_HIP, "hipGetSymbolAddress returned a null scratch address");
  d.ptr[dev] = ptr;
  *out = (uint8_t*)ptr;
  return MSAMP_OK;
}

msamp_status step_noalloc_impl(int32_t n, const int64_t* numel, const uint8_t* const* grad, int grad_fmt,
                               const msamp_meta* grad_meta, uint8_t* const* exp_avg,
                               msamp_meta* exp_avg_meta, uint16_t* const* exp_avg_sq,
                               uint16_t* const* weight, const msamp_adamw_hparams* hp, int64_t step,
                               void* stream_ptr) {
  g_last_error.clear();
  MSAMP_TRY(check_common(n, numel));
  if (n == 0) return MSAMP_OK;
  MSAMP_TRY(check_fmt(grad_fmt));
  MSAMP_TRY(check_hparams(hp, step));
  MSAMP_TRY(check_step_lists(false, n, numel, grad, grad_meta, exp_avg, exp_avg_meta, exp_avg_sq, weight,
                             nullptr, nullptr));
  NoAllocLayout l;
  MSAMP_TRY(noalloc_layout(n, numel, &l));

  hipStream_t s = (hipStream_t)stream_ptr;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(s, &cs);
  if (e != hipSuccess) return fail_hip(e, "hipStreamIsCapturing");
  if (cs != hipStreamCaptureStatusNone)
    return fail(MSAMP_E_INVALID_ARG,
                "msamp_adamw_o2_step_noalloc copies its tables from host memory at call time and "
                "cannot be captured into a graph");
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  uint8_t* base = nullptr;
  MSAMP_TRY(noalloc_scratch(dev, &base));

  NoAllocHost& h = noalloc_host();
  std::lock_guard<std::mutex> lk(h.mu);
  char* hb = h.image;
  std::memset(hb, 0, l.scratch_bytes + l.desc_bytes);  // amax words start at zero
  TensorDesc* hd = (TensorDesc*)(hb + l.scratch_bytes);
  for (int32_t t = 0; t < n; ++t) {
    TensorDesc d;
    std::memset(&d, 0, sizeof d);
    d.numel = numel[t];
    d.chunk = l.chunk_elems;
    d.p0 = grad[t];
    d.p1 = exp_avg[t];
    d.p2 = exp_avg_sq[t];
    d.p3 = weight[t];
    hd[t] = d;
  }
  ChunkRef* hc = (ChunkRef*)(hb + l.scratch_bytes + l.desc_bytes);
  for (int32_t t = 0, i = 0; t < n; ++t)
    for (int64_t j = 0, k = (numel[t] + l.chunk_elems - 1) / l.chunk_elems; j < k; ++j) hc[i++] = {t, (int32_t)j};
  // From pageable host memory the copy is synchronous: when it returns, the
  // earlier work on the stream has finished and the image has been read.
  e = hipMemcpyAsync(base, hb, l.total, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return fail_hip(e, "copy of the step tables into the static scratch");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail_hip(e, "copy of the step tables into the static scratch");

  uint32_t* amax_a = (uint32_t*)base;
  uint32_t* amax_b = amax_a + n;
  const TensorDesc* desc = (const TensorDesc*)(base + l.scratch_bytes);
  const ChunkRef* chunks = (const ChunkRef*)(base + l.scratch_bytes + l.desc_bytes);
  const StepConsts k = make_consts(hp, step, false);
  MSAMP_LAUNCH(MSAMP_KERNEL_STEP_PASS1, s,
               launch_step_pass1(grad_fmt, false, desc, chunks, l.nchunks, grad_meta, exp_avg_meta, amax_a, k, s));
  MSAMP_LAUNCH(MSAMP_KERNEL_O2_PASS2, s,
               launch_step_pass2(grad_fmt, false, false, desc, chunks, l.nchunks, grad_meta, exp_avg_meta, amax_a,
                                 amax_b, k, s));
  MSAMP_LAUNCH(MSAMP_KERNEL_FINALIZE, s,
               launch_step_finalize(n, amax_a, exp_avg_meta, nullptr, nullptr, 448.0f, s));
  return MSAMP_OK;
}

}  // namespace

extern "C" {

int msamp_abi_version(void) { return MSAMP_ABI_VERSION; }

const char* msamp_last_error(void) { return g_last_error.c_str(); }

const char* msamp_kernel_name(msamp_kernel_kind kind) {
  switch (kind) {
    case MSAMP_KERNEL_AMAX: return "amax";
    case MSAMP_KERNEL_QUANTIZE: return "quantize_fp8";
    case MSAMP_KERNEL_DEQUANTIZE: return "dequantize_fp8";
    case MSAMP_KERNEL_STEP_PASS1: return "step_pass1";
    case MSAMP_KERNEL_O2_PASS2: return "o2_pass2";
    case MSAMP_KERNEL_O3_PASS2: return "o3_pass2";
    case MSAMP_KERNEL_O3_PASS3: return "o3_pass3";
    case MSAMP_KERNEL_FINALIZE: return "finalize";
    case MSAMP_KERNEL_AMAX_FINALIZE: return "amax_finalize";
    case MSAMP_KERNEL_O2_DELAYED: return "o2_delayed";
    case MSAMP_KERNEL_RMW_PROBE: return "rmw_probe";
    case MSAMP_KERNEL_QUANTIZE_PASS1: return "quantize_pass1";
    case MSAMP_KERNEL_READ_PROBE: return "read_probe";
    case MSAMP_KERNEL_COPY_PROBE: return "copy_probe";
    case MSAMP_KERNEL_QP1_PROBE: return "qp1_probe";
    default: return "";
  }
}

msamp_status msamp_amax(int32_t n, const float* const* x, const int64_t* numel, msamp_meta* meta,
                        void* stream) {
  return guarded([&]() -> msamp_status {
    g_last_error.clear();
    MSAMP_TRY(check_count(n, numel));
    if (n == 0) return MSAMP_OK;
    MSAMP_TRY(check_meta(n, meta, "meta"));
    hipStream_t s = (hipStream_t)stream;
    const void* const* roles[1] = {(const void* const*)x};
    const char* names[1] = {"x"};
    Plan* p = nullptr;
    std::unique_lock<std::mutex> lease;  // held until the launches are enqueued
    MSAMP_TRY(get_plan(kPlanAmax, n, numel, roles, names, 1, true, s, &p, &lease));
    MetaFold fold;  // small lists: the completing workgroup writes meta[t].amax
    if (p->nchunks <= kFoldMaxChunks) {
      fold.done = p->done;
      fold.meta_a = meta;
      fold.amax_a = p->scratch_a;
    }
    MSAMP_LAUNCH(MSAMP_KERNEL_AMAX, s, launch_amax(p->desc, p->chunks, p->nchunks, p->scratch_a, s, fold));
    if (fold.done == nullptr)
      MSAMP_LAUNCH(MSAMP_KERNEL_AMAX_FINALIZE, s, launch_amax_finalize(n, p->scratch_a, meta, s));
    return MSAMP_OK;
  });
}

static msamp_status quantize_impl(int32_t n, const float* const* x, const int64_t* numel,
                                  msamp_fp8_format fmt, msamp_meta* meta, int32_t world,
                                  uint8_t* const* q, void* stream) {
  return guarded([&]() -> msamp_status {
    g_last_error.clear();
    MSAMP_TRY(check_count(n, numel));
    if (world < 1) return fail(MSAMP_E_INVALID_ARG, "world_size must be >= 1");
    if (n == 0) return MSAMP_OK;
    MSAMP_TRY(check_fmt((int)fmt));
    MSAMP_TRY(check_meta(n, meta, "meta"));
    hipStream_t s = (hipStream_t)stream;
    const void* const* roles[2] = {(const void* const*)x, (const void* const*)q};
    const char* names[2] = {"x", "q"};
    Plan* p = nullptr;
    std::unique_lock<std::mutex> lease;  // held until the launches are enqueued
    MSAMP_TRY(get_plan(kPlanQuantize, n, numel, roles, names, 2, true, s, &p, &lease));
    MSAMP_LAUNCH(MSAMP_KERNEL_QUANTIZE, s,
                 launch_quantize((int)fmt, p->desc, p->chunks, p->nchunks, meta, world, s));
    return MSAMP_OK;
  });
}

msamp_status msamp_quantize_fp8(int32_t n, const float* const* x, const int64_t* numel,
                                msamp_fp8_format fmt, msamp_meta* meta, uint8_t* const* q,
                                void* stream) {
  return quantize_impl(n, x, numel, fmt, meta, 1, q, stream);
}

msamp_status msamp_quantize_fp8_prescaled(int32_t n, const float* const* x, const int64_t* numel,
                                          msamp_fp8_format fmt, msamp_meta* meta,
                                          int32_t world_size, uint8_t* const* q, void* stream) {
  return quantize_impl(n, x, numel, fmt, meta, world_size, q, stream);
}

msamp_status msamp_dequantize_fp8(int32_t n, const uint8_t* const* q, const int64_t* numel,
                                  msamp_fp8_format fmt, const msamp_meta* meta,
                                  float* const* out, void* stream) {
  return guarded([&]() -> msamp_status {
    g_last_error.clear();
    MSAMP_TRY(check_count(n, numel));
    if (n == 0) return MSAMP_OK;
    MSAMP_TRY(check_fmt((int)fmt));
    MSAMP_TRY(check_meta(n, meta, "meta"));
    hipStream_t s = (hipStream_t)stream;
    const void* const* roles[2] = {(const void* const*)q, (const void* const*)out};
    const char* names[2] = {"q", "out"};
    Plan* p = nullptr;
    std::unique_lock<std::mutex> lease;  // held until the launches are enqueued
    MSAMP_TRY(get_plan(kPlanDequantize, n, numel, roles, names, 2, false, s, &p, &lease));
    MSAMP_LAUNCH(MSAMP_KERNEL_DEQUANTIZE, s,
                 launch_dequantize((int)fmt, p->desc, p->chunks, p->nchunks, meta, s));
    return MSAMP_OK;
  });
}

msamp_status msamp_adamw_o2_step(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                 msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                 uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                 uint16_t* const* exp_avg_sq, uint16_t* const* weight,
                                 const msamp_adamw_hparams* hp, int64_t step, void* stream) {
  return guarded([&]() {
    return step_impl(false, false, n, numel, grad, (int)grad_fmt, grad_meta, exp_avg, exp_avg_meta,
                     exp_avg_sq, weight, nullptr, nullptr, hp, step, stream);
  });
}

msamp_status msamp_adam_o2_step(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                uint16_t* const* exp_avg_sq, uint16_t* const* weight,
                                const msamp_adamw_hparams* hp, int64_t step, void* stream) {
  return guarded([&]() {
    return step_impl(false, true, n, numel, grad, (int)grad_fmt, grad_meta, exp_avg, exp_avg_meta,
                     exp_avg_sq, weight, nullptr, nullptr, hp, step, stream);
  });
}

msamp_status msamp_adamw_o3_step(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                 msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                 uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                 uint16_t* const* exp_avg_sq, uint16_t* const* master,
                                 uint8_t* const* weight_fp8, msamp_meta* weight_fp8_meta,
                                 const msamp_adamw_hparams* hp, int64_t step, void* stream) {
  return guarded([&]() {
    return step_impl(true, false, n, numel, grad, (int)grad_fmt, grad_meta, exp_avg, exp_avg_meta,
                     exp_avg_sq, master, weight_fp8, weight_fp8_meta, hp, step, stream);
  });
}

msamp_status msamp_adam_o3_step(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                uint16_t* const* exp_avg_sq, uint16_t* const* master,
                                uint8_t* const* weight_fp8, msamp_meta* weight_fp8_meta,
                                const msamp_adamw_hparams* hp, int64_t step, void* stream) {
  return guarded([&]() {
    return step_impl(true, true, n, numel, grad, (int)grad_fmt, grad_meta, exp_avg, exp_avg_meta,
                     exp_avg_sq, master, weight_fp8, weight_fp8_meta, hp, step, stream);
  });
}

static_assert(sizeof(msamp_step_constants) == sizeof(StepConsts), "constants layout");
static_assert(offsetof(msamp_step_constants, ibs) == offsetof(StepConsts, ibs), "constants layout");
static_assert(offsetof(msamp_step_constants, wd) == offsetof(StepConsts, wd), "constants layout");

msamp_status msamp_step_constants_compute(const msamp_adamw_hparams* hp, int64_t step, int coupled,
                                          msamp_step_constants* out) {
  return guarded([&]() -> msamp_status {
    g_last_error.clear();
    MSAMP_TRY(check_hparams(hp, step));
    if (out == nullptr) return fail(MSAMP_E_INVALID_ARG, "out is NULL");
    const StepConsts k = make_consts(hp, step, coupled != 0);
    std::memcpy(out, &k, sizeof k);
    return MSAMP_OK;
  });
}

msamp_status msamp_adamw_o2_step_devconst(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                          msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                          uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                          uint16_t* const* exp_avg_sq, uint16_t* const* weight,
                                          const msamp_step_constants* consts, int coupled,
                                          void* stream) {
  return guarded([&]() -> msamp_status {
    if (consts == nullptr) return fail(MSAMP_E_INVALID_ARG, "consts is NULL");
    return step_impl(false, coupled != 0, n, numel, grad, (int)grad_fmt, grad_meta, exp_avg,
                     exp_avg_meta, exp_avg_sq, weight, nullptr, nullptr, nullptr, 0, stream,
                     (const StepConsts*)consts);
  });
}

msamp_status msamp_adamw_o3_step_devconst(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                          msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                          uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                          uint16_t* const* exp_avg_sq, uint16_t* const* master,
                                          uint8_t* const* weight_fp8, msamp_meta* weight_fp8_meta,
                                          const msamp_step_constants* consts, int coupled,
                                          void* stream) {
  return guarded([&]() -> msamp_status {
    if (consts == nullptr) return fail(MSAMP_E_INVALID_ARG, "consts is NULL");
    return step_impl(true, coupled != 0, n, numel, grad, (int)grad_fmt, grad_meta, exp_avg,
                     exp_avg_meta, exp_avg_sq, master, weight_fp8, weight_fp8_meta, nullptr, 0, stream,
                     (const StepConsts*)consts);
  });
}

msamp_status msamp_adamw_o2_step_phase1(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                        msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                        uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                        uint16_t* const* exp_avg_sq, uint16_t* const* weight,
                                        const msamp_adamw_hparams* hp, int64_t step, int coupled,
                                        float* amax_m, void* stream) {
  return guarded([&]() {
    return phase_impl(1, false, coupled != 0, n, numel, grad, (int)grad_fmt, grad_meta, exp_avg,
                      exp_avg_meta, exp_avg_sq, weight, nullptr, nullptr, hp, step, amax_m, nullptr,
                      stream);
  });
}

msamp_status msamp_adamw_o2_step_phase2(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                        msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                        uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                        uint16_t* const* exp_avg_sq, uint16_t* const* weight,
                                        const msamp_adamw_hparams* hp, int64_t step, int coupled,
                                        const float* amax_m, void* stream) {
  return guarded([&]() {
    return phase_impl(2, false, coupled != 0, n, numel, grad, (int)grad_fmt, grad_meta, exp_avg,
                      exp_avg_meta, exp_avg_sq, weight, nullptr, nullptr, hp, step, nullptr, amax_m,
                      stream);
  });
}

msamp_status msamp_adamw_o3_step_phase1(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                        msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                        uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                        uint16_t* const* exp_avg_sq, uint16_t* const* master,
                                        uint8_t* const* weight_fp8, msamp_meta* weight_fp8_meta,
                                        const msamp_adamw_hparams* hp, int64_t step, int coupled,
                                        float* amax_m, void* stream) {
  return guarded([&]() {
    return phase_impl(1, true, coupled != 0, n, numel, grad, (int)grad_fmt, grad_meta, exp_avg,
                      exp_avg_meta, exp_avg_sq, master, weight_fp8, weight_fp8_meta, hp, step, amax_m,
                      nullptr, stream);
  });
}

msamp_status msamp_adamw_o3_step_phase2(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                        msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                        uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                        uint16_t* const* exp_avg_sq, uint16_t* const* master,
                                        uint8_t* const* weight_fp8, msamp_meta* weight_fp8_meta,
                                        const msamp_adamw_hparams* hp, int64_t step, int coupled,
                                        const float* amax_m, float* amax_w, void* stream) {
  return guarded([&]() {
    return phase_impl(2, true, coupled != 0, n, numel, grad, (int)grad_fmt, grad_meta, exp_avg,
                      exp_avg_meta, exp_avg_sq, master, weight_fp8, weight_fp8_meta, hp, step, amax_w,
                      amax_m, stream);
  });
}

msamp_status msamp_adamw_o3_step_phase3(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                        msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                        uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                        uint16_t* const* exp_avg_sq, uint16_t* const* master,
                                        uint8_t* const* weight_fp8, msamp_meta* weight_fp8_meta,
                                        const float* amax_w, void* stream) {
  return guarded([&]() {
    return phase_impl(3, true, false, n, numel, grad, (int)grad_fmt, grad_meta, exp_avg, exp_avg_meta,
                      exp_avg_sq, master, weight_fp8, weight_fp8_meta, nullptr, 0, nullptr, amax_w,
                      stream);
  });
}

msamp_status msamp_adamw_o2_step_delayed(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                         msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                         uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                         uint16_t* const* exp_avg_sq, uint16_t* const* weight,
                                         const msamp_adamw_hparams* hp, int64_t step, void* stream) {
  return guarded([&]() {
    return step_delayed_impl(n, numel, grad, (int)grad_fmt, grad_meta, exp_avg, exp_avg_meta,
                             exp_avg_sq, weight, hp, step, stream);
  });
}

msamp_status msamp_adamw_o2_step_scaled_v(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                          msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                          uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                          uint16_t* const* exp_avg_sq, msamp_meta* exp_avg_sq_meta,
                                          uint16_t* const* weight, const msamp_adamw_hparams* hp,
                                          int64_t step, void* stream) {
  return guarded([&]() {
    return step_scaled_v_impl(n, numel, grad, (int)grad_fmt, grad_meta, exp_avg, exp_avg_meta,
                              exp_avg_sq, exp_avg_sq_meta, weight, hp, step, stream);
  });
}

msamp_status msamp_adamw_o2_step_noalloc(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                         msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                         uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                         uint16_t* const* exp_avg_sq, uint16_t* const* weight,
                                         const msamp_adamw_hparams* hp, int64_t step, void* stream) {
  return guarded([&]() {
    return step_noalloc_impl(n, numel, grad, (int)grad_fmt, grad_meta, exp_avg, exp_avg_meta, exp_avg_sq,
                             weight, hp, step, stream);
  });
}

msamp_status msamp_quantize_adamw_o2_step(int32_t n, const int64_t* numel, const float* const* grad_f32,
                                          msamp_fp8_format grad_fmt, msamp_meta* grad_meta,
                                          uint8_t* const* grad, uint8_t* const* exp_avg,
                                          msamp_meta* exp_avg_meta, uint16_t* const* exp_avg_sq,
                                          uint16_t* const* weight, const msamp_adamw_hparams* hp,
                                          int64_t step, void* stream) {
  return guarded([&]() {
    return quantize_step_impl(false, false, n, numel, grad_f32, (int)grad_fmt, grad_meta, grad, exp_avg,
                              exp_avg_meta, exp_avg_sq, weight, nullptr, nullptr, hp, step, stream);
  });
}

msamp_status msamp_quantize_adam_o2_step(int32_t n, const int64_t* numel, const float* const* grad_f32,
                                         msamp_fp8_format grad_fmt, msamp_meta* grad_meta, uint8_t* const* grad,
                                         uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                         uint16_t* const* exp_avg_sq, uint16_t* const* weight,
                                         const msamp_adamw_hparams* hp, int64_t step, void* stream) {
  return guarded([&]() {
    return quantize_step_impl(false, true, n, numel, grad_f32, (int)grad_fmt, grad_meta, grad, exp_avg,
                              exp_avg_meta, exp_avg_sq, weight, nullptr, nullptr, hp, step, stream);
  });
}

msamp_status msamp_quantize_adamw_o2_step_devconst(int32_t n, const int64_t* numel, const float* const* grad_f32,
                                                   msamp_fp8_format grad_fmt, msamp_meta* grad_meta,
                                                   uint8_t* const* grad, uint8_t* const* exp_avg,
                                                   msamp_meta* exp_avg_meta, uint16_t* const* exp_avg_sq,
                                                   uint16_t* const* weight, const msamp_step_constants* consts,
                                                   int coupled, void* stream) {
  return guarded([&]() -> msamp_status {
    if (consts == nullptr) return fail(MSAMP_E_INVALID_ARG, "consts is NULL");
    return quantize_step_impl(false, coupled != 0, n, numel, grad_f32, (int)grad_fmt, grad_meta, grad, exp_avg,
                              exp_avg_meta, exp_avg_sq, weight, nullptr, nullptr, nullptr, 0, stream,
                              (const StepConsts*)consts);
  });
}

msamp_status msamp_quantize_adamw_o3_step(int32_t n, const int64_t* numel, const float* const* grad_f32,
                                          msamp_fp8_format grad_fmt, msamp_meta* grad_meta,
                                          uint8_t* const* grad, uint8_t* const* exp_avg,
                                          msamp_meta* exp_avg_meta, uint16_t* const* exp_avg_sq,
                                          uint16_t* const* master, uint8_t* const* weight_fp8,
                                          msamp_meta* weight_fp8_meta, const msamp_adamw_hparams* hp,
                                          int64_t step, void* stream) {
  return guarded([&]() {
    return quantize_step_impl(true, false, n, numel, grad_f32, (int)grad_fmt, grad_meta, grad, exp_avg,
                              exp_avg_meta, exp_avg_sq, master, weight_fp8, weight_fp8_meta, hp, step,
                              stream);
  });
}

msamp_status msamp_quantize_adam_o3_step(int32_t n, const int64_t* numel, const float* const* grad_f32,
                                         msamp_fp8_format grad_fmt, msamp_meta* grad_meta, uint8_t* const* grad,
                                         uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                         uint16_t* const* exp_avg_sq, uint16_t* const* master,
                                         uint8_t* const* weight_fp8, msamp_meta* weight_fp8_meta,
                                         const msamp_adamw_hparams* hp, int64_t step, void* stream) {
  return guarded([&]() {
    return quantize_step_impl(true, true, n, numel, grad_f32, (int)grad_fmt, grad_meta, grad, exp_avg,
                              exp_avg_meta, exp_avg_sq, master, weight_fp8, weight_fp8_meta, hp, step,
                              stream);
  });
}

msamp_status msamp_quantize_adamw_o3_step_devconst(int32_t n, const int64_t* numel, const float* const* grad_f32,
                                                   msamp_fp8_format grad_fmt, msamp_meta* grad_meta,
                                                   uint8_t* const* grad, uint8_t* const* exp_avg,
                                                   msamp_meta* exp_avg_meta, uint16_t* const* exp_avg_sq,
                                                   uint16_t* const* master, uint8_t* const* weight_fp8,
                                                   msamp_meta* weight_fp8_meta, const msamp_step_constants* consts,
                                                   int coupled, void* stream) {
  return guarded([&]() -> msamp_status {
    if (consts == nullptr) return fail(MSAMP_E_INVALID_ARG, "consts is NULL");
    return quantize_step_impl(true, coupled != 0, n, numel, grad_f32, (int)grad_fmt, grad_meta, grad, exp_avg,
                              exp_avg_meta, exp_avg_sq, master, weight_fp8, weight_fp8_meta, nullptr, 0, stream,
                              (const StepConsts*)consts);
  });
}

msamp_status msamp_release_cache(void) {
  return guarded([&]() -> msamp_status {
    g_last_error.clear();
    PlanCache& c = cache();
    std::lock_guard<std::mutex> lk(c.mu);
    int cur = -1;
    (void)hipGetDevice(&cur);
    for (auto& kv : c.map)
      for (auto& p : kv.second)
        if (!p->pinned) {
          (void)hipSetDevice(p->device);
          (void)hipDeviceSynchronize();
        }
    for (auto it = c.map.begin(); it != c.map.end();) {
      auto& vec = it->second;
      for (size_t i = vec.size(); i-- > 0;)
        if (!vec[i]->pinned) {
          c.bytes -= vec[i]->bytes;
          c.count -= 1;
          c.forget(vec[i].get());
          vec.erase(vec.begin() + (ptrdiff_t)i);
        }
      it = vec.empty() ? c.map.erase(it) : std::next(it);
    }
    if (cur >= 0) (void)hipSetDevice(cur);
    return MSAMP_OK;
  });
}

msamp_status msamp_unpin_captured_tables(void) {
  return guarded([&]() -> msamp_status {
    g_last_error.clear();
    PlanCache& c = cache();
    std::lock_guard<std::mutex> lk(c.mu);
    for (auto& kv : c.map)
      for (auto& p : kv.second) p->pinned = false;
    ++c.tick;  // no plan is exempt from the eviction below as the newest
    evict_locked(c);
    return MSAMP_OK;
  });
}

msamp_status msamp_cache_stats(int64_t* lists, int64_t* bytes, int64_t* pinned) {
  return guarded([&]() -> msamp_status {
    g_last_error.clear();
    PlanCache& c = cache();
    std::lock_guard<std::mutex> lk(c.mu);
    int64_t np = 0;
    for (auto& kv : c.map)
      for (auto& p : kv.second) np += p->pinned ? 1 : 0;
    if (lists) *lists = (int64_t)c.count;
    if (bytes) *bytes = (int64_t)c.bytes;
    if (pinned) *pinned = np;
    return MSAMP_OK;
  });
}

msamp_status msamp_quantize_pass1_probe(int32_t n, const int64_t* numel, const float* const* grad_f32,
                                        uint8_t* const* grad, uint8_t* const* exp_avg,
                                        uint16_t* const* exp_avg_sq, uint16_t* const* weight, void* stream) {
  return guarded([&]() -> msamp_status {
    g_last_error.clear();
    MSAMP_TRY(check_count(n, numel));
    if (n == 0) return MSAMP_OK;
    hipStream_t s = (hipStream_t)stream;
    const void* const* roles[6] = {(const void* const*)grad,       (const void* const*)exp_avg,
                                   (const void* const*)exp_avg_sq, (const void* const*)weight,
                                   nullptr,                        (const void* const*)grad_f32};
    const char* names[6] = {"grad", "exp_avg", "exp_avg_sq", "weight", nullptr, "grad_f32"};
    Plan* p = nullptr;
    std::unique_lock<std::mutex> lease;
    MSAMP_TRY(get_plan(kPlanQuantizeO2, n, numel, roles, names, 6, true, s, &p, &lease));
    MSAMP_LAUNCH(MSAMP_KERNEL_QP1_PROBE, s, launch_qp1_probe(p->desc, p->chunks, p->nchunks, s, wide_launch(p)));
    return MSAMP_OK;
  });
}

msamp_status msamp_stream_probe(msamp_stream_kind kind, const void* src, void* dst, int64_t bytes,
                                void* stream) {
  return guarded([&]() -> msamp_status {
    g_last_error.clear();
    if (kind != MSAMP_STREAM_READ && kind != MSAMP_STREAM_COPY)
      return fail(MSAMP_E_INVALID_ARG, "unknown stream probe kind");
    if (bytes < 0 || bytes % 16 != 0) return fail(MSAMP_E_INVALID_ARG, "bytes must be >= 0 and a multiple of 16");
    if (bytes == 0) return MSAMP_OK;
    if (src == nullptr) return fail(MSAMP_E_INVALID_ARG, "src is NULL");
    if (!aligned16(src)) return fail(MSAMP_E_MISALIGNED, "src is not 16-byte aligned");
    const bool copy = kind == MSAMP_STREAM_COPY;
    if (copy) {
      if (dst == nullptr) return fail(MSAMP_E_INVALID_ARG, "dst is NULL");
      if (!aligned16(dst)) return fail(MSAMP_E_MISALIGNED, "dst is not 16-byte aligned");
      const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
      if (a < b + (uintptr_t)bytes && b < a + (uintptr_t)bytes)
        return fail(MSAMP_E_INVALID_ARG, "src and dst overlap");
    }
    // one 256-thread workgroup per 16 KB: the launch must stay within 2^32 - 1 threads
    if ((bytes / 16 + 1023) / 1024 * 256 > (int64_t)UINT32_MAX) return fail(MSAMP_E_INVALID_ARG, "bytes too large");
    hipStream_t s = (hipStream_t)stream;
    MSAMP_LAUNCH(copy ? MSAMP_KERNEL_COPY_PROBE : MSAMP_KERNEL_READ_PROBE, s,
                 launch_stream_probe(copy, src, dst, bytes, s));
    return MSAMP_OK;
  });
}

msamp_status msamp_rmw_probe(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                             uint8_t* const* exp_avg, uint16_t* const* exp_avg_sq,
                             uint16_t* const* weight, void* stream) {
  return guarded([&]() -> msamp_status {
    g_last_error.clear();
    MSAMP_TRY(check_count(n, numel));
    if (n == 0) return MSAMP_OK;
    hipStream_t s = (hipStream_t)stream;
    const void* const* roles[4] = {(const void* const*)grad, (const void* const*)exp_avg,
                                   (const void* const*)exp_avg_sq, (const void* const*)weight};
    Plan* p = nullptr;
    std::unique_lock<std::mutex> lease;  // held until the launch is enqueued
    const char* names[4] = {"grad", "exp_avg", "exp_avg_sq", "weight"};
    MSAMP_TRY(get_plan(kPlanO2, n, numel, roles, names, 4, true, s, &p, &lease));
    MSAMP_LAUNCH(MSAMP_KERNEL_RMW_PROBE, s,
                 launch_rmw_probe(p->desc, p->chunks, p->nchunks, s, wide_update(p), p->split_update));
    return MSAMP_OK;
  });
}

msamp_status msamp_codec_probe(msamp_probe_op op, const void* in, void* out, int64_t n,
                               void* stream) {
  return guarded([&]() -> msamp_status {
    g_last_error.clear();
    if (n < 0) return fail(MSAMP_E_INVALID_ARG, "n < 0");
    if ((int)op < 0 || (int)op > (int)MSAMP_PROBE_F16_TO_F32)
      return fail(MSAMP_E_INVALID_ARG, "unknown probe op");
    if (n == 0) return MSAMP_OK;
    if (in == nullptr || out == nullptr) return fail(MSAMP_E_INVALID_ARG, "NULL buffer");
    if (!aligned16(in) || !aligned16(out)) return fail(MSAMP_E_MISALIGNED, "buffer not 16-byte aligned");
    hipError_t e = launch_codec_probe((int)op, in, out, n, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "codec probe");
    return MSAMP_OK;
  });
}

msamp_status msamp_profile_enable(int on) {
  return guarded([&]() -> msamp_status {
    g_last_error.clear();
    Profiler& p = profiler();
    std::lock_guard<std::mutex> lk(p.mu);
    if (on) {
      // discard earlier records; their events must have completed first
      for (auto& r : p.recs) (void)hipEventSynchronize(r.b);
      p.recycle_all();
      // create the events up front, so that the timed work does not
      for (size_t i = p.pool.size(); i < kProfilerReserve; ++i) {
        hipEvent_t e = nullptr;
        if (hipEventCreateWithFlags(&e, kProfilerEventFlags) != hipSuccess) break;
        p.pool.push_back(e);
      }
    }
    p.enabled = on != 0;
    return MSAMP_OK;
  });
}

msamp_status msamp_profile_select(uint32_t kind_mask) {
  return guarded([&]() -> msamp_status {
    g_last_error.clear();
    Profiler& p = profiler();
    std::lock_guard<std::mutex> lk(p.mu);
    p.mask = kind_mask;
    return MSAMP_OK;
  });
}

msamp_status msamp_profile_read(msamp_kernel_kind kind, int64_t* launches, double* total_ms) {
  return guarded([&]() -> msamp_status {
    g_last_error.clear();
    if (launches == nullptr || total_ms == nullptr)
      return fail(MSAMP_E_INVALID_ARG, "NULL output");
    Profiler& p = profiler();
    std::lock_guard<std::mutex> lk(p.mu);
    int64_t cnt = 0;
    double ms = 0.0;
    for (auto& r : p.recs) {
      if (r.kind != (int)kind) continue;
      hipError_t e = hipEventSynchronize(r.b);
      if (e != hipSuccess) return fail_hip(e, "hipEventSynchronize");
      float f = 0.0f;
      e = hipEventElapsedTime(&f, r.a, r.b);
      if (e != hipSuccess) return fail_hip(e, "hipEventElapsedTime");
      ms += (double)f;
      ++cnt;
    }
    *launches = cnt;
    *total_ms = ms;
    return MSAMP_OK;
  });
}

}  // extern "C"
