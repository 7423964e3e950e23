// Host-streamed experts with a device residency cache: the regime in which a
// model's routed experts (1.45 TB for K3) live in host memory and only a
// bounded set of them is resident in HBM.
//
// After "Deltafin's custom compiled runtime", section "CUDA pre-I/O planning
// and residency", and "How the native runtime works", section "Automatic
// PILOT prefetch and CUDA expert residency":
//  - a plan is frozen for the authoritative route union of one layer call
//    before any upload: hits keep their device slots, and the complete
//    ordered list of misses is returned;
//  - the finish call consumes that one plan and takes one host span per
//    reported miss; an all-hit plan uploads nothing;
//  - two pinned staging slabs alternate, so the host copy of one miss
//    overlaps the DMA of the previous one, and an event guards each slab
//    against reuse before its DMA has finished;
//  - eviction is one least-recently-used order across all layers;
//  - the slot pool is allocated with bounded retries (the request shrinks by
//    a quarter per failed attempt), sized from free memory with at least
//    2 GiB or 20% left over when no capacity is given;
//  - a terminal failure (a failed copy or event) poisons the cache: every
//    later call returns MOE_ERR_POISONED instead of continuing with
//    uncertain slot contents.
// Compute runs on the existing kernels: a slot holds one expert in the
// device layout, so the slot pool is a layer of `capacity` experts and the
// expert part of the layer runs on it with each route id replaced by its
// slot (moe_mxfp4_experts).  Every expert's arithmetic is the same as in the
// all-resident layer, so the output is the same bits.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>
#include <vector>

#include "moe_mxfp4.h"

struct moe_expert_cache {
  moe_layer_desc desc{};
  int n_layers = 0, E = 0, capacity = 0, max_ids = 0;
  size_t cb = 0, sb = 0;
  uint8_t* slot_codes = nullptr;   // device [capacity][cb]
  uint8_t* slot_scales = nullptr;  // device [capacity][sb]
  std::vector<int32_t> slot_of;    // [n_layers * E]: slot, or -1
  std::vector<int32_t> owner;      // [capacity]: layer * E + expert, or -1
  std::vector<uint64_t> last_use;  // [capacity]: tick of the last plan that used it
  std::vector<uint8_t> in_plan;    // [capacity]: used by the frozen plan
  uint64_t tick = 0;
  bool planned = false, plan_prefetch = false, poisoned = false;
  std::vector<int32_t> miss_slot;  // frozen plan: slot of each miss, in miss order
  std::vector<int32_t> miss_key;   // frozen plan: layer * E + expert of each miss
  uint8_t* slab[2] = {nullptr, nullptr};  // pinned staging, one expert each
  hipEvent_t slab_ev[2] = {nullptr, nullptr};
  bool slab_busy[2] = {false, false};
  int32_t* host_ids = nullptr;     // pinned [max_ids]: routes read back
  int32_t* host_slots = nullptr;   // pinned [max_ids]: routes as slots
  moe_cache_stats st{};
  int64_t fail_at = -1;            // test hook: the upload of this index fails (see moe_cache_create)
  int64_t uploads = 0;
  std::mutex mu;
};

namespace {

constexpr int kMaxCacheSlots = 4096;      // the expert kernels' E limit
constexpr int kStreamedMaxTokens = 4096;  // tokens per moe_cache_layer_forward call

moe_status cache_check_desc(const moe_layer_desc* d) { return moe_layer_check(d); }

// Slot for a miss: a free slot, else the least recently used one that the
// frozen plan does not use (-1 if none).
int pick_slot(moe_expert_cache* c) {
  int best = -1;
  for (int s = 0; s < c->capacity; ++s) {
    if (c->in_plan[s]) continue;
    if (c->owner[s] < 0) return s;
    if (best < 0 || c->last_use[s] < c->last_use[best]) best = s;
  }
  return best;
}

void release_plan(moe_expert_cache* c) {
  for (int s = 0; s < c->capacity; ++s) c->in_plan[s] = 0;
  c->miss_slot.clear();
  c->miss_key.clear();
  c->planned = false;
}

moe_status poison(moe_expert_cache* c) {
  c->poisoned = true;
  c->st.poisoned = 1;
  return MOE_ERR_POISONED;
}

}  // namespace

extern "C" {

moe_status moe_cache_create(const moe_layer_desc* desc, int32_t n_layers, int32_t capacity, int32_t max_retries,
                            moe_expert_cache** cache) {
  if (!cache) return MOE_ERR_NULL;
  *cache = nullptr;
  moe_status rc = cache_check_desc(desc);
  if (rc != MOE_OK) return rc;
  if (n_layers < 1 || n_layers > 4096 || capacity < 0 || max_retries < 0 || max_retries > 64) return MOE_ERR_SHAPE;
  size_t cb = 0, sb = 0;
  {
    size_t codes = 0, scales = 0;
    rc = moe_mxfp4_packed_bytes(desc, &codes, &scales);
    if (rc != MOE_OK) return rc;
    cb = codes / (size_t)desc->n_experts;
    sb = scales / (size_t)desc->n_experts;
  }
  size_t keys = (size_t)n_layers * (size_t)desc->n_experts;
  if (keys > (size_t)INT32_MAX) return MOE_ERR_OVERFLOW;
  int want = capacity;
  if (want == 0) {  // from free memory, keeping max(2 GiB, 20%) free
    size_t fr = 0, tot = 0;
    if (hipMemGetInfo(&fr, &tot) != hipSuccess) return MOE_ERR_DEVICE;
    size_t keep = tot / 5 > (size_t(2) << 30) ? tot / 5 : (size_t(2) << 30);
    size_t budget = fr > keep ? fr - keep : 0;
    size_t n = budget / (cb + sb);
    want = (int)(n < (size_t)kMaxCacheSlots ? n : (size_t)kMaxCacheSlots);
  }
  if (want > kMaxCacheSlots) want = kMaxCacheSlots;
  if (want < desc->top_k_max) return MOE_ERR_UNSUPPORTED;  // cannot hold one token's experts
  moe_expert_cache* c = new (std::nothrow) moe_expert_cache;
  if (!c) return MOE_ERR_DEVICE;
  c->desc = *desc;
  c->n_layers = n_layers;
  c->E = desc->n_experts;
  c->cb = cb;
  c->sb = sb;
  // bounded retries: shrink the request by a quarter after each failure
  int got = 0;
  for (int attempt = 0; attempt <= max_retries && want >= desc->top_k_max; ++attempt) {
    void* pc = nullptr;
    void* ps = nullptr;
    if (hipMalloc(&pc, (size_t)want * cb) == hipSuccess) {
      if (hipMalloc(&ps, (size_t)want * sb) == hipSuccess) {
        c->slot_codes = static_cast<uint8_t*>(pc);
        c->slot_scales = static_cast<uint8_t*>(ps);
        got = want;
        break;
      }
      (void)hipFree(pc);
    }
    (void)hipGetLastError();  // clear the failed allocation's error
    c->st.alloc_retries += 1;
    want -= want / 4 > 0 ? want / 4 : 1;
  }
  if (!got) {
    delete c;
    return MOE_ERR_DEVICE;
  }
  c->capacity = got;
  c->max_ids = kStreamedMaxTokens * desc->top_k_max;
  bool ok = true;
  for (int s = 0; s < 2 && ok; ++s) {
    ok = hipHostMalloc(reinterpret_cast<void**>(&c->slab[s]), cb + sb, hipHostMallocDefault) == hipSuccess &&
         hipEventCreateWithFlags(&c->slab_ev[s], hipEventDisableTiming) == hipSuccess;
  }
  ok = ok && hipHostMalloc(reinterpret_cast<void**>(&c->host_ids), (size_t)c->max_ids * 4, hipHostMallocDefault) ==
                 hipSuccess;
  ok = ok && hipHostMalloc(reinterpret_cast<void**>(&c->host_slots), (size_t)c->max_ids * 4,
                           hipHostMallocDefault) == hipSuccess;
  try {
    c->slot_of.assign(keys, -1);
    c->owner.assign((size_t)got, -1);
    c->last_use.assign((size_t)got, 0);
    c->in_plan.assign((size_t)got, 0);
  } catch (...) {
    ok = false;
  }
  c->st.struct_size = sizeof(moe_cache_stats);
  c->st.capacity = got;
  // Failure injection for tests of the poisoning path, forced from the host:
  // MOE_CACHE_FAIL_UPLOAD=n makes upload number n (counting from 0 over the
  // cache's life) report a failed copy without issuing it.
  if (const char* f = getenv("MOE_CACHE_FAIL_UPLOAD")) c->fail_at = atoll(f);
  if (!ok) {
    moe_cache_destroy(c);
    return MOE_ERR_DEVICE;
  }
  *cache = c;
  return MOE_OK;
}

moe_status moe_cache_destroy(moe_expert_cache* c) {
  if (!c) return MOE_OK;
  moe_status rc = MOE_OK;
  for (int s = 0; s < 2; ++s) {
    if (c->slab_ev[s]) {
      if (c->slab_busy[s] && hipEventSynchronize(c->slab_ev[s]) != hipSuccess) rc = MOE_ERR_DEVICE;
      if (hipEventDestroy(c->slab_ev[s]) != hipSuccess) rc = MOE_ERR_DEVICE;
    }
    if (c->slab[s] && hipHostFree(c->slab[s]) != hipSuccess) rc = MOE_ERR_DEVICE;
  }
  if (c->host_ids && hipHostFree(c->host_ids) != hipSuccess) rc = MOE_ERR_DEVICE;
  if (c->host_slots && hipHostFree(c->host_slots) != hipSuccess) rc = MOE_ERR_DEVICE;
  if (c->slot_codes && hipFree(c->slot_codes) != hipSuccess) rc = MOE_ERR_DEVICE;
  if (c->slot_scales && hipFree(c->slot_scales) != hipSuccess) rc = MOE_ERR_DEVICE;
  delete c;
  return rc;
}

moe_status moe_cache_slots(moe_expert_cache* c, void** slot_codes, void** slot_scales, int32_t* capacity) {
  if (!c || !slot_codes || !slot_scales || !capacity) return MOE_ERR_NULL;
  *slot_codes = c->slot_codes;
  *slot_scales = c->slot_scales;
  *capacity = c->capacity;
  return MOE_OK;
}

moe_status moe_cache_get_stats(moe_expert_cache* c, moe_cache_stats* out) {
  if (!c || !out) return MOE_ERR_NULL;
  if (out->struct_size != sizeof(moe_cache_stats)) return MOE_ERR_ABI;
  std::lock_guard<std::mutex> g(c->mu);
  *out = c->st;
  return MOE_OK;
}

moe_status moe_cache_plan(moe_expert_cache* c, int32_t layer, const int32_t* ids, int32_t n_ids, int32_t flags,
                          int32_t* slots_out, int32_t* miss_ids, int32_t* n_miss) {
  if (!c || !ids || !n_miss) return MOE_ERR_NULL;
  const bool prefetch = (flags & MOE_CACHE_PREFETCH) != 0;
  if (flags & ~MOE_CACHE_PREFETCH) return MOE_ERR_UNSUPPORTED;
  if (!prefetch && !slots_out) return MOE_ERR_NULL;
  std::lock_guard<std::mutex> g(c->mu);
  if (c->poisoned) return MOE_ERR_POISONED;
  if (c->planned) return MOE_ERR_STATE;
  if (layer < 0 || layer >= c->n_layers || n_ids < 1 || n_ids > c->max_ids) return MOE_ERR_RANGE;
  for (int i = 0; i < n_ids; ++i)
    if (ids[i] < 0 || ids[i] >= c->E) return MOE_ERR_RANGE;
  // the route union, in route order
  std::vector<int32_t> uni;
  uni.reserve((size_t)n_ids);
  for (int i = 0; i < n_ids; ++i) {
    bool seen = false;
    for (int32_t u : uni) seen = seen || u == ids[i];
    if (!seen) uni.push_back(ids[i]);
  }
  if ((int)uni.size() > c->capacity) return MOE_ERR_UNSUPPORTED;
  c->tick += 1;
  const int64_t base = (int64_t)layer * c->E;
  for (int32_t e : uni) {  // hits first: the plan keeps them resident
    const int s = c->slot_of[(size_t)(base + e)];
    if (s >= 0) {
      c->in_plan[s] = 1;
      c->last_use[s] = c->tick;
      if (!prefetch) c->st.hits += 1;
    }
  }
  int nm = 0;
  for (int32_t e : uni) {  // then the misses, in route order
    const size_t key = (size_t)(base + e);
    if (c->slot_of[key] >= 0) continue;
    const int s = pick_slot(c);  // exists: uni.size() <= capacity
    if (c->owner[s] >= 0) {
      c->slot_of[(size_t)c->owner[s]] = -1;
      c->st.evictions += 1;
    }
    c->owner[s] = (int32_t)key;
    c->slot_of[key] = s;
    c->last_use[s] = c->tick;
    c->in_plan[s] = 1;
    c->miss_slot.push_back(s);
    c->miss_key.push_back((int32_t)key);
    if (miss_ids) miss_ids[nm] = e;
    ++nm;
    if (prefetch)
      c->st.prefetched += 1;
    else
      c->st.misses += 1;
  }
  if (!prefetch)
    for (int i = 0; i < n_ids; ++i) slots_out[i] = c->slot_of[(size_t)(base + ids[i])];
  c->st.plans += 1;
  c->planned = true;
  c->plan_prefetch = prefetch;
  *n_miss = nm;
  return MOE_OK;
}

moe_status moe_cache_cancel(moe_expert_cache* c) {
  if (!c) return MOE_ERR_NULL;
  std::lock_guard<std::mutex> g(c->mu);
  if (!c->planned) return MOE_ERR_STATE;
  // the misses' slots hold nothing valid yet: they become free
  for (size_t i = 0; i < c->miss_slot.size(); ++i) {
    c->slot_of[(size_t)c->miss_key[i]] = -1;
    c->owner[(size_t)c->miss_slot[i]] = -1;
  }
  release_plan(c);
  return MOE_OK;
}

moe_status moe_cache_finish(moe_expert_cache* c, const void* const* miss_codes, const void* const* miss_scales,
                            int32_t host_pinned, void* stream) {
  if (!c) return MOE_ERR_NULL;
  std::lock_guard<std::mutex> g(c->mu);
  if (c->poisoned) return MOE_ERR_POISONED;
  if (!c->planned) return MOE_ERR_STATE;
  const size_t nm = c->miss_slot.size();
  if (nm && (!miss_codes || !miss_scales)) return MOE_ERR_NULL;
  for (size_t i = 0; i < nm; ++i)
    if (!miss_codes[i] || !miss_scales[i]) return MOE_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (size_t i = 0; i < nm; ++i) {
    if (c->uploads++ == c->fail_at) return poison(c);
    uint8_t* dc = c->slot_codes + (size_t)c->miss_slot[i] * c->cb;
    uint8_t* ds = c->slot_scales + (size_t)c->miss_slot[i] * c->sb;
    if (host_pinned) {  // direct DMA from the caller's pinned spans
      if (hipMemcpyAsync(dc, miss_codes[i], c->cb, hipMemcpyHostToDevice, s) != hipSuccess ||
          hipMemcpyAsync(ds, miss_scales[i], c->sb, hipMemcpyHostToDevice, s) != hipSuccess)
        return poison(c);
    } else {  // through the staging slabs, alternately
      const int k = (int)(i % 2);
      if (c->slab_busy[k] && hipEventSynchronize(c->slab_ev[k]) != hipSuccess) return poison(c);
      memcpy(c->slab[k], miss_codes[i], c->cb);
      memcpy(c->slab[k] + c->cb, miss_scales[i], c->sb);
      if (hipMemcpyAsync(dc, c->slab[k], c->cb, hipMemcpyHostToDevice, s) != hipSuccess ||
          hipMemcpyAsync(ds, c->slab[k] + c->cb, c->sb, hipMemcpyHostToDevice, s) != hipSuccess ||
          hipEventRecord(c->slab_ev[k], s) != hipSuccess)
        return poison(c);
      c->slab_busy[k] = true;
    }
    c->st.bytes_uploaded += (uint64_t)(c->cb + c->sb);
  }
  release_plan(c);
  return MOE_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- one streamed layer call

namespace {

#define CACHE_TRY(expr)              \
  do {                               \
    moe_status rc_ = (expr);         \
    if (rc_ != MOE_OK) return rc_;   \
  } while (0)

inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Workspace layout of moe_cache_layer_forward: logits [T][E], ids [T][k],
// weights [T][k], slot ids [T][k] (each 256-byte aligned), then the slot
// layer's forward workspace.
struct StreamLayout {
  size_t logits, ids, w, slots, fwd, fwd_bytes, total;
};

size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

moe_status stream_layout(moe_expert_cache* c, int32_t T, int32_t k, StreamLayout* L) {
  moe_layer_desc ds = c->desc;
  ds.n_experts = c->capacity;
  if (ds.top_k_max > ds.n_experts) ds.top_k_max = ds.n_experts;
  CACHE_TRY(moe_workspace_bytes(&ds, T, k, &L->fwd_bytes));
  size_t off = 0;
  L->logits = off;
  off = up256(off + (size_t)T * c->E * 4);
  L->ids = off;
  off = up256(off + (size_t)T * k * 4);
  L->w = off;
  off = up256(off + (size_t)T * k * 4);
  L->slots = off;
  off = up256(off + (size_t)T * k * 4);
  L->fwd = off;
  L->total = off + L->fwd_bytes;
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_cache_workspace_bytes(moe_expert_cache* c, int32_t n_tokens, int32_t k, size_t* bytes) {
  if (!c || !bytes) return MOE_ERR_NULL;
  if (n_tokens < 1 || n_tokens > kStreamedMaxTokens || k < 1 || k > c->desc.top_k_max) return MOE_ERR_SHAPE;
  StreamLayout L;
  CACHE_TRY(stream_layout(c, n_tokens, k, &L));
  *bytes = L.total;
  return MOE_OK;
}

moe_status moe_cache_layer_forward(moe_expert_cache* c, int32_t layer, const void* x, moe_dtype x_dtype,
                                   const float* router_w, const float* router_bias, const void* host_codes,
                                   const void* host_scales, int32_t host_pinned, int32_t n_tokens, int32_t k,
                                   float* out, int32_t* topk_idx_out, float* topk_w_out, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (!c || !x || !router_w || !host_codes || !host_scales || !out || !workspace) return MOE_ERR_NULL;
  if (c->poisoned) return MOE_ERR_POISONED;
  if (layer < 0 || layer >= c->n_layers) return MOE_ERR_RANGE;
  if (n_tokens < 1 || n_tokens > kStreamedMaxTokens || k < 1 || k > c->desc.top_k_max) return MOE_ERR_SHAPE;
  if (!al16(workspace)) return MOE_ERR_ALIGN;
  StreamLayout L;
  CACHE_TRY(stream_layout(c, n_tokens, k, &L));
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  float* logits = reinterpret_cast<float*>(ws + L.logits);
  int32_t* ids = reinterpret_cast<int32_t*>(ws + L.ids);
  float* w = reinterpret_cast<float*>(ws + L.w);
  int32_t* slots = reinterpret_cast<int32_t*>(ws + L.slots);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // routing on the device, then the route read back (the plan needs it)
  CACHE_TRY(moe_router_logits(&c->desc, x, x_dtype, router_w, router_bias, n_tokens, logits, stream));
  CACHE_TRY(moe_topk_softmax(logits, n_tokens, c->E, k, ids, w, stream));
  const int32_t P = n_tokens * k;
  if (hipMemcpyAsync(c->host_ids, ids, (size_t)P * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return MOE_ERR_DEVICE;
  int32_t n_miss = 0;
  std::vector<int32_t> miss((size_t)P);
  CACHE_TRY(moe_cache_plan(c, layer, c->host_ids, P, 0, c->host_slots, miss.data(), &n_miss));
  std::vector<const void*> mc((size_t)n_miss), ms((size_t)n_miss);
  for (int i = 0; i < n_miss; ++i) {
    mc[(size_t)i] = static_cast<const uint8_t*>(host_codes) + (size_t)miss[(size_t)i] * c->cb;
    ms[(size_t)i] = static_cast<const uint8_t*>(host_scales) + (size_t)miss[(size_t)i] * c->sb;
  }
  CACHE_TRY(moe_cache_finish(c, mc.data(), ms.data(), host_pinned, stream));
  if (hipMemcpyAsync(slots, c->host_slots, (size_t)P * 4, hipMemcpyHostToDevice, s) != hipSuccess)
    return MOE_ERR_DEVICE;
  moe_layer_desc ds = c->desc;
  ds.n_experts = c->capacity;
  if (ds.top_k_max > ds.n_experts) ds.top_k_max = ds.n_experts;
  CACHE_TRY(moe_mxfp4_experts(&ds, x, x_dtype, slots, w, c->slot_codes, c->slot_scales, n_tokens, k, out,
                              ws + L.fwd, L.fwd_bytes, stream));
  if (topk_idx_out && hipMemcpyAsync(topk_idx_out, ids, (size_t)P * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return MOE_ERR_DEVICE;
  if (topk_w_out && hipMemcpyAsync(topk_w_out, w, (size_t)P * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return MOE_ERR_DEVICE;
  return MOE_OK;
}

}  // extern "C"
