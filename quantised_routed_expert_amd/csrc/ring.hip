// Expert ring: an LRU cache of (layer, expert) blobs in HBM slots, filled from
// a vault in host memory ("The Ring Is an LRU Cache", Optimizations page;
// slot clamp [64, 4096] from the System Overview memory budget).
//
// The slot policy (hits, lazy LRU eviction that never takes a held slot,
// fresh ticks on every request, the claim histogram and the event log) lives
// in ring_policy.h, host code that the CPU tests also drive; this file adds
// the data movement.  Misses are copied with hipMemcpyAsync on the copy
// stream.  Before the copies of an acquisition, the copy stream waits for all
// work already enqueued on the compute stream (so no slot is overwritten while
// an earlier kernel may still read it); after them, the compute stream waits
// on the completion event of every slot it is handed.
// A vault layer in page-locked memory is copied directly.  A pageable layer
// goes through the ring's own pipeline: the threads of copy_pool.h copy the
// blob into one of kStages page-locked staging buffers while the DMA of the
// previous blob runs (the HIP runtime's own staging of pageable copies
// reaches about half of the link's page-locked rate).
// Every host buffer is sized at create; the acquire, release, prefetch and
// statistics calls allocate nothing and take no lock ("Zero Allocations, Zero
// Locks in the Token Loop").
#include <stdlib.h>
#include <string.h>

#include <new>
#include <vector>

#include "copy_pool.h"
#include "kernels.h"
#include "ring_policy.h"

namespace smoe {
int fail(int code, const char* fmt, ...);
}
using smoe::fail;

namespace smoe {

// Writes a layer's [E] expert table from pointers passed by value.
__global__ __launch_bounds__(256) void ring_table_kernel(RingTable t, const void** table, int E) {
  if ((int)threadIdx.x < E) table[threadIdx.x] = t.ptr[threadIdx.x];
}

hipError_t launch_ring_table(const RingTable& t, const void** table, int E, hipStream_t s) {
  hipLaunchKernelGGL(ring_table_kernel, dim3(1), dim3(256), 0, s, t, table, E);
  return hipGetLastError();
}

}  // namespace smoe

namespace {

constexpr int kStages = 4;         // page-locked staging buffers for pageable layers
constexpr int kCopyThreads = 8;    // host threads that fill a staging buffer
constexpr int kMaxRouted = smoe::kMaxPrefillTokens * smoe::kMaxTopK;  // routing entries of one chunk

}  // namespace

struct smoe_ring {
  smoe_ring_desc desc;
  smoe::RingPolicy pol;                 // slots, ticks, holds, claims, statistics, log
  std::vector<unsigned char> fill_recorded;
  std::vector<hipEvent_t> fill_done;    // per slot, recorded after its latest fill
  std::vector<const char*> vault;       // per layer: host base of its blobs
  std::vector<unsigned char> pageable;  // per layer: not page-locked (staged)
  std::vector<int> slots;               // scratch: the slots of one acquisition
  std::vector<int32_t> uni;             // scratch: a chunk's union in first-touch order
  std::vector<unsigned char> seen;      // scratch: [E] experts already in the union
  char* stage[kStages] = {};            // page-locked staging buffers (only with pageable layers)
  hipEvent_t stage_done[kStages] = {};
  unsigned char stage_used[kStages] = {};
  int next_stage = 0;
  smoe::CopyPool* pool = nullptr;
  int32_t* idx_host = nullptr;          // page-locked: a chunk's routing read back for acquire_routed
  hipEvent_t idx_ready = nullptr;
  hipEvent_t compute_mark = nullptr;
  unsigned long long h2d_bytes = 0;
};

static int hip_err(hipError_t e, const char* what) {
  return fail(SMOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Copies blob (layer, expert) into slot s on the copy stream -- directly from
// a page-locked layer, through a staging buffer from a pageable one -- and
// records the slot's fill event.  Returns 0 or SMOE_EHIP (message set).
static int fill_slot(smoe_ring* r, int layer, int expert, int s) {
  const smoe_ring_desc& d = r->desc;
  hipStream_t ps = (hipStream_t)d.copy_stream;
  const char* src = r->vault[layer] + (size_t)expert * d.vault_stride;
  char* dst = (char*)d.slab_dev + (size_t)s * d.slot_stride;
  hipError_t he;
  if (r->pageable[layer]) {
    // host copy into a free staging buffer while earlier DMAs run
    const int q = r->next_stage;
    r->next_stage = (q + 1) % kStages;
    he = r->stage_used[q] ? hipEventSynchronize(r->stage_done[q]) : hipSuccess;
    if (he == hipSuccess) {
      r->pool->copy(r->stage[q], src, d.slot_bytes);
      he = hipMemcpyAsync(dst, r->stage[q], d.slot_bytes, hipMemcpyHostToDevice, ps);
    }
    if (he == hipSuccess) {
      he = hipEventRecord(r->stage_done[q], ps);
      r->stage_used[q] = 1;
    }
  } else {
    he = hipMemcpyAsync(dst, src, d.slot_bytes, hipMemcpyHostToDevice, ps);
  }
  if (he == hipSuccess) he = hipEventRecord(r->fill_done[s], ps);
  if (he != hipSuccess) return hip_err(he, "fill");
  r->fill_recorded[s] = 1;
  r->h2d_bytes += d.slot_bytes;
  return 0;
}

// Orders the copy stream after the work already enqueued on compute_stream,
// so that no fill overwrites a slot an earlier kernel may still read.
static int order_copies(smoe_ring* r, void* compute_stream) {
  hipError_t he = hipEventRecord(r->compute_mark, (hipStream_t)compute_stream);
  if (he == hipSuccess) he = hipStreamWaitEvent((hipStream_t)r->desc.copy_stream, r->compute_mark, 0);
  if (he != hipSuccess) return hip_err(he, "ordering the copy stream after the compute stream");
  return 0;
}

// The acquisition of layer's experts[0..k) (validated): policy decisions,
// fills, then the compute stream's waits on every held slot's latest fill.
// r->slots[i] = slot of request i.
static int acquire_checked(smoe_ring* r, int layer, const int32_t* experts, int k, void* compute_stream) {
  if (int e = order_copies(r, compute_stream)) return e;
  const int rc = r->pol.acquire(layer, experts, k, [&](int expert, int s) { return fill_slot(r, layer, expert, s); },
                                r->slots.data());
  if (rc == smoe::RingPolicy::kNoSlot) return fail(SMOE_ENOSLOT, "every slot is held by the current acquisition");
  if (rc) return rc;
  // the compute stream may use a slot only once its latest fill has landed
  for (int s : r->pol.held()) {
    if (!r->fill_recorded[s]) continue;
    const hipError_t he = hipStreamWaitEvent((hipStream_t)compute_stream, r->fill_done[s], 0);
    if (he != hipSuccess) return hip_err(he, "hipStreamWaitEvent");
  }
  return SMOE_OK;
}

// Writes the layer's [E] device table: the slot of each acquired expert, NULL
// for the others (a kernel on compute_stream, after the fills' waits).
static int write_table(smoe_ring* r, const int32_t* experts, int k, void* table_dev, void* compute_stream) {
  smoe::RingTable t;
  memset(&t, 0, sizeof(t));
  for (int i = 0; i < k; ++i)
    t.ptr[experts[i]] = (const char*)r->desc.slab_dev + (size_t)r->slots[i] * r->desc.slot_stride;
  const hipError_t he = smoe::launch_ring_table(t, reinterpret_cast<const void**>(table_dev), r->desc.n_experts,
                                                (hipStream_t)compute_stream);
  if (he != hipSuccess) return hip_err(he, "expert table launch");
  return SMOE_OK;
}

static void destroy_resources(smoe_ring* r) {
  for (hipEvent_t ev : r->fill_done)
    if (ev) (void)hipEventDestroy(ev);
  for (int i = 0; i < kStages; ++i) {
    if (r->stage_done[i]) (void)hipEventDestroy(r->stage_done[i]);
    if (r->stage[i]) (void)hipHostFree(r->stage[i]);
  }
  if (r->idx_host) (void)hipHostFree(r->idx_host);
  if (r->idx_ready) (void)hipEventDestroy(r->idx_ready);
  if (r->compute_mark) (void)hipEventDestroy(r->compute_mark);
  delete r->pool;
}

extern "C" {

int smoe_ring_create(const smoe_ring_desc* d, smoe_ring** out) {
  if (!d || !out) return fail(SMOE_EINVAL, "NULL argument");
  *out = nullptr;
  if (d->n_slots < 64 || d->n_slots > 4096)
    return fail(SMOE_EINVAL, "n_slots=%d must be in [64, 4096]", d->n_slots);
  if (d->n_layers < 1 || d->n_experts < 1 || d->n_experts > smoe::kMaxExperts)
    return fail(SMOE_EINVAL, "n_layers=%d / n_experts=%d out of range", d->n_layers, d->n_experts);
  if (d->top_k < 1 || d->top_k > d->n_experts || d->top_k > smoe::kMaxTopK || d->n_slots < d->top_k)
    return fail(SMOE_EINVAL, "top_k=%d out of range for %d experts / %d slots", d->top_k, d->n_experts,
                d->n_slots);
  if (d->slot_bytes == 0 || d->slot_stride < d->slot_bytes || d->slot_stride % 16)
    return fail(SMOE_EINVAL, "slot_bytes/slot_stride invalid (stride must be >= bytes, multiple of 16)");
  if (!d->vault_layers || d->vault_stride < d->slot_bytes || !d->slab_dev)
    return fail(SMOE_EINVAL, "vault_layers / vault_stride / slab_dev invalid");
  for (int L = 0; L < d->n_layers; ++L)
    if (!d->vault_layers[L]) return fail(SMOE_EINVAL, "vault_layers[%d] is NULL", L);
  if (((uintptr_t)d->slab_dev & 15u) != 0) return fail(SMOE_EINVAL, "slab_dev must be 16-byte aligned");
  smoe_ring* r = new (std::nothrow) smoe_ring();
  if (!r) return fail(SMOE_ENOMEM, "host allocation failed");
  r->desc = *d;
  r->desc.vault_layers = nullptr;  // the caller's array need not outlive create
  const size_t n = (size_t)d->n_slots;
  bool any_pageable = false;
  try {  // every host container is sized here, once
    r->pol.setup(d->n_slots, d->n_layers, d->n_experts, d->log_capacity);
    r->vault.resize((size_t)d->n_layers);
    r->pageable.assign((size_t)d->n_layers, 0);
    r->fill_recorded.assign(n, 0);
    r->fill_done.assign(n, nullptr);
    r->slots.assign((size_t)(d->n_experts < d->n_slots ? d->n_experts : d->n_slots), -1);
    r->uni.reserve((size_t)d->n_experts);
    r->seen.assign((size_t)d->n_experts, 0);
  } catch (...) {
    delete r;
    return fail(SMOE_ENOMEM, "host allocation failed");
  }
  for (int L = 0; L < d->n_layers; ++L) {
    r->vault[L] = (const char*)d->vault_layers[L];
    hipPointerAttribute_t at;
    const hipError_t pe = hipPointerGetAttributes(&at, d->vault_layers[L]);
    if (pe != hipSuccess) (void)hipGetLastError();  // unregistered host memory
    r->pageable[L] = !(pe == hipSuccess && at.type == hipMemoryTypeHost);
    any_pageable |= r->pageable[L] != 0;
  }
  hipError_t e = hipEventCreateWithFlags(&r->compute_mark, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&r->idx_ready, hipEventDisableTiming);
  if (e == hipSuccess) e = hipHostMalloc((void**)&r->idx_host, kMaxRouted * sizeof(int32_t), hipHostMallocDefault);
  for (size_t i = 0; e == hipSuccess && i < n; ++i) e = hipEventCreateWithFlags(&r->fill_done[i], hipEventDisableTiming);
  for (int i = 0; e == hipSuccess && any_pageable && i < kStages; ++i) {
    e = hipEventCreateWithFlags(&r->stage_done[i], hipEventDisableTiming);
    if (e == hipSuccess) e = hipHostMalloc((void**)&r->stage[i], d->slot_bytes, hipHostMallocDefault);
  }
  if (e == hipSuccess && any_pageable) {
    r->pool = new (std::nothrow) smoe::CopyPool(kCopyThreads);
    if (!r->pool) e = hipErrorOutOfMemory;
  }
  if (e != hipSuccess) {
    destroy_resources(r);
    delete r;
    return hip_err(e, "ring set-up (events, page-locked buffers)");
  }
  *out = r;
  return SMOE_OK;
}

int smoe_ring_release(smoe_ring* r) {
  if (!r) return fail(SMOE_EINVAL, "NULL ring");
  r->pol.release();
  return SMOE_OK;
}

int smoe_ring_acquire(smoe_ring* r, int32_t layer, const int32_t* experts, int32_t k, const void** slot_ptrs,
                      void* compute_stream) {
  if (!r || !experts || !slot_ptrs) return fail(SMOE_EINVAL, "NULL argument");
  if (const char* msg = r->pol.check_request(layer, experts, k))
    return fail(SMOE_EINVAL, "acquire(layer=%d, k=%d): %s", layer, k, msg);
  if (int e = acquire_checked(r, layer, experts, k, compute_stream)) return e;
  for (int i = 0; i < k; ++i)
    slot_ptrs[i] = (const char*)r->desc.slab_dev + (size_t)r->slots[i] * r->desc.slot_stride;
  return SMOE_OK;
}

int smoe_ring_acquire_table(smoe_ring* r, int32_t layer, const int32_t* experts, int32_t k, void* table_dev,
                            void* compute_stream) {
  if (!r || !experts) return fail(SMOE_EINVAL, "NULL argument");
  if (!table_dev || ((uintptr_t)table_dev & 7u)) return fail(SMOE_EINVAL, "table_dev must be 8-byte aligned");
  if (const char* msg = r->pol.check_request(layer, experts, k))
    return fail(SMOE_EINVAL, "acquire(layer=%d, k=%d): %s", layer, k, msg);
  if (int e = acquire_checked(r, layer, experts, k, compute_stream)) return e;
  return write_table(r, experts, k, table_dev, compute_stream);
}

int smoe_ring_acquire_routed(smoe_ring* r, int32_t layer, int32_t n_tok, int32_t k, const int32_t* topk_idx_dev,
                             void* table_dev, int32_t* union_host, int32_t* n_union, void* compute_stream) {
  if (!r || !topk_idx_dev) return fail(SMOE_EINVAL, "NULL argument");
  if (!table_dev || ((uintptr_t)table_dev & 7u)) return fail(SMOE_EINVAL, "table_dev must be 8-byte aligned");
  if (n_tok < 1 || n_tok > smoe::kMaxPrefillTokens || k < 1 || k > smoe::kMaxTopK)
    return fail(SMOE_EINVAL, "n_tok=%d must be in [1, %d] and k=%d in [1, %d]", n_tok, smoe::kMaxPrefillTokens, k,
                smoe::kMaxTopK);
  if (layer < 0 || layer >= r->desc.n_layers) return fail(SMOE_EINVAL, "layer=%d out of range", layer);
  // the chunk's routing, read back once the router has written it
  hipStream_t cs = (hipStream_t)compute_stream;
  hipError_t he = hipMemcpyAsync(r->idx_host, topk_idx_dev, (size_t)n_tok * k * sizeof(int32_t),
                                 hipMemcpyDeviceToHost, cs);
  if (he == hipSuccess) he = hipEventRecord(r->idx_ready, cs);
  if (he == hipSuccess) he = hipEventSynchronize(r->idx_ready);
  if (he != hipSuccess) return hip_err(he, "reading the routing back");
  // union in first-touch order: t ascending, then rank; ids outside [0, E)
  // (never produced by the router) take no part
  const int E = r->desc.n_experts;
  memset(r->seen.data(), 0, (size_t)E);
  r->uni.clear();
  for (int i = 0; i < n_tok * k; ++i) {
    const int e = r->idx_host[i];
    if (e >= 0 && e < E && !r->seen[e]) {
      r->seen[e] = 1;
      r->uni.push_back(e);  // within the capacity reserved at create
    }
  }
  const int nu = (int)r->uni.size();
  if (nu == 0) return fail(SMOE_EINVAL, "the routing holds no expert in [0, %d)", E);
  if (const char* msg = r->pol.check_request(layer, r->uni.data(), nu))
    return fail(SMOE_EINVAL, "acquire_routed(layer=%d, union of %d): %s", layer, nu, msg);
  if (int e = acquire_checked(r, layer, r->uni.data(), nu, compute_stream)) return e;
  if (union_host) memcpy(union_host, r->uni.data(), (size_t)nu * sizeof(int32_t));
  if (n_union) *n_union = nu;
  return write_table(r, r->uni.data(), nu, table_dev, compute_stream);
}

int smoe_ring_prefetch(smoe_ring* r, int32_t layer, const int32_t* experts, int32_t n, int32_t* n_loaded,
                       void* compute_stream) {
  if (!r || (n > 0 && !experts)) return fail(SMOE_EINVAL, "NULL argument");
  const smoe_ring_desc& d = r->desc;
  if (n_loaded) *n_loaded = 0;
  if (layer < 0 || layer >= d.n_layers) return fail(SMOE_EINVAL, "layer=%d out of range", layer);
  if (n < 0 || n > d.n_experts) return fail(SMOE_EINVAL, "n=%d must be in [0, %d]", n, d.n_experts);
  for (int i = 0; i < n; ++i)
    if (experts[i] < 0 || experts[i] >= d.n_experts) return fail(SMOE_EINVAL, "expert %d out of range", experts[i]);
  bool ordered = false;
  int loaded = 0;
  const int rc = r->pol.prefetch(layer, experts, n,
                                 [&](int expert, int s) {
                                   if (!ordered) {  // loads must not overtake earlier compute
                                     if (int e = order_copies(r, compute_stream)) return e;
                                     ordered = true;
                                   }
                                   return fill_slot(r, layer, expert, s);
                                 },
                                 &loaded);
  if (n_loaded) *n_loaded = loaded;
  return rc ? rc : SMOE_OK;
}

int smoe_ring_hottest(const smoe_ring* r, int32_t n, int32_t* layers_out, int32_t* experts_out,
                      uint64_t* counts_out, int32_t* n_out) {
  if (!r || !n_out || (n > 0 && (!layers_out || !experts_out))) return fail(SMOE_EINVAL, "NULL argument");
  if (n < 0) return fail(SMOE_EINVAL, "n=%d < 0", n);
  // the claim histogram's scratch order lives in the handle (no allocation)
  *n_out = const_cast<smoe_ring*>(r)->pol.hottest(n, layers_out, experts_out, counts_out);
  return SMOE_OK;
}

int smoe_ring_stats(const smoe_ring* r, uint64_t* hits, uint64_t* misses, uint64_t* evictions,
                    uint64_t* h2d_bytes) {
  if (!r) return fail(SMOE_EINVAL, "NULL ring");
  if (hits) *hits = r->pol.hits();
  if (misses) *misses = r->pol.misses();
  if (evictions) *evictions = r->pol.evictions();
  if (h2d_bytes) *h2d_bytes = r->h2d_bytes;
  return SMOE_OK;
}

int smoe_ring_log(const smoe_ring* r, smoe_ring_event* events, size_t cap, size_t* n_out) {
  if (!r || !n_out || (cap && !events)) return fail(SMOE_EINVAL, "NULL argument");
  const std::vector<smoe_ring_event>& log = r->pol.log();
  const size_t n = log.size() < cap ? log.size() : cap;
  if (n) memcpy(events, log.data(), n * sizeof(smoe_ring_event));
  *n_out = n;
  return SMOE_OK;
}

int smoe_ring_destroy(smoe_ring* r) {
  if (!r) return SMOE_OK;
  if (r->pol.holding()) return fail(SMOE_EBUSY, "slots are still held: release first");
  // no copy into the caller's slab may outlive the handle
  for (size_t i = 0; i < r->fill_done.size(); ++i) {
    if (r->fill_recorded[i]) {
      const hipError_t e = hipEventSynchronize(r->fill_done[i]);
      if (e != hipSuccess) return hip_err(e, "waiting for pending fills");
    }
  }
  for (int i = 0; i < kStages; ++i) {
    if (r->stage_used[i]) {
      const hipError_t e = hipEventSynchronize(r->stage_done[i]);
      if (e != hipSuccess) return hip_err(e, "waiting for staged fills");
    }
  }
  destroy_resources(r);
  delete r;
  return SMOE_OK;
}

}  // extern "C"
