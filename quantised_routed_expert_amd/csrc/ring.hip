// Expert ring: an LRU cache of (layer, expert) blobs in HBM slots, filled from
// a vault in host memory ("The Ring Is an LRU Cache", Optimizations page;
// slot clamp [64, 4096] from the System Overview memory budget).
//
// Policy (host side, single-threaded per handle):
//   - a request for a resident (layer, expert) is a hit: no bytes move;
//   - a miss takes the lowest-index empty slot, else evicts the unpinned slot
//     with the oldest tick (lazy LRU; slots held by the current acquisition are
//     pinned and never evicted);
//   - every request, hit or load, stamps the slot with a fresh tick;
//   - slots keep their data and identity when released; nothing is ever wiped.
// Data movement: misses are copied with hipMemcpyAsync on the copy stream.
// Before the copies of an acquisition, the copy stream waits for all work
// already enqueued on the compute stream (so no slot is overwritten while an
// earlier kernel may still read it); after them, the compute stream waits on
// the completion event of every slot it is handed.
// A vault layer in page-locked memory is copied directly.  A pageable layer
// goes through the ring's own pipeline: a pool of host threads copies the
// blob into one of kStages page-locked staging buffers while the DMA of the
// previous blob runs (the HIP runtime's own staging of pageable copies
// reaches about half of the link's page-locked rate).
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <condition_variable>
#include <mutex>
#include <new>
#include <thread>
#include <vector>

#include "kernels.h"

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

// A fixed pool of host threads that copy one buffer in parallel parts.
class CopyPool {
 public:
  explicit CopyPool(int n) {
    for (int i = 0; i < n; ++i) th_.emplace_back([this, i] { run(i + 1); });
  }
  ~CopyPool() {
    {
      std::lock_guard<std::mutex> g(m_);
      stop_ = true;
    }
    cv_.notify_all();
    for (std::thread& t : th_) t.join();
  }
  // Copies `bytes` from src to dst with every pool thread and the caller.
  void copy(char* dst, const char* src, size_t bytes) {
    const int parts = (int)th_.size() + 1;
    {
      std::lock_guard<std::mutex> g(m_);
      dst_ = dst;
      src_ = src;
      bytes_ = bytes;
      parts_ = parts;
      pending_ = (int)th_.size();
      ++gen_;
    }
    cv_.notify_all();
    part(0);
    std::unique_lock<std::mutex> l(m_);
    done_.wait(l, [this] { return pending_ == 0; });
  }

 private:
  void part(int i) {
    const size_t per = ((bytes_ + parts_ - 1) / parts_ + 63) & ~(size_t)63;
    const size_t lo = (size_t)i * per;
    if (lo < bytes_) memcpy(dst_ + lo, src_ + lo, (bytes_ - lo < per ? bytes_ - lo : per));
  }
  void run(int i) {
    unsigned long long seen = 0;
    for (;;) {
      {
        std::unique_lock<std::mutex> l(m_);
        cv_.wait(l, [&] { return stop_ || gen_ != seen; });
        if (stop_) return;
        seen = gen_;
      }
      part(i);
      {
        std::lock_guard<std::mutex> g(m_);
        if (--pending_ == 0) done_.notify_one();
      }
    }
  }
  std::vector<std::thread> th_;
  std::mutex m_;
  std::condition_variable cv_, done_;
  char* dst_ = nullptr;
  const char* src_ = nullptr;
  size_t bytes_ = 0;
  int parts_ = 1, pending_ = 0;
  unsigned long long gen_ = 0;
  bool stop_ = false;
};

}  // namespace

struct smoe_ring {
  smoe_ring_desc desc;
  std::vector<long long> key;      // per slot: layer * E + expert, or -1 when empty
  std::vector<unsigned long long> tick;
  std::vector<unsigned char> pinned;
  std::vector<unsigned char> fill_recorded;
  std::vector<hipEvent_t> fill_done;  // per slot, recorded after its latest fill
  std::vector<int> where;          // (layer * E + expert) -> slot, or -1
  std::vector<unsigned long long> claims;  // (layer * E + expert) -> demand requests
  std::vector<int> held;           // slots of the current acquisition
  std::vector<const char*> vault;  // per layer: host base of its blobs
  std::vector<unsigned char> pageable;  // per layer: not page-locked (staged)
  char* stage[kStages] = {};       // page-locked staging buffers (only with pageable layers)
  hipEvent_t stage_done[kStages] = {};
  unsigned char stage_used[kStages] = {};
  int next_stage = 0;
  CopyPool* pool = nullptr;
  hipEvent_t compute_mark;
  unsigned long long now = 0;
  int n_filled = 0;                // empty slots are exactly [n_filled, n_slots)
  unsigned long long hits = 0, misses = 0, evictions = 0, h2d_bytes = 0, prefetches = 0;
  std::vector<smoe_ring_event> log;
};

static int hip_err(hipError_t e, const char* what) {
  return fail(SMOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// The slot a load takes: the lowest-index empty slot, else the unpinned slot
// with the oldest tick; -1 when every slot is pinned.
static int victim(const smoe_ring* r) {
  if (r->n_filled < r->desc.n_slots) return r->n_filled;
  unsigned long long best = ~0ull;
  int s = -1;
  for (int i = 0; i < r->desc.n_slots; ++i)
    if (!r->pinned[i] && r->tick[i] < best) {
      best = r->tick[i];
      s = i;
    }
  return s;
}

// Gives slot s to (layer, expert): drops its previous key (recorded in ev as
// the eviction) and copies the blob on the copy stream -- directly from a
// page-locked layer, through a staging buffer from a pageable one -- then
// records the slot's fill event.
static hipError_t load_slot(smoe_ring* r, int layer, int expert, int s, smoe_ring_event& ev) {
  const smoe_ring_desc& d = r->desc;
  hipStream_t ps = (hipStream_t)d.copy_stream;
  if (s == r->n_filled) {
    ++r->n_filled;
  } else {
    const long long old = r->key[s];
    r->where[old] = -1;
    ev.evicted_layer = (int)(old / d.n_experts);
    ev.evicted_expert = (int)(old % d.n_experts);
    ++r->evictions;
  }
  const long long kk = (long long)layer * d.n_experts + expert;
  r->key[s] = kk;
  r->where[kk] = s;
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
    if (he == hipSuccess) he = hipEventRecord(r->stage_done[q], ps);
    r->stage_used[q] = 1;
  } else {
    he = hipMemcpyAsync(dst, src, d.slot_bytes, hipMemcpyHostToDevice, ps);
  }
  if (he == hipSuccess) he = hipEventRecord(r->fill_done[s], ps);
  if (he == hipSuccess) {
    r->fill_recorded[s] = 1;
    r->h2d_bytes += d.slot_bytes;
  }
  return he;
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
  r->vault.resize((size_t)d->n_layers);
  r->pageable.assign((size_t)d->n_layers, 0);
  bool any_pageable = false;
  for (int L = 0; L < d->n_layers; ++L) {
    r->vault[L] = (const char*)d->vault_layers[L];
    hipPointerAttribute_t at;
    const hipError_t pe = hipPointerGetAttributes(&at, d->vault_layers[L]);
    if (pe != hipSuccess) (void)hipGetLastError();  // unregistered host memory
    r->pageable[L] = !(pe == hipSuccess && at.type == hipMemoryTypeHost);
    any_pageable |= r->pageable[L] != 0;
  }
  const size_t n = (size_t)d->n_slots;
  r->key.assign(n, -1);
  r->tick.assign(n, 0);
  r->pinned.assign(n, 0);
  r->fill_recorded.assign(n, 0);
  r->fill_done.assign(n, nullptr);
  r->where.assign((size_t)d->n_layers * d->n_experts, -1);
  r->claims.assign((size_t)d->n_layers * d->n_experts, 0);
  r->log.reserve(d->log_capacity);
  hipError_t e = hipEventCreateWithFlags(&r->compute_mark, hipEventDisableTiming);
  for (size_t i = 0; e == hipSuccess && i < n; ++i) e = hipEventCreateWithFlags(&r->fill_done[i], hipEventDisableTiming);
  for (int i = 0; e == hipSuccess && any_pageable && i < kStages; ++i) {
    e = hipEventCreateWithFlags(&r->stage_done[i], hipEventDisableTiming);
    if (e == hipSuccess) e = hipHostMalloc((void**)&r->stage[i], d->slot_bytes, hipHostMallocDefault);
  }
  if (e == hipSuccess && any_pageable) {
    r->pool = new (std::nothrow) CopyPool(kCopyThreads);
    if (!r->pool) e = hipErrorOutOfMemory;
  }
  if (e != hipSuccess) {
    for (hipEvent_t ev : r->fill_done)
      if (ev) (void)hipEventDestroy(ev);
    for (int i = 0; i < kStages; ++i) {
      if (r->stage_done[i]) (void)hipEventDestroy(r->stage_done[i]);
      if (r->stage[i]) (void)hipHostFree(r->stage[i]);
    }
    if (r->compute_mark) (void)hipEventDestroy(r->compute_mark);
    delete r->pool;
    delete r;
    return hip_err(e, "ring set-up (events, staging buffers)");
  }
  *out = r;
  return SMOE_OK;
}

int smoe_ring_release(smoe_ring* r) {
  if (!r) return fail(SMOE_EINVAL, "NULL ring");
  for (int s : r->held) r->pinned[s] = 0;
  r->held.clear();
  return SMOE_OK;
}

int smoe_ring_acquire(smoe_ring* r, int32_t layer, const int32_t* experts, int32_t k, const void** slot_ptrs,
                      void* compute_stream) {
  if (!r || !experts || !slot_ptrs) return fail(SMOE_EINVAL, "NULL argument");
  const smoe_ring_desc& d = r->desc;
  if (layer < 0 || layer >= d.n_layers) return fail(SMOE_EINVAL, "layer=%d out of range", layer);
  const int kmax = d.n_experts < d.n_slots ? d.n_experts : d.n_slots;
  if (k < 1 || k > kmax) return fail(SMOE_EINVAL, "k=%d must be in [1, %d]", k, kmax);
  for (int i = 0; i < k; ++i) {
    if (experts[i] < 0 || experts[i] >= d.n_experts) return fail(SMOE_EINVAL, "expert %d out of range", experts[i]);
    for (int j = 0; j < i; ++j)
      if (experts[j] == experts[i]) return fail(SMOE_EINVAL, "expert %d requested twice", experts[i]);
  }
  hipStream_t cs = (hipStream_t)compute_stream, ps = (hipStream_t)d.copy_stream;
  smoe_ring_release(r);
  // fills below must not overtake work already enqueued on the compute stream
  hipError_t he = hipEventRecord(r->compute_mark, cs);
  if (he == hipSuccess) he = hipStreamWaitEvent(ps, r->compute_mark, 0);
  if (he != hipSuccess) return hip_err(he, "ordering the copy stream after the compute stream");

  for (int rank = 0; rank < k; ++rank) {
    const long long kk = (long long)layer * d.n_experts + experts[rank];
    int s = r->where[kk];
    smoe_ring_event ev;
    ev.layer = layer;
    ev.rank = rank;
    ev.expert = experts[rank];
    ev.evicted_layer = -1;
    ev.evicted_expert = -1;
    ev.pad = 0;
    ++r->claims[kk];
    if (s >= 0) {
      ev.kind = 0;
      ++r->hits;
    } else {
      s = victim(r);
      if (s < 0) return fail(SMOE_ENOSLOT, "every slot is held by the current layer");
      he = load_slot(r, layer, experts[rank], s, ev);
      if (he != hipSuccess) return hip_err(he, "fill");
      ev.kind = 1;
      ++r->misses;
    }
    r->tick[s] = r->now++;
    r->pinned[s] = 1;
    r->held.push_back(s);
    ev.slot = s;
    if (r->log.size() < d.log_capacity) r->log.push_back(ev);
    slot_ptrs[rank] = (const char*)d.slab_dev + (size_t)s * d.slot_stride;
  }
  // the compute stream may use a slot only once its latest fill has landed
  for (int s : r->held) {
    if (!r->fill_recorded[s]) continue;
    he = hipStreamWaitEvent(cs, r->fill_done[s], 0);
    if (he != hipSuccess) return hip_err(he, "hipStreamWaitEvent");
  }
  return SMOE_OK;
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
  for (int i = 0; i < n; ++i) {
    const long long kk = (long long)layer * d.n_experts + experts[i];
    if (r->where[kk] >= 0) continue;  // resident: a bet that costs nothing
    const int s = victim(r);
    if (s < 0) break;                 // never displaces the current acquisition
    if (!ordered) {                   // loads must not overtake earlier compute
      hipError_t he = hipEventRecord(r->compute_mark, (hipStream_t)compute_stream);
      if (he == hipSuccess) he = hipStreamWaitEvent((hipStream_t)d.copy_stream, r->compute_mark, 0);
      if (he != hipSuccess) return hip_err(he, "ordering the copy stream after the compute stream");
      ordered = true;
    }
    smoe_ring_event ev;
    ev.layer = layer;
    ev.rank = i;
    ev.expert = experts[i];
    ev.kind = 2;
    ev.slot = s;
    ev.evicted_layer = -1;
    ev.evicted_expert = -1;
    ev.pad = 0;
    const hipError_t he = load_slot(r, layer, experts[i], s, ev);
    if (he != hipSuccess) return hip_err(he, "prefetch fill");
    r->tick[s] = r->now++;
    ++r->prefetches;
    ++loaded;
    if (r->log.size() < d.log_capacity) r->log.push_back(ev);
  }
  if (n_loaded) *n_loaded = loaded;
  return SMOE_OK;
}

int smoe_ring_hottest(const smoe_ring* r, int32_t n, int32_t* layers_out, int32_t* experts_out,
                      uint64_t* counts_out, int32_t* n_out) {
  if (!r || !n_out || (n > 0 && (!layers_out || !experts_out))) return fail(SMOE_EINVAL, "NULL argument");
  if (n < 0) return fail(SMOE_EINVAL, "n=%d < 0", n);
  std::vector<int> order;
  for (size_t i = 0; i < r->claims.size(); ++i)
    if (r->claims[i]) order.push_back((int)i);
  const size_t m = order.size() < (size_t)n ? order.size() : (size_t)n;
  std::partial_sort(order.begin(), order.begin() + m, order.end(), [r](int a, int b) {
    return r->claims[a] != r->claims[b] ? r->claims[a] > r->claims[b] : a < b;
  });
  for (size_t i = 0; i < m; ++i) {
    layers_out[i] = order[i] / r->desc.n_experts;
    experts_out[i] = order[i] % r->desc.n_experts;
    if (counts_out) counts_out[i] = r->claims[order[i]];
  }
  *n_out = (int32_t)m;
  return SMOE_OK;
}

int smoe_ring_acquire_table(smoe_ring* r, int32_t layer, const int32_t* experts, int32_t k, void* table_dev,
                            void* compute_stream) {
  if (!r || !experts) return fail(SMOE_EINVAL, "NULL argument");
  if (!table_dev || ((uintptr_t)table_dev & 7u)) return fail(SMOE_EINVAL, "table_dev must be 8-byte aligned");
  smoe::RingTable t;
  memset(&t, 0, sizeof(t));
  std::vector<const void*> ptrs((size_t)(k > 0 ? k : 1));
  if (int e = smoe_ring_acquire(r, layer, experts, k, ptrs.data(), compute_stream)) return e;
  for (int i = 0; i < k; ++i) t.ptr[experts[i]] = ptrs[i];
  const hipError_t he = smoe::launch_ring_table(t, reinterpret_cast<const void**>(table_dev), r->desc.n_experts,
                                                (hipStream_t)compute_stream);
  if (he != hipSuccess) return hip_err(he, "expert table launch");
  return SMOE_OK;
}

int smoe_ring_stats(const smoe_ring* r, uint64_t* hits, uint64_t* misses, uint64_t* evictions,
                    uint64_t* h2d_bytes) {
  if (!r) return fail(SMOE_EINVAL, "NULL ring");
  if (hits) *hits = r->hits;
  if (misses) *misses = r->misses;
  if (evictions) *evictions = r->evictions;
  if (h2d_bytes) *h2d_bytes = r->h2d_bytes;
  return SMOE_OK;
}

int smoe_ring_log(const smoe_ring* r, smoe_ring_event* events, size_t cap, size_t* n_out) {
  if (!r || !n_out || (cap && !events)) return fail(SMOE_EINVAL, "NULL argument");
  const size_t n = r->log.size() < cap ? r->log.size() : cap;
  if (n) memcpy(events, r->log.data(), n * sizeof(smoe_ring_event));
  *n_out = n;
  return SMOE_OK;
}

int smoe_ring_destroy(smoe_ring* r) {
  if (!r) return SMOE_OK;
  if (!r->held.empty()) return fail(SMOE_EBUSY, "slots are still held: release first");
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
  for (hipEvent_t ev : r->fill_done) (void)hipEventDestroy(ev);
  for (int i = 0; i < kStages; ++i) {
    if (r->stage_done[i]) (void)hipEventDestroy(r->stage_done[i]);
    if (r->stage[i]) (void)hipHostFree(r->stage[i]);
  }
  delete r->pool;
  (void)hipEventDestroy(r->compute_mark);
  delete r;
  return SMOE_OK;
}

}  // extern "C"
