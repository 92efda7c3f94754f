// Slot policy of the expert ring, host code only (no HIP): which slot a
// (layer, expert) request uses, what it evicts, and the bookkeeping of ticks,
// holds, claims, statistics and the event log.  The library's ring calls it
// around its copies; the CPU tests drive the same code directly.
//
// "The Ring Is an LRU Cache" (Optimizations page):
//   - a request for a resident (layer, expert) is a hit: no bytes move;
//   - a miss takes the lowest-index empty slot, else evicts the unheld slot
//     with the oldest tick (lazy least-recently-used; the slots of the current
//     acquisition are held and never evicted);
//   - every request, hit or load, stamps its slot with a fresh tick;
//   - released slots keep their data and identity; nothing is ever wiped.
// A speculative load (the Optimizations page's "ranks 9-16" bets, or an
// idle-time prewarm) takes the slot a miss would take, gets a fresh tick and
// no hold, and stops at the first bet for which every slot is held.
//
// Every container is sized once in setup(); the request paths allocate
// nothing ("Zero Allocations, Zero Locks in the Token Loop").  A slot's new
// identity is committed only after the caller's fill (the copy into the slot)
// was enqueued, so a failed fill leaves the policy as it was before that
// request.  Single-threaded per ring.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "../../include/smoe.h"

namespace smoe {

class RingPolicy {
 public:
  // Sizes every container (may throw std::bad_alloc).
  void setup(int n_slots, int n_layers, int n_experts, size_t log_capacity) {
    n_slots_ = n_slots;
    n_layers_ = n_layers;
    n_experts_ = n_experts;
    const size_t keys = (size_t)n_layers * (size_t)n_experts;
    key_.assign((size_t)n_slots, -1);
    tick_.assign((size_t)n_slots, 0);
    pinned_.assign((size_t)n_slots, 0);
    where_.assign(keys, -1);
    claims_.assign(keys, 0);
    held_.clear();
    held_.reserve((size_t)n_slots);
    order_.clear();
    order_.reserve(keys);
    log_.clear();
    log_.reserve(log_capacity);
    log_capacity_ = log_capacity;
  }

  int n_slots() const { return n_slots_; }
  int n_experts() const { return n_experts_; }
  bool holding() const { return !held_.empty(); }
  const std::vector<int>& held() const { return held_; }

  // Checks an acquisition request: layer in range, 1 <= k <= min(E, slots),
  // experts in range and distinct.  Returns 0 or a message.
  const char* check_request(int layer, const int32_t* experts, int k) const {
    if (layer < 0 || layer >= n_layers_) return "layer out of range";
    const int kmax = n_experts_ < n_slots_ ? n_experts_ : n_slots_;
    if (k < 1 || k > kmax) return "k must be in [1, min(E, n_slots)]";
    for (int i = 0; i < k; ++i) {
      if (experts[i] < 0 || experts[i] >= n_experts_) return "expert out of range";
      for (int j = 0; j < i; ++j)
        if (experts[j] == experts[i]) return "expert requested twice";
    }
    return nullptr;
  }

  // Drops the current holds (the slots stay resident).
  void release() {
    for (int s : held_) pinned_[s] = 0;
    held_.clear();
  }

  // The slot a load takes: the lowest-index empty slot, else the unheld slot
  // with the oldest tick; -1 when every slot is held.
  int victim() const {
    if (n_filled_ < n_slots_) return n_filled_;
    unsigned long long best = ~0ull;
    int s = -1;
    for (int i = 0; i < n_slots_; ++i)
      if (!pinned_[i] && tick_[i] < best) {
        best = tick_[i];
        s = i;
      }
    return s;
  }

  // A demand acquisition of layer's experts[0..k) in order, after an implicit
  // release.  fill(expert, slot) must enqueue the blob's copy into the slot
  // and return 0, or a nonzero error code that acquire() returns at once (the
  // requests before it stay committed and held).  slots_out[r] = slot of
  // request r.  Returns 0, kNoSlot when every slot is held, or fill's code.
  static constexpr int kNoSlot = -1;
  template <class Fill>
  int acquire(int layer, const int32_t* experts, int k, Fill&& fill, int* slots_out) {
    release();
    for (int r = 0; r < k; ++r) {
      const long long kk = (long long)layer * n_experts_ + experts[r];
      int s = where_[kk];
      smoe_ring_event ev = event(layer, r, experts[r]);
      if (s >= 0) {
        ev.kind = 0;
        ++hits_;
      } else {
        s = victim();
        if (s < 0) return kNoSlot;
        if (const int e = fill(experts[r], s)) return e;
        assign(s, kk, ev);
        ev.kind = 1;
        ++misses_;
      }
      ++claims_[kk];
      tick_[s] = now_++;
      pinned_[s] = 1;
      held_.push_back(s);
      ev.slot = s;
      record(ev);
      slots_out[r] = s;
    }
    return 0;
  }

  // Speculative loads of layer's experts[0..n): each one not resident is
  // loaded into the slot a miss would take (fresh tick, no hold); a resident
  // one is left untouched.  Stops at the first bet for which every slot is
  // held.  *loaded = loads issued.  Returns 0 or fill's code.
  template <class Fill>
  int prefetch(int layer, const int32_t* experts, int n, Fill&& fill, int* loaded) {
    *loaded = 0;
    for (int i = 0; i < n; ++i) {
      const long long kk = (long long)layer * n_experts_ + experts[i];
      if (where_[kk] >= 0) continue;  // resident: a bet that costs nothing
      const int s = victim();
      if (s < 0) break;               // never displaces the current acquisition
      if (const int e = fill(experts[i], s)) return e;
      smoe_ring_event ev = event(layer, i, experts[i]);
      assign(s, kk, ev);
      ev.kind = 2;
      ev.slot = s;
      tick_[s] = now_++;
      ++prefetches_;
      ++*loaded;
      record(ev);
    }
    return 0;
  }

  // The n most claimed (layer, expert) pairs: most claims first, ties to the
  // lower layer, then the lower expert.  Returns the number written.
  int hottest(int n, int32_t* layers, int32_t* experts, uint64_t* counts) {
    order_.clear();
    for (size_t i = 0; i < claims_.size(); ++i)
      if (claims_[i]) order_.push_back((int)i);
    const size_t m = order_.size() < (size_t)n ? order_.size() : (size_t)n;
    std::partial_sort(order_.begin(), order_.begin() + m, order_.end(), [this](int a, int b) {
      return claims_[a] != claims_[b] ? claims_[a] > claims_[b] : a < b;
    });
    for (size_t i = 0; i < m; ++i) {
      layers[i] = order_[i] / n_experts_;
      experts[i] = order_[i] % n_experts_;
      if (counts) counts[i] = claims_[order_[i]];
    }
    return (int)m;
  }

  unsigned long long hits() const { return hits_; }
  unsigned long long misses() const { return misses_; }
  unsigned long long evictions() const { return evictions_; }
  unsigned long long prefetches() const { return prefetches_; }
  const std::vector<smoe_ring_event>& log() const { return log_; }

 private:
  smoe_ring_event event(int layer, int rank, int expert) const {
    smoe_ring_event ev;
    ev.layer = layer;
    ev.rank = rank;
    ev.expert = expert;
    ev.kind = 0;
    ev.slot = -1;
    ev.evicted_layer = -1;
    ev.evicted_expert = -1;
    ev.pad = 0;
    return ev;
  }

  // Slot s now holds key kk; its previous key, if any, is evicted (recorded in ev).
  void assign(int s, long long kk, smoe_ring_event& ev) {
    if (s == n_filled_) {
      ++n_filled_;
    } else {
      const long long old = key_[s];
      where_[old] = -1;
      ev.evicted_layer = (int)(old / n_experts_);
      ev.evicted_expert = (int)(old % n_experts_);
      ++evictions_;
    }
    key_[s] = kk;
    where_[kk] = s;
  }

  void record(const smoe_ring_event& ev) {
    if (log_.size() < log_capacity_) log_.push_back(ev);
  }

  int n_slots_ = 0, n_layers_ = 0, n_experts_ = 0;
  int n_filled_ = 0;  // the empty slots are exactly [n_filled_, n_slots_)
  unsigned long long now_ = 0;
  unsigned long long hits_ = 0, misses_ = 0, evictions_ = 0, prefetches_ = 0;
  size_t log_capacity_ = 0;
  std::vector<long long> key_;               // per slot: layer * E + expert, or -1 when empty
  std::vector<unsigned long long> tick_;     // per slot: last request
  std::vector<unsigned char> pinned_;        // per slot: held by the current acquisition
  std::vector<int> where_;                   // (layer * E + expert) -> slot, or -1
  std::vector<unsigned long long> claims_;   // (layer * E + expert) -> demand requests
  std::vector<int> held_;                    // slots of the current acquisition
  std::vector<int> order_;                   // scratch of hottest()
  std::vector<smoe_ring_event> log_;
};

}  // namespace smoe
