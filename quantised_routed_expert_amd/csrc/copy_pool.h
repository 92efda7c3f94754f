// A fixed pool of host threads that copy one buffer in parallel parts, for
// the ring's fills from pageable vault memory (the HIP runtime's own staging
// of pageable copies reaches about half of the link's page-locked rate).
// Host code only.
//
// No mutex and no condition variable ("Zero Allocations, Zero Locks in the
// Token Loop", Optimizations page): a copy is handed out by publishing its
// arguments and bumping a 32-bit generation counter, and completion is a
// 32-bit countdown; idle threads sleep in std::atomic<>::wait (a futex on
// Linux), so they take no CPU time between copies.  The threads are started
// once, at construction.  copy() is called by one thread at a time.
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <thread>
#include <vector>

namespace smoe {

class CopyPool {
 public:
  explicit CopyPool(int n_threads) {
    th_.reserve((size_t)n_threads);
    for (int i = 0; i < n_threads; ++i) th_.emplace_back([this, i] { run(i + 1); });
  }

  ~CopyPool() {
    stop_.store(true, std::memory_order_relaxed);
    gen_.fetch_add(1, std::memory_order_release);
    gen_.notify_all();
    for (std::thread& t : th_) t.join();
  }

  CopyPool(const CopyPool&) = delete;
  CopyPool& operator=(const CopyPool&) = delete;

  // Copies `bytes` from src to dst with every pool thread and the caller;
  // returns when all parts are done.
  void copy(char* dst, const char* src, size_t bytes) {
    dst_ = dst;
    src_ = src;
    bytes_ = bytes;
    parts_ = (int)th_.size() + 1;
    pending_.store((int)th_.size(), std::memory_order_relaxed);
    gen_.fetch_add(1, std::memory_order_release);  // publishes the arguments above
    gen_.notify_all();
    part(0);
    for (int p = pending_.load(std::memory_order_acquire); p != 0; p = pending_.load(std::memory_order_acquire))
      pending_.wait(p, std::memory_order_acquire);
  }

 private:
  void part(int i) const {
    const size_t per = ((bytes_ + parts_ - 1) / parts_ + 63) & ~(size_t)63;
    const size_t lo = (size_t)i * per;
    if (lo < bytes_) memcpy(dst_ + lo, src_ + lo, bytes_ - lo < per ? bytes_ - lo : per);
  }

  void run(int i) {
    uint32_t seen = 0;
    for (;;) {
      uint32_t g;
      while ((g = gen_.load(std::memory_order_acquire)) == seen) gen_.wait(seen, std::memory_order_acquire);
      seen = g;
      if (stop_.load(std::memory_order_relaxed)) return;
      part(i);
      if (pending_.fetch_sub(1, std::memory_order_acq_rel) == 1) pending_.notify_one();
    }
  }

  std::vector<std::thread> th_;
  std::atomic<uint32_t> gen_{0};
  std::atomic<int> pending_{0};
  std::atomic<bool> stop_{false};
  // the current copy: written by copy() before the generation bump, read by
  // the threads after they observe it
  char* dst_ = nullptr;
  const char* src_ = nullptr;
  size_t bytes_ = 0;
  int parts_ = 1;
};

}  // namespace smoe
