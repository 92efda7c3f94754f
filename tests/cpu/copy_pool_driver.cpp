// Stress test of the ring's host copy pool (quantised_routed_expert_amd/csrc/
// copy_pool.h): many copies of assorted sizes and alignments through pools of
// several thread counts, each checked byte for byte; meant to run under
// ThreadSanitizer (and AddressSanitizer).  Prints "ok" and exits 0 on success.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "copy_pool.h"

int main(int argc, char** argv) {
  const int rounds = argc > 1 ? atoi(argv[1]) : 200;
  unsigned long long x = 0x9E3779B97F4A7C15ull;
  auto rnd = [&]() {
    x ^= x >> 12; x ^= x << 25; x ^= x >> 27;
    return x * 0x2545F4914F6CDD1Dull;
  };
  const size_t cap = 1 << 20;
  std::vector<char> src(cap + 64), dst(cap + 64);
  for (size_t i = 0; i < src.size(); ++i) src[i] = (char)(rnd() >> 56);
  for (int threads : {1, 3, 8}) {
    smoe::CopyPool pool(threads);
    for (int r = 0; r < rounds; ++r) {
      const size_t bytes = r % 7 == 0 ? 0 : (size_t)(rnd() % cap);
      const size_t so = rnd() % 64, d0 = rnd() % 64;
      memset(dst.data(), 0x5A, dst.size());
      pool.copy(dst.data() + d0, src.data() + so, bytes);
      if (memcmp(dst.data() + d0, src.data() + so, bytes) != 0) {
        printf("mismatch: threads %d round %d bytes %zu\n", threads, r, bytes);
        return 1;
      }
      for (size_t i = 0; i < d0; ++i)
        if (dst[i] != 0x5A) { printf("wrote before the destination\n"); return 1; }
      for (size_t i = d0 + bytes; i < dst.size(); ++i)
        if (dst[i] != 0x5A) { printf("wrote past the destination\n"); return 1; }
    }
  }
  printf("ok\n");
  return 0;
}
