// Test driver of the expert ring's slot policy (quantised_routed_expert_amd/
// csrc/ring_policy.h), the host code the library's ring runs, without HIP.
// Reads commands from stdin, one per line, and prints what the policy did:
//   setup n_slots n_layers n_experts log_capacity
//   fail N          make the N-th fill from now on fail (returns code 7)
//   acq L k e...    acquire (implicit release first) -> "acq rc slot..."
//   pre L n e...    speculative loads                -> "pre rc loaded"
//   rel             release
//   hot n           -> "hot m L E C L E C ..."
//   stats           -> "stats hits misses evictions prefetches"
//   log             -> one "ev L rank expert kind slot evL evE" line per event
// The fill callback only counts (and fails when told to).
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "ring_policy.h"

int main() {
  smoe::RingPolicy pol;
  long fill_calls = 0, fail_at = -1;
  auto fill = [&](int, int) -> int {
    ++fill_calls;
    return fill_calls == fail_at ? 7 : 0;
  };
  char cmd[32];
  while (scanf("%31s", cmd) == 1) {
    const std::string c(cmd);
    if (c == "setup") {
      int n, L, E;
      size_t cap;
      if (scanf("%d %d %d %zu", &n, &L, &E, &cap) != 4) return 2;
      pol.setup(n, L, E, cap);
    } else if (c == "fail") {
      long n;
      if (scanf("%ld", &n) != 1) return 2;
      fail_at = fill_calls + n;
    } else if (c == "acq" || c == "pre") {
      int L, k;
      if (scanf("%d %d", &L, &k) != 2) return 2;
      std::vector<int32_t> ex((size_t)k);
      for (int i = 0; i < k; ++i)
        if (scanf("%d", &ex[i]) != 1) return 2;
      if (c == "acq") {
        if (const char* msg = pol.check_request(L, ex.data(), k)) {
          printf("acq invalid %s\n", msg);
          continue;
        }
        std::vector<int> slots((size_t)k, -9);
        const int rc = pol.acquire(L, ex.data(), k, fill, slots.data());
        printf("acq %d", rc);
        for (int i = 0; i < k; ++i) printf(" %d", slots[i]);
        printf("\n");
      } else {
        int loaded = 0;
        const int rc = pol.prefetch(L, ex.data(), k, fill, &loaded);
        printf("pre %d %d\n", rc, loaded);
      }
    } else if (c == "rel") {
      pol.release();
    } else if (c == "hot") {
      int n;
      if (scanf("%d", &n) != 1) return 2;
      std::vector<int32_t> l((size_t)n + 1), e((size_t)n + 1);
      std::vector<uint64_t> cnt((size_t)n + 1);
      const int m = pol.hottest(n, l.data(), e.data(), cnt.data());
      printf("hot %d", m);
      for (int i = 0; i < m; ++i) printf(" %d %d %llu", l[i], e[i], (unsigned long long)cnt[i]);
      printf("\n");
    } else if (c == "stats") {
      printf("stats %llu %llu %llu %llu\n", pol.hits(), pol.misses(), pol.evictions(), pol.prefetches());
    } else if (c == "log") {
      for (const smoe_ring_event& ev : pol.log())
        printf("ev %d %d %d %d %d %d %d\n", ev.layer, ev.rank, ev.expert, ev.kind, ev.slot, ev.evicted_layer,
               ev.evicted_expert);
    } else {
      fprintf(stderr, "unknown command %s\n", cmd);
      return 2;
    }
  }
  return 0;
}
