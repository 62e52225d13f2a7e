// Drives the library's host-side resize planner (csrc/resize_plan.h) for
// tests/test_resize_plan.py: reads cases from stdin, writes each plan to
// stdout.  Built with the address and undefined-behaviour sanitizers.
//
// Input, per case: C C2, then C lines "key stamp".  Output, per case:
// "plan", C2 lines "key stamp order", "moves n" and n lines "src dst",
// "evicted n" and the n keys on one line.
#include <cstdio>
#include <vector>

#include "../expert_offload_serving_amd/csrc/resize_plan.h"

int main() {
  int C, C2;
  while (std::scanf("%d %d", &C, &C2) == 2) {
    std::vector<int32_t> key(C);
    std::vector<uint64_t> stamp(C);
    for (int s = 0; s < C; s++) {
      long long k;
      unsigned long long st;
      if (std::scanf("%lld %llu", &k, &st) != 2) return 2;
      key[s] = (int32_t)k;
      stamp[s] = st;
    }
    const moe::ResizePlan p = moe::plan_resize(key, stamp, C2, 12);
    std::printf("plan\n");
    for (int s = 0; s < C2; s++)
      std::printf("%d %llu %d\n", p.key[s], (unsigned long long)p.stamp[s], p.order[s]);
    std::printf("moves %zu\n", p.moves.size());
    for (const auto& m : p.moves) std::printf("%d %d\n", m.first, m.second);
    std::printf("evicted %zu\n", p.evicted.size());
    for (int k : p.evicted) std::printf("%d ", k);
    std::printf("\n");
  }
  return 0;
}
