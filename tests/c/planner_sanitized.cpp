// The host planner (paged_kv_gqa_amd/csrc/planner.cpp, plain C++17) driven under
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_planner_sanitized.py:
// random and extreme batches (up to 4096 requests, 2048 workers, 2M-token requests),
// the automatic tile and the plan, with the work list's invariants checked.
#include <algorithm>
#include <cstdio>
#include <random>
#include <vector>

#include "planner.hpp"

int main() {
  std::mt19937_64 rng(1);
  long plans = 0;
  for (int it = 0; it < 3000; ++it) {
    const int B = 1 + static_cast<int>(rng() % (it % 10 == 0 ? 4096 : 64));
    const int Hkv = 1 + static_cast<int>(rng() % 8);
    const int W = 1 + static_cast<int>(rng() % (it % 7 == 0 ? 2048 : 600));
    const bool fp8 = rng() % 2;
    const int P = fp8 ? 64 : 16 * (1 + static_cast<int>(rng() % 4));
    const int q_len = 1 + static_cast<int>(rng() % 4);
    const int max_len = (it % 13 == 0) ? 2000000 : 1 + static_cast<int>(rng() % 70000);
    std::vector<int32_t> sl(B);
    for (auto& x : sl) x = q_len + static_cast<int32_t>(rng() % max_len);
    const int64_t T = pkv::auto_tile_tokens(B, sl.data(), q_len, 8 * Hkv, Hkv, 128, P, fp8, W);
    if (T < 1 || T % pkv::tile_quantum(P, fp8) != 0) {
      std::printf("bad tile %lld\n", static_cast<long long>(T));
      return 1;
    }
    const pkv::PlanStats st = pkv::plan_stats(B, sl.data(), Hkv, T, W);
    std::vector<int32_t> items(4 * st.num_items + 4), offs(W + 1), rtb(B + 1);
    pkv::build_plan(B, sl.data(), Hkv, T, W, items.data(), offs.data(), rtb.data());
    if (offs[0] != 0 || offs[W] != st.num_items) {
      std::printf("bad worker offsets\n");
      return 1;
    }
    // every token of every (request, kv head) exactly once; slots a permutation
    int64_t tokens = 0, want = 0;
    std::vector<char> seen(st.num_items, 0);
    for (int64_t k = 0; k < st.num_items; ++k) {
      const int b = items[4 * k], i = items[4 * k + 2], slot = items[4 * k + 3];
      tokens += std::min<int64_t>(sl[b], (i + 1) * T) - i * T;
      if (slot < 0 || slot >= st.num_items || seen[slot]++) {
        std::printf("bad slot %d\n", slot);
        return 1;
      }
    }
    for (int b = 0; b < B; ++b) want += static_cast<int64_t>(sl[b]) * Hkv;
    if (tokens != want) {
      std::printf("tokens %lld != %lld\n", static_cast<long long>(tokens), static_cast<long long>(want));
      return 1;
    }
    ++plans;
  }
  std::printf("ok %ld plans\n", plans);
  return 0;
}
