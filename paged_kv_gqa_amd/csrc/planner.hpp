// Host tile planner: uniform KV tiles, longest-first greedy bin-packing onto W
// workers (HPC-Ops review, "How the kernels are organized around specific workload
// shapes"). Plain C++17 with no HIP dependency so it builds and runs on any host.
#pragma once

#include <cstdint>
#include <vector>

namespace pkv {

struct PlanStats {
  int64_t num_items = 0;
  int64_t makespan = 0;    // largest per-worker token load
  int64_t max_items = 0;   // most items on one worker
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tile-size quantum: the page size for bf16, lcm(page size, 64) for fp8.
int64_t tile_quantum(int page_size, bool fp8);

// Number of candidate tiles of the automatic rule: quantum * 2^k <= 65536, k >= 0
// (at least the quantum itself).
int auto_tile_candidates(int64_t quantum);

// Loads and item counts of the plan for tile size T without materialising it.
PlanStats plan_stats(int batch, const int32_t* seq_lens, int num_kv_heads, int64_t T,
                     int W);

// The automatic tile size (see pkv_plan_query).
int64_t auto_tile_tokens(int batch, const int32_t* seq_lens, int q_len, int num_q_heads,
                         int num_kv_heads, int head_dim, int page_size, bool fp8, int W);

// Materialise the plan into caller arrays (items [N][4], offsets [W+1], rtb [B+1]).
void build_plan(int batch, const int32_t* seq_lens, int num_kv_heads, int64_t T, int W,
                int32_t* items, int32_t* worker_offsets, int32_t* req_tile_base);

}  // namespace pkv
