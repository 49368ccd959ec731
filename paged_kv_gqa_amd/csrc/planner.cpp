// Host tile planner (see planner.hpp).
//
// Longest-first greedy placement of uniform KV tiles, in an exact fast form: every
// full tile costs T, more than any partial tile, so the full tiles are placed
// first; with all loads starting equal, the k-th full tile in (b, g, i) order lands
// on worker k mod W (each is the lowest-indexed least-loaded worker at its turn).
// Only the at most B*Hkv partial tiles (one per request and kv head) go through a
// (load, worker) min-heap, longest first, ties by (b, g).
#include "planner.hpp"

#include <algorithm>
#include <functional>
#include <numeric>
#include <queue>
#include <utility>

namespace pkv {

namespace {

constexpr int64_t kMaxAutoTile = 4096;

struct Partial {
  int64_t cost;
  int32_t b, g;
};

// Partial tiles of the plan in placement order.
std::vector<Partial> partial_tiles(int batch, const int32_t* seq_lens, int Hkv, int64_t T) {
  std::vector<Partial> out;
  for (int b = 0; b < batch; ++b) {
    const int64_t rem = seq_lens[b] % T;
    if (rem == 0) continue;
    for (int g = 0; g < Hkv; ++g) out.push_back({rem, b, g});
  }
  std::stable_sort(out.begin(), out.end(),
                   [](const Partial& x, const Partial& y) { return x.cost > y.cost; });
  return out;
}

int64_t full_tile_count(int batch, const int32_t* seq_lens, int Hkv, int64_t T) {
  int64_t f = 0;
  for (int b = 0; b < batch; ++b) f += seq_lens[b] / T;
  return f * Hkv;
}

using Slot = std::pair<int64_t, int32_t>;  // (load, worker)
using MinHeap = std::priority_queue<Slot, std::vector<Slot>, std::greater<Slot>>;

// Place the partial tiles; returns the worker of each, and updates loads / counts.
std::vector<int32_t> place_partials(const std::vector<Partial>& parts, int W,
                                    std::vector<int64_t>& loads,
                                    std::vector<int64_t>& counts) {
  std::vector<Slot> init(W);
  for (int w = 0; w < W; ++w) init[w] = {loads[w], w};
  MinHeap heap(std::greater<Slot>(), std::move(init));
  std::vector<int32_t> where(parts.size());
  for (size_t k = 0; k < parts.size(); ++k) {
    Slot s = heap.top();
    heap.pop();
    where[k] = s.second;
    loads[s.second] = s.first + parts[k].cost;
    counts[s.second] += 1;
    heap.push({loads[s.second], s.second});
  }
  return where;
}

}  // namespace

int64_t tile_quantum(int page_size, bool fp8) {
  if (!fp8) return page_size;
  return static_cast<int64_t>(page_size) * 64 / std::gcd(page_size, 64);
}

PlanStats plan_stats(int batch, const int32_t* seq_lens, int Hkv, int64_t T, int W) {
  const int64_t F = full_tile_count(batch, seq_lens, Hkv, T);
  std::vector<int64_t> counts(W), loads(W);
  for (int w = 0; w < W; ++w) {
    counts[w] = F / W + (w < F % W ? 1 : 0);
    loads[w] = counts[w] * T;
  }
  const std::vector<Partial> parts = partial_tiles(batch, seq_lens, Hkv, T);
  place_partials(parts, W, loads, counts);
  PlanStats st;
  st.num_items = F + static_cast<int64_t>(parts.size());
  st.makespan = *std::max_element(loads.begin(), loads.end());
  st.max_items = *std::max_element(counts.begin(), counts.end());
  return st;
}

int64_t auto_tile_tokens(int batch, const int32_t* seq_lens, int q_len, int num_q_heads,
                         int Hkv, int head_dim, int page_size, bool fp8, int W) {
  const int64_t quantum = tile_quantum(page_size, fp8);
  const int64_t eb = fp8 ? 1 : 2;
  const int64_t M = static_cast<int64_t>(num_q_heads / Hkv) * q_len;
  int64_t best_T = quantum, best_est = -1;
  for (int64_t T = quantum;; T *= 2) {
    const PlanStats st = plan_stats(batch, seq_lens, Hkv, T, W);
    const int64_t est = st.makespan * 2 * head_dim * eb +
                        (st.max_items + ceil_div(st.num_items, W)) * M * (head_dim + 1) * 4;
    if (best_est < 0 || est <= best_est) {  // ascending T: ties go to the larger tile
      best_T = T;
      best_est = est;
    }
    if (T * 2 > kMaxAutoTile) break;
  }
  return best_T;
}

void build_plan(int batch, const int32_t* seq_lens, int Hkv, int64_t T, int W,
                int32_t* items, int32_t* worker_offsets, int32_t* req_tile_base) {
  req_tile_base[0] = 0;
  for (int b = 0; b < batch; ++b)
    req_tile_base[b + 1] = req_tile_base[b] + static_cast<int32_t>(ceil_div(seq_lens[b], T));

  const int64_t F = full_tile_count(batch, seq_lens, Hkv, T);
  std::vector<int64_t> full(W), counts(W), loads(W);
  for (int w = 0; w < W; ++w) {
    full[w] = F / W + (w < F % W ? 1 : 0);
    counts[w] = full[w];
    loads[w] = full[w] * T;
  }
  const std::vector<Partial> parts = partial_tiles(batch, seq_lens, Hkv, T);
  const std::vector<int32_t> where = place_partials(parts, W, loads, counts);

  worker_offsets[0] = 0;
  for (int w = 0; w < W; ++w)
    worker_offsets[w + 1] = worker_offsets[w] + static_cast<int32_t>(counts[w]);

  auto put = [&](int64_t pos, int32_t b, int32_t g, int32_t i) {
    const int32_t nb = req_tile_base[b + 1] - req_tile_base[b];
    int32_t* it = items + 4 * pos;
    it[0] = b;
    it[1] = g;
    it[2] = i;
    it[3] = Hkv * req_tile_base[b] + g * nb + i;
  };
  // Full tiles: the k-th in (b, g, i) order is worker (k mod W)'s (k / W)-th item.
  int64_t k = 0;
  for (int b = 0; b < batch; ++b) {
    const int32_t nf = static_cast<int32_t>(seq_lens[b] / T);
    for (int g = 0; g < Hkv; ++g)
      for (int32_t i = 0; i < nf; ++i, ++k) put(worker_offsets[k % W] + k / W, b, g, i);
  }
  // Partial tiles follow each worker's full tiles, in placement order.
  std::vector<int64_t> cursor(W);
  for (int w = 0; w < W; ++w) cursor[w] = worker_offsets[w] + full[w];
  for (size_t p = 0; p < parts.size(); ++p) {
    const int32_t b = parts[p].b;
    put(cursor[where[p]]++, b, parts[p].g, static_cast<int32_t>(seq_lens[b] / T));
  }
}

}  // namespace pkv
