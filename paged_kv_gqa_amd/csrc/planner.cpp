// Host tile planner (see planner.hpp).
//
// Longest-first greedy placement of uniform KV tiles, in an exact fast form: every
// full tile costs T, more than any partial tile, so the full tiles are placed
// first; with all loads starting equal, the k-th full tile in (b, g, i) order lands
// on worker k mod W (each is the lowest-indexed least-loaded worker at its turn).
// Only the at most B*Hkv partial tiles (one per request and kv head) go through a
// (load, worker) tournament tree, longest first, ties by (b, g).
#include "planner.hpp"

#include <algorithm>
#include <cstdint>
#include <numeric>

namespace pkv {

namespace {

constexpr int64_t kMaxAutoTile = 65536;
// Automatic tile size, a bandwidth-sharing cost model (measured on MI355X): while k
// workers are busy each streams at min(chip / k, chip / kWorkerRatio), so the plan's
// streaming time in chip-token units is sum_j (l_j - l_(j-1)) * max(W - j + 1,
// kWorkerRatio) over the loads sorted ascending; each work item adds a fixed cost
// of ~kItemBytes of chip-wide streaming (~2.6 us at ~6.5 TB/s). The two constants
// are kept as a pair that picks the fastest measured power-of-two tile on every
// benchmark workload (one eight-wave workgroup alone streams at about chip / 240).
constexpr int64_t kWorkerRatio = 160;
constexpr int64_t kItemBytes = int64_t{1} << 24;

// Tournament tree over the workers' loads. A key packs (load, worker) into one
// 64-bit word, load in the high bits, so the smaller key is the less-loaded worker
// and, on equal loads, the lower index. Leaves hold the workers' keys, every inner
// node the smaller key of its children; raising the least-loaded worker's load
// re-plays its fixed-depth path to the root with one min per level.
class WorkerTree {
 public:
  static constexpr int kWorkerBits = 24;  // up to 16M workers; loads below 2^40 tokens
  void reset(const std::vector<int64_t>& loads) {
    const int W = static_cast<int>(loads.size());
    size_ = 1;
    while (size_ < W) size_ *= 2;
    node_.assign(2 * size_, UINT64_MAX);  // padding leaves never win
    for (int w = 0; w < W; ++w)
      node_[size_ + w] = (static_cast<uint64_t>(loads[w]) << kWorkerBits) | static_cast<uint64_t>(w);
    for (int i = size_ - 1; i >= 1; --i) node_[i] = std::min(node_[2 * i], node_[2 * i + 1]);
    root_ = node_[1];
  }
  // Add `cost` to the least-loaded worker (lowest index on ties); returns it. The
  // new minimum is carried up in a register (the siblings' keys are the only
  // loads), and the root stays cached for the next call.
  int32_t place(int64_t cost) {
    const int32_t w = static_cast<int32_t>(root_ & ((uint64_t{1} << kWorkerBits) - 1));
    int i = size_ + w;
    uint64_t v = root_ + (static_cast<uint64_t>(cost) << kWorkerBits);
    node_[i] = v;
    while (i > 1) {
      v = std::min(v, node_[i ^ 1]);
      i >>= 1;
      node_[i] = v;
    }
    root_ = v;
    return w;
  }

 private:
  int size_ = 1;
  uint64_t root_ = UINT64_MAX;
  std::vector<uint64_t> node_;
};

struct Scratch {
  std::vector<int64_t> loads, counts, full, sorted;
  std::vector<int32_t> reqs, nfull, rem;  // per request: full tiles, last-tile tokens
  std::vector<int32_t> tmp;               // radix-sort buffer
  std::vector<uint32_t> keys, tmp_keys;
  WorkerTree heap;
};

// Per-request tile counts for tile size T; returns the number of full tiles of one
// kv head. Divisions happen once per request here and nowhere in the loops below.
int64_t split_requests(int batch, const int32_t* seq_lens, int64_t T, Scratch& s) {
  s.nfull.resize(batch);
  s.rem.resize(batch);
  int64_t f = 0;
  for (int b = 0; b < batch; ++b) {
    const int32_t q = static_cast<int32_t>(seq_lens[b] / T);
    s.nfull[b] = q;
    s.rem[b] = seq_lens[b] - static_cast<int32_t>(q * T);
    f += q;
  }
  return f;
}

// The requests with a partial tile, longest partial tile first, ties by request
// index: a least-significant-digit radix sort (stable) of INT32_MAX - rem over the
// requests in index order, skipping the 8-bit digits on which all keys agree.
void partial_requests(int batch, Scratch& s) {
  s.reqs.clear();
  s.keys.clear();
  uint32_t all_or = 0, all_and = UINT32_MAX;
  for (int b = 0; b < batch; ++b)
    if (s.rem[b] != 0) {
      const uint32_t key = static_cast<uint32_t>(INT32_MAX - s.rem[b]);
      s.reqs.push_back(b);
      s.keys.push_back(key);
      all_or |= key;
      all_and &= key;
    }
  const size_t n = s.reqs.size();
  s.tmp.resize(n);
  s.tmp_keys.resize(n);
  for (int shift = 0; shift < 32; shift += 8) {
    if ((((all_or ^ all_and) >> shift) & 0xFF) == 0) continue;  // digit constant
    size_t count[257] = {0};
    for (size_t i = 0; i < n; ++i) ++count[((s.keys[i] >> shift) & 0xFF) + 1];
    for (int d = 0; d < 256; ++d) count[d + 1] += count[d];
    for (size_t i = 0; i < n; ++i) {
      const size_t pos = count[(s.keys[i] >> shift) & 0xFF]++;
      s.tmp[pos] = s.reqs[i];
      s.tmp_keys[pos] = s.keys[i];
    }
    s.reqs.swap(s.tmp);
    s.keys.swap(s.tmp_keys);
  }
}

// Streaming time of the per-worker loads in chip-token units (see kWorkerRatio):
// sum_j (l_j - l_(j-1)) * max(W - j + 1, R) over the loads sorted ascending. The
// weights exceed the busy-worker count only for the R - 1 largest loads, so this is
// the total plus sum (l_j - l_(j-1)) * (R - (W - j + 1)) over those positions; only
// the top R loads need sorting.
__int128 fluid_cost(std::vector<int64_t>& v, const std::vector<int64_t>& loads) {
  const int64_t W = static_cast<int64_t>(loads.size());
  const int64_t R = kWorkerRatio;
  int64_t total = 0, top = 0;
  for (int64_t x : loads) {
    total += x;
    top = std::max(top, x);
  }
  if (W <= R) return static_cast<__int128>(R) * top;  // every weight is R
  v.assign(loads.begin(), loads.end());
  std::nth_element(v.begin(), v.begin() + (W - R), v.end());
  std::sort(v.begin() + (W - R), v.end());
  __int128 extra = 0;
  for (int64_t i = W - R + 1; i < W; ++i)  // 0-based i has W - i busy workers
    extra += static_cast<__int128>(v[i] - v[i - 1]) * (R - (W - i));
  return total + extra;
}

// Full-tile phase: loads and counts after round-robin placement.
void full_phase(int64_t F, int64_t T, int W, Scratch& s) {
  s.full.assign(W, 0);
  s.loads.resize(W);
  s.counts.resize(W);
  for (int w = 0; w < W; ++w) {
    s.full[w] = F / W + (w < F % W ? 1 : 0);
    s.counts[w] = s.full[w];
    s.loads[w] = s.full[w] * T;
  }
}

}  // namespace

int64_t tile_quantum(int page_size, bool fp8) {
  if (!fp8) return page_size;
  return static_cast<int64_t>(page_size) * 64 / std::gcd(page_size, 64);
}

int auto_tile_candidates(int64_t quantum) {
  int n = 1;
  for (int64_t T = quantum; T * 2 <= kMaxAutoTile; T *= 2) ++n;
  return n;
}

namespace {

// Expects split_requests(T) to have filled s.nfull / s.rem.
PlanStats plan_stats_impl(int batch, int Hkv, int64_t T, int W, int64_t full_one_head, Scratch& s) {
  const int64_t F = full_one_head * Hkv;
  full_phase(F, T, W, s);
  partial_requests(batch, s);
  s.heap.reset(s.loads);
  for (int32_t b : s.reqs) {
    const int64_t cost = s.rem[b];
    for (int g = 0; g < Hkv; ++g) {
      const int32_t w = s.heap.place(cost);
      s.loads[w] += cost;
      s.counts[w] += 1;
    }
  }
  PlanStats st;
  st.num_items = F + static_cast<int64_t>(s.reqs.size()) * Hkv;
  st.makespan = *std::max_element(s.loads.begin(), s.loads.end());
  st.max_items = *std::max_element(s.counts.begin(), s.counts.end());
  return st;
}

}  // namespace

PlanStats plan_stats(int batch, const int32_t* seq_lens, int Hkv, int64_t T, int W) {
  Scratch s;
  const int64_t f = split_requests(batch, seq_lens, T, s);
  return plan_stats_impl(batch, Hkv, T, W, f, s);
}

int64_t auto_tile_tokens(int batch, const int32_t* seq_lens, int q_len, int num_q_heads,
                         int Hkv, int head_dim, int page_size, bool fp8, int W) {
  const int64_t quantum = tile_quantum(page_size, fp8);
  const int64_t kv = 2 * static_cast<int64_t>(head_dim) * (fp8 ? 1 : 2);  // bytes per token
  const int64_t M = static_cast<int64_t>(num_q_heads / Hkv) * q_len;
  const int64_t partial_bytes = M * (head_dim + 1) * 8;  // written, then read by combine
  int64_t total = 0, max_len = 0;
  for (int b = 0; b < batch; ++b) {
    total += seq_lens[b];
    max_len = std::max<int64_t>(max_len, seq_lens[b]);
  }
  total *= Hkv;
  std::vector<int64_t> cands;
  const int ncand = auto_tile_candidates(quantum);
  for (int k = 0; k < ncand; ++k) cands.push_back(quantum << k);
  // Candidates are quantum * 2^k, so floor(L / T) = floor(L / quantum) >> k.
  Scratch s;
  std::vector<int32_t> lq(batch);
  for (int b = 0; b < batch; ++b) lq[b] = static_cast<int32_t>(seq_lens[b] / quantum);
  s.nfull.resize(batch);
  s.rem.resize(batch);
  // Lower bound of every candidate first (O(B) each): fluid >= total (every phase
  // weighs at least its worker count) and fluid >= kWorkerRatio * makespan (every
  // phase weighs at least kWorkerRatio); the loads and item counts of the exact
  // full-tile phase only grow. Candidates are then simulated in increasing order of
  // their bound, and one whose bound cannot beat (or tie with a larger tile) the best
  // estimate so far is skipped. Ties go to the larger tile, independent of order.
  const int K = static_cast<int>(cands.size());
  std::vector<__int128> lower(K);
  std::vector<int64_t> fulls(K);
  for (int k = 0; k < K; ++k) {
    const int64_t T = cands[k];
    int64_t f = 0, partial = 0;
    for (int b = 0; b < batch; ++b) {
      const int32_t q = lq[b] >> k;
      f += q;
      partial += (seq_lens[b] != static_cast<int32_t>(q * T));
    }
    fulls[k] = f;
    const int64_t n_items = (f + partial) * Hkv;
    const int64_t full_per_worker = ceil_div(f * Hkv, W);
    // The makespan is also at least the largest single item, min(max L, T).
    const int64_t span_lb =
        std::max({ceil_div(total, W), full_per_worker * T, std::min<int64_t>(max_len, T)});
    const int64_t items_lb = std::max(ceil_div(n_items, W), full_per_worker);
    lower[k] = static_cast<__int128>(kv) * std::max(total, kWorkerRatio * span_lb) +
               static_cast<__int128>(items_lb) * kItemBytes +
               static_cast<__int128>(n_items) * partial_bytes;
  }
  std::vector<int> order(K);
  for (int k = 0; k < K; ++k) order[k] = k;
  std::sort(order.begin(), order.end(), [&](int a, int b) {
    return lower[a] < lower[b] || (lower[a] == lower[b] && a > b);
  });
  int64_t best_T = -1;
  __int128 best_est = -1;
  for (int k : order) {
    const int64_t T = cands[k];
    if (best_T >= 0 && (lower[k] > best_est || (lower[k] == best_est && T < best_T))) continue;
    for (int b = 0; b < batch; ++b) {
      const int32_t q = lq[b] >> k;
      s.nfull[b] = q;
      s.rem[b] = seq_lens[b] - static_cast<int32_t>(q * T);
    }
    const PlanStats st = plan_stats_impl(batch, Hkv, T, W, fulls[k], s);
    const __int128 est = static_cast<__int128>(kv) * fluid_cost(s.sorted, s.loads) +
                         static_cast<__int128>(st.max_items) * kItemBytes +
                         static_cast<__int128>(st.num_items) * partial_bytes;
    if (best_T < 0 || est < best_est || (est == best_est && T > best_T)) {
      best_T = T;
      best_est = est;
    }
  }
  return best_T;
}

void build_plan(int batch, const int32_t* seq_lens, int Hkv, int64_t T, int W,
                int32_t* items, int32_t* worker_offsets, int32_t* req_tile_base) {
  req_tile_base[0] = 0;
  for (int b = 0; b < batch; ++b)
    req_tile_base[b + 1] = req_tile_base[b] + static_cast<int32_t>(ceil_div(seq_lens[b], T));

  Scratch s;
  const int64_t F = split_requests(batch, seq_lens, T, s) * Hkv;
  full_phase(F, T, W, s);
  partial_requests(batch, s);
  s.heap.reset(s.loads);
  std::vector<int32_t> where;
  where.reserve(s.reqs.size() * Hkv);
  for (int32_t b : s.reqs) {
    const int64_t cost = s.rem[b];
    for (int g = 0; g < Hkv; ++g) {
      const int32_t w = s.heap.place(cost);
      s.counts[w] += 1;
      where.push_back(w);
    }
  }

  worker_offsets[0] = 0;
  for (int w = 0; w < W; ++w)
    worker_offsets[w + 1] = worker_offsets[w] + static_cast<int32_t>(s.counts[w]);

  auto put = [&](int64_t pos, int32_t b, int32_t g, int32_t i) {
    const int32_t nb = req_tile_base[b + 1] - req_tile_base[b];
    int32_t* it = items + 4 * pos;
    it[0] = b;
    it[1] = g;
    it[2] = i;
    it[3] = Hkv * req_tile_base[b] + g * nb + i;
  };
  // Full tiles: the k-th in (b, g, i) order is worker (k mod W)'s (k / W)-th item;
  // (w, round) track (k mod W, k / W) without dividing.
  int32_t w = 0, round = 0;
  for (int b = 0; b < batch; ++b) {
    const int32_t nf = s.nfull[b];
    for (int g = 0; g < Hkv; ++g)
      for (int32_t i = 0; i < nf; ++i) {
        put(static_cast<int64_t>(worker_offsets[w]) + round, b, g, i);
        if (++w == W) {
          w = 0;
          ++round;
        }
      }
  }
  // Partial tiles follow each worker's full tiles, in placement order.
  std::vector<int64_t>& cursor = s.loads;  // reused as per-worker write positions
  for (int w = 0; w < W; ++w) cursor[w] = worker_offsets[w] + s.full[w];
  size_t p = 0;
  for (int32_t b : s.reqs) {
    const int32_t last = s.nfull[b];
    for (int g = 0; g < Hkv; ++g, ++p) put(cursor[where[p]]++, b, g, last);
  }
}

}  // namespace pkv
