// Device-side tile planner: the uniform tiles and longest-first greedy bin-packing
// of the host planner (HPC-Ops review, "How the kernels are organized around
// specific workload shapes": tiles are assigned to the thread blocks before every
// decode step), computed on the GPU from device-resident seq_lens, so a decode step
// can be enqueued - or captured in a graph and replayed - with no host work.
//
// The output is bit-identical to the host plan. One workgroup builds a plan:
//   1. per request: n_b, its full tiles, the remainder tile's cost, prefix sums;
//   2. full tiles (cost T, listed first by the longest-first order) go round-robin:
//      the k-th one in (b, g, i) order to worker k mod W;
//   3. the remainder tiles (cost < T), sorted by (cost desc, b, g), are placed in
//      batches. With the worker keys (load, index) sorted ascending, l_0 <= l_1 <=
//      ..., and the next items costing c_k >= c_(k+1) >= ..., items k .. k+p-1 go to
//      the p least-loaded workers in that order whenever l_(p-1) < l_0 + c_(k+p-1):
//      each worker loaded in the batch ends above l_0 + c_(k+p-1) > l_j for every
//      later j of the batch, so one-at-a-time least-loaded placement picks exactly
//      these workers in this order. The batch taken is the exact one: it runs while
//      the key (l_j, j's worker) is below every key already raised in the batch
//      (which the condition above implies); after a batch the keys are sorted again.
//   4. write the items grouped by worker: full items first, then the worker's
//      remainder items in placement order.
// Worker keys live in registers, one per thread, sorted by a bitonic network whose
// short strides exchange within a wave. Keys are 32-bit: a worker's load is kept
// relative to the current least load, and during step 3 every load lies within T
// of it (each remainder tile costs less than T and goes to the least-loaded
// worker, and the full-tile loads differ by at most T), so (relative load, worker)
// fits in 32 bits for T < 2^18; the reference load is carried beside the keys.
// Automatic tile size: one workgroup per candidate tile builds that candidate's plan
// into scratch with its estimate (all candidates at once); a copy kernel then moves
// the plan with the lowest estimate (ties: the larger tile) into the outputs. The
// streaming term of the estimate uses the equivalent form
//   fluid = sum of the W - 160 smallest loads + 160 * largest load   (W > 160)
// of sum_j (l_j - l_(j-1)) * max(W - j + 1, 160) (summation by parts; 160 * largest
// load when W <= 160).
#include "kernels.hpp"

namespace pkv {
namespace {

// Threads of a planner workgroup: one per worker (and per request for the register
// sort of the request keys), so 256 or 512 when W and B allow it, else 1024 (fewer
// waves meet at each of the plan's barriers).
constexpr int kPT = 1024;
constexpr int kPTSmall = 512;
constexpr int kPTTiny = 256;
constexpr int kWorkerBits = 10;           // worker index in the low bits of a key
constexpr int kReqBits = 13;              // request index in the low bits of a key
constexpr long long kMaxTokenHeads = 1LL << 36;
constexpr long long kItemBytes = 1LL << 24;
constexpr int kWorkerRatio = 160;

typedef unsigned u32;

static_assert(kMaxDevicePlanWorkers <= kPT && kMaxDevicePlanWorkers <= (1 << kWorkerBits),
              "one thread and one key field per worker");
static_assert(kPTSmall % 64 == 0 && kPTSmall <= kPT && kPTTiny % 64 == 0 && kPTTiny <= kPTSmall,
              "planner workgroup sizes");
static_assert(kMaxDevicePlanBatch <= (1 << kReqBits), "request index field");
// Remainder-tile key (T - c) << kReqBits | b and worker key (relative load < 2T) <<
// kWorkerBits | w stay below 2^31, so ~0u is a sentinel above every key.
static_assert(kMaxDevicePlanTile <= (1 << 18) && 18 + kReqBits <= 31 && 19 + kWorkerBits <= 31,
              "32-bit keys");

template <int NT>
struct PlanLds {
  u32 rkey[kMaxDevicePlanBatch];        // remainder-tile keys ((T - c) << 13 | b), sorted
  int32_t fbx[kMaxDevicePlanBatch];     // exclusive prefix of full items (x Hkv)
  int32_t rtb[kMaxDevicePlanBatch];     // exclusive prefix of n_b
  int32_t len[kMaxDevicePlanBatch];     // seq_lens, read from global memory once
  u32 xbuf[2][NT];                      // exchange buffers of the register sort
  int32_t wcnt[kMaxDevicePlanWorkers];  // remainder items per worker
  int32_t woff[kMaxDevicePlanWorkers];  // first item of each worker
  long long red[5][NT / 64];
  u32 wmin[NT / 64];
  u32 kmin;                             // least worker key after a sort
  int first_miss;                       // first item that breaks the batch
};

// Where one plan goes: the outputs, or a candidate's region of the scratch.
struct PlanOut {
  int32_t* items;
  int32_t* worker_offsets;
  int32_t* req_tile_base;
  int32_t* info;
  int2* assign;  // (worker, position in its remainder list) of each remainder item
};

__device__ __forceinline__ u32 umin(u32 a, u32 b) { return a < b ? a : b; }
__device__ __forceinline__ u32 umax(u32 a, u32 b) { return a < b ? b : a; }

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// 32-bit value of lane (lane ^ j) for j in {1, 2, 4, 8, 16, 32}: quad permutes and
// row shifts (DPP) below 16, the gfx950 row-swap instructions at 16 and 32. Each
// swap returns the caller's value in one half of its result and the partner's in
// the other.
__device__ __forceinline__ unsigned lane_xor(unsigned v, int j, int lane) {
  switch (j) {
    case 1:
      return __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
    case 2:
      return __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
    case 4: {
      const unsigned up = __builtin_amdgcn_update_dpp(v, v, 0x104, 0xF, 0xF, false);  // lane + 4
      const unsigned dn = __builtin_amdgcn_update_dpp(v, v, 0x114, 0xF, 0xF, false);  // lane - 4
      return (lane & 4) ? dn : up;
    }
    case 8: {
      const unsigned up = __builtin_amdgcn_update_dpp(v, v, 0x108, 0xF, 0xF, false);
      const unsigned dn = __builtin_amdgcn_update_dpp(v, v, 0x118, 0xF, 0xF, false);
      return (lane & 8) ? dn : up;
    }
    case 16: {
      const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      return (lane & 16) ? r[0] : r[1];
    }
    default: {
      const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      return (lane & 32) ? r[0] : r[1];
    }
  }
}

// Ascending bitonic sort of one key per thread: thread t ends with the t-th smallest
// key of threads 0 .. N-1 (threads >= N hold ~0 and keep it). The network is
// unrolled, so every stage's stride is a constant: strides below 64 exchange within
// a wave (waves past N sit out), wider ones go through LDS, alternating two buffers
// so one barrier per stage suffices. Callers separate two calls by a workgroup
// barrier.
template <int N, int NT>
__device__ __forceinline__ u32 sort_keys_n(u32 x, PlanLds<NT>& sm) {
  const int tid = threadIdx.x, lane = tid & 63;
  const bool active = N >= NT || __builtin_amdgcn_readfirstlane(tid) < N;  // wave-uniform
  int buf = 0;
#pragma unroll
  for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      u32 y = x;
      if (j < 64) {
        if (active) y = lane_xor(x, j, lane);
      } else {
        if (tid < N) sm.xbuf[buf][tid] = x;
        __syncthreads();
        if (tid < N) y = sm.xbuf[buf][tid ^ j];
        buf ^= 1;
      }
      x = (((tid & k) == 0) == ((tid & j) == 0)) ? umin(x, y) : umax(x, y);
    }
  }
  return x;
}

// sort_keys_n for a power of two n <= NT known at run time (the request keys, once per
// plan; kept out of line, one copy of the ten networks).
template <int NT>
__device__ __attribute__((noinline)) u32 sort_keys(u32 x, int n, PlanLds<NT>& sm) {
  switch (n) {
    case 1: return x;
    case 2: return sort_keys_n<2>(x, sm);
    case 4: return sort_keys_n<4>(x, sm);
    case 8: return sort_keys_n<8>(x, sm);
    case 16: return sort_keys_n<16>(x, sm);
    case 32: return sort_keys_n<32>(x, sm);
    case 64: return sort_keys_n<64>(x, sm);
    case 128: return sort_keys_n<128>(x, sm);
    case 256: return sort_keys_n<256>(x, sm);
    case 512: return sort_keys_n<512>(x, sm);
    default: return sort_keys_n<NT>(x, sm);
  }
}

// Ascending bitonic sort of s[0, n) in LDS (n a power of two) for request counts
// above one key per thread. For strides j <= 64 the pairs of 64 consecutive
// pair indices stay in one aligned block of 128 elements owned by one wave, so those
// stages need only wave-level ordering.
template <int NT>
__device__ void lds_sort(u32* s, int n) {
  const int tid = threadIdx.x;
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int x = tid; x < (n >> 1); x += NT) {
        const int i = 2 * j * (x / j) + (x & (j - 1));
        const u32 a = s[i], b = s[i + j];
        if ((a > b) == ((i & k) == 0)) {
          s[i] = b;
          s[i + j] = a;
        }
      }
      const int jn = (j > 1) ? (j >> 1) : k;  // stride of the next stage
      if (j >= 128 || jn >= 128)
        __syncthreads();
      else
        wave_sync();
    }
  }
  __syncthreads();
}

// Exclusive prefix sums (in thread order) of a[0] and a[1] into pre; the workgroup
// totals of all five values into tot. Waves from `nact` threads on hold zeros.
template <int NT>
__device__ void block_scan5(const long long (&a)[5], long long (&pre)[2], long long (&tot)[5],
                            int nact, PlanLds<NT>& sm) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  long long inc[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) inc[i] = a[i];
  if (wid * 64 < nact) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const long long y = __shfl_up(inc[i], o);
        if (lane >= o) inc[i] += y;
      }
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int i = 0; i < 5; ++i) sm.red[i][wid] = inc[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    long long base = 0, t = 0;
    for (int w = 0; w < NT / 64; ++w) {
      const long long v = sm.red[i][w];
      base += (w < wid) ? v : 0;
      t += v;
    }
    tot[i] = t;
    if (i < 2) pre[i] = base + inc[i] - a[i];
  }
  __syncthreads();
}

// Workgroup maximum of v >= 0; waves from `nact` threads on hold zeros.
template <int NT>
__device__ long long block_max(long long v, int nact, PlanLds<NT>& sm) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (wid * 64 < nact) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
  }
  if (lane == 0) sm.red[0][wid] = v;
  __syncthreads();
  long long m = sm.red[0][0];
  for (int w = 1; w < NT / 64; ++w) m = max(m, sm.red[0][w]);
  __syncthreads();
  return m;
}

// Exclusive prefix minimum of v over threads 0 .. n-1 (thread order; ~0 for thread
// 0 and for threads >= n). Within a wave, a butterfly over the lane-exchange pattern of
// the sort (no LDS): at level j each lane takes its partner block's minimum, which
// counts towards the lane's prefix when the partner block lies below it (lane & j).
template <int NT>
__device__ u32 block_exclusive_min(u32 v, int n, PlanLds<NT>& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  u32 total = tid < n ? v : ~0u, excl = ~0u;
#pragma unroll
  for (int j = 1; j < 64; j <<= 1) {
    const u32 other = lane_xor(total, j, lane);
    if (lane & j) excl = umin(excl, other);
    total = umin(total, other);
  }
  if (lane == 0) sm.wmin[wid] = total;  // the wave's minimum, in every lane
  __syncthreads();
  u32 pre = excl;
  for (int w = 0; w < wid; ++w) pre = umin(pre, sm.wmin[w]);
  return tid < n ? pre : ~0u;
}

__device__ __forceinline__ int pow2_at_least(int x) {
  int n = 1;
  while (n < x) n <<= 1;
  return n;
}

template <int NT>
__device__ void write_empty_plan(const DevicePlanParams& p, const PlanOut& o, int status,
                                 long long T) {
  const int tid = threadIdx.x;
  for (int w = tid; w <= p.num_workers; w += NT) o.worker_offsets[w] = 0;
  for (int b = tid; b <= p.batch; b += NT) o.req_tile_base[b] = 0;
  if (tid == 0) {
    o.info[0] = status;
    o.info[1] = static_cast<int>(T);
    o.info[2] = 0;
    o.info[3] = 0;
  }
}

// Steps 1-4 for tile size T into `o`. Returns the status (uniform) and, when it is
// PKV_DEV_OK, the automatic rule's estimate in *est.
template <int NT>
__device__ int build_plan(const DevicePlanParams& p, long long T, PlanLds<NT>& sm, const PlanOut& o,
                          long long* est) {
  const int tid = threadIdx.x;
  const int B = p.batch, Hkv = p.num_kv_heads, W = p.num_workers;
  const int minL = max(1, p.q_len);
  const unsigned uT = static_cast<unsigned>(T);

  // 1. Per-request counts over a contiguous segment per thread.
  const int per = (B + NT - 1) / NT;
  const int b0 = min(B, tid * per), b1 = min(B, b0 + per);
  long long a[5] = {0, 0, 0, 0, 0};  // tiles, full tiles, tokens, bad lengths, remainders
  for (int b = b0; b < b1; ++b) {
    const int L = p.seq_lens[b];
    sm.len[b] = L;  // read back by this thread below, by all after the barriers
    if (L < minL) {
      a[3] = 1;
      continue;
    }
    const unsigned f = static_cast<unsigned>(L) / uT;
    const unsigned c = static_cast<unsigned>(L) - f * uT;
    a[0] += f + (c != 0);
    a[1] += f;
    a[2] += L;
    a[4] += (c != 0);
  }
  long long pre[2], tot[5];
  block_scan5(a, pre, tot, (B + per - 1) / max(per, 1), sm);
  const long long N = tot[0] * Hkv, F = tot[1] * Hkv, K = tot[4] * Hkv;
  int status = PKV_DEV_OK;
  if (tot[3] != 0)
    status = PKV_DEV_ERR_SEQ;
  else if (tot[2] * Hkv >= kMaxTokenHeads)
    status = PKV_DEV_ERR_UNSUPPORTED;
  else if (N > p.max_items)
    status = PKV_DEV_ERR_WORKSPACE;
  if (status != PKV_DEV_OK) {
    write_empty_plan<NT>(p, o, status, T);
    return status;
  }

  const int nB = pow2_at_least(max(B, 1));
  {
    int pn = static_cast<int>(pre[0]), pf = static_cast<int>(pre[1]);
    for (int b = b0; b < b1; ++b) {
      const unsigned L = static_cast<unsigned>(sm.len[b]);
      const unsigned f = L / uT;
      const unsigned c = L - f * uT;
      sm.rtb[b] = pn;
      sm.fbx[b] = pf * Hkv;
      o.req_tile_base[b] = pn;
      sm.rkey[b] = (c != 0) ? (((uT - c) << kReqBits) | static_cast<u32>(b)) : ~0u;
      pn += static_cast<int>(f + (c != 0));
      pf += static_cast<int>(f);
    }
    for (int b = B + tid; b < nB; b += NT) sm.rkey[b] = ~0u;
    if (tid == 0) o.req_tile_base[B] = static_cast<int>(tot[0]);
  }
  __syncthreads();
  if (nB <= NT) {
    const u32 key = sort_keys(tid < nB ? sm.rkey[tid] : ~0u, nB, sm);
    __syncthreads();
    if (tid < nB) sm.rkey[tid] = key;
  } else {
    lds_sort<NT>(sm.rkey, nB);
  }

  // 2. Loads after the round-robin of the full tiles, already in sorted order:
  // workers r .. W-1 carry base full tiles, workers 0 .. r-1 one more. Keys hold the
  // load relative to ref = base * T.
  const long long base = F / W;
  const int r = static_cast<int>(F - base * W);
  long long ref = base * T;
  u32 key = ~0u;
  if (tid < W) {
    const int w = (tid < W - r) ? r + tid : tid - (W - r);
    key = ((w < r ? uT : 0u) << kWorkerBits) | static_cast<u32>(w);
    sm.wcnt[w] = 0;
  }
  __syncthreads();

  // 3. Remainder tiles in batches of provably identical greedy placements: with the
  // keys sorted, item k + j goes to worker j while key_j is below every key already
  // raised in this batch (the keys hold the worker index, so this is the
  // least-loaded, lowest-index choice of a one-at-a-time placement).
  for (long long k = 0; k < K;) {
    const int lim = static_cast<int>(min(static_cast<long long>(W), K - k));
    u32 raised = ~0u;
    if (tid < lim) {
      const int x = static_cast<int>(k) + tid;
      const u32 c = uT - (sm.rkey[x / Hkv] >> kReqBits);  // tokens of the remainder tile
      raised = key + (c << kWorkerBits);
    }
    if (tid == 0) sm.first_miss = lim;
    const u32 below = block_exclusive_min(raised, lim, sm);
    // The first item that breaks the batch: each wave's first failing lane, found by a
    // ballot, so at most one LDS atomic per wave.
    const unsigned long long fails = __builtin_amdgcn_ballot_w64(tid < lim && key > below);
    if (fails != 0 && (tid & 63) == 0) atomicMin(&sm.first_miss, (tid & ~63) + __builtin_ctzll(fails));
    __syncthreads();
    const int np = sm.first_miss;
    if (tid < np) {
      const int w = static_cast<int>(key & ((1u << kWorkerBits) - 1));
      o.assign[k + tid] = make_int2(w, sm.wcnt[w]);
      sm.wcnt[w] += 1;
      key = raised;
    }
    // All NT keys are sorted (threads from W on hold the ~0u sentinel, above every
    // key), so the network is fixed at compile time and inlined.
    key = sort_keys_n<NT, NT>(key, sm);
    if (tid == 0) sm.kmin = key;
    __syncthreads();
    // Re-base the relative loads on the new least load (every key is at least kmin).
    const u32 d = sm.kmin >> kWorkerBits;
    if (tid < W) key -= d << kWorkerBits;
    ref += d;
    k += np;
  }

  // Estimate: fluid over the sorted loads (summation-by-parts form), most items on a
  // worker, partial bytes.
  // Thread t holds the t-th smallest load here, and worker t's item count (cnt, whose
  // exclusive prefix is worker t's first item in the list).
  long long term = 0, cnt = 0;
  if (tid < W) {
    const long long l = ref + static_cast<long long>(key >> kWorkerBits);
    term = (tid <= W - 1 - kWorkerRatio ? l : 0) + (tid == W - 1 ? kWorkerRatio * l : 0);
    cnt = base + (tid < r ? 1 : 0) + sm.wcnt[tid];
  }
  long long wpre[2], wtot[5];
  {
    const long long a[5] = {cnt, 0, term, 0, 0};
    block_scan5(a, wpre, wtot, W, sm);
  }
  const long long off = wpre[0], total = wtot[0], fluid = wtot[2];
  const long long max_items = block_max(cnt, W, sm);
  *est = p.kv_bytes_per_token * fluid + max_items * kItemBytes +
         N * p.rows * (p.head_dim + 1) * 8;

  // 4. Worker offsets, then the items.
  if (tid < W) {
    sm.woff[tid] = static_cast<int>(off);
    o.worker_offsets[tid] = static_cast<int>(off);
  }
  if (tid == 0) o.worker_offsets[W] = static_cast<int>(total);
  __syncthreads();

  int4* items = reinterpret_cast<int4*>(o.items);
  // Full items: the x-th in (b, g, i) order goes to worker x mod W at position x / W.
  // One (request, kv head) pair per thread and step: its f items are x0 .. x0 + f - 1
  // with x0 = fbx[b] + g f, so the worker and position advance without a division.
  if (F > 0) {
    for (int pq = tid; pq < B * Hkv; pq += NT) {
      const int b = pq / Hkv, g = pq - b * Hkv;
      const unsigned L = static_cast<unsigned>(sm.len[b]);
      const int f = static_cast<int>(L / uT);
      if (f == 0) continue;
      const int n = f + (L - static_cast<unsigned>(f) * uT != 0 ? 1 : 0);
      const int x0 = sm.fbx[b] + g * f;
      int pos = x0 / W;
      int w = x0 - pos * W;
      const int slot0 = Hkv * sm.rtb[b] + g * n;
#pragma unroll 4
      for (int i = 0; i < f; ++i) {
        items[sm.woff[w] + pos] = make_int4(b, g, i, slot0 + i);
        if (++w == W) {
          w = 0;
          ++pos;
        }
      }
    }
  }
  // Remainder items, in placement order after the worker's full items. The
  // placements were written by this workgroup before the barriers above.
  const int nK = static_cast<int>(K);
  for (int x = tid; x < nK; x += NT) {
    const int qv = x / Hkv;
    const int g = x - qv * Hkv;
    const int b = static_cast<int>(sm.rkey[qv] & ((1u << kReqBits) - 1));
    const int i = static_cast<int>(static_cast<unsigned>(sm.len[b]) / uT);
    const int2 asg = o.assign[x];
    const int fw = static_cast<int>(base) + (asg.x < r ? 1 : 0);
    items[sm.woff[asg.x] + fw + asg.y] = make_int4(b, g, i, Hkv * sm.rtb[b] + g * (i + 1) + i);
  }
  if (tid == 0) {
    o.info[0] = PKV_DEV_OK;
    o.info[1] = static_cast<int>(T);
    o.info[2] = static_cast<int>(N);
    o.info[3] = static_cast<int>(max_items);
  }
  return PKV_DEV_OK;
}

__device__ PlanOut candidate_out(const DevicePlanParams& p, int c) {
  char* base = p.cand_plans + static_cast<long long>(c) * p.cand_stride;
  PlanOut o;
  o.items = reinterpret_cast<int32_t*>(base);
  o.worker_offsets = reinterpret_cast<int32_t*>(base + p.cand_offsets_off);
  o.req_tile_base = reinterpret_cast<int32_t*>(base + p.cand_rtb_off);
  o.info = reinterpret_cast<int32_t*>(base + p.cand_info_off);
  o.assign = p.scratch_assign + static_cast<long long>(c) * p.batch * p.num_kv_heads;
  return o;
}

// Automatic tile: workgroup c builds the plan of tile quantum << c into scratch.
template <int NT>
__global__ __launch_bounds__(NT) void plan_candidates_kernel(const DevicePlanParams p) {
  __shared__ PlanLds<NT> sm;
  const int c = blockIdx.x;
  long long est = 0;
  const int st = build_plan(p, static_cast<long long>(p.quantum) << c, sm, candidate_out(p, c), &est);
  if (threadIdx.x == 0) {
    p.cand_est[c] = est;
    p.cand_status[c] = st;
  }
}

// Automatic tile: every workgroup finds the best candidate (lowest estimate, ties to
// the larger tile) and copies its share of that candidate's plan to the outputs.
__global__ __launch_bounds__(kPT) void plan_select_kernel(const DevicePlanParams p) {
  int best = -1;
  long long best_est = 0;
  for (int c = 0; c < p.num_candidates; ++c) {
    if (p.cand_status[c] != PKV_DEV_OK) continue;
    const long long e = p.cand_est[c];
    if (best < 0 || e <= best_est) {
      best = c;
      best_est = e;
    }
  }
  const int tid = threadIdx.x;
  if (best < 0) {  // nothing fits: report the largest candidate's status
    if (blockIdx.x == 0) {
      const int last = p.num_candidates - 1;
      const PlanOut o = {p.items, p.worker_offsets, p.req_tile_base, p.info, nullptr};
      write_empty_plan<kPT>(p, o, p.cand_status[last], static_cast<long long>(p.quantum) << last);
    }
    return;
  }
  const PlanOut src = candidate_out(p, best);
  const int N = src.info[2];
  const int4* from = reinterpret_cast<const int4*>(src.items);
  int4* to = reinterpret_cast<int4*>(p.items);
  for (int x = blockIdx.x * kPT + tid; x < N; x += gridDim.x * kPT) to[x] = from[x];
  if (blockIdx.x == 0) {
    for (int w = tid; w <= p.num_workers; w += kPT) p.worker_offsets[w] = src.worker_offsets[w];
    for (int b = tid; b <= p.batch; b += kPT) p.req_tile_base[b] = src.req_tile_base[b];
    if (tid < 4) p.info[tid] = src.info[tid];
  }
}

// Fixed tile: one workgroup builds the plan straight into the outputs.
template <int NT>
__global__ __launch_bounds__(NT) void plan_fixed_kernel(const DevicePlanParams p) {
  __shared__ PlanLds<NT> sm;
  const PlanOut o = {p.items, p.worker_offsets, p.req_tile_base, p.info, p.scratch_assign};
  long long est;
  build_plan(p, p.tile_tokens, sm, o, &est);
}

}  // namespace

hipError_t launch_plan_device(const DevicePlanParams& p, hipStream_t stream) {
  const bool tiny = p.num_workers <= kPTTiny && p.batch <= kPTTiny;
  const bool small = p.num_workers <= kPTSmall && p.batch <= kPTSmall;
  if (p.tile_tokens == 0) {
    if (tiny)
      hipLaunchKernelGGL(plan_candidates_kernel<kPTTiny>, dim3(p.num_candidates), dim3(kPTTiny), 0,
                         stream, p);
    else if (small)
      hipLaunchKernelGGL(plan_candidates_kernel<kPTSmall>, dim3(p.num_candidates), dim3(kPTSmall), 0,
                         stream, p);
    else
      hipLaunchKernelGGL(plan_candidates_kernel<kPT>, dim3(p.num_candidates), dim3(kPT), 0, stream, p);
    const long long blocks = (p.max_items + kPT - 1) / kPT;
    const int grid = static_cast<int>(blocks < 1 ? 1 : (blocks > 256 ? 256 : blocks));
    hipLaunchKernelGGL(plan_select_kernel, dim3(grid), dim3(kPT), 0, stream, p);
  } else {
    if (tiny)
      hipLaunchKernelGGL(plan_fixed_kernel<kPTTiny>, dim3(1), dim3(kPTTiny), 0, stream, p);
    else if (small)
      hipLaunchKernelGGL(plan_fixed_kernel<kPTSmall>, dim3(1), dim3(kPTSmall), 0, stream, p);
    else
      hipLaunchKernelGGL(plan_fixed_kernel<kPT>, dim3(1), dim3(kPT), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pkv
