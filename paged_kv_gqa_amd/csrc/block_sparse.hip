// Block-sparse decode: the sparse attention of the HALOps review (a precomputed block
// mask; masked-out KV tiles are skipped; per-tile FP8 scaling is kept) mapped onto the
// dense decode path.
//
// For every (request b, kv head g) this kernel compacts the attended logical pages -
// mask bit set, or the page holds one of the step's query tokens - into a block-table
// row of its own, storing phys * Hkv + g. Read as [num_pages * Hkv, 1, P, D], the
// cache [num_pages, Hkv, P, D] is the same memory, and entry phys * Hkv + g of that
// view is page phys of kv head g (the fp8 scales [num_pages, Hkv] likewise). Each
// (b, g) thus becomes a request of a one-kv-head problem whose length is the number
// of attended tokens. Only the last logical page can be partial and it is always
// attended, so the compacted row is an ordinary paged sequence: the query tokens stay
// its last tokens and the causal rule of the draft rows carries over unchanged.
#include "kernels.hpp"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kPagesPerThread = 16;  // consecutive pages per thread per pass

// One workgroup per (b, g). Each pass covers kThreads * kPagesPerThread pages: a
// thread loads the mask bytes and block-table entries of its pages (all in flight at
// once), counts the attended ones, and a workgroup exclusive scan of the counts gives
// its first output slot, so the output keeps the logical page order.
__global__ __launch_bounds__(kThreads) void block_sparse_compact_kernel(const BlockSparseParams p) {
  __shared__ int wave_tot[kThreads / 64];
  const int v = blockIdx.x;  // b * Hkv + g
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int b = v / p.num_kv_heads, g = v - b * p.num_kv_heads;
  const int L = p.seq_lens[b];
  if (L < 1 || L < p.q_len) {  // invalid length: passed on for the planner to report
    if (tid == 0) p.seq_lens_out[v] = L;
    return;
  }
  const int P = p.page_size;
  const int n = min((L + P - 1) / P, p.bt_stride);
  const int first_query_page = (L - p.q_len) / P;
  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.bt_stride;
  const uint8_t* mask = p.block_mask + static_cast<int64_t>(v) * p.mask_stride;
  int32_t* out = p.bt_out + static_cast<int64_t>(v) * p.bt_stride;
  int kept = 0;  // attended pages before this pass (uniform)
  for (int pass0 = 0; pass0 < n; pass0 += kThreads * kPagesPerThread) {
    const int p0 = pass0 + tid * kPagesPerThread;
    unsigned bits = 0;
    int32_t phys[kPagesPerThread];
#pragma unroll
    for (int s = 0; s < kPagesPerThread; ++s) {
      const int pg = p0 + s;
      phys[s] = 0;
      if (pg < n && (pg >= first_query_page || mask[pg] != 0)) {
        bits |= 1u << s;
        phys[s] = bt[pg];
      }
    }
    // Workgroup exclusive scan of the per-thread counts.
    const int cnt = __popc(bits);
    int inc = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o);
      if (lane >= o) inc += y;
    }
    if (lane == 63) wave_tot[wid] = inc;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
      const int t = wave_tot[w];
      before += (w < wid) ? t : 0;
      total += t;
    }
    __syncthreads();
    int pos = kept + before + inc - cnt;
#pragma unroll
    for (int s = 0; s < kPagesPerThread; ++s)
      if (bits & (1u << s)) out[pos++] = phys[s] * p.num_kv_heads + g;
    kept += total;
  }
  if (tid == 0) p.seq_lens_out[v] = L - (n - kept) * P;
}

}  // namespace

hipError_t launch_block_sparse_compact(const BlockSparseParams& p, hipStream_t stream) {
  const int rows = p.batch * p.num_kv_heads;
  hipLaunchKernelGGL(block_sparse_compact_kernel, dim3(rows), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
