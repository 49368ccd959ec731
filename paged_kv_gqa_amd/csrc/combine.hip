// Log-sum-exp merge of split-KV partials (the combine kernel of the HPC-Ops review,
// "How the kernels are organized around specific workload shapes").
//
// One wave per output row (b, t, h); each lane owns D/64 head dimensions. The
// n_b partials of the row are read in index order with a running maximum, so the
// result is deterministic. A request with a single tile still passes through here
// (the partial is already normalised; the merge only casts it to bf16).
#include "kernels.hpp"

#include <math.h>

namespace pkv {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.44269504088896341f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kRowsPerBlock = 4;

template <int D>
__global__ __launch_bounds__(64 * kRowsPerBlock) void combine_kernel(const CombineParams p) {
  constexpr int E = D / 64;
  const int total = p.batch * p.q_len * p.num_q_heads;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= total) return;
  const int lane = threadIdx.x & 63;
  const int h = row % p.num_q_heads;
  const int t = (row / p.num_q_heads) % p.q_len;
  const int b = row / (p.num_q_heads * p.q_len);
  const int g = h / p.group;
  const int r = t * p.group + (h - g * p.group);
  const int base = p.req_tile_base[b];
  const int nb = p.req_tile_base[b + 1] - base;
  const int64_t slot0 = static_cast<int64_t>(p.num_kv_heads) * base + static_cast<int64_t>(g) * nb;

  float mrun = -INFINITY, den = 0.f;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int i = 0; i < nb; ++i) {
    const int64_t rr = (slot0 + i) * p.rows + r;
    const float li = p.ws_lse[rr] * kLog2e;
    float o[E];
    if constexpr (E == 2) {
      const f32x2 v = *reinterpret_cast<const f32x2*>(p.ws_o + rr * D + 2 * lane);
      o[0] = v[0];
      o[1] = v[1];
    } else {
      o[0] = p.ws_o[rr * D + lane];
    }
    if (li == -INFINITY) continue;
    if (li > mrun) {
      const float sc = __builtin_amdgcn_exp2f(mrun - li);  // 0 when mrun = -inf
      den *= sc;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] *= sc;
      mrun = li;
    }
    const float w = __builtin_amdgcn_exp2f(li - mrun);
    den += w;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += w * o[e];
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  uint16_t* orow = p.out + static_cast<int64_t>(row) * D;
  if constexpr (E == 2) {
    f32x2 v = {acc[0] * inv, acc[1] * inv};
    *reinterpret_cast<bf16x2*>(orow + 2 * lane) = __builtin_convertvector(v, bf16x2);
  } else {
    orow[lane] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[0] * inv));
  }
  if (p.lse_out != nullptr && lane == 0)
    p.lse_out[row] = den > 0.f ? (mrun + __builtin_amdgcn_logf(den)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, int head_dim, hipStream_t stream) {
  const int total = p.batch * p.q_len * p.num_q_heads;
  const dim3 grid((total + kRowsPerBlock - 1) / kRowsPerBlock), block(64 * kRowsPerBlock);
  if (head_dim == 128)
    hipLaunchKernelGGL(combine_kernel<128>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(combine_kernel<64>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
