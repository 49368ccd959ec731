// Log-sum-exp merge of split-KV partials (the combine kernel of the HPC-Ops review,
// "How the kernels are organized around specific workload shapes").
//
// One wave per output row (b, t, h). The row's n_b split weights are computed in
// parallel, one split per lane: lane i reads lse_i, the wave takes the maximum and
// each lane forms w_i = exp(lse_i - max). The partial outputs are then accumulated
// in split order with the weights broadcast from their lanes; their loads do not
// depend on each other, so several are in flight at once (rows of at most 16 splits
// load them together with the lse values). Fixed summation order keeps the result
// deterministic. A request with a single tile is copied (its partial
// is already normalised: the output is cast to bf16, the lse passed through).
#include "kernels.hpp"

#include <math.h>

namespace pkv {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.44269504088896341f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kRowsPerBlock = 4;
constexpr int kUnroll = 8;
constexpr int kDirect = 16;  // rows of at most this many splits load all partials at once

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

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
  const float* lse = p.ws_lse + slot0 * p.rows + r;           // stride rows per split
  const float* o = p.ws_o + (slot0 * p.rows + r) * D + E * lane;  // stride rows * D per split
  const int64_t ostride = static_cast<int64_t>(p.rows) * D;

  // out is [B / split, Tq, split * Hq, D] (and lse_out likewise without D); with
  // split 1 the row index is the output row.
  int64_t orow_idx = row;
  if (p.request_split != 1) {
    const int qb = b / p.request_split, part = b - qb * p.request_split;
    orow_idx = ((static_cast<int64_t>(qb) * p.q_len + t) * p.request_split + part) * p.num_q_heads + h;
  }
  uint16_t* orow = p.out + orow_idx * D;
  if (nb == 1) {  // a single split is already normalised: cast it, pass its lse through
    if constexpr (E == 2) {
      const f32x2 v = *reinterpret_cast<const f32x2*>(o);
      *reinterpret_cast<bf16x2*>(orow + 2 * lane) = __builtin_convertvector(v, bf16x2);
    } else {
      orow[lane] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(o[0]));
    }
    if (p.lse_out != nullptr && lane == 0) p.lse_out[orow_idx] = lse[0];
    return;
  }

  if (nb <= kDirect) {  // the outputs load with the lse values
    float ov[kDirect][E];
#pragma unroll
    for (int u = 0; u < kDirect; ++u) {
      if (u < nb) {
        const float* src = o + u * ostride;
        if constexpr (E == 2) {
          const f32x2 v = *reinterpret_cast<const f32x2*>(src);
          ov[u][0] = v[0];
          ov[u][1] = v[1];
        } else {
          ov[u][0] = *src;
        }
      }
    }
    const float l = (lane < nb) ? lse[static_cast<int64_t>(lane) * p.rows] : -INFINITY;
    const float mx = wave_max(l) * kLog2e;
    const float m_use = (mx == -INFINITY) ? 0.f : mx;
    const float wl = (lane < nb) ? __builtin_amdgcn_exp2f(l * kLog2e - m_use) : 0.f;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll
    for (int u = 0; u < kDirect; ++u) {
      if (u < nb) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), u));
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += w * ov[u][e];
      }
    }
    const float den = wave_sum(wl);
    const float inv = den > 0.f ? 1.f / den : 0.f;
    if constexpr (E == 2) {
      f32x2 v = {acc[0] * inv, acc[1] * inv};
      *reinterpret_cast<bf16x2*>(orow + 2 * lane) = __builtin_convertvector(v, bf16x2);
    } else {
      orow[lane] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[0] * inv));
    }
    if (p.lse_out != nullptr && lane == 0)
      p.lse_out[orow_idx] = den > 0.f ? (m_use + __builtin_amdgcn_logf(den)) * kLn2 : -INFINITY;
    return;
  }

  float mloc = -INFINITY;
  for (int i = lane; i < nb; i += 64) mloc = fmaxf(mloc, lse[static_cast<int64_t>(i) * p.rows]);
  const float mx = wave_max(mloc) * kLog2e;  // -inf only if every split saw no key
  const float m_use = (mx == -INFINITY) ? 0.f : mx;

  float den = 0.f;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int i0 = 0; i0 < nb; i0 += 64) {
    const int i = i0 + lane;
    const float wl = (i < nb) ? __builtin_amdgcn_exp2f(lse[static_cast<int64_t>(i) * p.rows] * kLog2e - m_use) : 0.f;
    den += wl;
    const int cnt = min(64, nb - i0);
    int j = 0;
    for (; j + kUnroll <= cnt; j += kUnroll) {
      float ov[kUnroll][E];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const float* src = o + (i0 + j + u) * ostride;
        if constexpr (E == 2) {
          const f32x2 v = *reinterpret_cast<const f32x2*>(src);
          ov[u][0] = v[0];
          ov[u][1] = v[1];
        } else {
          ov[u][0] = *src;
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j + u));
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += w * ov[u][e];
      }
    }
    for (; j < cnt; ++j) {
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j));
      const float* src = o + (i0 + j) * ostride;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += w * src[e];
    }
  }
  den = wave_sum(den);
  const float inv = den > 0.f ? 1.f / den : 0.f;
  if constexpr (E == 2) {
    f32x2 v = {acc[0] * inv, acc[1] * inv};
    *reinterpret_cast<bf16x2*>(orow + 2 * lane) = __builtin_convertvector(v, bf16x2);
  } else {
    orow[lane] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[0] * inv));
  }
  if (p.lse_out != nullptr && lane == 0)
    p.lse_out[orow_idx] = den > 0.f ? (m_use + __builtin_amdgcn_logf(den)) * kLn2 : -INFINITY;
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
