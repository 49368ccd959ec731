// Fused KV append: the step's new k/v rows written into the paged cache, with the
// optional rotary embedding of the new q and k rows and, for an FP8 cache, per-page
// quantisation on write (the fused pre-processing of the HALOps README's decode
// attention; per-tile FP8 scaling as in the HALOps review).
//
// One workgroup per (request b, kv head g). Request b's Tq new tokens sit at
// positions L_b - Tq .. L_b - 1 and touch at most two pages (Tq <= 4 <= P).
// Rotation (half-split form, caller cos/sin tables): for i < D/2,
//   x[i] = x1*c - x2*s, x[i + D/2] = x2*c + x1*s,
// each product, sum and difference one IEEE float32 rounding (no fused multiply-add).
// FP8 pages (one scale per page and kv head, K and V apart), with a = the largest
// |value| of the page's new rows:
//   - new rows start at the page's first slot: scale = a / 448 (1 if a == 0);
//   - else the page keeps its scale s while a / s <= 448; otherwise the scale becomes
//     a / 448 and the page's earlier codes are re-encoded from their values code * s;
//   - codes round to the nearest e4m3fn value (ties to the even code), saturate at
//     +-448 and keep the sign.
#include "kernels.hpp"

// Every product, sum, difference and quotient below is its own IEEE float32 rounding:
// no multiply-add contraction in this file (the quantised codes depend on it), and
// float division is correctly rounded.
#pragma clang fp contract(off)

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxNew = 4;  // new rows per page and request (Tq <= 4)

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Exact value of an e4m3fn code (finite codes; 0x7F / 0xFF give NaN).
__device__ __forceinline__ float e4m3fn_value(uint32_t code) {
  const uint32_t sign = (code & 0x80u) << 24;
  const uint32_t e = (code >> 3) & 0xFu, m = code & 7u;
  if (e == 15u && m == 7u) return __uint_as_float(sign | 0x7FC00000u);
  if (e == 0u) {  // subnormal (and zero): m * 2^-9, exact
    const float v = static_cast<float>(m) * 0x1p-9f;
    return sign ? -v : v;
  }
  return __uint_as_float(sign | ((e + 120u) << 23) | (m << 20));
}

// e4m3fn code of a float32: nearest value, ties to the even code, saturating at 448,
// sign kept (a negative value that rounds to zero gives 0x80).
__device__ __forceinline__ uint32_t e4m3fn_code(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float ax = fabsf(x);
  if (ax != ax) return sign | 0x7Fu;
  if (ax >= 448.f) return sign | 0x7Eu;
  if (ax < 0x1p-6f) {  // subnormal range: multiples of 2^-9, rounding to 8 gives 2^-6
    const float q = __builtin_rintf(ax * 512.f);  // exact scaling; rint rounds half to even
    return sign | static_cast<uint32_t>(q);
  }
  const uint32_t au = __float_as_uint(ax);
  uint32_t e = ((au >> 23) & 0xFFu) - 127u + 7u;  // e4m3fn biased exponent, 1 .. 15
  uint32_t m = (au >> 20) & 7u;
  const uint32_t rest = au & 0xFFFFFu, half = 0x80000u;
  if (rest > half || (rest == half && (m & 1u))) {
    if (++m == 8u) {
      m = 0;
      ++e;
    }
  }
  const uint32_t code = (e << 3) | m;
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

__device__ __forceinline__ float block_max(float v, float* red) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float m = red[0];
  for (int w = 1; w < kThreads / 64; ++w) m = fmaxf(m, red[w]);
  __syncthreads();
  return m;
}

__global__ __launch_bounds__(kThreads) void kv_append_kernel(const KvAppendParams p) {
  __shared__ float rows[kMaxNew][kMaxHeadDim];
  __shared__ float red[kThreads / 64];
  __shared__ float page_scale;
  __shared__ int reencode;
  const int tid = threadIdx.x;
  const int b = blockIdx.x / p.num_kv_heads, g = blockIdx.x - b * p.num_kv_heads;
  const int Tq = p.q_len, D = p.head_dim, H = D / 2, P = p.page_size;
  const int L = p.seq_lens[b];
  if (L < Tq || L < 1 || L > p.bt_stride * P) return;  // outside the caller's contract
  const int first = L - Tq;
  const bool rope = p.rope_cos != nullptr;

  // Rotation of the new q rows of this kv head's query heads.
  if (rope && p.q_out != nullptr) {
    const int G = p.num_q_heads / p.num_kv_heads;
    for (int e = tid; e < Tq * G * H; e += kThreads) {
      const int t = e / (G * H), j = (e / H) % G, i = e % H;
      const int pos = first + t;
      const int64_t row = ((static_cast<int64_t>(b) * Tq + t) * p.num_q_heads + g * G + j) * D;
      const float x1 = bf16_to_f32(p.q[row + i]), x2 = bf16_to_f32(p.q[row + i + H]);
      const float c = p.rope_cos[static_cast<int64_t>(pos) * H + i];
      const float s = p.rope_sin[static_cast<int64_t>(pos) * H + i];
      const float r1 = x1 * c - x2 * s;
      const float r2 = x2 * c + x1 * s;
      p.q_out[row + i] = f32_to_bf16_rne(r1);
      p.q_out[row + i + H] = f32_to_bf16_rne(r2);
    }
  }

  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.bt_stride;
  const int64_t row_elems = D;
  for (int lp = first / P; lp <= (L - 1) / P; ++lp) {
    const int phys = bt[lp];
    const int o0 = max(first, lp * P) - lp * P;
    const int o1 = min(L, (lp + 1) * P) - lp * P;
    const int n = o1 - o0;                     // new rows in this page, 1 .. Tq
    const int t0 = lp * P + o0 - first;        // their first new-token index
    const int64_t slot = (static_cast<int64_t>(phys) * p.num_kv_heads + g) * P;  // row of offset 0
    for (int kind = 0; kind < 2; ++kind) {     // 0: K (rotated), 1: V
      const uint16_t* src = kind == 0 ? p.k_new : p.v_new;
      uint8_t* cache = kind == 0 ? p.k_cache : p.v_cache;
      const bool rot = rope && kind == 0;
      // The page's new rows as float32 (rotated for K).
      for (int e = tid; e < n * H; e += kThreads) {
        const int r = e / H, i = e - r * H;
        const int t = t0 + r;
        const int64_t in = ((static_cast<int64_t>(b) * Tq + t) * p.num_kv_heads + g) * D;
        float x1 = bf16_to_f32(src[in + i]), x2 = bf16_to_f32(src[in + i + H]);
        if (rot) {
          const int pos = first + t;
          const float c = p.rope_cos[static_cast<int64_t>(pos) * H + i];
          const float s = p.rope_sin[static_cast<int64_t>(pos) * H + i];
          const float r1 = x1 * c - x2 * s;
          const float r2 = x2 * c + x1 * s;
          x1 = r1;
          x2 = r2;
        }
        rows[r][i] = x1;
        rows[r][i + H] = x2;
      }
      __syncthreads();
      if (!p.fp8) {
        uint16_t* dst = reinterpret_cast<uint16_t*>(cache) + (slot + o0) * row_elems;
        for (int e = tid; e < n * D; e += kThreads) dst[e] = f32_to_bf16_rne(rows[e / D][e % D]);
        __syncthreads();
        continue;
      }
      float* scales = kind == 0 ? p.k_scale : p.v_scale;
      const int64_t sidx = static_cast<int64_t>(phys) * p.num_kv_heads + g;
      float a = 0.f;
      for (int e = tid; e < n * D; e += kThreads) a = fmaxf(a, fabsf(rows[e / D][e % D]));
      a = block_max(a, red);
      if (tid == 0) {
        float s = 1.f;
        int again = 0;
        if (o0 == 0) {
          s = a > 0.f ? a / 448.f : 1.f;
        } else {
          s = scales[sidx];
          if (!(a / s <= 448.f)) {
            s = a / 448.f;
            again = 1;
          }
        }
        page_scale = s;
        reencode = again;
      }
      __syncthreads();
      const float s = page_scale;
      uint8_t* page = cache + slot * row_elems;
      if (reencode) {  // earlier rows o < o0: their values under the new scale
        const float s_old = scales[sidx];
        for (int e = tid; e < o0 * D; e += kThreads) {
          const float v = e4m3fn_value(page[e]) * s_old;
          page[e] = static_cast<uint8_t>(e4m3fn_code(v / s));
        }
      }
      for (int e = tid; e < n * D; e += kThreads)
        page[o0 * row_elems + e] = static_cast<uint8_t>(e4m3fn_code(rows[e / D][e % D] / s));
      __syncthreads();  // every thread has read the old scale
      if (tid == 0) scales[sidx] = s;
    }
  }
}

}  // namespace

hipError_t launch_kv_append(const KvAppendParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(kv_append_kernel, dim3(p.batch * p.num_kv_heads), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
