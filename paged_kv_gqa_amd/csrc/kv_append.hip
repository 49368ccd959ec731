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

constexpr int kThreads = 256;  // four waves: (page 0, 1) x (K, V)

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

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Four consecutive bf16 values (8 bytes) -> float32.
__device__ __forceinline__ void load4(const uint16_t* src, float (&x)[4]) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(src);
  x[0] = __uint_as_float(w[0] << 16);
  x[1] = __uint_as_float(w[0] & 0xFFFF0000u);
  x[2] = __uint_as_float(w[1] << 16);
  x[3] = __uint_as_float(w[1] & 0xFFFF0000u);
}

__device__ __forceinline__ u32x2 pack4_bf16(const float (&x)[4]) {
  return u32x2{static_cast<uint32_t>(f32_to_bf16_rne(x[0])) | (static_cast<uint32_t>(f32_to_bf16_rne(x[1])) << 16),
               static_cast<uint32_t>(f32_to_bf16_rne(x[2])) | (static_cast<uint32_t>(f32_to_bf16_rne(x[3])) << 16)};
}

// Rotation of one lane's four pairs (x1[j], x2[j]) = (x[i0 + j], x[i0 + j + D/2]) of a
// row at position pos.
// (The tables need only 4-byte alignment: element loads.)
__device__ __forceinline__ void rotate4(float (&x1)[4], float (&x2)[4], const float* cos_row,
                                        const float* sin_row) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float c = cos_row[j], s = sin_row[j];
    const float r1 = x1[j] * c - x2[j] * s;
    const float r2 = x2[j] * c + x1[j] * s;
    x1[j] = r1;
    x2[j] = r2;
  }
}

// One workgroup of four waves per (request b, kv head g). Wave 2p + kind writes the
// new rows of touched page p (0: the page of the first new token, 1: the next one,
// if touched) of K (kind 0, rotated) or V (kind 1); each lane holds four rotation
// pairs (i0 .. i0+3 and the same + D/2 of one row), so the page's largest |value|
// is a wave reduction and no step waits for another wave. The page's old scale is
// loaded first, beside the rows. For FP8, one barrier then lets the whole workgroup
// re-encode page 0's earlier rows if its scale rose. Then every thread rotates the
// new q rows of the kv head's query heads.
__global__ __launch_bounds__(kThreads) void kv_append_kernel(const KvAppendParams p) {
  __shared__ int re_flag[2];          // page 0 of K / V needs its earlier rows re-encoded
  __shared__ float re_scale[2][2];    // (old, new) scale of page 0 of K / V
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x / p.num_kv_heads, g = blockIdx.x - b * p.num_kv_heads;
  const int Tq = p.q_len, D = p.head_dim, H = D / 2, P = p.page_size;
  const int L = p.seq_lens[b];
  if (L < Tq || L < 1 || L > p.bt_stride * P) return;  // outside the caller's contract
  const int first = L - Tq;
  const bool rope = p.rope_cos != nullptr;

  const int lp = first / P + (wid >> 1);
  const int kind = wid & 1;
  if (lp <= (L - 1) / P) {  // this wave's page is touched (wave-uniform)
    const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.bt_stride;
    const int64_t phys = bt[lp];
    const int o0 = max(first, lp * P) - lp * P;
    const int o1 = min(L, (lp + 1) * P) - lp * P;
    const int n = o1 - o0;                     // new rows in this page, 1 .. Tq
    const int t0 = lp * P + o0 - first;        // their first new-token index
    const int64_t sidx = phys * p.num_kv_heads + g;
    float* scales = kind == 0 ? p.k_scale : p.v_scale;
    const float s_old = p.fp8 ? scales[sidx] : 1.f;
    const uint16_t* src = kind == 0 ? p.k_new : p.v_new;
    uint8_t* cache = kind == 0 ? p.k_cache : p.v_cache;
    const int64_t slot = sidx * P;             // row 0 of the page's kv-head run

    const int e0 = 4 * lane;                   // first of this lane's four pairs
    const bool act = e0 < n * H;
    const int r = act ? e0 / H : 0, i0 = act ? e0 - r * H : 0;
    float x1[4] = {0.f, 0.f, 0.f, 0.f}, x2[4] = {0.f, 0.f, 0.f, 0.f};
    if (act) {
      const int t = t0 + r;
      const int64_t in = ((static_cast<int64_t>(b) * Tq + t) * p.num_kv_heads + g) * D;
      load4(src + in + i0, x1);
      load4(src + in + i0 + H, x2);
      if (rope && kind == 0) {
        const int64_t pos = first + t;
        rotate4(x1, x2, p.rope_cos + pos * H + i0, p.rope_sin + pos * H + i0);
      }
    }
    const int64_t row = slot + o0 + r;
    if (!p.fp8) {
      if (act) {
        uint16_t* dst = reinterpret_cast<uint16_t*>(cache) + row * D;
        *reinterpret_cast<u32x2*>(dst + i0) = pack4_bf16(x1);
        *reinterpret_cast<u32x2*>(dst + i0 + H) = pack4_bf16(x2);
      }
    } else {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) a = fmaxf(a, fmaxf(fabsf(x1[j]), fabsf(x2[j])));
      a = wave_max(a);
      float s = 1.f;
      bool again = false;
      if (o0 == 0) {
        s = a > 0.f ? a / 448.f : 1.f;
      } else {
        s = s_old;
        if (!(a / s <= 448.f)) {
          s = a / 448.f;
          again = true;
        }
      }
      if (wid < 2 && lane == 0) {  // page 0: whether its earlier rows need re-encoding
        re_flag[kind] = again ? 1 : 0;
        re_scale[kind][0] = s_old;
        re_scale[kind][1] = s;
      }
      if (act) {
        uint32_t c1 = 0, c2 = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c1 |= e4m3fn_code(x1[j] / s) << (8 * j);
          c2 |= e4m3fn_code(x2[j] / s) << (8 * j);
        }
        *reinterpret_cast<uint32_t*>(cache + row * D + i0) = c1;
        *reinterpret_cast<uint32_t*>(cache + row * D + i0 + H) = c2;
      }
      if (lane == 0) scales[sidx] = s;  // after this wave's reads of the old scale
    }
  }

  // A raised scale of page 0 re-encodes that page's earlier rows (o < o0) from their
  // values under the old scale; the whole workgroup shares the work. Those rows are
  // disjoint from the new ones written above.
  if (p.fp8) {
    __syncthreads();
    const int lp0 = first / P;
    const int o0 = first - lp0 * P;
#pragma unroll
    for (int kind = 0; kind < 2; ++kind) {
      if (re_flag[kind]) {
        const int64_t phys = p.block_table[static_cast<int64_t>(b) * p.bt_stride + lp0];
        uint8_t* page = (kind == 0 ? p.k_cache : p.v_cache) + (phys * p.num_kv_heads + g) * P * D;
        const float s_old = re_scale[kind][0], s = re_scale[kind][1];
        for (int e = 4 * tid; e < o0 * D; e += 4 * kThreads) {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(page + e);
          uint32_t out = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float v = e4m3fn_value((w >> (8 * j)) & 0xFFu) * s_old;
            out |= e4m3fn_code(v / s) << (8 * j);
          }
          *reinterpret_cast<uint32_t*>(page + e) = out;
        }
      }
    }
  }

  // Rotation of the new q rows of this kv head's query heads: four pairs per thread.
  if (rope && p.q_out != nullptr) {
    const int G = p.num_q_heads / p.num_kv_heads;
    for (int e = 4 * tid; e < Tq * G * H; e += 4 * kThreads) {
      const int t = e / (G * H), j = (e / H) % G, i0 = e % H;
      const int64_t pos = first + t;
      const int64_t qrow = ((static_cast<int64_t>(b) * Tq + t) * p.num_q_heads + g * G + j) * D;
      float x1[4], x2[4];
      load4(p.q + qrow + i0, x1);
      load4(p.q + qrow + i0 + H, x2);
      rotate4(x1, x2, p.rope_cos + pos * H + i0, p.rope_sin + pos * H + i0);
      *reinterpret_cast<u32x2*>(p.q_out + qrow + i0) = pack4_bf16(x1);
      *reinterpret_cast<u32x2*>(p.q_out + qrow + i0 + H) = pack4_bf16(x2);
    }
  }
}

}  // namespace

hipError_t launch_kv_append(const KvAppendParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(kv_append_kernel, dim3(p.batch * p.num_kv_heads), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
