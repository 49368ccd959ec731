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

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Exact value of an e4m3fn code (0x7F / 0xFF give NaN). Branch-free: the kernel is
// short enough that its instruction fetch shows, so the conversions are kept small.
__device__ __forceinline__ float e4m3fn_value(uint32_t code) {
  const uint32_t sign = (code & 0x80u) << 24;
  const uint32_t e = (code >> 3) & 0xFu, m = code & 7u;
  const float normal = __uint_as_float(sign | ((e + 120u) << 23) | (m << 20));
  const float sub = __uint_as_float(__float_as_uint(static_cast<float>(m) * 0x1p-9f) | sign);  // m * 2^-9
  const float nan = __uint_as_float(sign | 0x7FC00000u);
  return (e == 15u && m == 7u) ? nan : (e == 0u ? sub : normal);
}

// e4m3fn code of a float32: nearest value, ties to the even code, saturating at 448,
// sign kept (a negative value that rounds to zero gives 0x80). Branch-free:
// - |x| >= 2^-6: the float32 exponent and top 3 mantissa bits, rounded to nearest
//   even by adding 2^19 - 1 plus the kept lowest bit below them (a carry moves into the
//   exponent), rebiased from 127 to 7 and capped at 0x7E (448; 480 and up, and
//   infinity, would pass it);
// - |x| < 2^-6: the subnormal codes are the multiples of 2^-9, so the code is
//   rint(|x| * 512) (exact scaling; rint ties to even; 8 is 2^-6, the first normal);
// - NaN gives 0x7F.
__device__ __forceinline__ uint32_t e4m3fn_code(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float ax = fabsf(x);
  const uint32_t au = __float_as_uint(ax);
  const uint32_t normal = min(((au + 0x7FFFFu + ((au >> 20) & 1u)) >> 20) - (120u << 3), 0x7Eu);
  const uint32_t sub = static_cast<uint32_t>(__builtin_rintf(fminf(ax, 0x1p-6f) * 512.f));  // 0 .. 8
  uint32_t code = ax < 0x1p-6f ? sub : normal;
  code = (ax != ax) ? 0x7Fu : code;
  return sign | code;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

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

// Four consecutive table values (the tables need only 4-byte alignment: element loads;
// 16-byte loads where the tables allow them measured no faster).
__device__ __forceinline__ void load_row4(const float* src, float (&x)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = src[j];
}

// Rotation of one lane's four pairs (x1[j], x2[j]) = (x[i0 + j], x[i0 + j + D/2]) of a
// row by the table values (c[j], s[j]) of its position.
__device__ __forceinline__ void rotate4(float (&x1)[4], float (&x2)[4], const float (&c)[4],
                                        const float (&s)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float r1 = x1[j] * c[j] - x2[j] * s[j];
    const float r2 = x2[j] * c[j] + x1[j] * s[j];
    x1[j] = r1;
    x2[j] = r2;
  }
}

// Query-row quads a thread rotates with their loads issued up front (the rest, with
// more query heads or draft tokens, in a loop afterwards).
constexpr int kQPre = 2;

// One workgroup of kWaves waves per (request b, kv head g): four, or two when each
// request appends one token (which touches one page only). Wave 2p + kind writes the
// new rows of touched page p (0: the page of the first new token, 1: the next one,
// if touched) of K (kind 0, rotated) or V (kind 1); each lane holds four rotation
// pairs (i0 .. i0+3 and the same + D/2 of one row), so the page's largest |value|
// is a wave reduction and no step waits for another wave. Every thread also rotates
// four pairs of the new q rows of the kv head's query heads. All loads that need only
// the request's length (block-table entry, new k/v rows, q rows, rotation tables) are
// issued together, then the page scale (which needs the block-table entry); so the
// kernel waits for memory about twice before its stores. For FP8, one barrier then
// lets the whole workgroup re-encode page 0's earlier rows if its scale rose.
template <int kWaves>
__global__ __launch_bounds__(64 * kWaves) void kv_append_kernel(const KvAppendParams p) {
  constexpr int kThreads = 64 * kWaves;
  __shared__ int re_flag[2];          // page 0 of K / V needs its earlier rows re-encoded
  __shared__ float re_scale[2][2];    // (old, new) scale of page 0 of K / V
  __shared__ int64_t re_phys;         // physical page of page 0
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x / p.num_kv_heads, g = blockIdx.x - b * p.num_kv_heads;
  const int Tq = p.q_len, D = p.head_dim, H = D / 2, P = p.page_size;
  const int L = p.seq_lens[b];
  if (L < Tq || L < 1 || L > p.bt_stride * P) return;  // outside the caller's contract
  const int first = L - Tq;
  const bool rope = p.rope_cos != nullptr;

  // This wave's page and rows.
  const int lp = first / P + (wid >> 1);
  const int kind = wid & 1;
  const bool touched = lp <= (L - 1) / P;  // wave-uniform
  const int o0 = max(first, lp * P) - lp * P;
  const int o1 = min(L, (lp + 1) * P) - lp * P;
  const int n = o1 - o0;                   // new rows in this page, 1 .. Tq (if touched)
  const int t0 = lp * P + o0 - first;      // their first new-token index
  const int e0 = 4 * lane;                 // first of this lane's four pairs
  const bool act = touched && e0 < n * H;
  const int r = act ? e0 / H : 0, i0 = act ? e0 - r * H : 0;
  int64_t phys = 0;
  float x1[4] = {0.f, 0.f, 0.f, 0.f}, x2[4] = {0.f, 0.f, 0.f, 0.f};
  float kc[4], ks[4];
  const bool rot_k = rope && kind == 0;
  if (touched) {
    phys = p.block_table[static_cast<int64_t>(b) * p.bt_stride + lp];
    if (act) {
      const uint16_t* src = kind == 0 ? p.k_new : p.v_new;
      const int64_t in = ((static_cast<int64_t>(b) * Tq + t0 + r) * p.num_kv_heads + g) * D;
      load4(src + in + i0, x1);
      load4(src + in + i0 + H, x2);
      if (rot_k) {
        const int64_t pos = first + t0 + r;
        load_row4(p.rope_cos + pos * H + i0, kc);
        load_row4(p.rope_sin + pos * H + i0, ks);
      }
    }
  }

  // The first q quads of this thread: rows of query heads g*G .. g*G+G-1.
  const int G = p.num_q_heads / p.num_kv_heads;
  const int qn = (rope && p.q_out != nullptr) ? Tq * G * H : 0;
  float qx1[kQPre][4], qx2[kQPre][4], qc[kQPre][4], qs[kQPre][4];
  int64_t qrow[kQPre];
  int qi0[kQPre];
  // Thread order for the q quads starts at the second wave, so that with one new token
  // (two waves) the V wave rotates q while the K wave rotates k.
  const int qtid = (tid + 64) % kThreads;
#pragma unroll
  for (int k = 0; k < kQPre; ++k) {
    const int e = 4 * qtid + 4 * kThreads * k;
    qrow[k] = -1;
    if (e < qn) {
      const int t = e / (G * H), j = (e / H) % G;
      qi0[k] = e % H;
      const int64_t pos = first + t;
      qrow[k] = ((static_cast<int64_t>(b) * Tq + t) * p.num_q_heads + g * G + j) * D;
      load4(p.q + qrow[k] + qi0[k], qx1[k]);
      load4(p.q + qrow[k] + qi0[k] + H, qx2[k]);
      load_row4(p.rope_cos + pos * H + qi0[k], qc[k]);
      load_row4(p.rope_sin + pos * H + qi0[k], qs[k]);
    }
  }

  // The page scale (FP8): the one load that waits for the block-table entry.
  const int64_t sidx = phys * p.num_kv_heads + g;
  float* scales = kind == 0 ? p.k_scale : p.v_scale;
  const float s_old = (p.fp8 && touched) ? scales[sidx] : 1.f;

#pragma unroll
  for (int k = 0; k < kQPre; ++k) {
    if (qrow[k] >= 0) {
      rotate4(qx1[k], qx2[k], qc[k], qs[k]);
      *reinterpret_cast<u32x2*>(p.q_out + qrow[k] + qi0[k]) = pack4_bf16(qx1[k]);
      *reinterpret_cast<u32x2*>(p.q_out + qrow[k] + qi0[k] + H) = pack4_bf16(qx2[k]);
    }
  }
  for (int e = 4 * qtid + 4 * kThreads * kQPre; e < qn; e += 4 * kThreads) {
    const int t = e / (G * H), j = (e / H) % G, qi = e % H;
    const int64_t pos = first + t;
    const int64_t row = ((static_cast<int64_t>(b) * Tq + t) * p.num_q_heads + g * G + j) * D;
    float y1[4], y2[4], c[4], sn[4];
    load4(p.q + row + qi, y1);
    load4(p.q + row + qi + H, y2);
    load_row4(p.rope_cos + pos * H + qi, c);
    load_row4(p.rope_sin + pos * H + qi, sn);
    rotate4(y1, y2, c, sn);
    *reinterpret_cast<u32x2*>(p.q_out + row + qi) = pack4_bf16(y1);
    *reinterpret_cast<u32x2*>(p.q_out + row + qi + H) = pack4_bf16(y2);
  }

  if (touched) {
    uint8_t* cache = kind == 0 ? p.k_cache : p.v_cache;
    const int64_t row = sidx * P + o0 + r;  // row o0 + r of the page's kv-head run
    if (act && rot_k) rotate4(x1, x2, kc, ks);
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
          // A "raised" scale equal to the old one (a / s rounds just above 448 while
          // a / 448 rounds back to s) would re-encode every earlier code to itself: the
          // round trip code value * s / s moves a value by at most 2^-23 relative, far
          // below half an e4m3fn step, while s lies in [2^-100, 2^118] (no float32
          // underflow or overflow on the way). So that re-encode is skipped.
          again = !(s == s_old && s_old >= 0x1p-100f && s_old <= 0x1p118f);
        }
      }
      if (wid < 2 && lane == 0) {  // page 0: whether its earlier rows need re-encoding
        re_flag[kind] = again ? 1 : 0;
        re_scale[kind][0] = s_old;
        re_scale[kind][1] = s;
        if (kind == 0) re_phys = phys;
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
  // values under the old scale; the whole workgroup shares the work, each thread
  // loading all of its 16-byte units before converting any (one wait for memory).
  // Those rows are disjoint from the new ones written above.
  if (p.fp8) {
    __syncthreads();
    const int nflag = re_flag[0] + re_flag[1];
    if (nflag != 0) {
      const int o0p = first - (first / P) * P;
      const int units = o0p * D / 16;  // 16-byte units of the earlier rows of one page
      const int kfirst = re_flag[0] ? 0 : 1;
      const int64_t run = (re_phys * p.num_kv_heads + g) * P * D;
      const int total = nflag * units;  // units of the flagged kinds, kfirst's first
      constexpr int kBatch = 4;
      for (int f0 = 0; f0 < total; f0 += kBatch * kThreads) {
        u32x4 w[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int f = f0 + j * kThreads + tid;
          if (f < total) {
            const int kd = f < units ? kfirst : 1;
            const uint8_t* page = (kd == 0 ? p.k_cache : p.v_cache) + run;
            w[j] = *reinterpret_cast<const u32x4*>(page + 16 * static_cast<int64_t>(f < units ? f : f - units));
          }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int f = f0 + j * kThreads + tid;
          if (f < total) {
            const int kd = f < units ? kfirst : 1;
            uint8_t* page = (kd == 0 ? p.k_cache : p.v_cache) + run;
            const float so = re_scale[kd][0], sn = re_scale[kd][1];
            uint32_t* dst = reinterpret_cast<uint32_t*>(page + 16 * static_cast<int64_t>(f < units ? f : f - units));
#pragma unroll 1
            for (int i = 0; i < 4; ++i) {
              const uint32_t word = i == 0 ? w[j].x : i == 1 ? w[j].y : i == 2 ? w[j].z : w[j].w;
              uint32_t o = 0;
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) {
                const float v = e4m3fn_value((word >> (8 * jj)) & 0xFFu) * so;
                o |= e4m3fn_code(v / sn) << (8 * jj);
              }
              dst[i] = o;
            }
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_kv_append(const KvAppendParams& p, hipStream_t stream) {
  if (p.q_len == 1)
    hipLaunchKernelGGL(kv_append_kernel<2>, dim3(p.batch * p.num_kv_heads), dim3(128), 0, stream, p);
  else
    hipLaunchKernelGGL(kv_append_kernel<4>, dim3(p.batch * p.num_kv_heads), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
