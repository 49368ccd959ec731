// Variable-length causal prefill attention over the paged KV cache (the HALOps
// README's variable-length GQA prefill), on the gfx950 matrix cores.
//
// Work item = (request b, kv head g, head group of GWI query heads, 64-token query
// tile). Each wave takes 16 query tokens and HPW = min(GWI, 2) of the group's heads,
// so a workgroup has 4 * GWI / HPW waves (8 for four-head groups: two waves per SIMD,
// whose matrix products and exponentials the hardware interleaves). The workgroup
// walks the tile's causal key range in 32-key blocks; each block is staged into LDS
// once for all of the group's heads. Query token t of request b sits at position
// L_b - n_b + t and sees keys j <= that position.
//
// Per block, with v_mfma_f32_16x16x32_bf16 (lane l: row / column l % 16, k-group
// l / 16):
// - S^T = K . Q^T: K rows come from LDS, the Q^T fragments stay in registers for the
//   whole tile. Lane (n, gq) gets keys 16h + 4gq + v of query n for the two 16-key
//   halves h.
// - Online softmax in log2 units, c = scale * log2(e) (times the page's K scale for
//   FP8): p = 2^(s c - m) with one fused multiply-add before the exponential. The
//   running maximum m is raised only when a block exceeds it by more than 8, so the
//   accumulator is rescaled rarely; the row's probability sum l is kept in fp32 and
//   is the output's normaliser and the log-sum-exp's argument.
// - P enters the matrix cores as bf16. Where a block's largest probability may be a
//   large share of the row's sum (a row's first block, rows that see few keys, sharp
//   rows), the low bf16 part p - bf16(p) is multiplied into V as well, so the weights
//   that dominate an output are carried to about 16 bits.
// - O^T += V^T . P^T: the two S^T halves of a lane pack into the 8 k-values of P^T's
//   B operand directly (keys 4gq + 0..3 and 16 + 4gq + 0..3); V is staged into LDS
//   transposed, in that same key order, so V^T's A operand is one 16-byte LDS read.
// - The next block's K and V are loaded into registers while the current one is
//   computed (double-buffered stage, one barrier per block).
// FP8 (e4m3fn) K/V bytes are widened to bf16 exactly; with 64-token pages a 32-key
// block lies in one page, so its K scale multiplies the scores and its V scale P.
#include "kernels.hpp"

#include <math.h>

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTileTokens = 64;     // query tokens per work item (4 token slices x 16)
constexpr int kBlockKeys = 32;
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kLn2 = 0.69314718055994531f;
// A row's running maximum is raised only when a block's maximum exceeds it by more
// than this (log2 units), so probabilities stay <= 2^8.
constexpr float kRescaleSlack = 8.f;
// P's low bf16 part is multiplied into V as well on a block where some row's largest
// probability p_max may exceed a quarter of the row's sum after the block: tested as
// 3 p_max > (sum before the block), which holds whenever p_max > (sum after) / 4.
constexpr float kLowPartTest = 3.f;

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ float bf16_lo(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(unsigned u) { return __uint_as_float(u & 0xffff0000u); }

// Four e4m3fn bytes -> four bf16 (two dwords), exact.
__device__ __forceinline__ u32x2 fp8x4_to_bf16(unsigned w) {
  u32x2 r;
  r[0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  r[1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  return r;
}

// Reductions over the four lanes n, n + 16, n + 32, n + 48 (one query row); every
// lane of the row gets the same bits.
__device__ __forceinline__ float group_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Position of key k (0..31) of a block in the P^T / V^T operand order: lane group gq
// holds keys 4gq + 0..3 of half 0 then of half 1.
__device__ __forceinline__ int key_slot(int k) {
  const int h = k >> 4, r = k & 15;
  return 8 * (r >> 2) + 4 * h + (r & 3);
}

// Heads per work item GWI (1, 2, 4); each wave takes 16 tokens x HPW heads.
template <int GWI>
struct WaveCfg {
  static constexpr int kHeadsPerWave = GWI > 2 ? 2 : GWI;
  static constexpr int kWaves = 4 * GWI / kHeadsPerWave;
  static constexpr int kThreads = 64 * kWaves;
};

template <int D, bool FP8>
struct PCfg {
  static constexpr int kEb = FP8 ? 1 : 2;
  static constexpr int kRowBytes = D * kEb;
  static constexpr int kRowUnits = kRowBytes / 16;        // 16-byte units per K/V row
  static constexpr int kBlockUnits = kBlockKeys * kRowUnits;
  static constexpr int kSteps = D / 32;                   // MFMA k-steps over D
  static constexpr int kDimBlocks = D / 16;               // 16-dim blocks of O^T
  static constexpr int kDimsPerUnit = 16 / kEb;           // head dims in one 16-byte unit
};

// Head dimension of k-step s, lane group gq, element e (fp8: one 16-byte read of a
// row serves two k-steps), as in the decode kernel.
template <bool FP8>
__device__ __forceinline__ int op_dim(int s, int gq, int e) {
  if (FP8) return 64 * (s >> 1) + 16 * gq + 8 * (s & 1) + e;
  return 32 * s + 8 * gq + e;
}

// LDS (bytes): K rows [32] of kKStride = row bytes + 16, and V^T rows [D] of
// kVStride = 80 (32 bf16 keys in operand order + 16). The padding puts the 16 rows
// that 16 lanes read at once in disjoint bank groups, and leaves each lane one base
// address with constant offsets.
template <int D, bool FP8>
struct Stage {
  static constexpr int kKStride = PCfg<D, FP8>::kRowBytes + 16;
  static constexpr int kVStride = 2 * kBlockKeys + 16;
  alignas(16) uint8_t k[kBlockKeys * kKStride];
  alignas(16) uint8_t vt[D * kVStride];
};

struct TileCtx {
  const int32_t* __restrict__ bt;
  int64_t head_off, page_bytes;
  int L, page_size, row_bytes;
};

// Global byte offset of 16-byte unit `unit` of key j (callers keep j < L).
__device__ __forceinline__ int64_t unit_offset(const TileCtx& c, int j, int unit) {
  const int page = j / c.page_size;
  return static_cast<int64_t>(c.bt[page]) * c.page_bytes + c.head_off +
         static_cast<int64_t>(j - page * c.page_size) * c.row_bytes + 16 * unit;
}

// 16-byte units of one block per thread (fp8 D=64 has fewer units than threads).
template <int D, bool FP8, int NT>
struct BlockRegs {
  static constexpr int kUnits = (PCfg<D, FP8>::kBlockUnits + NT - 1) / NT;
  u32x4 k[kUnits];
  u32x4 v[kUnits];
};

// Load block kb's K and V units of this thread (zeros past the sequence end).
template <int D, bool FP8, int NT>
__device__ __forceinline__ void load_block(BlockRegs<D, FP8, NT>& r, const TileCtx& c,
                                           const uint8_t* __restrict__ kc,
                                           const uint8_t* __restrict__ vc, int kb, int tid) {
  using C = PCfg<D, FP8>;
#pragma unroll
  for (int i = 0; i < BlockRegs<D, FP8, NT>::kUnits; ++i) {
    const int u = tid + NT * i;
    const int row = u / C::kRowUnits, unit = u % C::kRowUnits;
    const int j = kb * kBlockKeys + row;
    if (u < C::kBlockUnits && j < c.L) {
      const int64_t off = unit_offset(c, j, unit);
      r.k[i] = *reinterpret_cast<const u32x4*>(kc + off);
      r.v[i] = *reinterpret_cast<const u32x4*>(vc + off);
    } else {
      r.k[i] = u32x4{0u, 0u, 0u, 0u};
      r.v[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// K rows as loaded; V transposed into operand key order (fp8 widened to bf16).
template <int D, bool FP8, int NT>
__device__ __forceinline__ void stage_block(Stage<D, FP8>& st, const BlockRegs<D, FP8, NT>& r, int tid) {
  using C = PCfg<D, FP8>;
  using S = Stage<D, FP8>;
#pragma unroll
  for (int i = 0; i < BlockRegs<D, FP8, NT>::kUnits; ++i) {
    const int u = tid + NT * i;
    if (u >= C::kBlockUnits) break;
    const int row = u / C::kRowUnits, unit = u % C::kRowUnits;
    *reinterpret_cast<u32x4*>(st.k + row * S::kKStride + 16 * unit) = r.k[i];
    const int ks = key_slot(row);
    const int d0 = unit * C::kDimsPerUnit;
    unsigned w[8];
    if constexpr (FP8) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 x = fp8x4_to_bf16(r.v[i][q]);
        w[2 * q] = x[0];
        w[2 * q + 1] = x[1];
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = r.v[i][q];
    }
    uint8_t* col = st.vt + d0 * S::kVStride + 2 * ks;
#pragma unroll
    for (int e = 0; e < C::kDimsPerUnit; ++e) {
      const unsigned word = w[e >> 1];
      *reinterpret_cast<uint16_t*>(col + e * S::kVStride) =
          static_cast<uint16_t>((e & 1) ? (word >> 16) : (word & 0xffffu));
    }
  }
}

// One 32-key block for this wave's 16 query tokens and HPW heads (lane (n, gq): query
// n). diag: the block reaches past some token's position, so keys j > pos are masked.
// The rare cases (masking, raising the maximum, the low part of P) are uniform
// branches inside one body, so the accumulators keep one register assignment.
template <int D, bool FP8, int HPW>
__device__ __forceinline__ void attend_block(const Stage<D, FP8>& st,
                                             const u32x4 (&qf)[HPW][PCfg<D, FP8>::kSteps],
                                             f32x4 (&acc)[HPW][PCfg<D, FP8>::kDimBlocks],
                                             float (&m)[HPW], float (&l)[HPW], bool diag, int j0,
                                             int pos, int n, int gq, float c, float v_mul) {
  using C = PCfg<D, FP8>;
  using S = Stage<D, FP8>;
  // K operands: key 16h + n, dims op_dim(s, gq, 0..7).
  const uint8_t* kbase = st.k + n * S::kKStride + 16 * gq;
  u32x4 kop[2][C::kSteps];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint8_t* krow = kbase + 16 * h * S::kKStride;
    if constexpr (FP8) {
#pragma unroll
      for (int u = 0; u < C::kSteps / 2; ++u) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(krow + 64 * u);
        const u32x2 a = fp8x4_to_bf16(x[0]), bq = fp8x4_to_bf16(x[1]);
        const u32x2 c2 = fp8x4_to_bf16(x[2]), d2 = fp8x4_to_bf16(x[3]);
        kop[h][2 * u] = u32x4{a[0], a[1], bq[0], bq[1]};
        kop[h][2 * u + 1] = u32x4{c2[0], c2[1], d2[0], d2[1]};
      }
    } else {
#pragma unroll
      for (int s = 0; s < C::kSteps; ++s) kop[h][s] = *reinterpret_cast<const u32x4*>(krow + 64 * s);
    }
  }
  // Raw scores S^T: lane (n, gq) holds keys j0 + 16h + 4gq + v of query n.
  f32x4 sacc[HPW][2];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sacc[hh][h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < C::kSteps; ++s) sacc[hh][h] = mfma_bf16(kop[h][s], qf[hh][s], sacc[hh][h]);
    }
  if (diag) {
    const int lim = pos - j0 - 4 * gq;  // key 16h + v of this lane is visible iff 16h + v <= lim
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (16 * h + v > lim) sacc[hh][h][v] = -INFINITY;
  }
  // Row maxima of the block (raw units; c > 0 keeps the order).
  float cmax[HPW];
  bool raise = false;
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    float x = fmaxf(fmaxf(sacc[hh][0][0], sacc[hh][0][1]), fmaxf(sacc[hh][0][2], sacc[hh][0][3]));
    x = fmaxf(x, fmaxf(fmaxf(sacc[hh][1][0], sacc[hh][1][1]), fmaxf(sacc[hh][1][2], sacc[hh][1][3])));
    cmax[hh] = group_max(x);
    raise |= cmax[hh] * c > m[hh] + kRescaleSlack;
  }
  if (__builtin_amdgcn_ballot_w64(raise)) {
    __asm__ volatile("");  // keeps this rare path a branch (not a select on every block)
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const float mc = cmax[hh] * c;
      const bool up = mc > m[hh] + kRescaleSlack;
      const float alpha = up ? __builtin_amdgcn_exp2f(m[hh] - mc) : 1.f;  // m = -inf gives 0
#pragma unroll
      for (int bl = 0; bl < C::kDimBlocks; ++bl) acc[hh][bl] *= alpha;
      l[hh] *= alpha;
      m[hh] = up ? mc : m[hh];
    }
  }
  // Probabilities p = 2^(s c - m) (times the V scale for FP8), the row sums, and P^T
  // packed to bf16.
  float pv[HPW][8];
  u32x4 ph[HPW];
  bool low = false;
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const float negm = m[hh] == -INFINITY ? 0.f : -m[hh];
    const float pmax = __builtin_amdgcn_exp2f(fmaf(cmax[hh], c, negm));
    low |= kLowPartTest * pmax > l[hh];
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pv[hh][e] = __builtin_amdgcn_exp2f(fmaf(sacc[hh][e >> 2][e & 3], c, negm));
      rs += pv[hh][e];
    }
    l[hh] += group_sum(rs);
    if constexpr (FP8) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[hh][e] *= v_mul;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) ph[hh][e] = pack_bf16(pv[hh][2 * e], pv[hh][2 * e + 1]);
  }
  // V^T operands: dims 16bl + n, keys in operand order.
  u32x4 vop[C::kDimBlocks];
#pragma unroll
  for (int bl = 0; bl < C::kDimBlocks; ++bl)
    vop[bl] = *reinterpret_cast<const u32x4*>(st.vt + (16 * bl + n) * S::kVStride + 16 * gq);
  if (__builtin_amdgcn_ballot_w64(low)) {
    __asm__ volatile("");
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      u32x4 pl;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pl[e] = pack_bf16(pv[hh][2 * e] - bf16_lo(ph[hh][e]), pv[hh][2 * e + 1] - bf16_hi(ph[hh][e]));
#pragma unroll
      for (int bl = 0; bl < C::kDimBlocks; ++bl) acc[hh][bl] = mfma_bf16(vop[bl], pl, acc[hh][bl]);
    }
  }
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
    for (int bl = 0; bl < C::kDimBlocks; ++bl) acc[hh][bl] = mfma_bf16(vop[bl], ph[hh], acc[hh][bl]);
}

template <int D, bool FP8, int GWI>
__global__ __launch_bounds__(WaveCfg<GWI>::kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_kernel(const PrefillParams p) {
  using C = PCfg<D, FP8>;
  using W = WaveCfg<GWI>;
  constexpr int HPW = W::kHeadsPerWave;
  constexpr int NT = W::kThreads;
  __shared__ Stage<D, FP8> stage[2];
  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slice = wid & 3, head_pair = wid >> 2;
  const int lane = tid & 63, n = lane & 15, gq = lane >> 4;

  const int4 item = reinterpret_cast<const int4*>(p.items)[blockIdx.x];
  const int b = item.x, g = item.y, hg = item.z, t0 = item.w;
  const int G = p.num_q_heads / p.num_kv_heads;
  if (b < 0 || b >= p.batch || g < 0 || g >= p.num_kv_heads || hg < 0 || (hg + 1) * GWI > G || t0 < 0)
    return;  // not an item of this batch (uniform over the workgroup)
  const int q0 = p.cu_q[b];
  const int nq = p.cu_q[b + 1] - q0;
  const int L = p.kv_lens[b];
  if (t0 >= nq || L < nq || L > p.bt_stride * p.page_size) return;  // outside the contract
  const int h0 = g * G + hg * GWI + head_pair * HPW;  // this wave's first query head
  const int first_pos = L - nq;                       // position of query token 0

  TileCtx ctx;
  ctx.bt = p.block_table + static_cast<int64_t>(b) * p.bt_stride;
  ctx.row_bytes = C::kRowBytes;
  ctx.head_off = static_cast<int64_t>(g) * p.page_size * C::kRowBytes;
  ctx.page_bytes = static_cast<int64_t>(p.num_kv_heads) * p.page_size * C::kRowBytes;
  ctx.L = L;
  ctx.page_size = p.page_size;

  // This lane's query token and its causal limit (rows past the request's end reuse
  // the last position and are not written).
  const int tw = t0 + 16 * slice;
  const int t = tw + n;
  const bool valid = t < nq;
  const int pos = first_pos + (valid ? t : nq - 1);
  const int wave_tokens = max(0, min(16, nq - tw));
  const int wave_end = wave_tokens > 0 ? first_pos + tw + wave_tokens : 0;  // keys needed
  const int wave_first_pos = first_pos + tw;
  const int tile_end = first_pos + min(t0 + kTileTokens, nq);            // keys of the item
  const int nblocks = (tile_end + kBlockKeys - 1) / kBlockKeys;
  const int wave_blocks = (wave_end + kBlockKeys - 1) / kBlockKeys;

  // Softmax scale in log2 units; a negative scale is taken as |scale| with Q negated
  // (exact in bf16), so c > 0 below.
  float qk_log2 = p.scale * kLog2e;
  const unsigned qflip = qk_log2 < 0.f ? 0x80008000u : 0u;
  qk_log2 = fabsf(qk_log2);

  // Q^T fragments (B operand): query token t, dims op_dim(s, gq, 0..7).
  u32x4 qf[HPW][C::kSteps];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const uint16_t* qrow = p.q + (static_cast<int64_t>(q0 + (valid ? t : 0)) * p.num_q_heads + h0 + hh) * D;
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) {
      qf[hh][s] = valid ? *reinterpret_cast<const u32x4*>(qrow + op_dim<FP8>(s, gq, 0))
                        : u32x4{0u, 0u, 0u, 0u};
      qf[hh][s] ^= u32x4{qflip, qflip, qflip, qflip};
    }
  }

  f32x4 acc[HPW][C::kDimBlocks];
  float m[HPW], l[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
#pragma unroll
    for (int bl = 0; bl < C::kDimBlocks; ++bl) acc[hh][bl] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[hh] = -INFINITY;
    l[hh] = 0.f;
  }

  // Double-buffered stage: block kb is written into stage[kb & 1] while the other
  // buffer may still be read; the one barrier per block separates both uses.
  BlockRegs<D, FP8, NT> regs;
  load_block<D, FP8, NT>(regs, ctx, p.k_cache, p.v_cache, 0, tid);
  for (int kb = 0; kb < nblocks; ++kb) {
    Stage<D, FP8>& st = stage[kb & 1];
    stage_block<D, FP8, NT>(st, regs, tid);
    __syncthreads();
    if (kb + 1 < nblocks) load_block<D, FP8, NT>(regs, ctx, p.k_cache, p.v_cache, kb + 1, tid);
    if (kb < wave_blocks) {
      const int j0 = kb * kBlockKeys;
      float c = qk_log2, v_mul = 1.f;
      if constexpr (FP8) {
        const int64_t sidx = static_cast<int64_t>(ctx.bt[j0 / p.page_size]) * p.num_kv_heads + g;
        c = qk_log2 * p.k_scale[sidx];
        v_mul = p.v_scale[sidx];
      }
      attend_block<D, FP8, HPW>(st, qf, acc, m, l, j0 + kBlockKeys - 1 > wave_first_pos, j0, pos,
                                n, gq, c, v_mul);
    }
  }

  // Rows to the output: lane (n, gq) holds dims 16bl + 4gq + v of query n; l is the
  // row's fp32 probability sum (the same in the row's four lanes).
  if (!valid) return;
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const float inv = l[hh] > 0.f ? 1.f / l[hh] : 0.f;
    const int64_t row = static_cast<int64_t>(q0 + t) * p.num_q_heads + h0 + hh;
    uint16_t* orow = p.out + row * D;
#pragma unroll
    for (int bl = 0; bl < C::kDimBlocks; ++bl) {
      const int d = 16 * bl + 4 * gq;
      const u32x2 w = {pack_bf16(acc[hh][bl][0] * inv, acc[hh][bl][1] * inv),
                       pack_bf16(acc[hh][bl][2] * inv, acc[hh][bl][3] * inv)};
      *reinterpret_cast<u32x2*>(orow + d) = w;
    }
    if (p.lse != nullptr && gq == 0)
      p.lse[row] = l[hh] > 0.f ? (m[hh] + __builtin_amdgcn_logf(l[hh])) * kLn2 : -INFINITY;
  }
}

template <int D, bool FP8, int GWI>
void launch_one(const PrefillParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_kernel<D, FP8, GWI>), dim3(static_cast<unsigned>(p.num_items)),
                     dim3(WaveCfg<GWI>::kThreads), 0, stream, p);
}

template <int D, bool FP8>
void launch_heads(const PrefillParams& p, int heads_per_item, hipStream_t stream) {
  switch (heads_per_item) {
    case 1: launch_one<D, FP8, 1>(p, stream); break;
    case 2: launch_one<D, FP8, 2>(p, stream); break;
    default: launch_one<D, FP8, 4>(p, stream); break;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int head_dim, bool fp8, int heads_per_item,
                          hipStream_t stream) {
  if (head_dim == 128) {
    if (fp8) launch_heads<128, true>(p, heads_per_item, stream);
    else launch_heads<128, false>(p, heads_per_item, stream);
  } else {
    if (fp8) launch_heads<64, true>(p, heads_per_item, stream);
    else launch_heads<64, false>(p, heads_per_item, stream);
  }
  return hipGetLastError();
}

}  // namespace pkv
