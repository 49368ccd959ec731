// Split-KV partial attention for paged-KV GQA decode on gfx950.
//
// One persistent workgroup per planner worker walks its work items (b, g, i): the
// uniform KV tiles that the per-step greedy bin-packing assigned to it (HPC-Ops
// review, "How the kernels are organized around specific workload shapes"). For
// each tile it writes a softmax-normalised partial output and its log-sum-exp, to
// be merged by the combine kernel.
//
// Mapping onto CDNA4 (wave64, MFMA 16x16x32 bf16):
// - The waves of a workgroup split a tile into 32-token chunks, round-robin. A chunk
//   is two 16-token halves; each half lies inside one page because pages and tiles
//   are multiples of 16 tokens.
// - Operands are swapped so the KV tokens fill the MFMA's 16-row side and the
//   M = G*Tq query rows of the kv head sit on the 16-column side (the "swap A/B"
//   idea of the HPC-Ops launch article, section on aligning task traits with the
//   hardware, re-derived for MFMA). M <= 16 is one column block; up to 64 rows (wide
//   GQA groups with draft tokens) take NB = 2 or 4 blocks that share every K/V
//   operand. Lane l owns query row 16*nb + l % 16 of block nb for the whole softmax,
//   so row max, row sum and rescale factors never leave the lane except for one
//   exchange across the four 16-lane groups.
// - K and V stream from HBM with non-temporal 16-byte loads, each wave instruction
//   reading 1 KB of whole 128-byte lines of a 16-token half: on MI355X only
//   full-line non-temporal reads reach ~6.8 TB/s on a random 4 KB page gather
//   (half-line or cached reads stop near 6.1 TB/s). Each wave stages its chunk in
//   its own LDS region:
//   - K as stored (bf16 or e4m3fn), in XOR-swizzled 16-byte units, read back in the
//     MFMA operand layout (lane l: token l % 16 of a half, bytes 16*(l/16) + 64*u of
//     its row), so QK^T needs no shuffling;
//   - V as 16-bit rows with a padded row stride, read back transposed by gfx950's
//     ds_read_b64_tr_b16: P.V contracts over tokens, and the transposing read hands
//     each lane four consecutive tokens of one head dimension, the operand layout V^T
//     needs.
// - FP8 (OCP e4m3fn) K bytes are widened to bf16 with the gfx950 conversion
//   instruction (exact) and the page's K scale multiplies the scores (one scale per
//   page and kv head; a 16-token half lies in one page). FP8 V bytes are
//   converted on their way into LDS to fp16 (code x 2^e, exact: the conversion
//   instruction applies a power-of-two scale), so P.V runs in fp16; the rest of the
//   page's V scale, v_scale / 2^e in [1, 2), multiplies P.
// - P enters the matrix cores as 16-bit numbers: fp16 for FP8 KV (2^-12 relative
//   rounding), bf16 for bf16 KV (2^-9). With bf16, on a chunk where some row's
//   largest weight may be a large share of that row's sum (a wave's first chunk of an
//   item, rows that see few keys, a score far above the earlier ones), the low bf16
//   part p - bf16(p) is multiplied into V as well, so the weights that dominate an
//   output carry about 16 bits.
// - The next chunk's loads are issued into the same registers as soon as the
//   current chunk sits in LDS, so each wave keeps one chunk (16 KB for bf16) in
//   flight while its matrix and vector work runs.
#include "kernels.hpp"

#include <math.h>

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLn2 = 0.69314718055994531f;
// A chunk also multiplies the low bf16 part of P into V when, for some row, three
// times the lane's largest new weight exceeds the lane's share of the row's sum so
// far. That holds whenever a weight exceeds a quarter of the row's sum after the
// chunk (the weight's own lane sees 4p > p + its earlier sum).
constexpr float kLowPartTest = 3.f;

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

// Two floats -> packed fp16 pair (round to nearest even; v_cvt_pk_f16_f32).
__device__ __forceinline__ unsigned pack_f16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, f16x2));
}

__device__ __forceinline__ float bf16_lo(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(unsigned u) { return __uint_as_float(u & 0xffff0000u); }

// Eight e4m3fn bytes (two dwords) -> eight bf16 (four dwords), exact.
__device__ __forceinline__ u32x4 fp8x8_to_bf16(unsigned w0, unsigned w1) {
  u32x4 r;
  r[0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
  r[1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
  r[2] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
  r[3] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
  return r;
}

// Eight e4m3fn bytes -> eight fp16 values of code x scale, for a power-of-two scale
// (exact while the result stays in fp16's normal and subnormal range).
__device__ __forceinline__ u32x4 fp8x8_to_f16(unsigned w0, unsigned w1, float scale) {
  u32x4 r;
  r[0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, scale, false));
  r[1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, scale, true));
  r[2] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, scale, false));
  r[3] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, scale, true));
  return r;
}

// Transposing LDS read of four 16-bit values: in each 16-lane group, lanes 4k..4k+3
// address row k of a 4 x 16 tile and lane i receives column i (rows 0..3).
__device__ __forceinline__ u32x2 read_tr16(const uint8_t* p) {
  const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, x);
}

// Max over the four 16-lane groups (lanes n, n+16, n+32, n+48) with the gfx950
// lane-swap instructions: each swap returns the value and its partner in every lane.
__device__ __forceinline__ float group_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float max8(const float (&a)[8]) {
  return fmaxf(fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])),
               fmaxf(fmaxf(a[4], a[5]), fmaxf(a[6], a[7])));
}

template <int D, bool FP8, int NB>
struct Cfg {
  static constexpr int kEb = FP8 ? 1 : 2;        // bytes per KV element
  static constexpr int kSteps = D / 32;           // MFMA k-steps over the head dimension
  static constexpr int kLoads = D * kEb / 64;     // 16-byte loads per lane per half
  static constexpr int kBlocks = D / 16;          // 16-wide head-dim blocks of the output
  static constexpr int kRowBytes = D * kEb;
  static constexpr int kUnits = kRowBytes / 16;   // 16-byte units per token row
  // Rows per 256 bytes is a power of two; the swizzle uses rows / (256 / kRowBytes).
  static constexpr int kRowShift = kRowBytes == 256 ? 0 : (kRowBytes == 128 ? 1 : 2);
  // One column block: two waves per SIMD. Two or four blocks hold 2-4x the
  // accumulators and query fragments: one wave per SIMD, with twice the registers.
  static constexpr int kWaves = NB == 1 ? 8 : 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kRows = 16 * NB;
  // bf16 KV: P.V in bf16, with P's low part on chunks that need it. FP8 KV: P.V in
  // fp16 (V = code x scale converted on staging), precise enough without it.
  static constexpr bool kLowPart = !FP8;
  // Per-wave LDS (bytes): K rows [32] as stored, then V rows [32] as 16-bit with a
  // stride of 2D + 32 bytes (the four rows of a transposing read fall in disjoint
  // bank groups). After an item's last chunk the region holds the wave's
  // unnormalised output rows, kMergeBlocks column blocks [16][D] fp32 at a time.
  static constexpr int kKBytes = 32 * kRowBytes;
  static constexpr int kVStride = 2 * D + 32;
  static constexpr int kStageBytes = kKBytes + 32 * kVStride;
  static constexpr int kMergeBlocks =
      kStageBytes / (16 * D * 4) < NB ? kStageBytes / (16 * D * 4) : NB;
  static constexpr int kMergeRounds = (NB + kMergeBlocks - 1) / kMergeBlocks;
  // Four column blocks keep their query fragments in LDS (per wave, [NB][kSteps]
  // 16-byte units in lane order) instead of 64 registers.
  static constexpr bool kQInLds = NB > 2;
  static constexpr int kQBytes = kQInLds ? NB * kSteps * 64 * 16 : 0;
  static constexpr int kWaveBytes = kStageBytes + kQBytes;
  static_assert(kMergeBlocks >= 1, "a column block's rows must fit a wave's region");
};

// Head-dimension index that k-step s, lane group gq, element e of a QK^T operand
// holds. bf16: one 16-byte K unit per step. fp8: one 16-byte unit serves two steps.
template <bool FP8>
__device__ __forceinline__ int op_dim(int s, int gq, int e) {
  if (FP8) return 64 * (s >> 1) + 16 * gq + 8 * (s & 1) + e;
  return 32 * s + 8 * gq + e;
}

struct ItemCtx {
  const int32_t* __restrict__ bt;  // block-table row of the request
  int64_t head_off;                // byte offset of kv head g inside a page
  int64_t page_bytes;              // bytes of one page (all heads)
  int tile_start, tile_end, page_size, row_bytes;
  unsigned page_magic;             // ceil(2^32 / page_size)
};

// Page of token j (0 <= j < 2^31) and j's row inside it, without a division: with
// m = ceil(2^32 / P) the estimate floor(j m / 2^32) exceeds j / P by less than 1/2,
// so it is the quotient or one more.
__device__ __forceinline__ int page_of(int j, unsigned magic, int P, int* row) {
  int q = static_cast<int>(__umulhi(static_cast<unsigned>(j), magic));
  int r = j - q * P;
  if (r < 0) {
    q -= 1;
    r += P;
  }
  *row = r;
  return q;
}

// Byte offsets of the two 16-token halves of a chunk (wave-uniform; the block-table
// reads are scalar loads) and their physical pages, which index the FP8 page scales.
// A half past the tile end re-reads half 0 (masked later).
struct HalfOffsets {
  int64_t off[2];
  int64_t phys[2];
};

__device__ __forceinline__ HalfOffsets chunk_offsets(const ItemCtx& it, int chunk) {
  HalfOffsets r;
  const int j0 = it.tile_start + 32 * chunk;
  // Both block-table entries are read before either is used (two scalar loads in
  // flight at once). Half 1 lies in half 0's page or the next one.
  int row0, row1;
  const int page0 = page_of(j0, it.page_magic, it.page_size, &row0);
  int page1 = page0;
  row1 = row0;
  if (j0 + 16 < it.tile_end) {
    row1 = row0 + 16;
    if (row1 >= it.page_size) {
      row1 -= it.page_size;
      page1 += 1;
    }
  }
  const int64_t phys0 = it.bt[page0];
  const int64_t phys1 = it.bt[page1];
  r.phys[0] = phys0;
  r.phys[1] = phys1;
  r.off[0] = phys0 * it.page_bytes + it.head_off + static_cast<int64_t>(row0) * it.row_bytes;
  r.off[1] = phys1 * it.page_bytes + it.head_off + static_cast<int64_t>(row1) * it.row_bytes;
  return r;
}

// One chunk as loaded: [K/V][half][instruction], 16 bytes per lane each.
template <int D, bool FP8, int NB>
struct Raw {
  u32x4 r[2][2][Cfg<D, FP8, NB>::kLoads];
};

// Issue the chunk's loads: instruction j of half h reads bytes j*1024 + 16*lane of
// the half's contiguous 16-row run (whole cache lines, non-temporal).
template <int D, bool FP8, int NB>
__device__ __forceinline__ void load_raw(Raw<D, FP8, NB>& raw, const uint8_t* __restrict__ kc,
                                         const uint8_t* __restrict__ vc, const HalfOffsets& ho,
                                         int lane) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int j = 0; j < Cfg<D, FP8, NB>::kLoads; ++j) {
      const int64_t off = ho.off[h] + j * 1024 + lane * 16;
      raw.r[0][h][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kc + off));
      raw.r[1][h][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vc + off));
    }
  }
}

// K stage slot of 16-byte unit `unit` of chunk row `row` (0..31). The unit index is
// XOR-ed with the row's position among the rows that share a 256-byte bank window,
// so 16 lanes reading one unit column of 16 rows hit 16 distinct 16-byte bank groups.
template <int D, bool FP8, int NB>
__device__ __forceinline__ int k_slot(int row, int unit) {
  using C = Cfg<D, FP8, NB>;
  return row * C::kUnits + (unit ^ ((row >> C::kRowShift) & (C::kUnits - 1)));
}

// Stage a loaded chunk. V rows at or past `valid` (tokens past the tile end, which
// may be unwritten cache memory) are stored as zeros, so that a zero probability
// never meets a NaN in P.V. FP8 V codes of half h are stored as fp16 code x
// v_pow2[h] (a power of two).
template <int D, bool FP8, int NB>
__device__ __forceinline__ void stage_write(uint8_t* __restrict__ st, const Raw<D, FP8, NB>& raw,
                                            int lane, int valid, const float (&v_pow2)[2]) {
  using C = Cfg<D, FP8, NB>;
  u32x4* const kst = reinterpret_cast<u32x4*>(st);
  uint8_t* const vst = st + C::kKBytes;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < C::kLoads; ++j) {
      const int pos = j * 1024 + lane * 16;
      const int row = 16 * h + pos / C::kRowBytes;
      const int unit = (pos % C::kRowBytes) / 16;
      kst[k_slot<D, FP8, NB>(row, unit)] = raw.r[0][h][j];
      const u32x4 v = raw.r[1][h][j];
      if constexpr (FP8) {
        u32x4* dst = reinterpret_cast<u32x4*>(vst + row * C::kVStride + 32 * unit);
        dst[0] = fp8x8_to_f16(v[0], v[1], v_pow2[h]);
        dst[1] = fp8x8_to_f16(v[2], v[3], v_pow2[h]);
      } else {
        *reinterpret_cast<u32x4*>(vst + row * C::kVStride + 16 * unit) = v;
      }
    }
  if (valid < 32) {  // a tile's last chunk only (wave-uniform): overwrite the tail rows
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < C::kLoads; ++j) {
        const int pos = j * 1024 + lane * 16;
        const int row = 16 * h + pos / C::kRowBytes;
        const int unit = (pos % C::kRowBytes) / 16;
        if (row >= valid) {
          u32x4* dst = reinterpret_cast<u32x4*>(vst + row * C::kVStride + (FP8 ? 32 : 16) * unit);
          dst[0] = u32x4{0u, 0u, 0u, 0u};
          if constexpr (FP8) dst[1] = u32x4{0u, 0u, 0u, 0u};
        }
      }
  }
}

// K operands of half h: lane (n, gq) takes bytes 64u + 16gq of token row 16h + n;
// fp8 units widen to two bf16 operand steps.
template <int D, bool FP8, int NB>
__device__ __forceinline__ void read_k(const uint8_t* __restrict__ st, u32x4 (&kop)[D / 32], int h,
                                       int n, int gq) {
  using C = Cfg<D, FP8, NB>;
  const u32x4* const kst = reinterpret_cast<const u32x4*>(st);
#pragma unroll
  for (int u = 0; u < C::kLoads; ++u) {
    const u32x4 kr = kst[k_slot<D, FP8, NB>(16 * h + n, 4 * u + gq)];
    if constexpr (FP8) {
      kop[2 * u] = fp8x8_to_bf16(kr[0], kr[1]);
      kop[2 * u + 1] = fp8x8_to_bf16(kr[2], kr[3]);
    } else {
      kop[u] = kr;
    }
  }
}

// Online-softmax state of the rows a lane owns (one per column block): running
// maximum m (log2 units), the sum of the weights P.V used (the output's normaliser)
// and the sum of the unrounded weights (the log-sum-exp's argument). Each lane
// holds the sums of its own tokens; the row's four lanes are added at the end.
template <int NB>
struct RowState {
  float m[NB], lsum[NB], lexact[NB];
};

// Online-softmax update of one 32-token chunk for every column block. acc[nb][bl]
// holds O^T of head-dim block bl (lane: dims 16bl + 4gq + v, query row 16nb + n).
// bf16 KV with one column block forms P's low parts only when the chunk needs them;
// wider items form them with the high parts (fewer live registers: the unrounded
// weights are not kept across the products) and read K once per block.
template <int D, bool FP8, int NB, class QGet>
__device__ __forceinline__ void process_chunk(const uint8_t* __restrict__ st, const QGet& qget,
                                              f32x4 (&acc)[NB][D / 16], RowState<NB>& rs, int j0,
                                              const int (&lim)[NB], const float (&c_qk)[2],
                                              const float (&p_mul)[2], int n, int gq) {
  using C = Cfg<D, FP8, NB>;
  constexpr bool kLow = C::kLowPart;
  constexpr bool kEagerLow = kLow && NB > 1;
  float pv[kLow && !kEagerLow ? NB : 1][8];
  u32x4 ph[NB], pl[kEagerLow ? NB : 1];
  float psum[NB], plsum[kEagerLow ? NB : 1];
  bool low = false;
  // S^T = K . Q^T: lane (n, gq) gets tokens 16h + 4gq + v of query row 16nb + n.
  f32x4 sacc1[NB == 1 ? 2 : 1];
  if constexpr (NB == 1) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 kop[C::kSteps];
      read_k<D, FP8, NB>(st, kop, h, n, gq);
      sacc1[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < C::kSteps; ++s) sacc1[h] = mfma_bf16(kop[s], qget(0, s), sacc1[h]);
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    f32x4 sacc[2];
    if constexpr (NB == 1) {
      sacc[0] = sacc1[0];
      sacc[1] = sacc1[1];
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 kop[C::kSteps];
        read_k<D, FP8, NB>(st, kop, h, n, gq);
        sacc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < C::kSteps; ++s) sacc[h] = mfma_bf16(kop[s], qget(nb, s), sacc[h]);
      }
    }
    float sv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = j0 + 16 * (e >> 2) + 4 * gq + (e & 3);
      sv[e] = (j < lim[nb]) ? sacc[e >> 2][e & 3] * c_qk[e >> 2] : -INFINITY;
    }
    const float lane_max = max8(sv);
    const float m_new = fmaxf(rs.m[nb], group_max(lane_max));
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(rs.m[nb] - m_use);
    rs.lsum[nb] *= alpha;
    rs.lexact[nb] *= alpha;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int bl = 0; bl < C::kBlocks; ++bl) acc[nb][bl] *= alpha;
    }
    rs.m[nb] = m_new;
    if constexpr (kLow) low |= kLowPartTest * __builtin_amdgcn_exp2f(lane_max - m_use) > rs.lexact[nb];
    float p[8], pexact = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = __builtin_amdgcn_exp2f(sv[e] - m_use);
      pexact += p[e];
    }
    rs.lexact[nb] += pexact;
    if constexpr (FP8) {  // P.V weights carry the V scale's non-power-of-two part
#pragma unroll
      for (int e = 0; e < 4; ++e)
        ph[nb][e] = pack_f16(p[2 * e] * p_mul[e >> 1], p[2 * e + 1] * p_mul[e >> 1]);
    } else {
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ph[nb][e] = pack_bf16(p[2 * e], p[2 * e + 1]);
        ps += bf16_lo(ph[nb][e]) + bf16_hi(ph[nb][e]);
      }
      psum[nb] = ps;
    }
    if constexpr (kEagerLow) {
      float ls = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pl[nb][e] = pack_bf16(p[2 * e] - bf16_lo(ph[nb][e]), p[2 * e + 1] - bf16_hi(ph[nb][e]));
        ls += bf16_lo(pl[nb][e]) + bf16_hi(pl[nb][e]);
      }
      plsum[nb] = ls;
    } else if constexpr (kLow) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[nb][e] = p[e];
    }
  }

  // V^T operands: dims 16bl + n, tokens 4gq + 0..3 then 16 + 4gq + 0..3 (lane (n, gq)
  // addresses row 4gq + n / 4, dims 16bl + 4 (n % 4) of each four-row tile).
  const uint8_t* const vbase = st + C::kKBytes + (4 * gq + (n >> 2)) * C::kVStride + 8 * (n & 3);
  auto read_v = [&](int bl) {
    const u32x2 lo = read_tr16(vbase + 32 * bl);
    const u32x2 hi = read_tr16(vbase + 16 * C::kVStride + 32 * bl);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  // O^T += V^T . P^T: the lane's eight weights (tokens 4gq + 0..3, 16 + 4gq + 0..3)
  // are exactly the k-values of P^T's B operand.
  auto pv_mfma = [&](u32x4 v, u32x4 w, f32x4 c) { return FP8 ? mfma_f16(v, w, c) : mfma_bf16(v, w, c); };
  if constexpr (kEagerLow) {
    // Wide items: one V operand at a time, high and (when needed) low parts
    // accumulated on the matrix core (the accumulators live in AGPRs).
    const bool low_chunk = __builtin_amdgcn_ballot_w64(low) != 0;
#pragma unroll
    for (int bl = 0; bl < C::kBlocks; ++bl) {
      const u32x4 vop = read_v(bl);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb][bl] = mfma_bf16(vop, ph[nb], acc[nb][bl]);
      if (low_chunk) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb][bl] = mfma_bf16(vop, pl[nb], acc[nb][bl]);
      }
    }
    if (low_chunk) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) psum[nb] += plsum[nb];
    }
  } else {
    u32x4 vop[C::kBlocks];
#pragma unroll
    for (int bl = 0; bl < C::kBlocks; ++bl) vop[bl] = read_v(bl);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int bl = 0; bl < C::kBlocks; ++bl) acc[nb][bl] = pv_mfma(vop[bl], ph[nb], acc[nb][bl]);
    if constexpr (kLow) {
      if (__builtin_amdgcn_ballot_w64(low)) {
        // The low part goes through a fresh accumulator and is added in place, so the
        // accumulators keep their registers whichever way this branch goes.
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          u32x4 pln;
          float ls = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pln[e] = pack_bf16(pv[nb][2 * e] - bf16_lo(ph[nb][e]), pv[nb][2 * e + 1] - bf16_hi(ph[nb][e]));
            ls += bf16_lo(pln[e]) + bf16_hi(pln[e]);
          }
          psum[nb] += ls;
#pragma unroll
          for (int bl = 0; bl < C::kBlocks; ++bl)
            acc[nb][bl] += mfma_bf16(vop[bl], pln, f32x4{0.f, 0.f, 0.f, 0.f});
        }
      }
    }
  }
  // bf16 KV: the normaliser is the sum of the weights P.V used, so V = 1 gives
  // exactly 1. FP8 KV: the unrounded sum (fp16 weights are within 2^-12 of it).
  if constexpr (!FP8) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) rs.lsum[nb] += psum[nb];
  }
}

// Scalar shape arguments of the decode kernel.
struct DecodeShape {
  int q_len, num_q_heads, num_kv_heads, group, rows, page_size, bt_stride, tile_tokens;
  int request_split;  // work-list request b is part b % split of the caller's request b / split
  float qk_scale_log2;
  unsigned page_magic;  // ceil(2^32 / page_size)
};

// Wave-uniform description of one work item.
struct ItemInfo {
  ItemCtx it;
  int b, g, slot, L, nchunks;
};

template <int D, bool FP8, int NB>
__device__ __forceinline__ ItemInfo item_info(const int32_t* __restrict__ items,
                                              const int32_t* __restrict__ seq_lens,
                                              const int32_t* __restrict__ block_table,
                                              const DecodeShape& sh, int itx) {
  using C = Cfg<D, FP8, NB>;
  ItemInfo r;
  r.b = items[4 * itx + 0];
  r.g = items[4 * itx + 1];
  const int ti = items[4 * itx + 2];
  r.slot = items[4 * itx + 3];
  r.L = seq_lens[r.b];
  r.it.bt = block_table + static_cast<int64_t>(r.b) * sh.bt_stride;
  r.it.row_bytes = C::kRowBytes;
  r.it.head_off = static_cast<int64_t>(r.g) * sh.page_size * C::kRowBytes;
  r.it.page_bytes = static_cast<int64_t>(sh.num_kv_heads) * sh.page_size * C::kRowBytes;
  r.it.tile_start = ti * sh.tile_tokens;
  r.it.tile_end = min(r.L, r.it.tile_start + sh.tile_tokens);
  r.it.page_size = sh.page_size;
  r.it.page_magic = sh.page_magic;
  r.nchunks = (r.it.tile_end - r.it.tile_start + 31) >> 5;
  return r;
}

template <int D, bool FP8, int NB>
__global__ __launch_bounds__((Cfg<D, FP8, NB>::kThreads), kDecodeGroupsPerCU) void decode_partial_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ k_cache,
    const uint8_t* __restrict__ v_cache, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ items,
    const int32_t* __restrict__ worker_offsets, const int32_t* __restrict__ tile_dev,
    float* __restrict__ ws_o, float* __restrict__ ws_lse, uint16_t* __restrict__ out,
    float* __restrict__ lse_out, const DecodeShape sh_arg) {
  using C = Cfg<D, FP8, NB>;
  constexpr int kWaves = C::kWaves;
  constexpr int kThreads = C::kThreads;
  // The tile size comes from the launch, or from device memory when a device-built
  // plan chose it.
  DecodeShape sh = sh_arg;
  if (tile_dev != nullptr) sh.tile_tokens = __builtin_amdgcn_readfirstlane(tile_dev[0]);
  __shared__ __attribute__((aligned(16))) uint8_t lds_stage[kWaves][C::kWaveBytes];
  __shared__ float lds_m[kWaves][C::kRows];
  __shared__ float lds_l[kWaves][C::kRows];
  __shared__ float lds_le[kWaves][C::kRows];

  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int n = lane & 15;   // query row owned by this lane (and K/V row it reads)
  const int gq = lane >> 4;  // 16-lane group
  uint8_t* const my_stage = lds_stage[wid];

  const int M = sh.rows;
  const int Tq = sh.q_len;
  const int G = sh.group;
  const int first = worker_offsets[blockIdx.x];
  const int last = worker_offsets[blockIdx.x + 1];

  // The wave's work is a stream of units (item, chunk): chunks wid, wid + kWaves, ...
  // of each of the worker's items. `raw` always holds the next unit's K/V in flight,
  // so an item's first chunk is loaded while the previous item is still being
  // computed and merged. With one column block `qf_next` prefetches the query
  // fragments of that item as well; wider items load theirs when the item starts
  // (their registers go to the extra accumulators).
  constexpr bool kPrefetchQ = NB == 1;
  Raw<D, FP8, NB> raw;
  u32x4 qf_next[kPrefetchQ ? NB : 1][C::kSteps];
  // FP8: the K and V page scales of the unit in flight (one per 16-token half, whose
  // pages may differ), loaded with its K/V so that their dependent loads (block-table
  // entry, then scale) stay off the compute path.
  float ksc_next[2] = {1.f, 1.f}, vsc_next[2] = {1.f, 1.f};
  int u_itx = -1, u_c = 0;
  ItemInfo u_info;
  auto find_unit = [&](int from) {  // first unit of this wave in items >= from
    u_itx = -1;
    for (int x = from; x < last; ++x) {
      const ItemInfo inf = item_info<D, FP8, NB>(items, seq_lens, block_table, sh, x);
      if (wid < inf.nchunks) {
        u_itx = x;
        u_c = wid;
        u_info = inf;
        return;
      }
    }
  };
  // Query fragments of kv head g of work-list request b: row r = 16nb + n is draft
  // token r / G of query head g*G + r % G (rows r >= M are zero).
  auto load_q = [&](u32x4 (&dst)[NB][C::kSteps], int b, int g) {
    // q is [B / split, Tq, split * Hq, D]; with split 1 this is [B, Tq, Hq, D].
    const int split = sh.request_split;
    const int64_t qb = (split == 1) ? b : b / split;
    const int part = (split == 1) ? 0 : b - static_cast<int>(qb) * split;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int r = 16 * nb + n;
      if (r < M) {
        const int t = r / G;
        const int head = g * G + (r - t * G);
        const uint16_t* qrow = q + (((qb * Tq + t) * split + part) * sh.num_q_heads + head) * D;
#pragma unroll
        for (int s = 0; s < C::kSteps; ++s)
          dst[nb][s] = *reinterpret_cast<const u32x4*>(qrow + op_dim<FP8>(s, gq, 0));
      } else {
#pragma unroll
        for (int s = 0; s < C::kSteps; ++s) dst[nb][s] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto issue_unit = [&]() {
    if (u_itx < 0) return;
    const HalfOffsets ho = chunk_offsets(u_info.it, u_c);
    load_raw<D, FP8, NB>(raw, k_cache, v_cache, ho, lane);
    if constexpr (FP8) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t sidx = ho.phys[h] * sh.num_kv_heads + u_info.g;
        ksc_next[h] = k_scale[sidx];
        vsc_next[h] = v_scale[sidx];
      }
    }
    if constexpr (kPrefetchQ) {
      if (u_c == wid) load_q(qf_next, u_info.b, u_info.g);  // first chunk of an item
    }
  };
  find_unit(first);
  issue_unit();

  for (int itx = first; itx < last; ++itx) {
    const ItemInfo cur = (u_itx == itx) ? u_info
                                        : item_info<D, FP8, NB>(items, seq_lens, block_table, sh, itx);
    // Causal limit of each row (draft token t sees keys up to L - Tq + t); padding
    // rows r >= M see the whole tile.
    int lim[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int r = 16 * nb + n;
      lim[nb] = cur.it.tile_end;
      if (r < M) lim[nb] = min(lim[nb], cur.L - Tq + r / G + 1);
    }
    u32x4 qf[C::kQInLds ? 1 : NB][C::kSteps];
    u32x4* const qlds = reinterpret_cast<u32x4*>(my_stage + C::kStageBytes);
    if constexpr (kPrefetchQ) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int s = 0; s < C::kSteps; ++s) qf[nb][s] = qf_next[nb][s];
    } else if (u_itx == itx) {
      if constexpr (C::kQInLds) {
        u32x4 qt[NB][C::kSteps];
        load_q(qt, cur.b, cur.g);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int s = 0; s < C::kSteps; ++s) qlds[(nb * C::kSteps + s) * 64 + lane] = qt[nb][s];
      } else {
        load_q(qf, cur.b, cur.g);
      }
    }
    auto qget = [&](int nb, int s) -> u32x4 {
      if constexpr (C::kQInLds)
        return qlds[(nb * C::kSteps + s) * 64 + lane];
      else
        return qf[nb][s];
    };

    f32x4 acc[NB][C::kBlocks];
    RowState<NB> rs;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int bl = 0; bl < C::kBlocks; ++bl) acc[nb][bl] = f32x4{0.f, 0.f, 0.f, 0.f};
      rs.m[nb] = -INFINITY;
      rs.lsum[nb] = 0.f;
      rs.lexact[nb] = 0.f;
    }

    while (u_itx == itx) {
      const int c = u_c;
      const int j0 = cur.it.tile_start + 32 * c;
      // This unit's page scales are used before issue_unit loads the next unit's. The V
      // scale splits into v_pow2 = 2^e, applied exactly when V is converted to fp16,
      // and p_mul = v_scale / 2^e, in [1, 2) while e lies in [-15, 7].
      float c_qk[2] = {sh.qk_scale_log2, sh.qk_scale_log2}, p_mul[2] = {1.f, 1.f},
            v_pow2[2] = {1.f, 1.f};
      if constexpr (FP8) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          c_qk[h] *= ksc_next[h];
          int e;
          (void)frexpf(vsc_next[h], &e);
          const int e1 = min(max(e - 1, -15), 7);
          v_pow2[h] = ldexpf(1.f, e1);
          p_mul[h] = ldexpf(vsc_next[h], -e1);
        }
      }
      stage_write<D, FP8, NB>(my_stage, raw, lane, cur.it.tile_end - j0, v_pow2);
      if (c + kWaves < cur.nchunks)
        u_c = c + kWaves;
      else
        find_unit(itx + 1);
      issue_unit();
      process_chunk<D, FP8, NB>(my_stage, qget, acc, rs, j0, lim, c_qk, p_mul, n, gq);
    }

    // A request cut into one tile has its final rows here: with `out` set they are
    // written there too (work-list requests are the caller's when out is set).
    const bool direct = out != nullptr && cur.it.tile_start == 0 && cur.it.tile_end == cur.L;
    // Wave result -> LDS: row max and full row sums, then the unnormalised rows of
    // kMergeBlocks column blocks per round, merged across the waves.
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float ls = FP8 ? rs.lexact[nb] : rs.lsum[nb];
      float le = rs.lexact[nb];
      ls += __shfl_xor(ls, 16);
      ls += __shfl_xor(ls, 32);
      le += __shfl_xor(le, 16);
      le += __shfl_xor(le, 32);
      if (gq == 0) {
        lds_m[wid][16 * nb + n] = rs.m[nb];
        lds_l[wid][16 * nb + n] = ls;
        lds_le[wid][16 * nb + n] = le;
      }
    }
    float* const my_rows = reinterpret_cast<float*>(my_stage);
#pragma unroll
    for (int round = 0; round < C::kMergeRounds; ++round) {
      if (round > 0) __syncthreads();  // the previous round's rows have been merged
#pragma unroll
      for (int k = 0; k < C::kMergeBlocks; ++k) {
        const int nb = round * C::kMergeBlocks + k;
        if (nb < NB) {
#pragma unroll
          for (int bl = 0; bl < C::kBlocks; ++bl)
            *reinterpret_cast<f32x4*>(my_rows + (16 * k + n) * D + 16 * bl + 4 * gq) = acc[nb][bl];
        }
      }
      __syncthreads();

      // Merge the waves' partial softmax states of this round's rows and write them.
      const int r0 = 16 * C::kMergeBlocks * round;
      const int r1 = min(M, r0 + 16 * C::kMergeBlocks);
      float* wo = ws_o + static_cast<int64_t>(cur.slot) * M * D;
      for (int e = r0 * D + tid; e < r1 * D; e += kThreads) {
        const int r = e / D, d = e - r * D;
        float mx = lds_m[0][r];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, lds_m[w][r]);
        float o = 0.f;
        if (mx != -INFINITY) {
          float num = 0.f, den = 0.f;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) {
            const float f = __builtin_amdgcn_exp2f(lds_m[w][r] - mx);
            num += f * reinterpret_cast<const float*>(lds_stage[w])[(r - r0) * D + d];
            den += f * lds_l[w][r];
          }
          o = num / den;
        }
        wo[e] = o;
        if (direct) {  // what the combine writes for a single split: bf16(o)
          const int t = r / G, head = cur.g * G + (r - t * G);
          out[((static_cast<int64_t>(cur.b) * Tq + t) * sh.num_q_heads + head) * D + d] =
              __builtin_bit_cast(uint16_t, static_cast<__bf16>(o));
        }
      }
    }
    for (int r = tid; r < M; r += kThreads) {
      float mx = lds_m[0][r];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, lds_m[w][r]);
      float lse = -INFINITY;
      if (mx != -INFINITY) {
        float den = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) den += __builtin_amdgcn_exp2f(lds_m[w][r] - mx) * lds_le[w][r];
        lse = (mx + __builtin_amdgcn_logf(den)) * kLn2;
      }
      ws_lse[static_cast<int64_t>(cur.slot) * M + r] = lse;
      if (direct && lse_out != nullptr) {  // the combine passes a single split's lse through
        const int t = r / G, head = cur.g * G + (r - t * G);
        lse_out[(static_cast<int64_t>(cur.b) * Tq + t) * sh.num_q_heads + head] = lse;
      }
    }
    __syncthreads();
  }
}

template <int D, bool FP8, int NB>
void launch_one(const DecodeParams& p, int num_workers, hipStream_t stream) {
  const unsigned magic =
      static_cast<unsigned>(((1ull << 32) + static_cast<unsigned>(p.page_size) - 1) /
                            static_cast<unsigned>(p.page_size));
  const DecodeShape sh = {p.q_len,     p.num_q_heads, p.num_kv_heads, p.group,
                          p.rows,      p.page_size,   p.bt_stride,    p.tile_tokens,
                          p.request_split, p.qk_scale_log2, magic};
  hipLaunchKernelGGL((decode_partial_kernel<D, FP8, NB>), dim3(num_workers),
                     dim3(Cfg<D, FP8, NB>::kThreads), 0, stream, p.q, p.k_cache, p.v_cache,
                     p.k_scale, p.v_scale, p.block_table, p.seq_lens, p.items, p.worker_offsets,
                     p.tile_tokens_dev, p.ws_o, p.ws_lse, p.out, p.lse_out, sh);
}

template <int D, bool FP8>
void launch_rows(const DecodeParams& p, int num_workers, hipStream_t stream) {
  if (p.rows <= 16)
    launch_one<D, FP8, 1>(p, num_workers, stream);
  else if (p.rows <= 32)
    launch_one<D, FP8, 2>(p, num_workers, stream);
  else
    launch_one<D, FP8, 4>(p, num_workers, stream);
}

}  // namespace

hipError_t launch_decode_partial(const DecodeParams& p, int head_dim, bool fp8, int num_workers,
                                 hipStream_t stream) {
  if (head_dim == 128) {
    if (fp8)
      launch_rows<128, true>(p, num_workers, stream);
    else
      launch_rows<128, false>(p, num_workers, stream);
  } else {
    if (fp8)
      launch_rows<64, true>(p, num_workers, stream);
    else
      launch_rows<64, false>(p, num_workers, stream);
  }
  return hipGetLastError();
}

}  // namespace pkv
