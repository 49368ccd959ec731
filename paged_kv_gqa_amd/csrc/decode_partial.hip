// Split-KV partial attention for paged-KV GQA decode on gfx950.
//
// One persistent workgroup per planner worker walks its work items (b, g, i): the
// uniform KV tiles that the per-step greedy bin-packing assigned to it (HPC-Ops
// review, "How the kernels are organized around specific workload shapes"). For
// each tile it writes a softmax-normalised partial output and its log-sum-exp, to
// be merged by the combine kernel.
//
// Mapping onto CDNA4 (wave64, MFMA 16x16x32 bf16):
// - The waves of a workgroup (kDecodeWaves, eight: one workgroup per CU) split a tile
//   into 32-token chunks, round-robin.
//   A chunk is two 16-token halves; each half lies inside one page because pages
//   and tiles are multiples of 16 tokens.
// - Operands are swapped so the KV tokens fill the MFMA's 16-row side and the
//   M = G*Tq query rows of the kv head sit on the 16-column side (the "swap A/B"
//   idea of the HPC-Ops launch article, section on aligning task traits with the
//   hardware, re-derived for MFMA). Lane l owns query row n = l % 16 for the whole
//   softmax, so row max, row sum and rescale factors never leave the lane except
//   for one exchange across the four 16-lane groups.
// - K and V stream from HBM with non-temporal 16-byte loads, each wave instruction
//   reading 1 KB of whole 128-byte lines of a 16-token half: on MI355X only
//   full-line non-temporal reads reach ~6.8 TB/s on a random 4 KB page gather
//   (half-line or cached reads stop near 6.1 TB/s). Each wave stages its chunk in
//   its own LDS region (XOR-swizzled 16-byte units, so the reads below hit distinct
//   banks) and reads it back in the MFMA operand layout: lane l holds token l % 16 of
//   a half, bytes 16*(l/16) + 64*u of its row. QK^T then needs no shuffling. P.V
//   contracts over tokens, so V is transposed on the matrix core: an MFMA of the V
//   half against a 0/1 selection matrix returns, in each lane, four consecutive
//   tokens of one head dimension - the operand layout P.V needs - exactly (products
//   by 1 and sums of zeros), in fp32, then packed back to bf16.
// - FP8 (OCP e4m3fn) K/V bytes are widened to bf16 with the gfx950 conversion
//   instruction (exact). The per-(page, kv head) scales are applied outside the
//   products: the K scale multiplies the scores, the V scale multiplies P before P.V.
// - The next chunk's loads are issued into the same registers as soon as the
//   current chunk sits in LDS, so each wave keeps one chunk (16 KB for bf16) in
//   flight while its matrix and vector work runs.
#include "kernels.hpp"

#include <math.h>

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = kDecodeWaves;
constexpr int kThreads = kWaves * 64;
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
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

// Max over the four 16-lane groups (lanes n, n+16, n+32, n+48) with the gfx950
// lane-swap instructions: each swap returns the value and its partner in every lane.
__device__ __forceinline__ float group_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <int D, bool FP8>
struct Cfg {
  static constexpr int kEb = FP8 ? 1 : 2;        // bytes per KV element
  static constexpr int kSteps = D / 32;           // MFMA k-steps over the head dimension
  static constexpr int kLoads = D * kEb / 64;     // 16-byte loads per lane per half
  static constexpr int kBlocks = D / 16;          // 16-wide head-dim blocks of the output
  static constexpr int kRowBytes = D * kEb;
  static constexpr int kUnits = kRowBytes / 16;   // 16-byte units per token row
  // Rows per 256 bytes is a power of two; the swizzle uses rows / (256 / kRowBytes).
  static constexpr int kRowShift = kRowBytes == 256 ? 0 : (kRowBytes == 128 ? 1 : 2);
  // Per-wave LDS: K and V stage (2 x 32 rows) or the wave's epilogue rows, whichever
  // is larger, in 16-byte units.
  static constexpr int kStageVec = 2 * 32 * kUnits > 4 * D ? 2 * 32 * kUnits : 4 * D;
};

// Head-dimension index that k-step s, lane group gq, element e of an MFMA operand
// holds. bf16: one 16-byte load per step. fp8: one 16-byte load serves two steps.
template <bool FP8>
__device__ __forceinline__ int op_dim(int s, int gq, int e) {
  if (FP8) return 64 * (s >> 1) + 16 * gq + 8 * (s & 1) + e;
  return 32 * s + 8 * gq + e;
}

// Head-dimension index of output value v in block (s, c) of lane group gq: the
// selection matrix c picks operand column k = 16c + r, r = 4*gq + v.
template <bool FP8>
__device__ __forceinline__ int out_dim(int s, int c, int gq, int v) {
  const int k = 16 * c + 4 * gq + v;
  return op_dim<FP8>(s, k >> 3, k & 7);
}

struct ItemCtx {
  const int32_t* __restrict__ bt;  // block-table row of the request
  int64_t head_off;                // byte offset of kv head g inside a page
  int64_t page_bytes;              // bytes of one page (all heads)
  int tile_start, tile_end, page_size, row_bytes;
};

// Byte offsets of the two 16-token halves of a chunk (wave-uniform; the block-table
// reads are scalar loads). A half past the tile end re-reads half 0 (masked later).
// phys0: physical page of half 0, which holds the whole chunk when pages are 64
// tokens (fp8), so it also indexes the chunk's page scales.
struct HalfOffsets {
  int64_t off[2];
  int64_t phys0;
};

__device__ __forceinline__ HalfOffsets chunk_offsets(const ItemCtx& it, int chunk) {
  HalfOffsets r;
  const int j0 = it.tile_start + 32 * chunk;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int jh = j0 + 16 * h;
    if (jh >= it.tile_end) jh = j0;
    const int page = jh / it.page_size;
    const int64_t phys = it.bt[page];
    if (h == 0) r.phys0 = phys;
    r.off[h] = phys * it.page_bytes + it.head_off +
               static_cast<int64_t>(jh - page * it.page_size) * it.row_bytes;
  }
  return r;
}

// One chunk as loaded: [K/V][half][instruction], 16 bytes per lane each.
template <int D, bool FP8>
struct Raw {
  u32x4 r[2][2][Cfg<D, FP8>::kLoads];
};

// Issue the chunk's loads: instruction j of half h reads bytes j*1024 + 16*lane of
// the half's contiguous 16-row run (whole cache lines, non-temporal).
template <int D, bool FP8>
__device__ __forceinline__ void load_raw(Raw<D, FP8>& raw, const uint8_t* __restrict__ kc,
                                         const uint8_t* __restrict__ vc, const HalfOffsets& ho,
                                         int lane) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int j = 0; j < Cfg<D, FP8>::kLoads; ++j) {
      const int64_t off = ho.off[h] + j * 1024 + lane * 16;
      raw.r[0][h][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kc + off));
      raw.r[1][h][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vc + off));
    }
  }
}

// Stage slot of 16-byte unit `unit` of chunk row `row` (0..31) of K (kv 0) or V (1).
// The unit index is XOR-ed with the row's position among the rows that share a
// 256-byte bank window, so 16 lanes reading one unit column of 16 rows hit 16
// distinct 16-byte bank groups.
template <int D, bool FP8>
__device__ __forceinline__ int stage_slot(int kv, int row, int unit) {
  using C = Cfg<D, FP8>;
  return (kv * 32 + row) * C::kUnits + (unit ^ ((row >> C::kRowShift) & (C::kUnits - 1)));
}

template <int D, bool FP8>
__device__ __forceinline__ void stage_write(u32x4* __restrict__ st, const Raw<D, FP8>& raw, int lane) {
  using C = Cfg<D, FP8>;
#pragma unroll
  for (int kv = 0; kv < 2; ++kv)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < C::kLoads; ++j) {
        const int pos = j * 1024 + lane * 16;
        st[stage_slot<D, FP8>(kv, 16 * h + pos / C::kRowBytes, (pos % C::kRowBytes) / 16)] = raw.r[kv][h][j];
      }
}

// Read the chunk back in MFMA operand layout: lane (n, gq) takes, for each half and
// 16-byte piece u, bytes 64u + 16gq of token row n; fp8 pieces widen to two bf16
// operand steps.
template <int D, bool FP8>
__device__ __forceinline__ void stage_read(const u32x4* __restrict__ st, u32x4 (&kop)[2][D / 32],
                                           u32x4 (&vop)[2][D / 32], int n, int gq) {
  using C = Cfg<D, FP8>;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int u = 0; u < C::kLoads; ++u) {
      const u32x4 kr = st[stage_slot<D, FP8>(0, 16 * h + n, 4 * u + gq)];
      const u32x4 vr = st[stage_slot<D, FP8>(1, 16 * h + n, 4 * u + gq)];
      if constexpr (FP8) {
        kop[h][2 * u] = fp8x8_to_bf16(kr[0], kr[1]);
        kop[h][2 * u + 1] = fp8x8_to_bf16(kr[2], kr[3]);
        vop[h][2 * u] = fp8x8_to_bf16(vr[0], vr[1]);
        vop[h][2 * u + 1] = fp8x8_to_bf16(vr[2], vr[3]);
      } else {
        kop[h][u] = kr;
        vop[h][u] = vr;
      }
    }
  }
}

// Online-softmax update of one 32-token chunk. acc[blk] holds O^T for head-dim
// block blk (lane: rows 4*gq+v of the block, column n); m in log2 units.
template <int D, bool FP8>
__device__ __forceinline__ void process_chunk(u32x4 (&kop)[2][D / 32], u32x4 (&vop)[2][D / 32],
                                              const u32x4 (&qf)[D / 32],
                                              const u32x4 (&sel)[2], f32x4 (&acc)[D / 16],
                                              float& m, float& lsum, float& lexact, int j0, int lim,
                                              int tile_end, float c_qk, float v_mul, int n,
                                              int gq) {
  using C = Cfg<D, FP8>;
  // Tokens at or past the tile end may be unwritten cache memory: zero their V so
  // that a zero probability cannot meet a NaN in P.V. Lane l loaded token l % 16.
  if (j0 + 32 > tile_end) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (j0 + 16 * h + n >= tile_end) {
#pragma unroll
        for (int s = 0; s < C::kSteps; ++s) vop[h][s] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  // S^T = K . Q^T: lane (n, gq) gets tokens 16h + 4gq + v of query row n.
  f32x4 st[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    st[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) st[h] = mfma_bf16(kop[h][s], qf[s], st[h]);
  }
  float sv[8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = j0 + 16 * h + 4 * gq + v;
      sv[4 * h + v] = (j < lim) ? st[h][v] * c_qk : -INFINITY;
    }
  }
  float cm = sv[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) cm = fmaxf(cm, sv[e]);
  cm = group_max(cm);
  const float m_new = fmaxf(m, cm);
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(m - m_use);
  unsigned pk[4];
  float psum = 0.f, pexact = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float p0 = __builtin_amdgcn_exp2f(sv[2 * e] - m_use);
    const float p1 = __builtin_amdgcn_exp2f(sv[2 * e + 1] - m_use);
    const unsigned u = pack_bf16(p0, p1);
    psum += bf16_lo(u) + bf16_hi(u);   // normaliser: the rounded weights P.V sees
    pexact += p0 + p1;                 // log-sum-exp: the unrounded weights
    pk[e] = FP8 ? pack_bf16(p0 * v_mul, p1 * v_mul) : u;
  }
  lsum = lsum * alpha + psum;
  lexact = lexact * alpha + pexact;
  if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
    for (int b = 0; b < C::kBlocks; ++b) acc[b] *= alpha;
  }
  m = m_new;
  const u32x4 pb = {pk[0], pk[1], pk[2], pk[3]};

  // V^T via the selection MFMA, then O^T += V^T . P^T.
#pragma unroll
  for (int s = 0; s < C::kSteps; ++s) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      const f32x4 x0 = mfma_bf16(vop[0][s], sel[c], zero);
      const f32x4 x1 = mfma_bf16(vop[1][s], sel[c], zero);
      const u32x4 va = {pack_bf16(x0[0], x0[1]), pack_bf16(x0[2], x0[3]),
                        pack_bf16(x1[0], x1[1]), pack_bf16(x1[2], x1[3])};
      acc[2 * s + c] = mfma_bf16(va, pb, acc[2 * s + c]);
    }
  }
}

// Scalar shape arguments of the decode kernel.
struct DecodeShape {
  int q_len, num_q_heads, num_kv_heads, group, rows, page_size, bt_stride, tile_tokens;
  int request_split;  // work-list request b is part b % split of the caller's request b / split
  float qk_scale_log2;
};

// Wave-uniform description of one work item.
struct ItemInfo {
  ItemCtx it;
  int b, g, slot, L, nchunks;
};

template <int D, bool FP8>
__device__ __forceinline__ ItemInfo item_info(const int32_t* __restrict__ items,
                                              const int32_t* __restrict__ seq_lens,
                                              const int32_t* __restrict__ block_table,
                                              const DecodeShape& sh, int itx) {
  using C = Cfg<D, FP8>;
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
  r.nchunks = (r.it.tile_end - r.it.tile_start + 31) >> 5;
  return r;
}

template <int D, bool FP8>
__global__ __launch_bounds__(kThreads, kDecodeGroupsPerCU) void decode_partial_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ k_cache,
    const uint8_t* __restrict__ v_cache, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ items,
    const int32_t* __restrict__ worker_offsets, const int32_t* __restrict__ tile_dev,
    float* __restrict__ ws_o, float* __restrict__ ws_lse, const DecodeShape sh_arg) {
  using C = Cfg<D, FP8>;
  // The tile size comes from the launch, or from device memory when a device-built
  // plan chose it.
  DecodeShape sh = sh_arg;
  if (tile_dev != nullptr) sh.tile_tokens = __builtin_amdgcn_readfirstlane(tile_dev[0]);
  // Each wave's region stages its chunks and, after its last chunk of an item,
  // holds its unnormalised output rows [16][D] for the merge.
  __shared__ u32x4 lds_stage[kWaves][C::kStageVec];
  __shared__ float lds_m[kWaves][kMaxRows];
  __shared__ float lds_l[kWaves][kMaxRows];
  __shared__ float lds_le[kWaves][kMaxRows];

  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int n = lane & 15;   // query row owned by this lane (and K/V row it reads)
  const int gq = lane >> 4;  // 16-lane group
  u32x4* const my_stage = lds_stage[wid];

  // Selection matrices: sel[c] has a 1 where operand k = 16c + n (bf16 1.0 = 0x3f80).
  u32x4 sel[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int e = 16 * c + n - 8 * gq;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      sel[c][w] = (e == 2 * w ? 0x3f80u : 0u) | (e == 2 * w + 1 ? 0x3f800000u : 0u);
  }

  const int M = sh.rows;
  const int Tq = sh.q_len;
  const int G = sh.group;
  const int first = worker_offsets[blockIdx.x];
  const int last = worker_offsets[blockIdx.x + 1];

  // The wave's work is a stream of units (item, chunk): chunks wid, wid + kWaves, ... of
  // each of the worker's items. `raw` always holds the next unit's K/V in flight, and
  // `qf_next` the query fragment of its item, so an item's first chunk is loaded
  // while the previous item is still being computed and merged.
  Raw<D, FP8> raw;
  u32x4 qf_next[C::kSteps];
  // FP8: the K and V page scales of the unit in flight, loaded with its K/V so that
  // their dependent loads (block-table entry, then scale) stay off the compute path.
  float ksc_next = 1.f, vsc_next = 1.f;
  int u_itx = -1, u_c = 0;
  ItemInfo u_info;
  auto find_unit = [&](int from) {  // first unit of this wave in items >= from
    u_itx = -1;
    for (int x = from; x < last; ++x) {
      const ItemInfo inf = item_info<D, FP8>(items, seq_lens, block_table, sh, x);
      if (wid < inf.nchunks) {
        u_itx = x;
        u_c = wid;
        u_info = inf;
        return;
      }
    }
  };
  auto issue_unit = [&]() {
    if (u_itx < 0) return;
    const HalfOffsets ho = chunk_offsets(u_info.it, u_c);
    load_raw<D, FP8>(raw, k_cache, v_cache, ho, lane);
    if constexpr (FP8) {
      const int64_t sidx = ho.phys0 * sh.num_kv_heads + u_info.g;
      ksc_next = k_scale[sidx];
      vsc_next = v_scale[sidx];
    }
    if (u_c == wid) {  // first chunk of an item: fetch that item's query fragment
      if (n < M) {
        const int t = n / G;
        const int head = u_info.g * G + (n - t * G);
        // q is [B / split, Tq, split * Hq, D]; with split 1 this is [B, Tq, Hq, D].
        const int split = sh.request_split;
        const int64_t qb = (split == 1) ? u_info.b : u_info.b / split;
        const int part = (split == 1) ? 0 : u_info.b - static_cast<int>(qb) * split;
        const uint16_t* qrow =
            q + (((qb * Tq + t) * split + part) * sh.num_q_heads + head) * D;
#pragma unroll
        for (int s = 0; s < C::kSteps; ++s)
          qf_next[s] = *reinterpret_cast<const u32x4*>(qrow + op_dim<FP8>(s, gq, 0));
      } else {
#pragma unroll
        for (int s = 0; s < C::kSteps; ++s) qf_next[s] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  find_unit(first);
  issue_unit();

  for (int itx = first; itx < last; ++itx) {
    const ItemInfo cur = (u_itx == itx) ? u_info
                                        : item_info<D, FP8>(items, seq_lens, block_table, sh, itx);
    // Causal limit of row n (draft token t sees keys up to L - Tq + t); padding rows
    // n >= M see the whole tile.
    int lim = cur.it.tile_end;
    if (n < M) lim = min(lim, cur.L - Tq + n / G + 1);
    u32x4 qf[C::kSteps];
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) qf[s] = qf_next[s];

    f32x4 acc[C::kBlocks];
#pragma unroll
    for (int bl = 0; bl < C::kBlocks; ++bl) acc[bl] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, lsum = 0.f, lexact = 0.f;

    while (u_itx == itx) {
      const int c = u_c;
      stage_write<D, FP8>(my_stage, raw, lane);
      float c_qk = sh.qk_scale_log2, v_mul = 1.f;
      if constexpr (FP8) {  // this unit's scales, before issue_unit loads the next's
        c_qk = sh.qk_scale_log2 * ksc_next;
        v_mul = vsc_next;
      }
      if (c + kWaves < cur.nchunks)
        u_c = c + kWaves;
      else
        find_unit(itx + 1);
      issue_unit();
      u32x4 kop[2][C::kSteps], vop[2][C::kSteps];
      stage_read<D, FP8>(my_stage, kop, vop, n, gq);
      process_chunk<D, FP8>(kop, vop, qf, sel, acc, m, lsum, lexact, cur.it.tile_start + 32 * c, lim,
                            cur.it.tile_end, c_qk, v_mul, n, gq);
    }

    // Wave result -> LDS: row max, full row sums, unnormalised O.
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    lexact += __shfl_xor(lexact, 16);
    lexact += __shfl_xor(lexact, 32);
    if (gq == 0) {
      lds_m[wid][n] = m;
      lds_l[wid][n] = lsum;
      lds_le[wid][n] = lexact;
    }
    float* const my_rows = reinterpret_cast<float*>(my_stage);   // [16][D]
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int v = 0; v < 4; ++v) my_rows[n * D + out_dim<FP8>(s, c, gq, v)] = acc[2 * s + c][v];
    __syncthreads();

    // Merge the waves' partial softmax states and write the item's partial.
    float* wo = ws_o + static_cast<int64_t>(cur.slot) * M * D;
    for (int e = tid; e < M * D; e += kThreads) {
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
          num += f * reinterpret_cast<const float*>(lds_stage[w])[r * D + d];
          den += f * lds_l[w][r];
        }
        o = num / den;
      }
      wo[e] = o;
    }
    if (tid < M) {
      float mx = lds_m[0][tid];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, lds_m[w][tid]);
      float lse = -INFINITY;
      if (mx != -INFINITY) {
        float den = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) den += __builtin_amdgcn_exp2f(lds_m[w][tid] - mx) * lds_le[w][tid];
        lse = (mx + __builtin_amdgcn_logf(den)) * kLn2;
      }
      ws_lse[static_cast<int64_t>(cur.slot) * M + tid] = lse;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_decode_partial(const DecodeParams& p, int head_dim, bool fp8, int num_workers,
                                 hipStream_t stream) {
  const dim3 grid(num_workers), block(kThreads);
  const DecodeShape sh = {p.q_len,     p.num_q_heads, p.num_kv_heads, p.group,
                          p.rows,      p.page_size,   p.bt_stride,    p.tile_tokens,
                          p.request_split, p.qk_scale_log2};
#define PKV_LAUNCH(DIM, F8)                                                                   \
  hipLaunchKernelGGL((decode_partial_kernel<DIM, F8>), grid, block, 0, stream, p.q, p.k_cache, \
                     p.v_cache, p.k_scale, p.v_scale, p.block_table, p.seq_lens, p.items,     \
                     p.worker_offsets, p.tile_tokens_dev, p.ws_o, p.ws_lse, sh)
  if (head_dim == 128) {
    if (fp8)
      PKV_LAUNCH(128, true);
    else
      PKV_LAUNCH(128, false);
  } else {
    if (fp8)
      PKV_LAUNCH(64, true);
    else
      PKV_LAUNCH(64, false);
  }
#undef PKV_LAUNCH
  return hipGetLastError();
}

}  // namespace pkv
