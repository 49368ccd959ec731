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
//   accumulator is rescaled rarely; the row's probability sum l is kept in fp32 (each
//   lane sums its keys; the row's four lanes are added at the end) and is the output's
//   normaliser and the log-sum-exp's argument.
// - P enters the matrix cores as bf16. Where a block's largest probability may be a
//   large share of the row's sum (a row's first block, rows that see few keys, sharp
//   rows), the low bf16 part p - bf16(p) is multiplied into V as well, so the weights
//   that dominate an output are carried to about 16 bits.
// - O^T += V^T . P^T: the two S^T halves of a lane pack into the 8 k-values of P^T's
//   B operand directly (keys 4gq + 0..3 and 16 + 4gq + 0..3). V is staged row-major;
//   gfx950's transposing LDS read (ds_read_b64_tr_b16: in each 16-lane group, lanes
//   4k..4k+3 address row k of a 4 x 16 tile of 16-bit values and lane i receives
//   column i) gives lane (n, gq) the four keys 4gq + 0..3 (then 16 + 4gq + 0..3) of
//   head dim 16bl + n, i.e. V^T's A operand, in two reads.
// - Blocks are software-pipelined: while block kb's exponentials run, the wave reads
//   block kb + 1's K operands and issues its score products, so matrix, vector and LDS
//   work overlap inside one wave. The stage is triple-buffered with one barrier per
//   block; the K/V loads for the stage run one block ahead, the block-table entries
//   one block earlier still.
// FP8 (e4m3fn) K/V bytes are widened to bf16 exactly when staged, once per workgroup
// and spread over all of its threads; each 16-key half of a block lies in one page,
// whose K scale multiplies that half's scores and whose V scale its P.
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
  static constexpr int kRowBytes = D * kEb;               // one K or V row in the cache
  static constexpr int kSteps = D / 32;                   // MFMA k-steps over D
  static constexpr int kDimBlocks = D / 16;               // 16-dim blocks of O^T
};

// Head dimension of k-step s, lane group gq, element e of the S^T operands.
__device__ __forceinline__ int op_dim(int s, int gq, int e) { return 32 * s + 8 * gq + e; }

// LDS (bytes), bf16 rows: K rows [32] of stride 2D + 16 (16 lanes reading one 16-byte
// unit of rows n = 0..15 hit disjoint bank groups) and V rows [32] of stride 2D + 32
// (the four rows of a transposing read hit disjoint bank groups). Each lane reads at
// one base address plus constant offsets.
template <int D>
struct Stage {
  static constexpr int kKStride = 2 * D + 16;
  static constexpr int kVStride = 2 * D + 32;
  alignas(16) uint8_t k[kBlockKeys * kKStride];
  alignas(16) uint8_t v[kBlockKeys * kVStride];
};

// A block's K (and V) bytes split into equal units, one per thread where the
// workgroup has enough threads: 16-byte units for bf16; for fp8, whose block holds half
// the bytes, units of 8 (or 4) bytes when 16-byte units would leave threads idle, so
// that every wave shares the widening to bf16.
template <int D, bool FP8, int NT>
struct Units {
  static constexpr int kRowBytes = PCfg<D, FP8>::kRowBytes;
  static constexpr int kFit = kBlockKeys * kRowBytes / NT;  // bytes per thread
  static constexpr int kBytes = !FP8 || kFit >= 16 ? 16 : (kFit >= 8 ? 8 : 4);
  static constexpr int kWords = kBytes / 4;
  static constexpr int kRowUnits = kRowBytes / kBytes;     // units per cache row
  static constexpr int kBlockUnits = kBlockKeys * kRowUnits;
  static constexpr int kPerThread = (kBlockUnits + NT - 1) / NT;
};

template <int N>
using uvec = unsigned __attribute__((ext_vector_type(N)));

// This thread's units of one block, with each unit's page walk: the physical page and
// in-page row of the next block to load, and the logical page and in-page row of the
// block after it (advanced by 32 keys per block, so no division by the page size).
template <int D, bool FP8, int NT>
struct BlockRegs {
  using U = Units<D, FP8, NT>;
  static constexpr int kUnits = U::kPerThread;
  uvec<U::kWords> k[kUnits];
  uvec<U::kWords> v[kUnits];
  int phys[kUnits], load_off[kUnits];
  int walk_page[kUnits], walk_off[kUnits];
};

template <int D, bool FP8, int NT>
__device__ __forceinline__ void walk_init(BlockRegs<D, FP8, NT>& r, int page_size, int tid) {
  using U = Units<D, FP8, NT>;
#pragma unroll
  for (int i = 0; i < U::kPerThread; ++i) {
    const int row = (tid + NT * i) / U::kRowUnits;  // < 32 for staging units
    r.walk_page[i] = row / page_size;
    r.walk_off[i] = row % page_size;
  }
}

// Look up the physical pages of the walked block (last_page clamps rows past the
// sequence end, which are not loaded) and advance the walk by one block.
template <int D, bool FP8, int NT>
__device__ __forceinline__ void block_pages(BlockRegs<D, FP8, NT>& r, const int32_t* __restrict__ bt,
                                            int last_page, int page_size, int tid) {
  using U = Units<D, FP8, NT>;
#pragma unroll
  for (int i = 0; i < U::kPerThread; ++i) {
    const bool staged = tid + NT * i < U::kBlockUnits;
    r.phys[i] = staged ? bt[min(r.walk_page[i], last_page)] : 0;
    r.load_off[i] = r.walk_off[i];
    int off = r.walk_off[i] + kBlockKeys, page = r.walk_page[i];
    while (off >= page_size) {  // at most twice (page_size >= 16)
      off -= page_size;
      ++page;
    }
    r.walk_off[i] = off;
    r.walk_page[i] = page;
  }
}

// Load block kb's K and V units of this thread (zeros past the sequence end).
template <int D, bool FP8, int NT>
__device__ __forceinline__ void load_block(BlockRegs<D, FP8, NT>& r, const uint8_t* __restrict__ kc,
                                           const uint8_t* __restrict__ vc, int64_t page_bytes,
                                           int64_t head_off, int kb, int L, int tid) {
  using U = Units<D, FP8, NT>;
  using V = uvec<U::kWords>;
#pragma unroll
  for (int i = 0; i < U::kPerThread; ++i) {
    const int u = tid + NT * i;
    const int row = u / U::kRowUnits, unit = u % U::kRowUnits;
    if (u < U::kBlockUnits && kb * kBlockKeys + row < L) {
      const int64_t off = static_cast<int64_t>(r.phys[i]) * page_bytes + head_off +
                          r.load_off[i] * U::kRowBytes + U::kBytes * unit;
      r.k[i] = *reinterpret_cast<const V*>(kc + off);
      r.v[i] = *reinterpret_cast<const V*>(vc + off);
    } else {
      r.k[i] = V{};
      r.v[i] = V{};
    }
  }
}

// K and V rows into LDS as bf16 (fp8 widened exactly), row-major.
template <int D, bool FP8, int NT>
__device__ __forceinline__ void stage_block(Stage<D>& st, const BlockRegs<D, FP8, NT>& r, int tid) {
  using U = Units<D, FP8, NT>;
  using S = Stage<D>;
#pragma unroll
  for (int i = 0; i < U::kPerThread; ++i) {
    const int u = tid + NT * i;
    if (u >= U::kBlockUnits) break;
    const int row = u / U::kRowUnits, unit = u % U::kRowUnits;
    uint8_t* kd = st.k + row * S::kKStride;
    uint8_t* vd = st.v + row * S::kVStride;
    if constexpr (FP8) {  // each dword of 4 codes -> 8 bytes of bf16
      uvec<2 * U::kWords> kw, vw;
#pragma unroll
      for (int w = 0; w < U::kWords; ++w) {
        const u32x2 ka = fp8x4_to_bf16(r.k[i][w]), va = fp8x4_to_bf16(r.v[i][w]);
        kw[2 * w] = ka[0];
        kw[2 * w + 1] = ka[1];
        vw[2 * w] = va[0];
        vw[2 * w + 1] = va[1];
      }
      *reinterpret_cast<uvec<2 * U::kWords>*>(kd + 2 * U::kBytes * unit) = kw;
      *reinterpret_cast<uvec<2 * U::kWords>*>(vd + 2 * U::kBytes * unit) = vw;
    } else {
      *reinterpret_cast<u32x4*>(kd + 16 * unit) = r.k[i];
      *reinterpret_cast<u32x4*>(vd + 16 * unit) = r.v[i];
    }
  }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposing LDS read of four 16-bit values (see the header).
__device__ __forceinline__ u32x2 read_tr16(const uint8_t* p) {
  const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, x);
}

// A load whose address is the same in every lane, through the scalar data cache (the
// constant address space): it is waited for apart from the vector loads in flight.
template <typename T>
__device__ __forceinline__ T load_uniform(const T* ptr, int64_t i) {
  return ((const __attribute__((address_space(4))) T*)(ptr))[i];
}

__device__ __forceinline__ float max8(const float (&a)[8]) {
  return fmaxf(fmaxf(fmaxf(a[0], a[1]), a[2]),
               fmaxf(fmaxf(fmaxf(a[3], a[4]), a[5]), fmaxf(a[6], a[7])));
}

// Online-softmax state of one query row and head: running maximum m (log2 units;
// -inf before the first block), negm = -m (+inf before the first block, so that the
// first block always raises m), and this lane's share of the probability sum (the
// row's four lanes are added at the end).
struct RowState {
  float m, negm, l;
};

// K operands of one staged block: key 16h + n, dims op_dim(s, gq, 0..7).
template <int D>
__device__ __forceinline__ void read_k(const Stage<D>& st, int n, int gq,
                                       u32x4 (&kop)[2][PCfg<D, false>::kSteps]) {
  using S = Stage<D>;
  const uint8_t* kbase = st.k + n * S::kKStride + 16 * gq;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int s = 0; s < PCfg<D, false>::kSteps; ++s)
      kop[h][s] = *reinterpret_cast<const u32x4*>(kbase + 16 * h * S::kKStride + 64 * s);
}

// Raw scores S^T = K . Q^T of one block: lane (n, gq) gets keys 16h + 4gq + v of query n.
template <int D, int HPW>
__device__ __forceinline__ void score_block(const u32x4 (&kop)[2][PCfg<D, false>::kSteps],
                                            const u32x4 (&qf)[HPW][PCfg<D, false>::kSteps],
                                            f32x4 (&sacc)[HPW][2]) {
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sacc[hh][h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < PCfg<D, false>::kSteps; ++s) sacc[hh][h] = mfma_bf16(kop[h][s], qf[hh][s], sacc[hh][h]);
    }
}

// V^T operands of one staged block: dims 16bl + n, keys 4gq + 0..3 then 16 + 4gq + 0..3
// (two transposing reads; lane (n, gq) addresses row 4gq + n / 4, dims 16bl + 4 (n % 4)).
template <int D>
__device__ __forceinline__ void read_v(const Stage<D>& st, int n, int gq,
                                       u32x4 (&vop)[PCfg<D, false>::kDimBlocks]) {
  using S = Stage<D>;
  const uint8_t* vbase = st.v + (4 * gq + (n >> 2)) * S::kVStride + 8 * (n & 3);
#pragma unroll
  for (int bl = 0; bl < PCfg<D, false>::kDimBlocks; ++bl) {
    const u32x2 lo = read_tr16(vbase + 32 * bl);
    const u32x2 hi = read_tr16(vbase + 16 * S::kVStride + 32 * bl);
    vop[bl] = u32x4{lo[0], lo[1], hi[0], hi[1]};
  }
}

// Online softmax of one block's scores for this wave's 16 query tokens and HPW heads
// (lane (n, gq): query n), first part. diag: the block reaches past some token's
// position, so keys j > pos are masked. Per key the exponent argument a = s c - m is
// formed; the row maximum needs a cross-lane reduction only when some lane sees a > 8
// (m must be raised), a rare branch that rescales the accumulators. Out: the
// arguments and each head's largest argument on this lane.
template <int D, bool FP8, int HPW>
__device__ __forceinline__ void softmax_args(bool diag, int j0, int pos, int gq,
                                             f32x4 (&sacc)[HPW][2],
                                             f32x4 (&acc)[HPW][PCfg<D, FP8>::kDimBlocks],
                                             RowState (&rs)[HPW], const float (&c)[2],
                                             float (&arg)[HPW][8], float (&amax)[HPW]) {
  using C = PCfg<D, FP8>;
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
  // Exponent arguments a = s c - m (masked keys: -inf, since c > 0) and their lane max.
  bool raise = false;
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
#pragma unroll
    for (int e = 0; e < 8; ++e) arg[hh][e] = fmaf(sacc[hh][e >> 2][e & 3], c[e >> 2], rs[hh].negm);
    amax[hh] = max8(arg[hh]);
    raise |= amax[hh] > kRescaleSlack;
  }
  if (__builtin_amdgcn_ballot_w64(raise)) {
    __asm__ volatile("");  // keeps this rare path a branch (not a select on every block)
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      float raw[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) raw[e] = sacc[hh][e >> 2][e & 3];
      // The row's block maximum in log2 units (c > 0 in both halves).
      const float mc = group_max(fmaxf(fmaxf(fmaxf(raw[0], raw[1]), fmaxf(raw[2], raw[3])) * c[0],
                                       fmaxf(fmaxf(raw[4], raw[5]), fmaxf(raw[6], raw[7])) * c[1]));
      // Lanes whose row keeps its maximum multiply by 1 (no divergent branch, so the
      // accumulators are scaled in place).
      const bool up = mc > rs[hh].m + kRescaleSlack;  // the same in the row's four lanes
      const float alpha = up ? __builtin_amdgcn_exp2f(rs[hh].m - mc) : 1.f;  // m = -inf: 0
#pragma unroll
      for (int bl = 0; bl < C::kDimBlocks; ++bl) acc[hh][bl] *= alpha;
      rs[hh].l *= alpha;
      rs[hh].m = up ? mc : rs[hh].m;
      rs[hh].negm = up ? -mc : rs[hh].negm;
#pragma unroll
      for (int e = 0; e < 8; ++e) arg[hh][e] = fmaf(raw[e], c[e >> 2], rs[hh].negm);
      amax[hh] = max8(arg[hh]);
    }
  }
}

// Second part: probabilities p = 2^a (times the V scale for FP8), this lane's sums, P^T
// packed to bf16 in ph, and whether the low bf16 part of P must be multiplied into V
// as well. The low-part test uses this lane's largest p and sum: if a row's largest p
// exceeds a quarter of the row's sum after the block, the lane that holds it sees
// 3 p > (its sum before the block).
template <bool FP8, int HPW>
__device__ __forceinline__ void softmax_probs(const float (&arg)[HPW][8], const float (&amax)[HPW],
                                              RowState (&rs)[HPW], const float (&v_mul)[2],
                                              float (&pv)[HPW][8], u32x4 (&ph)[HPW], bool& low) {
  low = false;
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    low |= kLowPartTest * __builtin_amdgcn_exp2f(amax[hh]) > rs[hh].l;
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pv[hh][e] = __builtin_amdgcn_exp2f(arg[hh][e]);
      sum += pv[hh][e];
    }
    rs[hh].l += sum;
    if constexpr (FP8) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[hh][e] *= v_mul[e >> 2];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) ph[hh][e] = pack_bf16(pv[hh][2 * e], pv[hh][2 * e + 1]);
  }
}

// O^T += V^T . P^T for one block, plus the low bf16 part of P where asked.
template <int D, int HPW>
__device__ __forceinline__ void pv_block(const u32x4 (&vop)[PCfg<D, false>::kDimBlocks],
                                         const float (&pv)[HPW][8], const u32x4 (&ph)[HPW], bool low,
                                         f32x4 (&acc)[HPW][PCfg<D, false>::kDimBlocks]) {
  constexpr int kDimBlocks = PCfg<D, false>::kDimBlocks;
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
    for (int bl = 0; bl < kDimBlocks; ++bl) acc[hh][bl] = mfma_bf16(vop[bl], ph[hh], acc[hh][bl]);
  if (__builtin_amdgcn_ballot_w64(low)) {
    // The low part goes through a fresh accumulator and is added in place, so the
    // accumulators keep their registers whichever way this branch goes.
    __asm__ volatile("");
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      u32x4 pl;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pl[e] = pack_bf16(pv[hh][2 * e] - bf16_lo(ph[hh][e]), pv[hh][2 * e + 1] - bf16_hi(ph[hh][e]));
#pragma unroll
      for (int bl = 0; bl < kDimBlocks; ++bl)
        acc[hh][bl] += mfma_bf16(vop[bl], pl, f32x4{0.f, 0.f, 0.f, 0.f});
    }
  }
}

template <int D, bool FP8, int GWI>
__global__ __launch_bounds__(WaveCfg<GWI>::kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_kernel(const PrefillParams p) {
  using C = PCfg<D, FP8>;
  using W = WaveCfg<GWI>;
  constexpr int HPW = W::kHeadsPerWave;
  constexpr int NT = W::kThreads;
  __shared__ Stage<D> stage[3];
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

  const int32_t* __restrict__ bt = p.block_table + static_cast<int64_t>(b) * p.bt_stride;
  const int64_t head_off = static_cast<int64_t>(g) * p.page_size * C::kRowBytes;
  const int64_t page_bytes = static_cast<int64_t>(p.num_kv_heads) * p.page_size * C::kRowBytes;

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
      qf[hh][s] = valid ? *reinterpret_cast<const u32x4*>(qrow + op_dim(s, gq, 0))
                        : u32x4{0u, 0u, 0u, 0u};
      qf[hh][s] ^= u32x4{qflip, qflip, qflip, qflip};
    }
  }

  f32x4 acc[HPW][C::kDimBlocks];
  RowState rs[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
#pragma unroll
    for (int bl = 0; bl < C::kDimBlocks; ++bl) acc[hh][bl] = f32x4{0.f, 0.f, 0.f, 0.f};
    rs[hh] = RowState{-INFINITY, INFINITY, 0.f};
  }

  // Triple-buffered stage, one barrier per block. In step kb the workgroup stages block
  // kb + 1 and each wave then reads block kb + 1's K operands and block kb's V operands,
  // so block kb + 1's score products are issued around block kb's softmax and the LDS
  // reads overlap vector and matrix work. A buffer written in step kb last held block
  // kb - 2, whose reads all ended before the barrier of step kb - 1. The K/V loads run
  // one block ahead of the staging, the block-table entries (and FP8 page scales) one
  // block ahead of the loads that use them.
  using R = BlockRegs<D, FP8, NT>;
  const int last_page = (L - 1) / p.page_size;
  R regs;
  walk_init<D, FP8, NT>(regs, p.page_size, tid);
  block_pages<D, FP8, NT>(regs, bt, last_page, p.page_size, tid);
  load_block<D, FP8, NT>(regs, p.k_cache, p.v_cache, page_bytes, head_off, 0, L, tid);
  stage_block<D, FP8, NT>(stage[0], regs, tid);
  if (nblocks > 1) {
    block_pages<D, FP8, NT>(regs, bt, last_page, p.page_size, tid);
    load_block<D, FP8, NT>(regs, p.k_cache, p.v_cache, page_bytes, head_off, 1, L, tid);
    if (nblocks > 2) block_pages<D, FP8, NT>(regs, bt, last_page, p.page_size, tid);
  }
  __syncthreads();
  f32x4 sacc[HPW][2] = {};
  if (wave_blocks > 0) {
    u32x4 kop[2][C::kSteps];
    read_k<D>(stage[0], n, gq, kop);
    score_block<D, HPW>(kop, qf, sacc);
  }
  // FP8 page scales of the block being computed, one per 16-key half (a half lies in
  // one page; the two may differ when pages are shorter than 32 keys or not aligned to
  // blocks), and the physical pages of the next block's halves.
  // With pages a multiple of 32 keys a block lies in one page: its second half takes
  // the first half's scales, with no second lookup.
  // The logical page (and row in it) of each half's first key is advanced by one block
  // per step, so no division by the page size per block; pages past the last clamp to
  // it (keys past the length are masked).
  float ksc[2] = {1.f, 1.f}, vsc[2] = {1.f, 1.f};
  int scale_page[2] = {0, 0};
  int hpg[2] = {0, 0}, hrow[2] = {0, 0};  // logical page and row of half h's first key
  auto half_phys = [&](int h) { return load_uniform(bt, min(hpg[h], last_page)); };
  auto half_advance = [&](int h) {  // by one block of keys
    hrow[h] += kBlockKeys;
    while (hrow[h] >= p.page_size) {
      hrow[h] -= p.page_size;
      ++hpg[h];
    }
  };
  const int scale_halves = (p.page_size % kBlockKeys == 0) ? 1 : 2;
  if constexpr (FP8) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h < scale_halves) {
        hpg[h] = (16 * h) / p.page_size;
        hrow[h] = 16 * h - hpg[h] * p.page_size;
        const int64_t sidx = static_cast<int64_t>(half_phys(h)) * p.num_kv_heads + g;
        ksc[h] = load_uniform(p.k_scale, sidx);
        vsc[h] = load_uniform(p.v_scale, sidx);
        half_advance(h);
        scale_page[h] = half_phys(h);
      }
    }
  }
  int cur = 0, nxt = 1;  // stage buffers of blocks kb and kb + 1
  for (int kb = 0; kb < nblocks; ++kb) {
    float ksc_next[2] = {1.f, 1.f}, vsc_next[2] = {1.f, 1.f};
    if (kb + 1 < nblocks) {
      stage_block<D, FP8, NT>(stage[nxt], regs, tid);
      __syncthreads();
      if (kb + 2 < nblocks) {
        load_block<D, FP8, NT>(regs, p.k_cache, p.v_cache, page_bytes, head_off, kb + 2, L, tid);
        if (kb + 3 < nblocks) block_pages<D, FP8, NT>(regs, bt, last_page, p.page_size, tid);
      }
      if constexpr (FP8) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (h < scale_halves) {
            const int64_t sidx = static_cast<int64_t>(scale_page[h]) * p.num_kv_heads + g;
            ksc_next[h] = load_uniform(p.k_scale, sidx);
            vsc_next[h] = load_uniform(p.v_scale, sidx);
            if (kb + 2 < nblocks) {
              half_advance(h);
              scale_page[h] = half_phys(h);
            }
          }
        }
      }
    }
    if (kb < wave_blocks) {
      const int j0 = kb * kBlockKeys;
      const bool diag = j0 + kBlockKeys - 1 > wave_first_pos;
      // c > 0 keeps masked keys at a = -inf (a zero scale acts as the smallest normal one).
      // With one scale lookup per block the second half takes the first half's scales.
      const float ksc1 = scale_halves == 2 ? ksc[1] : ksc[0];
      const float vs[2] = {vsc[0], scale_halves == 2 ? vsc[1] : vsc[0]};
      const float c[2] = {fmaxf(qk_log2 * ksc[0], 1.17549435e-38f),
                          fmaxf(qk_log2 * ksc1, 1.17549435e-38f)};
      float pv[HPW][8];
      u32x4 ph[HPW];
      bool low;
      u32x4 vop[C::kDimBlocks];
      float arg[HPW][8], amax[HPW];
      softmax_args<D, FP8, HPW>(diag, j0, pos, gq, sacc, acc, rs, c, arg, amax);
      // The next block's scores, issued among this block's exponentials (unused after
      // the wave's last block, whose next buffer then holds an earlier block).
      {
        u32x4 kop[2][C::kSteps];
        read_k<D>(stage[nxt], n, gq, kop);
        score_block<D, HPW>(kop, qf, sacc);
      }
      softmax_probs<FP8, HPW>(arg, amax, rs, vs, pv, ph, low);
      read_v<D>(stage[cur], n, gq, vop);
      pv_block<D, HPW>(vop, pv, ph, low, acc);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ksc[h] = ksc_next[h];
      vsc[h] = vsc_next[h];
    }
    cur = nxt;
    nxt = nxt == 2 ? 0 : nxt + 1;
  }

  // Rows to the output: lane (n, gq) holds dims 16bl + 4gq + v of query n; the row's
  // probability sum is the sum of its four lanes' shares.
  float lrow[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) lrow[hh] = group_sum(rs[hh].l);
  if (!valid) return;
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const float inv = lrow[hh] > 0.f ? 1.f / lrow[hh] : 0.f;
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
      p.lse[row] = lrow[hh] > 0.f ? (rs[hh].m + __builtin_amdgcn_logf(lrow[hh])) * kLn2 : -INFINITY;
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
