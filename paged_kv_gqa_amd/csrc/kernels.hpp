// Device-side parameter blocks and launchers shared by the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pkv {

// Waves per decode workgroup (one workgroup = one planner worker).
constexpr int kDecodeWaves = 4;
// Decode workgroups resident per compute unit that the default worker count assumes.
constexpr int kDecodeGroupsPerCU = 2;
// Largest M = G * Tq one work item may carry (one MFMA column block).
constexpr int kMaxRows = 16;

struct DecodeParams {
  const uint16_t* q;          // bf16 [B, Tq, Hq, D]
  const uint8_t* k_cache;     // [num_pages, Hkv, P, D] bf16 or e4m3fn
  const uint8_t* v_cache;
  const float* k_scale;       // [num_pages, Hkv] (fp8 only)
  const float* v_scale;
  const int32_t* block_table; // [B, bt_stride]
  const int32_t* seq_lens;    // [B]
  const int32_t* items;       // [N][4] (b, g, i, slot)
  const int32_t* worker_offsets;
  float* ws_o;                // [num_partials, M, D]
  float* ws_lse;              // [num_partials, M]
  int q_len, num_q_heads, num_kv_heads, group, rows, page_size, bt_stride, tile_tokens;
  float qk_scale_log2;        // softmax scale * log2(e)
};

struct CombineParams {
  const float* ws_o;
  const float* ws_lse;
  const int32_t* req_tile_base;  // [B + 1]
  uint16_t* out;                 // bf16 [B, Tq, Hq, D]
  float* lse_out;                // [B, Tq, Hq] or null
  int batch, q_len, num_q_heads, num_kv_heads, group, rows;
};

hipError_t launch_decode_partial(const DecodeParams& p, int head_dim, bool fp8,
                                 int num_workers, hipStream_t stream);

hipError_t launch_combine(const CombineParams& p, int head_dim, hipStream_t stream);

}  // namespace pkv
