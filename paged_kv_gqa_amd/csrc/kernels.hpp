// Device-side parameter blocks and launchers shared by the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pkv {

// Waves per decode workgroup (one workgroup = one planner worker).
constexpr int kDecodeWaves = 8;
// Decode workgroups resident per compute unit that the default worker count assumes.
constexpr int kDecodeGroupsPerCU = 1;
// Largest M = G * Tq one work item may carry (four MFMA column blocks).
constexpr int kMaxRows = 64;

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
  const int32_t* tile_tokens_dev;  // if set, T is read from here instead of tile_tokens
  int q_len, num_q_heads, num_kv_heads, group, rows, page_size, bt_stride, tile_tokens;
  int request_split;          // work-list request b = part b % split of request b / split
  float qk_scale_log2;        // softmax scale * log2(e)
  uint16_t* out;              // bf16 [B, Tq, Hq, D] or null: single-tile requests' final rows
  float* lse_out;             // [B, Tq, Hq] or null
};

struct CombineParams {
  const float* ws_o;
  const float* ws_lse;
  const int32_t* req_tile_base;  // [B + 1]
  uint16_t* out;                 // bf16 [B, Tq, Hq, D]
  float* lse_out;                // [B, Tq, Hq] or null
  int batch, q_len, num_q_heads, num_kv_heads, group, rows;
  int request_split;             // as in DecodeParams
};

struct BlockSparseParams {
  const int32_t* block_table;    // [B, bt_stride]
  const int32_t* seq_lens;       // [B]
  const uint8_t* block_mask;     // [B, Hkv, mask_stride]
  int32_t* bt_out;               // [B * Hkv, bt_stride]: phys * Hkv + g of attended pages
  int32_t* seq_lens_out;         // [B * Hkv]
  int batch, num_kv_heads, q_len, page_size, bt_stride, mask_stride;
};

hipError_t launch_block_sparse_compact(const BlockSparseParams& p, hipStream_t stream);

// Largest head dimension of any kernel.
constexpr int kMaxHeadDim = 128;

struct KvAppendParams {
  const uint16_t* k_new;         // bf16 [B, Tq, Hkv, D]
  const uint16_t* v_new;
  const uint16_t* q;             // bf16 [B, Tq, Hq, D], rotated into q_out (may alias)
  uint16_t* q_out;               // or null
  const float* rope_cos;         // [max_pos, D/2] or null (no rotation)
  const float* rope_sin;
  uint8_t* k_cache;              // [num_pages, Hkv, P, D] bf16 or e4m3fn
  uint8_t* v_cache;
  float* k_scale;                // [num_pages, Hkv] (fp8)
  float* v_scale;
  const int32_t* block_table;    // [B, bt_stride]
  const int32_t* seq_lens;       // [B], counting the new tokens
  int batch, q_len, num_q_heads, num_kv_heads, head_dim, page_size, bt_stride;
  bool fp8;
};

hipError_t launch_kv_append(const KvAppendParams& p, hipStream_t stream);

// Query tokens per prefill work item, and query heads one item covers at most.
constexpr int kPrefillTileTokens = 64;
constexpr int kPrefillMaxHeadsPerItem = 4;

struct PrefillParams {
  const uint16_t* q;             // bf16 [total, Hq, D]
  const int32_t* cu_q;           // [B + 1]
  const int32_t* kv_lens;        // [B]
  const int32_t* block_table;    // [B, bt_stride]
  const int32_t* items;          // [num_items][4] (b, g, head group, first token)
  const uint8_t* k_cache;        // [num_pages, Hkv, P, D] bf16 or e4m3fn
  const uint8_t* v_cache;
  const float* k_scale;          // [num_pages, Hkv] (fp8)
  const float* v_scale;
  uint16_t* out;                 // bf16 [total, Hq, D]
  float* lse;                    // [total, Hq] or null
  int64_t num_items;
  int batch, num_q_heads, num_kv_heads, page_size, bt_stride;
  float scale;
};

hipError_t launch_prefill(const PrefillParams& p, int head_dim, bool fp8, int heads_per_item,
                          hipStream_t stream);

// Device planner limits: one thread per worker, the requests sorted in LDS.
constexpr int kMaxDevicePlanWorkers = 1024;
constexpr int kMaxDevicePlanBatch = 4096;
// Largest fixed tile (tokens) a device-built plan takes (its keys are 32-bit).
constexpr int kMaxDevicePlanTile = 1 << 18;
// Candidate tiles of the automatic rule: quantum << c, c < num_candidates <= 16.
constexpr int kMaxDevicePlanCandidates = 16;

// Status codes the device planner writes (the pkv_status values).
constexpr int PKV_DEV_OK = 0;
constexpr int PKV_DEV_ERR_UNSUPPORTED = -2;
constexpr int PKV_DEV_ERR_WORKSPACE = -4;
constexpr int PKV_DEV_ERR_SEQ = -6;

struct DevicePlanParams {
  const int32_t* seq_lens;    // device [B]
  int32_t* items;             // [max_items][4]
  int32_t* worker_offsets;    // [W + 1]
  int32_t* req_tile_base;     // [B + 1]
  int32_t* info;              // [4] status, T, N, most items on one worker
  long long* cand_est;        // scratch [kMaxDevicePlanCandidates]
  int32_t* cand_status;       // scratch [kMaxDevicePlanCandidates]
  int2* scratch_assign;       // scratch [candidates][B * Hkv]: (worker, position) of
                              // each remainder item
  char* cand_plans;           // scratch: one plan per candidate tile (automatic tile)
  long long cand_stride, cand_offsets_off, cand_rtb_off, cand_info_off;
  long long max_items;
  long long tile_tokens;      // 0 = automatic
  long long kv_bytes_per_token;
  int batch, q_len, num_kv_heads, num_workers, quantum, num_candidates, rows, head_dim;
};

hipError_t launch_plan_device(const DevicePlanParams& p, hipStream_t stream);

hipError_t launch_decode_partial(const DecodeParams& p, int head_dim, bool fp8,
                                 int num_workers, hipStream_t stream);

hipError_t launch_combine(const CombineParams& p, int head_dim, hipStream_t stream);

}  // namespace pkv
