// C ABI of libpkv.so (declared in include/pkv.h): argument validation, status
// reporting, the host planner entry points and the kernel launches.
#include "pkv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstddef>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "planner.hpp"
#include "status.hpp"
#include "validate.hpp"

namespace {

thread_local std::string g_last_error;

}  // namespace

int pkv::fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

namespace {

using pkv::fail;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr float kLog2e = 1.44269504088896341f;

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Shape rules shared by every entry point.
int check_shape(int q_len, int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                int kv_format) {
  if (kv_format != PKV_KV_BF16 && kv_format != PKV_KV_FP8_E4M3FN)
    return fail(PKV_ERR_INVALID_ARG, "kv_format %d is not a pkv_kv_format", kv_format);
  if (num_q_heads < 1 || num_kv_heads < 1 || q_len < 1 || head_dim < 1 || page_size < 1)
    return fail(PKV_ERR_INVALID_ARG, "sizes must be positive (q_len %d, heads %d/%d, D %d, P %d)",
                q_len, num_q_heads, num_kv_heads, head_dim, page_size);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
  if (page_size % 16 != 0)
    return fail(PKV_ERR_UNSUPPORTED, "page_size %d is not a multiple of 16", page_size);
  if (num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_UNSUPPORTED, "num_q_heads %d is not a multiple of num_kv_heads %d",
                num_q_heads, num_kv_heads);
  if (q_len > 4) return fail(PKV_ERR_UNSUPPORTED, "q_len %d (supported: 1..4)", q_len);
  const int rows = (num_q_heads / num_kv_heads) * q_len;
  if (rows > pkv::kMaxRows)
    return fail(PKV_ERR_UNSUPPORTED, "group size x q_len = %d rows per kv head (max %d)", rows,
                pkv::kMaxRows);
  return PKV_OK;
}

int check_seq_lens(int batch, const int32_t* seq_lens_h, int q_len) {
  for (int b = 0; b < batch; ++b) {
    const int32_t L = seq_lens_h[b];
    if (L < 1 || L < q_len)
      return fail(PKV_ERR_SEQ, "seq_lens[%d] = %d (needs >= max(1, q_len = %d))", b, L, q_len);
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported shape or format";
    case PKV_ERR_ALIGNMENT: return "device pointer not 16-byte aligned";
    case PKV_ERR_WORKSPACE: return "workspace too small";
    case PKV_ERR_HIP: return "HIP runtime error";
    case PKV_ERR_SEQ: return "sequence length shorter than the query tokens or zero";
    default: return "unknown status";
  }
}

const char* pkv_last_error(void) { return g_last_error.c_str(); }

int pkv_plan_query(int batch, const int32_t* seq_lens_h, int q_len, int num_q_heads,
                   int num_kv_heads, int head_dim, int page_size, int kv_format, int tile_tokens,
                   int num_workers, int32_t* tile_tokens_out, int64_t* num_items_out,
                   int64_t* num_partials_out) {
  if (batch < 0) return fail(PKV_ERR_INVALID_ARG, "batch %d < 0", batch);
  if ((batch > 0 && seq_lens_h == nullptr) || tile_tokens_out == nullptr ||
      num_items_out == nullptr || num_partials_out == nullptr)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (num_workers < 1) return fail(PKV_ERR_INVALID_ARG, "num_workers %d < 1", num_workers);
  if (tile_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "tile_tokens %d < 0", tile_tokens);
  int st = check_shape(q_len, num_q_heads, num_kv_heads, head_dim, page_size, kv_format);
  if (st != PKV_OK) return st;
  st = check_seq_lens(batch, seq_lens_h, q_len);
  if (st != PKV_OK) return st;
  const bool fp8 = kv_format == PKV_KV_FP8_E4M3FN;
  const int64_t quantum = pkv::tile_quantum(page_size, fp8);
  int64_t T = tile_tokens;
  if (T == 0) {
    T = pkv::auto_tile_tokens(batch, seq_lens_h, q_len, num_q_heads, num_kv_heads, head_dim,
                              page_size, fp8, num_workers);
  } else if (T % quantum != 0) {
    return fail(PKV_ERR_UNSUPPORTED, "tile_tokens %d is not a multiple of the quantum %lld",
                tile_tokens, static_cast<long long>(quantum));
  }
  const pkv::PlanStats s = pkv::plan_stats(batch, seq_lens_h, num_kv_heads, T, num_workers);
  if (s.num_items > INT32_MAX / 4)
    return fail(PKV_ERR_UNSUPPORTED, "plan of %lld items is too large",
                static_cast<long long>(s.num_items));
  *tile_tokens_out = static_cast<int32_t>(T);
  *num_items_out = s.num_items;
  *num_partials_out = s.num_items;
  return PKV_OK;
}

int pkv_plan(int batch, const int32_t* seq_lens_h, int q_len, int num_kv_heads, int tile_tokens,
             int num_workers, int32_t* items_h, int32_t* worker_offsets_h,
             int32_t* req_tile_base_h) {
  if (batch < 0) return fail(PKV_ERR_INVALID_ARG, "batch %d < 0", batch);
  if ((batch > 0 && (seq_lens_h == nullptr || items_h == nullptr)) ||
      worker_offsets_h == nullptr || req_tile_base_h == nullptr)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (num_workers < 1) return fail(PKV_ERR_INVALID_ARG, "num_workers %d < 1", num_workers);
  if (tile_tokens < 1) return fail(PKV_ERR_INVALID_ARG, "tile_tokens %d < 1", tile_tokens);
  if (num_kv_heads < 1 || q_len < 1)
    return fail(PKV_ERR_INVALID_ARG, "num_kv_heads %d and q_len %d must be positive", num_kv_heads,
                q_len);
  const int st = check_seq_lens(batch, seq_lens_h, q_len);
  if (st != PKV_OK) return st;
  pkv::build_plan(batch, seq_lens_h, num_kv_heads, tile_tokens, num_workers, items_h,
                  worker_offsets_h, req_tile_base_h);
  return PKV_OK;
}

int pkv_default_num_workers(int device, int kv_format, int head_dim, int* out) {
  if (out == nullptr) return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (kv_format != PKV_KV_BF16 && kv_format != PKV_KV_FP8_E4M3FN)
    return fail(PKV_ERR_INVALID_ARG, "kv_format %d is not a pkv_kv_format", kv_format);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
  int cus = 0;
  const hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess)
    return fail(PKV_ERR_HIP, "hipDeviceGetAttribute(device %d): %s", device, hipGetErrorString(e));
  *out = cus * pkv::kDecodeGroupsPerCU;
  return PKV_OK;
}

int pkv_workspace_bytes(int64_t num_partials, int rows_per_partial, int head_dim, size_t* out) {
  if (out == nullptr) return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (num_partials < 0 || rows_per_partial < 1 || head_dim < 1)
    return fail(PKV_ERR_INVALID_ARG, "bad sizes (partials %lld, rows %d, D %d)",
                static_cast<long long>(num_partials), rows_per_partial, head_dim);
  const size_t o = static_cast<size_t>(num_partials) * rows_per_partial * head_dim * 4;
  const size_t l = static_cast<size_t>(num_partials) * rows_per_partial * 4;
  *out = align256(o) + align256(l);
  return PKV_OK;
}

int pkv_decode_partial(const pkv_decode_args* a, void* stream) {
  if (a == nullptr) return fail(PKV_ERR_INVALID_ARG, "null args");
  // ABI 1 callers pass the struct without its last field.
  constexpr size_t kV1Size = offsetof(pkv_decode_args, tile_tokens_dev);
  if (a->struct_size < kV1Size)
    return fail(PKV_ERR_INVALID_ARG, "struct_size %zu < %zu", a->struct_size, kV1Size);
  const bool has_tile_dev =
      a->struct_size >= offsetof(pkv_decode_args, tile_tokens_dev) + sizeof(a->tile_tokens_dev);
  const bool has_split =
      a->struct_size >= offsetof(pkv_decode_args, request_split) + sizeof(a->request_split);
  const bool has_out = a->struct_size >= offsetof(pkv_decode_args, lse_out) + sizeof(a->lse_out);
  void* const direct_out = has_out ? a->out : nullptr;
  float* const direct_lse = has_out ? a->lse_out : nullptr;
  const int32_t* tile_dev = has_tile_dev ? a->tile_tokens_dev : nullptr;
  const int split = (has_split && a->request_split != 0) ? a->request_split : 1;
  int st = check_shape(a->q_len, a->num_q_heads, a->num_kv_heads, a->head_dim, a->page_size,
                       a->kv_format);
  if (st != PKV_OK) return st;
  if (a->batch < 0 || a->num_items < 0 || a->num_partials < a->num_items || a->num_pages < 0)
    return fail(PKV_ERR_INVALID_ARG, "negative size or num_partials < num_items");
  if (a->num_workers < 1) return fail(PKV_ERR_INVALID_ARG, "num_workers %d < 1", a->num_workers);
  if (split < 1 || a->batch % split != 0)
    return fail(PKV_ERR_INVALID_ARG, "request_split %d does not divide batch %d", split, a->batch);
  const bool fp8 = a->kv_format == PKV_KV_FP8_E4M3FN;
  const int64_t quantum = pkv::tile_quantum(a->page_size, fp8);
  if (tile_dev == nullptr && (a->tile_tokens < 1 || a->tile_tokens % quantum != 0))
    return fail(PKV_ERR_UNSUPPORTED, "tile_tokens %d is not a positive multiple of %lld",
                a->tile_tokens, static_cast<long long>(quantum));
  if (tile_dev != nullptr && !aligned(tile_dev, 4))
    return fail(PKV_ERR_ALIGNMENT, "tile_tokens_dev misaligned");
  if (a->num_items == 0) return PKV_OK;
  if (a->batch < 1 || a->num_pages < 1)
    return fail(PKV_ERR_INVALID_ARG, "work items given for an empty batch or cache");
  const int max_pages = static_cast<int>(pkv::ceil_div(INT32_MAX, a->page_size));
  if (a->bt_stride < 1 || a->bt_stride > max_pages)
    return fail(PKV_ERR_INVALID_ARG, "bt_stride %d out of range", a->bt_stride);
  if (!a->q || !a->k_cache || !a->v_cache || !a->block_table || !a->seq_lens || !a->items ||
      !a->worker_offsets || !a->req_tile_base || !a->workspace)
    return fail(PKV_ERR_INVALID_ARG, "null device pointer");
  if (fp8 != (a->k_scale != nullptr) || fp8 != (a->v_scale != nullptr))
    return fail(PKV_ERR_INVALID_ARG, "k_scale/v_scale must be given exactly for fp8 KV");
  if (!aligned(a->q, 16) || !aligned(a->k_cache, 16) || !aligned(a->v_cache, 16) ||
      !aligned(a->workspace, 16))
    return fail(PKV_ERR_ALIGNMENT, "q, k_cache, v_cache and workspace must be 16-byte aligned");
  if (!aligned(a->block_table, 4) || !aligned(a->seq_lens, 4) || !aligned(a->items, 16) ||
      !aligned(a->worker_offsets, 4) || (fp8 && (!aligned(a->k_scale, 4) || !aligned(a->v_scale, 4))))
    return fail(PKV_ERR_ALIGNMENT, "int32/fp32 arrays misaligned (items need 16 bytes)");
  const int rows = (a->num_q_heads / a->num_kv_heads) * a->q_len;
  size_t need = 0;
  pkv_workspace_bytes(a->num_partials, rows, a->head_dim, &need);
  if (a->workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", a->workspace_bytes, need);
  if (!std::isfinite(a->scale)) return fail(PKV_ERR_INVALID_ARG, "scale is not finite");
  if (direct_out == nullptr && direct_lse != nullptr)
    return fail(PKV_ERR_INVALID_ARG, "lse_out without out");
  if (direct_out != nullptr && split != 1)
    return fail(PKV_ERR_INVALID_ARG, "out needs request_split 1");
  if ((direct_out != nullptr && !aligned(direct_out, 16)) ||
      (direct_lse != nullptr && !aligned(direct_lse, 4)))
    return fail(PKV_ERR_ALIGNMENT, "out must be 16-byte aligned, lse_out 4-byte");

  pkv::DecodeParams p;
  p.q = static_cast<const uint16_t*>(a->q);
  p.k_cache = static_cast<const uint8_t*>(a->k_cache);
  p.v_cache = static_cast<const uint8_t*>(a->v_cache);
  p.k_scale = a->k_scale;
  p.v_scale = a->v_scale;
  p.block_table = a->block_table;
  p.seq_lens = a->seq_lens;
  p.items = a->items;
  p.worker_offsets = a->worker_offsets;
  p.ws_o = static_cast<float*>(a->workspace);
  p.ws_lse = reinterpret_cast<float*>(static_cast<char*>(a->workspace) +
                                      align256(static_cast<size_t>(a->num_partials) * rows *
                                               a->head_dim * 4));
  p.q_len = a->q_len;
  p.num_q_heads = a->num_q_heads;
  p.num_kv_heads = a->num_kv_heads;
  p.group = a->num_q_heads / a->num_kv_heads;
  p.rows = rows;
  p.page_size = a->page_size;
  p.bt_stride = a->bt_stride;
  p.tile_tokens = a->tile_tokens;
  p.tile_tokens_dev = tile_dev;
  p.request_split = split;
  p.qk_scale_log2 = a->scale * kLog2e;
  p.out = static_cast<uint16_t*>(direct_out);
  p.lse_out = direct_lse;
  if (pkv::validate_enabled()) {
    st = pkv::validate_decode(a, tile_dev, static_cast<hipStream_t>(stream));
    if (st != PKV_OK) return st;
  }
  const hipError_t e = pkv::launch_decode_partial(p, a->head_dim, fp8, a->num_workers,
                                                  static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "decode_partial launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

namespace {

// Scratch of pkv_plan_device: candidate estimates and statuses, the remainder-item
// placements of each plan being built and, for the automatic tile, one whole plan
// per candidate tile.
struct DevicePlanLayout {
  size_t assign_off, plans_off, plan_stride, offsets_off, rtb_off, info_off, total;
};

DevicePlanLayout device_plan_layout(int batch, int Hkv, int W, int64_t max_items, int ncand) {
  DevicePlanLayout l;
  const size_t assign = 8 * static_cast<size_t>(batch) * Hkv;
  l.assign_off = 256;
  l.plans_off = align256(l.assign_off + assign * (ncand > 0 ? ncand : 1));
  l.offsets_off = align256(16 * static_cast<size_t>(max_items > 0 ? max_items : 1));
  l.rtb_off = l.offsets_off + align256(4 * (static_cast<size_t>(W) + 1));
  l.info_off = l.rtb_off + align256(4 * (static_cast<size_t>(batch) + 1));
  l.plan_stride = l.info_off + 256;
  l.total = ncand > 0 ? l.plans_off + l.plan_stride * ncand : l.assign_off + assign;
  return l;
}

}  // namespace

int pkv_plan_device_scratch_bytes(int batch, int num_kv_heads, int page_size, int kv_format,
                                  int tile_tokens, int num_workers, int64_t max_items,
                                  size_t* out) {
  if (out == nullptr) return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (batch < 0 || num_kv_heads < 1 || page_size < 1 || tile_tokens < 0 || num_workers < 1 ||
      max_items < 0)
    return fail(PKV_ERR_INVALID_ARG, "size out of range (batch %d, kv heads %d, P %d, T %d, W %d, "
                "max_items %lld)", batch, num_kv_heads, page_size, tile_tokens, num_workers,
                static_cast<long long>(max_items));
  if (kv_format != PKV_KV_BF16 && kv_format != PKV_KV_FP8_E4M3FN)
    return fail(PKV_ERR_INVALID_ARG, "kv_format %d is not a pkv_kv_format", kv_format);
  const int ncand = tile_tokens == 0
                        ? pkv::auto_tile_candidates(pkv::tile_quantum(page_size, kv_format != 0))
                        : 0;
  *out = device_plan_layout(batch, num_kv_heads, num_workers, max_items, ncand).total;
  return PKV_OK;
}

int pkv_plan_device(const int32_t* seq_lens, int batch, int q_len, int num_q_heads,
                    int num_kv_heads, int head_dim, int page_size, int kv_format,
                    int tile_tokens, int num_workers, int64_t max_items, int32_t* items,
                    int32_t* worker_offsets, int32_t* req_tile_base, int32_t* info,
                    void* scratch, size_t scratch_bytes, void* stream) {
  int st = check_shape(q_len, num_q_heads, num_kv_heads, head_dim, page_size, kv_format);
  if (st != PKV_OK) return st;
  if (batch < 0 || num_workers < 1 || tile_tokens < 0 || max_items < 0)
    return fail(PKV_ERR_INVALID_ARG, "negative size (batch %d, W %d, T %d, max_items %lld)", batch,
                num_workers, tile_tokens, static_cast<long long>(max_items));
  if (batch > pkv::kMaxDevicePlanBatch || num_workers > pkv::kMaxDevicePlanWorkers ||
      max_items > INT32_MAX / 4 || tile_tokens > pkv::kMaxDevicePlanTile)
    return fail(PKV_ERR_UNSUPPORTED, "device plan limits: batch %d (max %d), W %d (max %d), "
                "max_items %lld, tile_tokens %d (max %d)", batch, pkv::kMaxDevicePlanBatch,
                num_workers, pkv::kMaxDevicePlanWorkers, static_cast<long long>(max_items),
                tile_tokens, pkv::kMaxDevicePlanTile);
  const bool fp8 = kv_format == PKV_KV_FP8_E4M3FN;
  const int64_t quantum = pkv::tile_quantum(page_size, fp8);
  if (tile_tokens % quantum != 0)
    return fail(PKV_ERR_UNSUPPORTED, "tile_tokens %d is not a multiple of the quantum %lld",
                tile_tokens, static_cast<long long>(quantum));
  if ((batch > 0 && seq_lens == nullptr) || items == nullptr || worker_offsets == nullptr ||
      req_tile_base == nullptr || info == nullptr || scratch == nullptr)
    return fail(PKV_ERR_INVALID_ARG, "null device pointer");
  if (!aligned(items, 16) || !aligned(scratch, 16) || !aligned(seq_lens, 4) ||
      !aligned(worker_offsets, 4) || !aligned(req_tile_base, 4) || !aligned(info, 4))
    return fail(PKV_ERR_ALIGNMENT, "items and scratch need 16 bytes, int32 arrays 4");
  const int ncand = tile_tokens == 0 ? pkv::auto_tile_candidates(quantum) : 0;
  if (ncand > pkv::kMaxDevicePlanCandidates)
    return fail(PKV_ERR_UNSUPPORTED, "too many candidate tiles");
  const DevicePlanLayout lay = device_plan_layout(batch, num_kv_heads, num_workers, max_items, ncand);
  if (scratch_bytes < lay.total)
    return fail(PKV_ERR_WORKSPACE, "scratch %zu bytes < %zu needed", scratch_bytes, lay.total);

  pkv::DevicePlanParams p;
  p.seq_lens = seq_lens;
  p.items = items;
  p.worker_offsets = worker_offsets;
  p.req_tile_base = req_tile_base;
  p.info = info;
  p.cand_est = static_cast<long long*>(scratch);
  p.cand_status = reinterpret_cast<int32_t*>(static_cast<char*>(scratch) +
                                             8 * pkv::kMaxDevicePlanCandidates);
  p.scratch_assign = reinterpret_cast<int2*>(static_cast<char*>(scratch) + lay.assign_off);
  p.cand_plans = static_cast<char*>(scratch) + lay.plans_off;
  p.cand_stride = static_cast<long long>(lay.plan_stride);
  p.cand_offsets_off = static_cast<long long>(lay.offsets_off);
  p.cand_rtb_off = static_cast<long long>(lay.rtb_off);
  p.cand_info_off = static_cast<long long>(lay.info_off);
  p.max_items = max_items;
  p.tile_tokens = tile_tokens;
  p.kv_bytes_per_token = 2LL * head_dim * (fp8 ? 1 : 2);
  p.batch = batch;
  p.q_len = q_len;
  p.num_kv_heads = num_kv_heads;
  p.num_workers = num_workers;
  p.quantum = static_cast<int>(quantum);
  p.num_candidates = pkv::auto_tile_candidates(quantum);
  p.rows = (num_q_heads / num_kv_heads) * q_len;
  p.head_dim = head_dim;
  const hipError_t e = pkv::launch_plan_device(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "plan_device launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

int pkv_block_sparse_compact(const int32_t* block_table, const int32_t* seq_lens,
                             const uint8_t* block_mask, int batch, int num_kv_heads,
                             int q_len, int page_size, int bt_stride, int mask_stride,
                             int64_t num_pages, int32_t* bt_out, int32_t* seq_lens_out,
                             void* stream) {
  if (batch < 0 || num_kv_heads < 1 || q_len < 1 || page_size < 1 || bt_stride < 1 ||
      mask_stride < bt_stride || num_pages < 0)
    return fail(PKV_ERR_INVALID_ARG, "sizes out of range (batch %d, kv heads %d, q_len %d, P %d, "
                "bt_stride %d, mask_stride %d)", batch, num_kv_heads, q_len, page_size, bt_stride,
                mask_stride);
  if (num_pages * num_kv_heads > INT32_MAX)
    return fail(PKV_ERR_UNSUPPORTED, "num_pages x num_kv_heads = %lld does not fit int32",
                static_cast<long long>(num_pages * num_kv_heads));
  if (batch == 0) return PKV_OK;
  if (!block_table || !seq_lens || !block_mask || !bt_out || !seq_lens_out)
    return fail(PKV_ERR_INVALID_ARG, "null device pointer");
  if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(bt_out, 4) ||
      !aligned(seq_lens_out, 4))
    return fail(PKV_ERR_ALIGNMENT, "int32 arrays must be 4-byte aligned");
  pkv::BlockSparseParams p;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.block_mask = block_mask;
  p.bt_out = bt_out;
  p.seq_lens_out = seq_lens_out;
  p.batch = batch;
  p.num_kv_heads = num_kv_heads;
  p.q_len = q_len;
  p.page_size = page_size;
  p.bt_stride = bt_stride;
  p.mask_stride = mask_stride;
  if (pkv::validate_enabled()) {
    const int vst = pkv::validate_block_sparse(block_table, seq_lens, batch, page_size, bt_stride,
                                               num_pages, static_cast<hipStream_t>(stream));
    if (vst != PKV_OK) return vst;
  }
  const hipError_t e = pkv::launch_block_sparse_compact(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "block_sparse_compact launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

int pkv_block_sparse_lengths(int batch, const int32_t* seq_lens_h, const uint8_t* block_mask_h,
                             int num_kv_heads, int q_len, int page_size, int mask_stride,
                             int32_t* lengths_out_h) {
  if (batch < 0 || num_kv_heads < 1 || q_len < 1 || page_size < 1 || mask_stride < 1)
    return fail(PKV_ERR_INVALID_ARG, "sizes out of range");
  if (batch > 0 && (!seq_lens_h || !block_mask_h || !lengths_out_h))
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  const int st = check_seq_lens(batch, seq_lens_h, q_len);
  if (st != PKV_OK) return st;
  for (int b = 0; b < batch; ++b) {
    const int L = seq_lens_h[b];
    const int n = static_cast<int>(pkv::ceil_div(L, page_size));
    if (n > mask_stride)
      return fail(PKV_ERR_INVALID_ARG, "request %d has %d pages, mask_stride is %d", b, n,
                  mask_stride);
    const int first_query_page = (L - q_len) / page_size;
    for (int g = 0; g < num_kv_heads; ++g) {
      const uint8_t* m = block_mask_h + (static_cast<int64_t>(b) * num_kv_heads + g) * mask_stride;
      // Nonzero bytes among the pages before the query pages, eight at a time: a
      // byte's high bit of ((x & 0x7f..) + 0x7f..) | x is set iff the byte is nonzero.
      int attended = 0, pg = 0;
      for (; pg + 8 <= first_query_page; pg += 8) {
        uint64_t x;
        std::memcpy(&x, m + pg, 8);
        const uint64_t lo7 = 0x7f7f7f7f7f7f7f7fULL;
        attended += __builtin_popcountll((((x & lo7) + lo7) | x) & ~lo7);
      }
      for (; pg < first_query_page; ++pg) attended += (m[pg] != 0);
      lengths_out_h[b * num_kv_heads + g] = L - (first_query_page - attended) * page_size;
    }
  }
  return PKV_OK;
}

int pkv_kv_append(const pkv_kv_append_args* a, void* stream) {
  if (a == nullptr) return fail(PKV_ERR_INVALID_ARG, "null args");
  if (a->struct_size < sizeof(pkv_kv_append_args))
    return fail(PKV_ERR_INVALID_ARG, "struct_size %zu < %zu", a->struct_size,
                sizeof(pkv_kv_append_args));
  int st = check_shape(a->q_len, a->num_q_heads, a->num_kv_heads, a->head_dim, a->page_size,
                       a->kv_format);
  if (st != PKV_OK) return st;
  if (a->batch < 0 || a->num_pages < 0 || a->bt_stride < 1)
    return fail(PKV_ERR_INVALID_ARG, "sizes out of range (batch %d, pages %lld, bt_stride %d)",
                a->batch, static_cast<long long>(a->num_pages), a->bt_stride);
  if (a->batch == 0) return PKV_OK;
  const bool fp8 = a->kv_format == PKV_KV_FP8_E4M3FN;
  if (!a->k_new || !a->v_new || !a->k_cache || !a->v_cache || !a->block_table || !a->seq_lens)
    return fail(PKV_ERR_INVALID_ARG, "null device pointer");
  if (fp8 != (a->k_scale != nullptr) || fp8 != (a->v_scale != nullptr))
    return fail(PKV_ERR_INVALID_ARG, "k_scale/v_scale must be given exactly for fp8 KV");
  if ((a->rope_cos == nullptr) != (a->rope_sin == nullptr))
    return fail(PKV_ERR_INVALID_ARG, "rope_cos and rope_sin go together");
  if ((a->q == nullptr) != (a->q_out == nullptr))
    return fail(PKV_ERR_INVALID_ARG, "q and q_out go together");
  if (a->rope_cos != nullptr &&
      static_cast<int64_t>(a->max_pos) < static_cast<int64_t>(a->bt_stride) * a->page_size)
    return fail(PKV_ERR_INVALID_ARG, "max_pos %d < bt_stride x page_size", a->max_pos);
  if (!aligned(a->k_new, 16) || !aligned(a->v_new, 16) || !aligned(a->k_cache, 16) ||
      !aligned(a->v_cache, 16) || (a->q && (!aligned(a->q, 16) || !aligned(a->q_out, 16))) ||
      !aligned(a->block_table, 4) || !aligned(a->seq_lens, 4) ||
      (a->rope_cos && (!aligned(a->rope_cos, 4) || !aligned(a->rope_sin, 4))) ||
      (fp8 && (!aligned(a->k_scale, 4) || !aligned(a->v_scale, 4))))
    return fail(PKV_ERR_ALIGNMENT, "rows and caches need 16 bytes, tables 4");
  pkv::KvAppendParams p;
  p.k_new = static_cast<const uint16_t*>(a->k_new);
  p.v_new = static_cast<const uint16_t*>(a->v_new);
  p.q = static_cast<const uint16_t*>(a->q);
  p.q_out = static_cast<uint16_t*>(a->q_out);
  p.rope_cos = a->rope_cos;
  p.rope_sin = a->rope_sin;
  p.k_cache = static_cast<uint8_t*>(a->k_cache);
  p.v_cache = static_cast<uint8_t*>(a->v_cache);
  p.k_scale = a->k_scale;
  p.v_scale = a->v_scale;
  p.block_table = a->block_table;
  p.seq_lens = a->seq_lens;
  p.batch = a->batch;
  p.q_len = a->q_len;
  p.num_q_heads = a->num_q_heads;
  p.num_kv_heads = a->num_kv_heads;
  p.head_dim = a->head_dim;
  p.page_size = a->page_size;
  p.bt_stride = a->bt_stride;
  p.fp8 = fp8;
  if (pkv::validate_enabled()) {
    const int vst = pkv::validate_kv_append(a, static_cast<hipStream_t>(stream));
    if (vst != PKV_OK) return vst;
  }
  const hipError_t e = pkv::launch_kv_append(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "kv_append launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

namespace {

int prefill_heads_per_item(int num_q_heads, int num_kv_heads) {
  const int G = num_q_heads / num_kv_heads;
  return G < pkv::kPrefillMaxHeadsPerItem ? G : pkv::kPrefillMaxHeadsPerItem;
}

int check_prefill_heads(int num_q_heads, int num_kv_heads) {
  if (num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_UNSUPPORTED, "num_q_heads %d is not a multiple of num_kv_heads %d",
                num_q_heads, num_kv_heads);
  const int G = num_q_heads / num_kv_heads;
  if (G != 1 && G != 2 && G % 4 != 0)
    return fail(PKV_ERR_UNSUPPORTED, "group size %d (supported: 1, 2, multiples of 4)", G);
  return PKV_OK;
}

}  // namespace

int pkv_prefill_plan_size(int batch, const int32_t* q_lens_h, int num_q_heads, int num_kv_heads,
                          int64_t* num_items_out) {
  if (batch < 0 || num_items_out == nullptr || (batch > 0 && q_lens_h == nullptr))
    return fail(PKV_ERR_INVALID_ARG, "bad arguments");
  const int st = check_prefill_heads(num_q_heads, num_kv_heads);
  if (st != PKV_OK) return st;
  const int groups = (num_q_heads / num_kv_heads) / prefill_heads_per_item(num_q_heads, num_kv_heads);
  int64_t n = 0;
  for (int b = 0; b < batch; ++b) {
    if (q_lens_h[b] < 0) return fail(PKV_ERR_INVALID_ARG, "q_lens[%d] = %d < 0", b, q_lens_h[b]);
    n += pkv::ceil_div(q_lens_h[b], pkv::kPrefillTileTokens);
  }
  *num_items_out = n * num_kv_heads * groups;
  return PKV_OK;
}

int pkv_prefill_plan(int batch, const int32_t* q_lens_h, const int32_t* kv_lens_h, int num_q_heads,
                     int num_kv_heads, int32_t* items_h) {
  int64_t total = 0;
  int st = pkv_prefill_plan_size(batch, q_lens_h, num_q_heads, num_kv_heads, &total);
  if (st != PKV_OK) return st;
  if (total > 0 && (kv_lens_h == nullptr || items_h == nullptr))
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (total > INT32_MAX / 4) return fail(PKV_ERR_UNSUPPORTED, "too many prefill items");
  const int groups = (num_q_heads / num_kv_heads) / prefill_heads_per_item(num_q_heads, num_kv_heads);
  struct Item {
    int64_t keys;
    int32_t b, g, hg, t0;
  };
  std::vector<Item> v;
  v.reserve(static_cast<size_t>(total));
  for (int b = 0; b < batch; ++b) {
    const int n = q_lens_h[b], L = kv_lens_h[b];
    if (L < n) return fail(PKV_ERR_INVALID_ARG, "kv_lens[%d] = %d < q_len %d", b, L, n);
    for (int t0 = 0; t0 < n; t0 += pkv::kPrefillTileTokens) {
      const int64_t keys = static_cast<int64_t>(L - n) + std::min(t0 + pkv::kPrefillTileTokens, n);
      for (int g = 0; g < num_kv_heads; ++g)
        for (int hg = 0; hg < groups; ++hg) v.push_back({keys, b, g, hg, t0});
    }
  }
  // Heaviest first; the stable sort keeps (b, g, group, tile) order among equals.
  std::stable_sort(v.begin(), v.end(), [](const Item& x, const Item& y) { return x.keys > y.keys; });
  for (size_t i = 0; i < v.size(); ++i) {
    items_h[4 * i + 0] = v[i].b;
    items_h[4 * i + 1] = v[i].g;
    items_h[4 * i + 2] = v[i].hg;
    items_h[4 * i + 3] = v[i].t0;
  }
  return PKV_OK;
}

int pkv_prefill(const pkv_prefill_args* a, void* stream) {
  if (a == nullptr) return fail(PKV_ERR_INVALID_ARG, "null args");
  if (a->struct_size < sizeof(pkv_prefill_args))
    return fail(PKV_ERR_INVALID_ARG, "struct_size %zu < %zu", a->struct_size, sizeof(pkv_prefill_args));
  if (a->kv_format != PKV_KV_BF16 && a->kv_format != PKV_KV_FP8_E4M3FN)
    return fail(PKV_ERR_INVALID_ARG, "kv_format %d is not a pkv_kv_format", a->kv_format);
  if (a->head_dim != 64 && a->head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", a->head_dim);
  if (a->page_size < 16 || a->page_size % 16 != 0)
    return fail(PKV_ERR_UNSUPPORTED, "page_size %d is not a multiple of 16", a->page_size);
  const bool fp8 = a->kv_format == PKV_KV_FP8_E4M3FN;
  int st = check_prefill_heads(a->num_q_heads, a->num_kv_heads);
  if (st != PKV_OK) return st;
  if (a->batch < 0 || a->num_items < 0 || a->num_pages < 0 || a->bt_stride < 1)
    return fail(PKV_ERR_INVALID_ARG, "sizes out of range");
  if (a->num_items == 0) return PKV_OK;
  if (a->num_items > INT32_MAX) return fail(PKV_ERR_UNSUPPORTED, "too many prefill items");
  if (!a->q || !a->cu_q || !a->kv_lens || !a->block_table || !a->items || !a->k_cache ||
      !a->v_cache || !a->out)
    return fail(PKV_ERR_INVALID_ARG, "null device pointer");
  if (fp8 != (a->k_scale != nullptr) || fp8 != (a->v_scale != nullptr))
    return fail(PKV_ERR_INVALID_ARG, "k_scale/v_scale must be given exactly for fp8 KV");
  if (!std::isfinite(a->scale)) return fail(PKV_ERR_INVALID_ARG, "scale is not finite");
  if (!aligned(a->q, 16) || !aligned(a->out, 16) || !aligned(a->k_cache, 16) ||
      !aligned(a->v_cache, 16) || !aligned(a->items, 16) || !aligned(a->cu_q, 4) ||
      !aligned(a->kv_lens, 4) || !aligned(a->block_table, 4) || (a->lse && !aligned(a->lse, 4)))
    return fail(PKV_ERR_ALIGNMENT, "q, out, caches and items need 16 bytes");
  pkv::PrefillParams p;
  p.q = static_cast<const uint16_t*>(a->q);
  p.cu_q = a->cu_q;
  p.kv_lens = a->kv_lens;
  p.block_table = a->block_table;
  p.items = a->items;
  p.k_cache = static_cast<const uint8_t*>(a->k_cache);
  p.v_cache = static_cast<const uint8_t*>(a->v_cache);
  p.k_scale = a->k_scale;
  p.v_scale = a->v_scale;
  p.out = static_cast<uint16_t*>(a->out);
  p.lse = a->lse;
  p.num_items = a->num_items;
  p.batch = a->batch;
  p.num_q_heads = a->num_q_heads;
  p.num_kv_heads = a->num_kv_heads;
  p.page_size = a->page_size;
  p.bt_stride = a->bt_stride;
  p.scale = a->scale;
  if (pkv::validate_enabled()) {
    st = pkv::validate_prefill(a, prefill_heads_per_item(a->num_q_heads, a->num_kv_heads),
                               static_cast<hipStream_t>(stream));
    if (st != PKV_OK) return st;
  }
  const hipError_t e = pkv::launch_prefill(p, a->head_dim, fp8,
                                           prefill_heads_per_item(a->num_q_heads, a->num_kv_heads),
                                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

static_assert(pkv::PKV_DEV_OK == PKV_OK && pkv::PKV_DEV_ERR_SEQ == PKV_ERR_SEQ &&
                  pkv::PKV_DEV_ERR_UNSUPPORTED == PKV_ERR_UNSUPPORTED &&
                  pkv::PKV_DEV_ERR_WORKSPACE == PKV_ERR_WORKSPACE,
              "device status codes are the pkv_status values");
static_assert(8 * pkv::kMaxDevicePlanCandidates + 4 * pkv::kMaxDevicePlanCandidates <= 256,
              "candidate scratch fits the first 256 bytes");

int pkv_combine(const void* workspace, size_t workspace_bytes, int64_t num_partials,
                const int32_t* req_tile_base, int batch, int q_len, int num_q_heads,
                int num_kv_heads, int head_dim, void* out, float* lse_out, void* stream) {
  return pkv_combine_split(workspace, workspace_bytes, num_partials, req_tile_base, batch, q_len,
                           num_q_heads, num_kv_heads, head_dim, 1, out, lse_out, stream);
}

int pkv_combine_split(const void* workspace, size_t workspace_bytes, int64_t num_partials,
                      const int32_t* req_tile_base, int batch, int q_len, int num_q_heads,
                      int num_kv_heads, int head_dim, int request_split, void* out,
                      float* lse_out, void* stream) {
  const int st = check_shape(q_len, num_q_heads, num_kv_heads, head_dim, 16, PKV_KV_BF16);
  if (st != PKV_OK) return st;
  if (batch < 0 || num_partials < 0)
    return fail(PKV_ERR_INVALID_ARG, "batch %d / num_partials %lld negative", batch,
                static_cast<long long>(num_partials));
  if (request_split < 1 || batch % request_split != 0)
    return fail(PKV_ERR_INVALID_ARG, "request_split %d does not divide batch %d", request_split,
                batch);
  if (batch == 0) return PKV_OK;
  if (static_cast<int64_t>(batch) * q_len * num_q_heads > INT32_MAX / 64)
    return fail(PKV_ERR_UNSUPPORTED, "too many output rows");
  if (!workspace || !req_tile_base || !out) return fail(PKV_ERR_INVALID_ARG, "null device pointer");
  if (!aligned(workspace, 16) || !aligned(out, 16) || !aligned(req_tile_base, 4) ||
      (lse_out && !aligned(lse_out, 4)))
    return fail(PKV_ERR_ALIGNMENT, "workspace and out must be 16-byte aligned");
  const int rows = (num_q_heads / num_kv_heads) * q_len;
  size_t need = 0;
  pkv_workspace_bytes(num_partials, rows, head_dim, &need);
  if (workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  pkv::CombineParams p;
  p.ws_o = static_cast<const float*>(workspace);
  p.ws_lse = reinterpret_cast<const float*>(
      static_cast<const char*>(workspace) +
      align256(static_cast<size_t>(num_partials) * rows * head_dim * 4));
  p.req_tile_base = req_tile_base;
  p.out = static_cast<uint16_t*>(out);
  p.lse_out = lse_out;
  p.batch = batch;
  p.q_len = q_len;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = num_q_heads / num_kv_heads;
  p.rows = rows;
  p.request_split = request_split;
  if (pkv::validate_enabled()) {
    const int vst = pkv::validate_combine(req_tile_base, batch, num_kv_heads, num_partials,
                                          static_cast<hipStream_t>(stream));
    if (vst != PKV_OK) return vst;
  }
  const hipError_t e = pkv::launch_combine(p, head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "combine launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

}  // extern "C"
