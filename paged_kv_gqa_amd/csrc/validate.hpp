// Synchronous checks of the device-resident arguments that the kernels take on
// trust, run when the environment sets PKV_VALIDATE (non-empty, not "0"). Each
// drains the call's stream, copies the lengths, block-table rows and work lists to
// the host and checks them there, so a bad index or length comes back as a
// pkv_status (with pkv_last_error) instead of reaching a kernel. Debugging aid: every
// checked call waits for the GPU.
#pragma once

#include <hip/hip_runtime.h>

#include "pkv.h"

namespace pkv {

bool validate_enabled();

// While one of these lives, validate_enabled() is false on this thread (entry points
// that must not allocate, even host memory, run without the checks).
class ValidateOff {
 public:
  ValidateOff();
  ~ValidateOff();
  ValidateOff(const ValidateOff&) = delete;
  ValidateOff& operator=(const ValidateOff&) = delete;

 private:
  bool prev_;
};

// seq_lens in [max(1, q_len), bt_stride * P], the block-table entries of every used
// page in [0, num_pages), and the work list: worker offsets ascending from 0 to at
// most num_items, n_b = ceil(L_b / T) tiles per request in req_tile_base, and every
// listed item (b, g, i, slot) inside the batch with slot = Hkv * req_tile_base[b] +
// g * n_b + i < num_partials. An empty work list (an error plan of the device
// planner) is accepted as such. tile_dev: the device tile, or null.
int validate_decode(const pkv_decode_args* a, const int32_t* tile_dev, hipStream_t stream);

// req_tile_base ascending from 0 with Hkv * req_tile_base[batch] <= num_partials.
int validate_combine(const int32_t* req_tile_base, int batch, int num_kv_heads,
                     int64_t num_partials, hipStream_t stream);

// cu_q ascending from 0, kv_lens[b] >= the request's query count and <= bt_stride *
// P, the used block-table entries in [0, num_pages), every item inside the batch.
int validate_prefill(const pkv_prefill_args* a, int heads_per_item, hipStream_t stream);

// seq_lens in [q_len, bt_stride * P], used block-table entries in [0, num_pages).
int validate_kv_append(const pkv_kv_append_args* a, hipStream_t stream);

// Block-table entries of the pages each request uses in [0, num_pages).
int validate_block_sparse(const int32_t* block_table, const int32_t* seq_lens, int batch,
                          int page_size, int bt_stride, int64_t num_pages, hipStream_t stream);

}  // namespace pkv
