// PKV_VALIDATE checks (see validate.hpp).
#include "validate.hpp"

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "kernels.hpp"
#include "status.hpp"

namespace pkv {

namespace {
thread_local bool t_validate_off = false;
}  // namespace

bool validate_enabled() {
  if (t_validate_off) return false;
  const char* e = std::getenv("PKV_VALIDATE");
  return e != nullptr && e[0] != '\0' && std::strcmp(e, "0") != 0;
}

ValidateOff::ValidateOff() : prev_(t_validate_off) { t_validate_off = true; }
ValidateOff::~ValidateOff() { t_validate_off = prev_; }

namespace {

int drain(hipStream_t stream) {
  const hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "PKV_VALIDATE: stream: %s", hipGetErrorString(e));
  return PKV_OK;
}

// Copy n elements of device (or mapped host) memory to the host.
template <typename T>
int fetch(std::vector<T>& dst, const T* src, size_t n) {
  dst.assign(n, T{});
  if (n == 0) return PKV_OK;
  const hipError_t e = hipMemcpy(dst.data(), src, n * sizeof(T), hipMemcpyDefault);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "PKV_VALIDATE: copy: %s", hipGetErrorString(e));
  return PKV_OK;
}

int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Block-table entries of the first ceil(len_b / P) pages of every row (none where
// len_b is 0).
int check_pages(const int32_t* block_table, const std::vector<int32_t>& len, int bt_stride,
                int page_size, int64_t num_pages) {
  const int B = static_cast<int>(len.size());
  std::vector<int32_t> bt;
  int st = fetch(bt, block_table, static_cast<size_t>(B) * bt_stride);
  if (st != PKV_OK) return st;
  for (int b = 0; b < B; ++b) {
    const int64_t np = std::min<int64_t>(ceil_div64(std::max(len[b], 0), page_size), bt_stride);
    for (int64_t p = 0; p < np; ++p) {
      const int32_t e = bt[static_cast<size_t>(b) * bt_stride + p];
      if (e < 0 || e >= num_pages)
        return fail(PKV_ERR_INVALID_ARG, "PKV_VALIDATE: block_table[%d][%lld] = %d is outside [0, %lld)",
                    b, static_cast<long long>(p), e, static_cast<long long>(num_pages));
    }
  }
  return PKV_OK;
}

int check_lengths(const std::vector<int32_t>& len, int min_len, int bt_stride, int page_size,
                  const char* name) {
  for (size_t b = 0; b < len.size(); ++b) {
    if (len[b] < min_len)
      return fail(PKV_ERR_SEQ, "PKV_VALIDATE: %s[%zu] = %d < %d", name, b, len[b], min_len);
    if (static_cast<int64_t>(len[b]) > static_cast<int64_t>(bt_stride) * page_size)
      return fail(PKV_ERR_INVALID_ARG, "PKV_VALIDATE: %s[%zu] = %d exceeds the block table (%d pages of %d)",
                  name, b, len[b], bt_stride, page_size);
  }
  return PKV_OK;
}

}  // namespace

int validate_decode(const pkv_decode_args* a, const int32_t* tile_dev, hipStream_t stream) {
  int st = drain(stream);
  if (st != PKV_OK) return st;
  const int B = a->batch, W = a->num_workers, Hkv = a->num_kv_heads;
  std::vector<int32_t> L, offs, rtb, items;
  if ((st = fetch(L, a->seq_lens, B)) != PKV_OK) return st;
  if ((st = check_lengths(L, std::max(1, a->q_len), a->bt_stride, a->page_size, "seq_lens")) != PKV_OK)
    return st;
  if ((st = check_pages(a->block_table, L, a->bt_stride, a->page_size, a->num_pages)) != PKV_OK) return st;
  if ((st = fetch(offs, a->worker_offsets, static_cast<size_t>(W) + 1)) != PKV_OK) return st;
  if (offs[0] != 0)
    return fail(PKV_ERR_INVALID_ARG, "PKV_VALIDATE: worker_offsets[0] = %d, not 0", offs[0]);
  for (int w = 0; w < W; ++w)
    if (offs[w + 1] < offs[w])
      return fail(PKV_ERR_INVALID_ARG, "PKV_VALIDATE: worker_offsets decrease at %d", w);
  const int64_t N = offs[W];
  if (N > a->num_items)
    return fail(PKV_ERR_INVALID_ARG, "PKV_VALIDATE: worker_offsets[%d] = %lld > num_items %lld", W,
                static_cast<long long>(N), static_cast<long long>(a->num_items));
  if (N == 0) return PKV_OK;  // an empty work list reads nothing
  int32_t T = a->tile_tokens;
  if (tile_dev != nullptr) {
    std::vector<int32_t> t;
    if ((st = fetch(t, tile_dev, 1)) != PKV_OK) return st;
    T = t[0];
  }
  if (T < 1) return fail(PKV_ERR_INVALID_ARG, "PKV_VALIDATE: tile size %d", T);
  if ((st = fetch(rtb, a->req_tile_base, static_cast<size_t>(B) + 1)) != PKV_OK) return st;
  if (rtb[0] != 0) return fail(PKV_ERR_INVALID_ARG, "PKV_VALIDATE: req_tile_base[0] = %d, not 0", rtb[0]);
  for (int b = 0; b < B; ++b) {
    const int64_t nb = ceil_div64(L[b], T);
    if (rtb[b + 1] - rtb[b] != nb)
      return fail(PKV_ERR_INVALID_ARG, "PKV_VALIDATE: request %d has %d tiles in req_tile_base, "
                  "seq_lens[%d] = %d needs %lld of %d tokens (plan and lengths differ)", b,
                  rtb[b + 1] - rtb[b], b, L[b], static_cast<long long>(nb), T);
  }
  if (static_cast<int64_t>(Hkv) * rtb[B] > a->num_partials)
    return fail(PKV_ERR_INVALID_ARG, "PKV_VALIDATE: %lld partials needed, num_partials %lld",
                static_cast<long long>(static_cast<int64_t>(Hkv) * rtb[B]),
                static_cast<long long>(a->num_partials));
  if ((st = fetch(items, a->items, static_cast<size_t>(N) * 4)) != PKV_OK) return st;
  for (int64_t x = 0; x < N; ++x) {
    const int32_t b = items[4 * x], g = items[4 * x + 1], i = items[4 * x + 2], slot = items[4 * x + 3];
    const bool in = b >= 0 && b < B && g >= 0 && g < Hkv && i >= 0 && i < rtb[b + 1] - rtb[b];
    if (!in || static_cast<int64_t>(slot) !=
                   static_cast<int64_t>(Hkv) * rtb[b] + static_cast<int64_t>(g) * (rtb[b + 1] - rtb[b]) + i)
      return fail(PKV_ERR_INVALID_ARG, "PKV_VALIDATE: item %lld = (%d, %d, %d, %d) is not a tile of the plan",
                  static_cast<long long>(x), b, g, i, slot);
  }
  return PKV_OK;
}

int validate_combine(const int32_t* req_tile_base, int batch, int num_kv_heads,
                     int64_t num_partials, hipStream_t stream) {
  int st = drain(stream);
  if (st != PKV_OK) return st;
  std::vector<int32_t> rtb;
  if ((st = fetch(rtb, req_tile_base, static_cast<size_t>(batch) + 1)) != PKV_OK) return st;
  if (rtb[0] != 0) return fail(PKV_ERR_INVALID_ARG, "PKV_VALIDATE: req_tile_base[0] = %d, not 0", rtb[0]);
  for (int b = 0; b < batch; ++b)
    if (rtb[b + 1] < rtb[b])
      return fail(PKV_ERR_INVALID_ARG, "PKV_VALIDATE: req_tile_base decreases at %d", b);
  if (static_cast<int64_t>(num_kv_heads) * rtb[batch] > num_partials)
    return fail(PKV_ERR_INVALID_ARG, "PKV_VALIDATE: %lld partials read, num_partials %lld",
                static_cast<long long>(static_cast<int64_t>(num_kv_heads) * rtb[batch]),
                static_cast<long long>(num_partials));
  return PKV_OK;
}

int validate_prefill(const pkv_prefill_args* a, int heads_per_item, hipStream_t stream) {
  int st = drain(stream);
  if (st != PKV_OK) return st;
  const int B = a->batch;
  std::vector<int32_t> cu, kl, items;
  if ((st = fetch(cu, a->cu_q, static_cast<size_t>(B) + 1)) != PKV_OK) return st;
  if ((st = fetch(kl, a->kv_lens, B)) != PKV_OK) return st;
  if (cu[0] != 0) return fail(PKV_ERR_INVALID_ARG, "PKV_VALIDATE: cu_q[0] = %d, not 0", cu[0]);
  std::vector<int32_t> used(B, 0);  // kv length of requests with query tokens
  for (int b = 0; b < B; ++b) {
    const int n = cu[b + 1] - cu[b];
    if (n < 0) return fail(PKV_ERR_INVALID_ARG, "PKV_VALIDATE: cu_q decreases at %d", b);
    if (kl[b] < n)
      return fail(PKV_ERR_SEQ, "PKV_VALIDATE: kv_lens[%d] = %d < its %d query tokens", b, kl[b], n);
    if (static_cast<int64_t>(kl[b]) > static_cast<int64_t>(a->bt_stride) * a->page_size)
      return fail(PKV_ERR_INVALID_ARG, "PKV_VALIDATE: kv_lens[%d] = %d exceeds the block table", b, kl[b]);
    used[b] = n > 0 ? kl[b] : 0;
  }
  if ((st = check_pages(a->block_table, used, a->bt_stride, a->page_size, a->num_pages)) != PKV_OK)
    return st;
  if ((st = fetch(items, a->items, static_cast<size_t>(a->num_items) * 4)) != PKV_OK) return st;
  const int groups = (a->num_q_heads / a->num_kv_heads) / heads_per_item;
  for (int64_t x = 0; x < a->num_items; ++x) {
    const int32_t b = items[4 * x], g = items[4 * x + 1], hg = items[4 * x + 2], t0 = items[4 * x + 3];
    const bool in = b >= 0 && b < B && g >= 0 && g < a->num_kv_heads && hg >= 0 && hg < groups &&
                    t0 >= 0 && t0 < cu[b + 1] - cu[b] && t0 % kPrefillTileTokens == 0;
    if (!in)
      return fail(PKV_ERR_INVALID_ARG, "PKV_VALIDATE: item %lld = (%d, %d, %d, %d) is outside the batch",
                  static_cast<long long>(x), b, g, hg, t0);
  }
  return PKV_OK;
}

int validate_kv_append(const pkv_kv_append_args* a, hipStream_t stream) {
  int st = drain(stream);
  if (st != PKV_OK) return st;
  std::vector<int32_t> L;
  if ((st = fetch(L, a->seq_lens, a->batch)) != PKV_OK) return st;
  if ((st = check_lengths(L, std::max(1, a->q_len), a->bt_stride, a->page_size, "seq_lens")) != PKV_OK)
    return st;
  return check_pages(a->block_table, L, a->bt_stride, a->page_size, a->num_pages);
}

int validate_block_sparse(const int32_t* block_table, const int32_t* seq_lens, int batch,
                          int page_size, int bt_stride, int64_t num_pages, hipStream_t stream) {
  int st = drain(stream);
  if (st != PKV_OK) return st;
  std::vector<int32_t> L;
  if ((st = fetch(L, seq_lens, batch)) != PKV_OK) return st;
  return check_pages(block_table, L, bt_stride, page_size, num_pages);
}

}  // namespace pkv
