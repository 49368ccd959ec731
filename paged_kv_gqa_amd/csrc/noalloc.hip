// pkv_decode_noalloc: a whole decode step (pkv_decode_partial, then pkv_combine on
// the same stream) whose split-KV partials live in a library-owned device array
// instead of a caller workspace, for callers that cannot allocate device memory.
//
// The array is a file-scope __device__ symbol, so each GPU the library runs on holds
// its own copy (kNoAllocScratchBytes) from the code object's load until the process
// ends. In host code its name is only a stand-in: the device address is taken once
// per device with hipGetSymbolAddress (that device current) and kept; only that
// address ever reaches a kernel. Every call on a GPU shares the GPU's array, which
// keeps the last call's contents. Nothing in it needs to start at zero (decode_partial
// writes every slot the combine reads), and calls that overlap on one GPU (other
// streams or threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pkv.h"
#include "status.hpp"
#include "validate.hpp"

namespace {

constexpr size_t kNoAllocScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __attribute__((aligned(256))) unsigned char scratch[kNoAllocScratchBytes];

std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_status[kMaxDevices];

// Device address of this device's array (set-up on the first call on each device).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return pkv::fail(PKV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "device %d (at most %d devices)", dev, kMaxDevices);
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = (g_status[dev] == hipSuccess) ? p : nullptr;
  });
  if (g_status[dev] != hipSuccess || g_scratch[dev] == nullptr)
    return pkv::fail(PKV_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                     hipGetErrorString(g_status[dev]));
  *out = g_scratch[dev];
  return PKV_OK;
}

}  // namespace

extern "C" int pkv_decode_noalloc(const pkv_decode_args* a, void* out, float* lse_out,
                                  void* stream) {
  if (a == nullptr) return pkv::fail(PKV_ERR_INVALID_ARG, "null args");
  if (a->struct_size < sizeof(pkv_decode_args))
    return pkv::fail(PKV_ERR_INVALID_ARG, "struct_size %zu < %zu", a->struct_size,
                     sizeof(pkv_decode_args));
  if (a->num_kv_heads < 1 || a->num_q_heads < 1 || a->q_len < 1 || a->head_dim < 1)
    return pkv::fail(PKV_ERR_INVALID_ARG, "sizes must be positive");
  const int rows = (a->num_q_heads / a->num_kv_heads) * a->q_len;
  size_t need = 0;
  int st = pkv_workspace_bytes(a->num_partials, rows > 0 ? rows : 1, a->head_dim, &need);
  if (st != PKV_OK) return st;
  if (need > kNoAllocScratchBytes)
    return pkv::fail(PKV_ERR_WORKSPACE,
                     "%lld partials of %d rows x %d need %zu bytes; the static scratch holds %zu",
                     static_cast<long long>(a->num_partials), rows, a->head_dim, need,
                     kNoAllocScratchBytes);
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != PKV_OK) return st;
  pkv_decode_args d = *a;
  d.struct_size = sizeof(pkv_decode_args);
  d.workspace = ws;
  d.workspace_bytes = kNoAllocScratchBytes;
  // The host-side PKV_VALIDATE checks copy arrays into host vectors; this entry point
  // makes no allocation of any kind, so it runs without them.
  pkv::ValidateOff no_validate;
  st = pkv_decode_partial(&d, stream);
  if (st != PKV_OK) return st;
  return pkv_combine_split(ws, kNoAllocScratchBytes, d.num_partials, d.req_tile_base, d.batch,
                           d.q_len, d.num_q_heads, d.num_kv_heads, d.head_dim,
                           d.request_split != 0 ? d.request_split : 1, out, lse_out, stream);
}
