// HBM read-bandwidth probes for the roofline (measurement only; built as
// libpkv_probe.so and loaded by the bench, not part of libpkv.so).
//
// HBM3E's 8 TB/s is the part's specification; these kernels measure what this part
// actually delivers for the two read patterns that bound the decode kernel:
// - a contiguous stream (grid-stride, 16 bytes per lane, 16 loads in flight per lane);
// - a gather of 4 KB pages in random order, each wave reading two pages at a time as
//   1 KB contiguous (whole-line) loads, the access pattern of decode's K/V gather at
//   page size 16 (one 16-token page of one kv head is 4 KB in bf16).
// Both use non-temporal loads, as the decode kernel does, and fold what they read
// into a value that is stored only if it equals a constant, so no load is dropped.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kStreamUnroll = 16;
constexpr unsigned kNever = 0x9E3779B9u;

__device__ __forceinline__ unsigned fold(u32x4 v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ p,
                                                               size_t n16, unsigned* sink) {
  unsigned acc = 0;
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
  size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  for (; i + (kStreamUnroll - 1) * stride < n16; i += kStreamUnroll * stride) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= fold(v[u]);
  }
  for (; i < n16; i += stride) acc ^= fold(__builtin_nontemporal_load(p + i));
  if (acc == kNever) sink[0] = acc;
}

// Wave w reads pages perm[w * per_wave ...], two per iteration.
__global__ __launch_bounds__(kThreads) void page_gather_kernel(const uint8_t* __restrict__ p,
                                                               const int32_t* __restrict__ perm,
                                                               int npages, int per_wave,
                                                               unsigned* sink) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6));
  unsigned acc = 0;
  const int c0 = wave * per_wave;
  const int c1 = min(npages, c0 + per_wave);
  for (int c = c0; c < c1; c += 2) {
    const int pg[2] = {perm[c], perm[min(c + 1, c1 - 1)]};
    u32x4 v[8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        v[4 * h + u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
            p + static_cast<size_t>(pg[h]) * 4096 + u * 1024 + lane * 16));
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= fold(v[u]);
  }
  if (acc == kNever) sink[0] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from the 16-byte aligned device buffer `buf`.
// sink: a device unsigned. Returns a hipError_t.
int pkvp_stream_read(const void* buf, size_t bytes, unsigned* sink, int grid, void* stream) {
  if (buf == nullptr || sink == nullptr || grid < 1 || bytes % 16 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf), bytes / 16,
                     sink);
  return hipGetLastError();
}

// Reads the npages 4 KB pages of `buf` in the order of perm (device int32[npages], a
// permutation of 0 .. npages-1). Returns a hipError_t.
int pkvp_page_gather(const void* buf, const int32_t* perm, int npages, unsigned* sink, int grid,
                     void* stream) {
  if (buf == nullptr || perm == nullptr || sink == nullptr || grid < 1 || npages < 1)
    return hipErrorInvalidValue;
  const int waves = grid * (kThreads / 64);
  int per_wave = (npages + waves - 1) / waves;
  per_wave += per_wave & 1;  // pages are taken two at a time
  hipLaunchKernelGGL(page_gather_kernel, dim3(grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(buf), perm,
                     npages, per_wave, sink);
  return hipGetLastError();
}

}  // extern "C"
