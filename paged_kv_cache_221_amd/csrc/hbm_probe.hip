// hbm_probe.hip -- loads-only kernels that give the benchmark its HBM read
// ceilings (see include/pa_probe.h): a contiguous sweep, and the block walk
// of a paged decode call without the attention.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pa_probe.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 512;
constexpr unsigned kMagic = 0x9e3779b9u;

__device__ inline unsigned fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

__global__ __launch_bounds__(kThreads) void read_linear_kernel(const u32x4* __restrict__ src,
                                                               int64_t n16, uint32_t* sink) {
  const int64_t T = gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * n16 / T, hi = (int64_t)(blockIdx.x + 1) * n16 / T;
  constexpr int U = 8;  // loads in flight per thread
  unsigned acc = 0;
  int64_t i = lo + threadIdx.x;
  for (; i + (U - 1) * kThreads < hi; i += U * kThreads) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= fold(v[u]);
  }
  for (; i < hi; i += kThreads) acc ^= fold(__builtin_nontemporal_load(src + i));
  if (acc == kMagic) sink[blockIdx.x * kThreads + threadIdx.x] = acc;
}

// One block of `block_bytes` per pool per step, each thread loading
// block_bytes / 8192 pieces of 16 bytes of K and of V (every load instruction
// of the workgroup covers 8 KiB contiguously); two blocks in flight.
__global__ __launch_bounds__(kThreads) void read_blocks_kernel(const char* __restrict__ kp,
                                                               const char* __restrict__ vp,
                                                               int64_t pool_blocks, int block_bytes,
                                                               const int32_t* __restrict__ list,
                                                               int64_t n, uint32_t* sink) {
  constexpr int kMaxPieces = 8;  // block_bytes <= 64 KiB
  const int pieces = block_bytes / (kThreads * 16);
  const int64_t T = gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * n / T, hi = (int64_t)(blockIdx.x + 1) * n / T;
  unsigned acc = 0;
  for (int64_t b = lo; b < hi; b += 2) {
    u32x4 r[2][2 * kMaxPieces];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      // past the share's end: nothing is loaded (a duplicate block would
      // count bytes the decode call does not read)
      const int64_t idx = b + d < hi ? b + d : hi - 1;
      const int64_t pb = list[idx];
      const bool ok = b + d < hi && pb >= 0 && pb < pool_blocks;
      const u32x4* k = reinterpret_cast<const u32x4*>(kp + (ok ? pb : 0) * block_bytes);
      const u32x4* v = reinterpret_cast<const u32x4*>(vp + (ok ? pb : 0) * block_bytes);
#pragma unroll
      for (int j = 0; j < kMaxPieces; ++j) {
        if (ok && j < pieces) {
          r[d][j] = __builtin_nontemporal_load(k + threadIdx.x + j * kThreads);
          r[d][kMaxPieces + j] = __builtin_nontemporal_load(v + threadIdx.x + j * kThreads);
        } else {
          r[d][j] = r[d][kMaxPieces + j] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int j = 0; j < 2 * kMaxPieces; ++j) acc ^= fold(r[d][j]);
  }
  if (acc == kMagic) sink[blockIdx.x * kThreads + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

int pa_probe_read_linear(const void* src, size_t bytes, uint32_t* sink, int grid, void* stream) {
  if (src == nullptr || sink == nullptr || grid <= 0 || bytes % 16 != 0) return -1;
  read_linear_kernel<<<dim3((unsigned)grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(src), (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int pa_probe_read_blocks(const void* k_pool, const void* v_pool, int64_t pool_blocks,
                         int block_bytes, const int32_t* blocks, int64_t num_blocks,
                         uint32_t* sink, int grid, void* stream) {
  if (k_pool == nullptr || v_pool == nullptr || blocks == nullptr || sink == nullptr ||
      grid <= 0 || pool_blocks <= 0 || num_blocks <= 0 || block_bytes <= 0 ||
      block_bytes % (kThreads * 16) != 0 || block_bytes > 8 * kThreads * 16)
    return -1;
  read_blocks_kernel<<<dim3((unsigned)grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const char*>(k_pool), static_cast<const char*>(v_pool), pool_blocks,
      block_bytes, blocks, num_blocks, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
