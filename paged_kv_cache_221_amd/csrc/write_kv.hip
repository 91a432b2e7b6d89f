// write_kv.hip -- the slot_mapping-driven KV write [P1 §02; P3 §1.4] and the
// copy-on-write block copy [P2 写时复制].
//
// Each new token's K row and V row (Hkv * D elements each, contiguous in both
// the input and the cache) is copied into the slot slot_mapping names, as
// raw 16-byte vectors: the write is a bit-exact copy whatever the dtype.
// One workgroup per token; its threads stride over the K then the V vectors.
// The block copy moves whole blocks (block_size token rows) the same way,
// one workgroup per (source, destination) pair.
#include "attn_tile.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kWriteThreads = 256;

__global__ __launch_bounds__(kWriteThreads) void write_kv_kernel(
    const u32x4* __restrict__ k_new, const u32x4* __restrict__ v_new, u32x4* __restrict__ k_cache,
    u32x4* __restrict__ v_cache, const int64_t* __restrict__ slot_mapping, int vecs_per_row,
    int64_t num_slots) {
  const int64_t t = blockIdx.x;
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;  // padding token, or outside the pool
  const u32x4* ksrc = k_new + t * vecs_per_row;
  const u32x4* vsrc = v_new + t * vecs_per_row;
  u32x4* kdst = k_cache + slot * vecs_per_row;
  u32x4* vdst = v_cache + slot * vecs_per_row;
  for (int i = threadIdx.x; i < 2 * vecs_per_row; i += kWriteThreads) {
    if (i < vecs_per_row) {
      kdst[i] = ksrc[i];
    } else {
      vdst[i - vecs_per_row] = vsrc[i - vecs_per_row];
    }
  }
}

__global__ __launch_bounds__(kWriteThreads) void copy_blocks_kernel(
    u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache, const int32_t* __restrict__ src_dst,
    int64_t vecs_per_block, int num_blocks) {
  const int32_t src = src_dst[2 * (int64_t)blockIdx.x];
  const int32_t dst = src_dst[2 * (int64_t)blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const u32x4* ks = k_cache + src * vecs_per_block;
  const u32x4* vs = v_cache + src * vecs_per_block;
  u32x4* kd = k_cache + dst * vecs_per_block;
  u32x4* vd = v_cache + dst * vecs_per_block;
  // four vectors of K and four of V in flight per thread before the stores
  constexpr int kBatch = 4;
  for (int64_t i0 = threadIdx.x; i0 < vecs_per_block; i0 += kBatch * kWriteThreads) {
    u32x4 a[kBatch], b[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int64_t i = i0 + j * kWriteThreads;
      if (i < vecs_per_block) {
        a[j] = ks[i];
        b[j] = vs[i];
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int64_t i = i0 + j * kWriteThreads;
      if (i < vecs_per_block) {
        kd[i] = a[j];
        vd[i] = b[j];
      }
    }
  }
}

}  // namespace

hipError_t launch_copy_blocks(const pa_kv_cache* c, const int32_t* src_dst, int num_pairs,
                              hipStream_t stream) {
  if (num_pairs <= 0) return hipSuccess;
  const int elem = c->dtype == PA_F32 ? 4 : 2;
  const int64_t block_bytes = (int64_t)c->block_size * c->num_kv_heads * c->head_dim * elem;
  copy_blocks_kernel<<<dim3((unsigned)num_pairs), dim3(kWriteThreads), 0, stream>>>(
      static_cast<u32x4*>(c->k_cache), static_cast<u32x4*>(c->v_cache), src_dst, block_bytes / 16,
      c->num_blocks);
  return hipGetLastError();
}

hipError_t launch_write_kv(const pa_kv_cache* c, const void* k_new, const void* v_new,
                           const int64_t* slot_mapping, int num_tokens, hipStream_t stream) {
  if (num_tokens <= 0) return hipSuccess;
  const int elem = c->dtype == PA_F32 ? 4 : 2;
  const int64_t row_bytes = (int64_t)c->num_kv_heads * c->head_dim * elem;
  const int vecs_per_row = (int)(row_bytes / 16);
  const int64_t num_slots = (int64_t)c->num_blocks * c->block_size;
  write_kv_kernel<<<dim3((unsigned)num_tokens), dim3(kWriteThreads), 0, stream>>>(
      static_cast<const u32x4*>(k_new), static_cast<const u32x4*>(v_new),
      static_cast<u32x4*>(c->k_cache), static_cast<u32x4*>(c->v_cache), slot_mapping,
      vecs_per_row, num_slots);
  return hipGetLastError();
}

}  // namespace pa
