// write_kv.hip -- the slot_mapping-driven KV write [P1 §02; P3 §1.4].
//
// Each new token's K row and V row (Hkv * D elements each, contiguous in both
// the input and the cache) is copied into the slot slot_mapping names, as
// raw 16-byte vectors: the write is a bit-exact copy whatever the dtype.
// One workgroup per token; its threads stride over the K then the V vectors.
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

}  // namespace

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
