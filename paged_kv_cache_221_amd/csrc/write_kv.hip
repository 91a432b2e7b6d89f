// write_kv.hip -- the slot_mapping-driven KV write [P1 §02; P3 §1.4] and the
// copy-on-write block copy [P2 写时复制].
//
// Each new token's K row and V row (Hkv * D elements each, contiguous in both
// the input and the cache) is copied into the slot slot_mapping names, as
// raw 16-byte vectors: the write is a bit-exact copy whatever the dtype (an
// E4M3 cache instead stores the quantised codes of bf16 rows [P3 §4.1]).
// One workgroup per token; its threads stride over the K then the V vectors.
// The block copy moves whole blocks (block_size token rows) the same way,
// one workgroup per (source, destination) pair. The rotary-embedding variant
// of the write rotates q and K first [P2 步骤 3: RoPE].
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

// KV write into an E4M3 cache: bf16 rows in, each element divided by the
// cache's scale (fp32, correctly rounded) and stored as its E4M3 code. Each
// thread converts 8 elements (16 bytes in, 8 bytes out).
__global__ __launch_bounds__(kWriteThreads) void write_kv_fp8_kernel(
    const u32x4* __restrict__ k_new, const u32x4* __restrict__ v_new,
    u32x2* __restrict__ k_cache, u32x2* __restrict__ v_cache,
    const int64_t* __restrict__ slot_mapping, int groups_per_row, int64_t num_slots,
    float k_scale, float v_scale) {
  const int64_t t = blockIdx.x;
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;
  for (int i = threadIdx.x; i < 2 * groups_per_row; i += kWriteThreads) {
    const bool is_k = i < groups_per_row;
    const int gidx = is_k ? i : i - groups_per_row;
    const u32x4 x = (is_k ? k_new : v_new)[t * groups_per_row + gidx];
    const float sc = is_k ? k_scale : v_scale;
    const unsigned w[4] = {x.x, x.y, x.z, x.w};
    unsigned c[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[2 * j] = e4m3_code(__fdiv_rn(__uint_as_float(w[j] << 16), sc));
      c[2 * j + 1] = e4m3_code(__fdiv_rn(__uint_as_float(w[j] & 0xffff0000u), sc));
    }
    const u32x2 out = {c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                       c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
    (is_k ? k_cache : v_cache)[slot * groups_per_row + gidx] = out;
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
  // kBatch vectors of K and as many of V in flight per thread before the
  // stores (a whole 16-token block pair of 8 heads x 128 bf16 at 8); the
  // copied bytes are not read again by this kernel, so they stream past the
  // caches
  constexpr int kBatch = 8;
  for (int64_t i0 = threadIdx.x; i0 < vecs_per_block; i0 += kBatch * kWriteThreads) {
    u32x4 a[kBatch], b[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int64_t i = i0 + j * kWriteThreads;
      if (i < vecs_per_block) {
        a[j] = __builtin_nontemporal_load(ks + i);
        b[j] = __builtin_nontemporal_load(vs + i);
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int64_t i = i0 + j * kWriteThreads;
      if (i < vecs_per_block) {
        __builtin_nontemporal_store(a[j], kd + i);
        __builtin_nontemporal_store(b[j], vd + i);
      }
    }
  }
}

// Storage <-> fp32 for the rotary embedding (round to nearest even back).
template <class E>
__device__ inline float to_f32(typename E::storage v);
template <>
__device__ inline float to_f32<Bf16>(uint16_t v) {
  return __uint_as_float((unsigned)v << 16);
}
template <>
__device__ inline float to_f32<F16>(uint16_t v) {
  return (float)__builtin_bit_cast(_Float16, v);
}
template <>
__device__ inline float to_f32<F32>(float v) {
  return v;
}
template <class E>
__device__ inline typename E::storage from_f32(float f) {
  if constexpr (sizeof(typename E::storage) == 4) {
    return f;
  } else {
    return E::from_float(f);
  }
}

// Rotary position embedding fused with the KV write: one workgroup per token.
// Each rotated pair (a, b) of a query or key head becomes
// (a cos - b sin, b cos + a sin) in fp32 with the angle of its position;
// q is rotated in place, the rotated K and the raw V go to the token's slot.
template <class E>
__global__ __launch_bounds__(kWriteThreads) void rope_write_kv_kernel(
    typename E::storage* __restrict__ q, const typename E::storage* __restrict__ k_new,
    const typename E::storage* __restrict__ v_new, typename E::storage* __restrict__ k_cache,
    typename E::storage* __restrict__ v_cache, const int64_t* __restrict__ slot_mapping,
    const int32_t* __restrict__ positions, const float* __restrict__ cos_sin, int max_position,
    int rotary_dim, int neox, int num_heads, int num_kv_heads, int head_dim, int64_t num_slots) {
  using S = typename E::storage;
  const int64_t t = blockIdx.x;
  const int pos = positions[t];
  if (pos < 0 || pos >= max_position) return;  // outside the table: token left alone
  const int half = rotary_dim / 2;
  const float* cs = cos_sin + (int64_t)pos * rotary_dim;
  auto pair = [&](int j, int* ia, int* ib) {
    *ia = neox ? j : 2 * j;
    *ib = neox ? j + half : 2 * j + 1;
  };
  // queries, in place
  for (int i = threadIdx.x; i < num_heads * half; i += kWriteThreads) {
    const int h = i / half, j = i - h * half;
    int ia, ib;
    pair(j, &ia, &ib);
    S* row = q + (t * num_heads + h) * head_dim;
    const float a = to_f32<E>(row[ia]), b = to_f32<E>(row[ib]);
    const float c = cs[j], sn = cs[half + j];
    row[ia] = from_f32<E>(a * c - b * sn);
    row[ib] = from_f32<E>(b * c + a * sn);
  }
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;  // padding token, or outside the pool
  const int64_t row_elems = (int64_t)num_kv_heads * head_dim;
  const S* ks = k_new + t * row_elems;
  const S* vs = v_new + t * row_elems;
  S* kd = k_cache + slot * row_elems;
  S* vd = v_cache + slot * row_elems;
  for (int i = threadIdx.x; i < num_kv_heads * half; i += kWriteThreads) {
    const int h = i / half, j = i - h * half;
    int ia, ib;
    pair(j, &ia, &ib);
    const float a = to_f32<E>(ks[h * head_dim + ia]), b = to_f32<E>(ks[h * head_dim + ib]);
    const float c = cs[j], sn = cs[half + j];
    kd[h * head_dim + ia] = from_f32<E>(a * c - b * sn);
    kd[h * head_dim + ib] = from_f32<E>(b * c + a * sn);
  }
  const int rest = head_dim - rotary_dim;  // dimensions past rotary_dim pass through
  for (int i = threadIdx.x; i < num_kv_heads * rest; i += kWriteThreads) {
    const int h = i / rest, d = rotary_dim + (i - h * rest);
    kd[h * head_dim + d] = ks[h * head_dim + d];
  }
  for (int64_t i = threadIdx.x; i < row_elems; i += kWriteThreads) vd[i] = vs[i];
}

// The same step for an E4M3 cache: q is rotated in place as for a bf16
// cache; the rotated K row, rounded to bf16 exactly as the bf16 path stores
// it, and the V row are then quantised as pa_write_kv quantises a bf16 row
// (x / scale in fp32, nearest E4M3 code, ties to even, saturating at 448).
__global__ __launch_bounds__(kWriteThreads) void rope_write_kv_fp8_kernel(
    uint16_t* __restrict__ q, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, const int64_t* __restrict__ slot_mapping,
    const int32_t* __restrict__ positions, const float* __restrict__ cos_sin, int max_position,
    int rotary_dim, int neox, int num_heads, int num_kv_heads, int head_dim, int64_t num_slots,
    float k_scale, float v_scale) {
  const int64_t t = blockIdx.x;
  const int pos = positions[t];
  if (pos < 0 || pos >= max_position) return;  // outside the table: token left alone
  const int half = rotary_dim / 2;
  const float* cs = cos_sin + (int64_t)pos * rotary_dim;
  auto pair = [&](int j, int* ia, int* ib) {
    *ia = neox ? j : 2 * j;
    *ib = neox ? j + half : 2 * j + 1;
  };
  auto code = [](uint16_t bf, float scale) {
    return (uint8_t)e4m3_code(__fdiv_rn(__uint_as_float((unsigned)bf << 16), scale));
  };
  for (int i = threadIdx.x; i < num_heads * half; i += kWriteThreads) {
    const int h = i / half, j = i - h * half;
    int ia, ib;
    pair(j, &ia, &ib);
    uint16_t* row = q + (t * num_heads + h) * head_dim;
    const float a = to_f32<Bf16>(row[ia]), b = to_f32<Bf16>(row[ib]);
    const float c = cs[j], sn = cs[half + j];
    row[ia] = from_f32<Bf16>(a * c - b * sn);
    row[ib] = from_f32<Bf16>(b * c + a * sn);
  }
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;  // padding token, or outside the pool
  const int64_t row_elems = (int64_t)num_kv_heads * head_dim;
  const uint16_t* ks = k_new + t * row_elems;
  const uint16_t* vs = v_new + t * row_elems;
  uint8_t* kd = k_cache + slot * row_elems;
  uint8_t* vd = v_cache + slot * row_elems;
  for (int i = threadIdx.x; i < num_kv_heads * half; i += kWriteThreads) {
    const int h = i / half, j = i - h * half;
    int ia, ib;
    pair(j, &ia, &ib);
    const float a = to_f32<Bf16>(ks[h * head_dim + ia]), b = to_f32<Bf16>(ks[h * head_dim + ib]);
    const float c = cs[j], sn = cs[half + j];
    kd[h * head_dim + ia] = code(from_f32<Bf16>(a * c - b * sn), k_scale);
    kd[h * head_dim + ib] = code(from_f32<Bf16>(b * c + a * sn), k_scale);
  }
  const int rest = head_dim - rotary_dim;  // dimensions past rotary_dim: quantised as they are
  for (int i = threadIdx.x; i < num_kv_heads * rest; i += kWriteThreads) {
    const int h = i / rest, d = rotary_dim + (i - h * rest);
    kd[h * head_dim + d] = code(ks[h * head_dim + d], k_scale);
  }
  for (int64_t i = threadIdx.x; i < row_elems; i += kWriteThreads) vd[i] = code(vs[i], v_scale);
}

// N consecutive floats from an address aligned to 4N bytes (N = 2, 4 or 8).
template <int N>
__device__ inline void load_floats(const float* p, float (&out)[N]) {
  if constexpr (N == 2) {
    const float2 x = *reinterpret_cast<const float2*>(p);
    out[0] = x.x;
    out[1] = x.y;
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const float4 x = *reinterpret_cast<const float4*>(p + i);
      out[i] = x.x;
      out[i + 1] = x.y;
      out[i + 2] = x.z;
      out[i + 3] = x.w;
    }
  }
}

// The same step in 16-byte vectors (V = 16 / element size elements), for
// rotary_dim a multiple of 16 and 16-byte aligned rows: a NeoX unit is the V
// pairs (i, i + rotary_dim/2) for i in [V u, V u + V), two vectors; a GPT-J
// unit is the V/2 adjacent pairs of one vector. Dimensions past rotary_dim of
// K and all of V are copied as vectors; q's stay in place.
template <class E, bool NEOX>
__global__ __launch_bounds__(kWriteThreads) void rope_write_kv_vec_kernel(
    typename E::storage* __restrict__ q, const typename E::storage* __restrict__ k_new,
    const typename E::storage* __restrict__ v_new, typename E::storage* __restrict__ k_cache,
    typename E::storage* __restrict__ v_cache, const int64_t* __restrict__ slot_mapping,
    const int32_t* __restrict__ positions, const float* __restrict__ cos_sin, int max_position,
    int rotary_dim, int num_heads, int num_kv_heads, int head_dim, int64_t num_slots) {
  using S = typename E::storage;
  constexpr int V = 16 / (int)sizeof(S);
  constexpr int NP = NEOX ? V : V / 2;  // pairs per unit
  const int64_t t = blockIdx.x;
  const int pos = positions[t];
  if (pos < 0 || pos >= max_position) return;  // outside the table: token left alone
  const int half = rotary_dim / 2;
  const int units = NEOX ? half / V : rotary_dim / V;  // rotation units per head row
  const float* cs = cos_sin + (int64_t)pos * rotary_dim;

  // rotates unit u of the head row src into dst (dst may equal src)
  auto rotate = [&](const S* src, S* dst, int u) {
    const int j0 = u * NP;  // first pair of the unit
    float c[NP], sn[NP];
    load_floats<NP>(cs + j0, c);
    load_floats<NP>(cs + half + j0, sn);
    if constexpr (NEOX) {
      const u32x4 va = *reinterpret_cast<const u32x4*>(src + V * u);
      const u32x4 vb = *reinterpret_cast<const u32x4*>(src + V * u + half);
      S a[V], b[V];
      __builtin_memcpy(a, &va, 16);
      __builtin_memcpy(b, &vb, 16);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float fa = to_f32<E>(a[e]), fb = to_f32<E>(b[e]);
        a[e] = from_f32<E>(fa * c[e] - fb * sn[e]);
        b[e] = from_f32<E>(fb * c[e] + fa * sn[e]);
      }
      u32x4 oa, ob;
      __builtin_memcpy(&oa, a, 16);
      __builtin_memcpy(&ob, b, 16);
      *reinterpret_cast<u32x4*>(dst + V * u) = oa;
      *reinterpret_cast<u32x4*>(dst + V * u + half) = ob;
    } else {
      const u32x4 vx = *reinterpret_cast<const u32x4*>(src + V * u);
      S x[V];
      __builtin_memcpy(x, &vx, 16);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const float fa = to_f32<E>(x[2 * p]), fb = to_f32<E>(x[2 * p + 1]);
        x[2 * p] = from_f32<E>(fa * c[p] - fb * sn[p]);
        x[2 * p + 1] = from_f32<E>(fb * c[p] + fa * sn[p]);
      }
      u32x4 o;
      __builtin_memcpy(&o, x, 16);
      *reinterpret_cast<u32x4*>(dst + V * u) = o;
    }
  };

  // queries, in place
  for (int i = threadIdx.x; i < num_heads * units; i += kWriteThreads) {
    const int h = i / units;
    S* row = q + (t * num_heads + h) * head_dim;
    rotate(row, row, i - h * units);
  }
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;  // padding token, or outside the pool
  const int64_t row_elems = (int64_t)num_kv_heads * head_dim;
  const S* ks = k_new + t * row_elems;
  S* kd = k_cache + slot * row_elems;
  for (int i = threadIdx.x; i < num_kv_heads * units; i += kWriteThreads) {
    const int h = i / units;
    rotate(ks + h * head_dim, kd + h * head_dim, i - h * units);
  }
  // K dims past rotary_dim, then all of V, as 16-byte vectors
  const int rest = (head_dim - rotary_dim) / V;  // vectors per head row
  for (int i = threadIdx.x; i < num_kv_heads * rest; i += kWriteThreads) {
    const int h = i / rest;
    const int64_t e = (int64_t)h * head_dim + rotary_dim + V * (i - h * rest);
    *reinterpret_cast<u32x4*>(kd + e) = *reinterpret_cast<const u32x4*>(ks + e);
  }
  const u32x4* vs = reinterpret_cast<const u32x4*>(v_new + t * row_elems);
  u32x4* vd = reinterpret_cast<u32x4*>(v_cache + slot * row_elems);
  for (int64_t i = threadIdx.x; i < row_elems / V; i += kWriteThreads) vd[i] = vs[i];
}

}  // namespace

hipError_t launch_rope_write_kv(const pa_kv_cache* c, void* q, int num_heads, const void* k_new,
                                const void* v_new, const int64_t* slot_mapping,
                                const int32_t* positions, const float* cos_sin, int max_position,
                                int rotary_dim, int neox, int num_tokens, hipStream_t stream) {
  if (num_tokens <= 0) return hipSuccess;
  const int64_t num_slots = (int64_t)c->num_blocks * c->block_size;
  const dim3 grid((unsigned)num_tokens), block(kWriteThreads);
  if (c->dtype == PA_FP8_E4M3) {
    rope_write_kv_fp8_kernel<<<grid, block, 0, stream>>>(
        static_cast<uint16_t*>(q), static_cast<const uint16_t*>(k_new),
        static_cast<const uint16_t*>(v_new), static_cast<uint8_t*>(c->k_cache),
        static_cast<uint8_t*>(c->v_cache), slot_mapping, positions, cos_sin, max_position,
        rotary_dim, neox, num_heads, c->num_kv_heads, c->head_dim, num_slots, c->k_scale,
        c->v_scale);
    return hipGetLastError();
  }
  auto aligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  const bool vec = rotary_dim % 16 == 0 && c->head_dim % 8 == 0 && aligned(q) &&
                   aligned(k_new) && aligned(v_new) && aligned(c->k_cache) &&
                   aligned(c->v_cache) && aligned(cos_sin);
  if (vec) {
    switch (c->dtype) {
#define PA_ROPE_VEC(E)                                                                           \
  if (neox)                                                                                      \
    rope_write_kv_vec_kernel<E, true><<<grid, block, 0, stream>>>(                               \
        static_cast<E::storage*>(q), static_cast<const E::storage*>(k_new),                      \
        static_cast<const E::storage*>(v_new), static_cast<E::storage*>(c->k_cache),            \
        static_cast<E::storage*>(c->v_cache), slot_mapping, positions, cos_sin, max_position,    \
        rotary_dim, num_heads, c->num_kv_heads, c->head_dim, num_slots);                         \
  else                                                                                           \
    rope_write_kv_vec_kernel<E, false><<<grid, block, 0, stream>>>(                              \
        static_cast<E::storage*>(q), static_cast<const E::storage*>(k_new),                      \
        static_cast<const E::storage*>(v_new), static_cast<E::storage*>(c->k_cache),            \
        static_cast<E::storage*>(c->v_cache), slot_mapping, positions, cos_sin, max_position,    \
        rotary_dim, num_heads, c->num_kv_heads, c->head_dim, num_slots);                         \
  break;
      case PA_BF16: PA_ROPE_VEC(Bf16)
      case PA_F16: PA_ROPE_VEC(F16)
      case PA_F32: PA_ROPE_VEC(F32)
#undef PA_ROPE_VEC
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (c->dtype) {
#define PA_ROPE_LAUNCH(E)                                                                        \
  rope_write_kv_kernel<E><<<grid, block, 0, stream>>>(                                          \
      static_cast<E::storage*>(q), static_cast<const E::storage*>(k_new),                        \
      static_cast<const E::storage*>(v_new), static_cast<E::storage*>(c->k_cache),              \
      static_cast<E::storage*>(c->v_cache), slot_mapping, positions, cos_sin, max_position,      \
      rotary_dim, neox, num_heads, c->num_kv_heads, c->head_dim, num_slots);                     \
  break;
    case PA_BF16: PA_ROPE_LAUNCH(Bf16)
    case PA_F16: PA_ROPE_LAUNCH(F16)
    case PA_F32: PA_ROPE_LAUNCH(F32)
#undef PA_ROPE_LAUNCH
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const pa_kv_cache* c, const int32_t* src_dst, int num_pairs,
                              hipStream_t stream) {
  if (num_pairs <= 0) return hipSuccess;
  const int elem = c->dtype == PA_F32 ? 4 : c->dtype == PA_FP8_E4M3 ? 1 : 2;
  const int64_t block_bytes = (int64_t)c->block_size * c->num_kv_heads * c->head_dim * elem;
  copy_blocks_kernel<<<dim3((unsigned)num_pairs), dim3(kWriteThreads), 0, stream>>>(
      static_cast<u32x4*>(c->k_cache), static_cast<u32x4*>(c->v_cache), src_dst, block_bytes / 16,
      c->num_blocks);
  return hipGetLastError();
}

hipError_t launch_write_kv(const pa_kv_cache* c, const void* k_new, const void* v_new,
                           const int64_t* slot_mapping, int num_tokens, hipStream_t stream) {
  if (num_tokens <= 0) return hipSuccess;
  if (c->dtype == PA_FP8_E4M3) {
    const int groups = c->num_kv_heads * c->head_dim / 8;
    write_kv_fp8_kernel<<<dim3((unsigned)num_tokens), dim3(kWriteThreads), 0, stream>>>(
        static_cast<const u32x4*>(k_new), static_cast<const u32x4*>(v_new),
        static_cast<u32x2*>(c->k_cache), static_cast<u32x2*>(c->v_cache), slot_mapping, groups,
        (int64_t)c->num_blocks * c->block_size, c->k_scale, c->v_scale);
    return hipGetLastError();
  }
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
