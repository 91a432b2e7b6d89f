// attn_tile.h -- one wavefront's share of paged attention on gfx950.
//
// A wave owns a "row tile" of 16 query rows that read the same KV head: the
// GQA group of query heads of one or more tokens ([P1 §04]: query head h
// reads KV head h / (Hq/Hkv), no copy). It streams 16-token KV blocks,
// located through the block table ([P2 paging], [P3 §3.5]), and keeps the
// scores and probabilities in registers (the FlashAttention principle of
// [P1 §04] and [P3 §3.4]: S and P never reach HBM), with an online softmax.
//
// Both products run on the matrix cores, as 16x16 tiles:
//   S^T[key][row] = K[key][:] . Q[row][:]          (A = K rows, B = Q rows)
//   O^T[dim][row] += V^T[dim][key] . P^T[key][row]  (A = V^T,    B = P^T)
// The output layout of the first product (lane l holds keys 4*(l/16)+i of
// row l%16) is exactly the B-operand layout the second product needs, so P
// goes from one MFMA to the next without leaving the lane. The A operand of
// the second product wants, per lane, four keys of one dimension; choosing
// dimension slot m of chunk c to be dim (D/16)*m + c makes every lane's data a
// contiguous run of D/16 elements of each of its four key rows, so V is read
// straight from HBM with wide loads and never transposed through LDS. Rows
// of the softmax state (m, l) and of O^T both sit at lane%16, so the rescale
// is lane-local too.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kBlockTokens = 16;  // tokens per KV block (block_size)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ inline float neg_inf() { return -__builtin_huge_valf(); }
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ inline float xor_shuffle(float v, int mask) { return __shfl_xor(v, mask, kWave); }

// ----------------------------------------------------------- element types
struct Bf16 {
  using storage = uint16_t;
  __device__ static uint16_t from_float(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);  // round to nearest even
    return (uint16_t)(u >> 16);
  }
  __device__ static f32x4 mma_qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static f32x4 mma_pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
  }
};

struct F16 {
  using storage = uint16_t;
  __device__ static uint16_t from_float(float f) {
    _Float16 h = (_Float16)f;  // hardware conversion, round to nearest even
    return __builtin_bit_cast(uint16_t, h);
  }
  __device__ static f32x4 mma_qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static f32x4 mma_pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
};

struct F32 {
  using storage = float;
};

// --------------------------------------------------- operand load / compute
// Ops<E, D> knows how one wave loads a 16-token KV block in MFMA operand
// layout, how it computes the 16x16 score tile and how it accumulates P.V.
template <class E, int D>
struct Ops;

// 16-bit storage: QK with 16x16x32 (8 elements per lane per 32-dim chunk),
// PV with 16x16x16 (4 keys per lane).
template <class E, int D>
struct Ops16 {
  static_assert(D == 64 || D == 128, "head_dim");
  using storage = uint16_t;
  static constexpr int kQk = D / 32;   // QK chunks
  static constexpr int kVe = D / 16;   // V elements per (lane, key)
  static constexpr int kChunks = D / 16;
  struct VVec { unsigned w[kVe / 2]; };
  struct KV {
    u32x4 k[kQk];
    VVec v[4];
  };
  struct Q {
    u32x4 q[kQk];
  };
  using P = u32x2;

  // kblk/vblk point at (key 0 of the block, this KV head, dim 0); rs is the
  // element stride between consecutive keys (Hkv * D).
  __device__ static void load(KV& kv, const storage* kblk, const storage* vblk, int64_t rs,
                              int lane) {
    const int m = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int c = 0; c < kQk; ++c)
      kv.k[c] = *reinterpret_cast<const u32x4*>(kblk + m * rs + 32 * c + 8 * grp);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const storage* src = vblk + (4 * grp + i) * rs + kVe * m;
      if constexpr (kVe == 8) {
        u32x4 t = *reinterpret_cast<const u32x4*>(src);
        kv.v[i].w[0] = t.x; kv.v[i].w[1] = t.y; kv.v[i].w[2] = t.z; kv.v[i].w[3] = t.w;
      } else {
        u32x2 t = *reinterpret_cast<const u32x2*>(src);
        kv.v[i].w[0] = t.x; kv.v[i].w[1] = t.y;
      }
    }
  }
  __device__ static void load_q(Q& q, const storage* qrow, bool valid, int lane) {
    const int grp = lane >> 4;
#pragma unroll
    for (int c = 0; c < kQk; ++c) {
      q.q[c] = valid ? *reinterpret_cast<const u32x4*>(qrow + 32 * c + 8 * grp)
                     : u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ static void zero_v(KV& kv, int i) {
#pragma unroll
    for (int w = 0; w < kVe / 2; ++w) kv.v[i].w[w] = 0u;
  }
  __device__ static f32x4 scores(const KV& kv, const Q& q) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kQk; ++c) acc = E::mma_qk(kv.k[c], q.q[c], acc);
    return acc;
  }
  __device__ static P pack_p(const float (&p)[4]) {
    P r;
    r.x = (unsigned)E::from_float(p[0]) | ((unsigned)E::from_float(p[1]) << 16);
    r.y = (unsigned)E::from_float(p[2]) | ((unsigned)E::from_float(p[3]) << 16);
    return r;
  }
  __device__ static void pv(f32x4 (&o)[kChunks], const KV& kv, P p) {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int w = c >> 1;
      u32x2 a;
      if ((c & 1) == 0) {
        a.x = (kv.v[0].w[w] & 0xffffu) | (kv.v[1].w[w] << 16);
        a.y = (kv.v[2].w[w] & 0xffffu) | (kv.v[3].w[w] << 16);
      } else {
        a.x = (kv.v[0].w[w] >> 16) | (kv.v[1].w[w] & 0xffff0000u);
        a.y = (kv.v[2].w[w] >> 16) | (kv.v[3].w[w] & 0xffff0000u);
      }
      o[c] = E::mma_pv(a, p, o[c]);
    }
  }
  __device__ static storage to_storage(float f) { return E::from_float(f); }
};

template <int D>
struct Ops<Bf16, D> : Ops16<Bf16, D> {};
template <int D>
struct Ops<F16, D> : Ops16<F16, D> {};

// fp32 storage: QK and PV with 16x16x4 (one element per lane per MFMA).
template <int D>
struct Ops<F32, D> {
  static_assert(D == 64 || D == 128, "head_dim");
  using storage = float;
  static constexpr int kKv = D / 16;   // 4-float K vectors per lane
  static constexpr int kVe = D / 16;   // V elements per (lane, key)
  static constexpr int kChunks = D / 16;
  struct KV {
    f32x4 k[kKv];
    float v[4][kVe];
  };
  struct Q {
    f32x4 q[kKv];
  };
  struct P {
    float p[4];
  };

  __device__ static void load(KV& kv, const storage* kblk, const storage* vblk, int64_t rs,
                              int lane) {
    const int m = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int j = 0; j < kKv; ++j)
      kv.k[j] = *reinterpret_cast<const f32x4*>(kblk + m * rs + 16 * j + 4 * grp);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const storage* src = vblk + (4 * grp + i) * rs + kVe * m;
#pragma unroll
      for (int w = 0; w < kVe / 4; ++w) {
        f32x4 t = *reinterpret_cast<const f32x4*>(src + 4 * w);
        kv.v[i][4 * w + 0] = t.x; kv.v[i][4 * w + 1] = t.y;
        kv.v[i][4 * w + 2] = t.z; kv.v[i][4 * w + 3] = t.w;
      }
    }
  }
  __device__ static void load_q(Q& q, const storage* qrow, bool valid, int lane) {
    const int grp = lane >> 4;
#pragma unroll
    for (int j = 0; j < kKv; ++j)
      q.q[j] = valid ? *reinterpret_cast<const f32x4*>(qrow + 16 * j + 4 * grp)
                     : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __device__ static void zero_v(KV& kv, int i) {
#pragma unroll
    for (int e = 0; e < kVe; ++e) kv.v[i][e] = 0.f;
  }
  __device__ static f32x4 scores(const KV& kv, const Q& q) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kKv; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kv.k[j][e], q.q[j][e], acc, 0, 0, 0);
    return acc;
  }
  __device__ static P pack_p(const float (&p)[4]) {
    P r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.p[i] = p[i];
    return r;
  }
  __device__ static void pv(f32x4 (&o)[kChunks], const KV& kv, const P& p) {
#pragma unroll
    for (int c = 0; c < kChunks; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv.v[i][c], p.p[i], o[c], 0, 0, 0);
  }
  __device__ static storage to_storage(float f) { return f; }
};

// ------------------------------------------------------------ row tile state
template <int D>
struct RowState {
  float m;  // running max of the row's scores, log2 domain (replicated per row)
  float l;  // this lane's partial sum of exp2(s - m) (summed across lanes at the end)
  f32x4 o[D / 16];
  __device__ void init() {
    m = neg_inf();
    l = 0.f;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
};

// Describes where one wave's KV blocks live.
template <class Storage>
struct KvView {
  const Storage* k;        // k_cache + kv_head * D
  const Storage* v;        // v_cache + kv_head * D
  int64_t rs;              // elements between consecutive keys: Hkv * D
  const int32_t* table;    // this request's block-table row
  int num_blocks;          // pool size, for the out-of-pool guard
};

// One block: mask, online softmax update, P.V accumulation.
// key_end: keys >= key_end are invisible to this lane's row.
// seq_len: keys >= seq_len do not exist (their V may hold anything).
template <class E, int D>
__device__ inline void consume_block(RowState<D>& st, typename Ops<E, D>::KV& kv,
                                     const typename Ops<E, D>::Q& q, int key0, int key_end,
                                     int seq_len, float scale_log2, int lane) {
  using O = Ops<E, D>;
  const int grp = lane >> 4;
  if (key0 + kBlockTokens > seq_len) {  // wave-uniform: the request's last block
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (key0 + 4 * grp + i >= seq_len) O::zero_v(kv, i);
  }
  f32x4 acc = O::scores(kv, q);
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = key0 + 4 * grp + i;
    s[i] = key < key_end ? acc[i] * scale_log2 : neg_inf();
  }
  float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  mx = fmaxf(mx, xor_shuffle(mx, 16));
  mx = fmaxf(mx, xor_shuffle(mx, 32));
  const float m_new = fmaxf(st.m, mx);
  const float m_use = m_new == neg_inf() ? 0.f : m_new;
  // An unchanged maximum (including a row that has seen no key yet) keeps
  // alpha exactly 1, so the rescale below is skipped when no row moved.
  const float alpha = st.m == m_new ? 1.0f : fast_exp2(st.m - m_use);
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = fast_exp2(s[i] - m_use);
  st.l = st.l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
  st.m = m_new;
  if (__any(alpha != 1.0f)) {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) st.o[c] *= alpha;
  }
  O::pv(st.o, kv, O::pack_p(p));
}

// Streams blocks [b_begin, b_end) with stride b_step through one row tile,
// loading block n+1 while block n is consumed. All control is wave-uniform.
template <class E, int D>
__device__ inline void stream_blocks(RowState<D>& st, const typename Ops<E, D>::Q& q,
                                     const KvView<typename Ops<E, D>::storage>& kv_view,
                                     int b_begin, int b_end, int b_step, int key_end,
                                     int seq_len, float scale_log2, int lane) {
  using O = Ops<E, D>;
  using KV = typename O::KV;
  if (b_begin >= b_end) return;
  const int64_t block_elems = (int64_t)kBlockTokens * kv_view.rs;
  auto block_id = [&](int b) -> int {
    int pb = kv_view.table[b];
    return (pb >= 0 && pb < kv_view.num_blocks) ? pb : -1;
  };
  auto load = [&](KV& kv, int pb) {
    const int64_t base = (int64_t)(pb < 0 ? 0 : pb) * block_elems;
    O::load(kv, kv_view.k + base, kv_view.v + base, kv_view.rs, lane);
  };
  KV buf0, buf1;
  int b = b_begin;
  int pb0 = block_id(b);
  load(buf0, pb0);
  while (true) {
    int bn = b + b_step;
    int pb1 = -1;
    if (bn < b_end) {
      pb1 = block_id(bn);
      load(buf1, pb1);
    }
    if (pb0 >= 0)
      consume_block<E, D>(st, buf0, q, b * kBlockTokens, key_end, seq_len, scale_log2, lane);
    if (bn >= b_end) break;
    b = bn;
    bn = b + b_step;
    pb0 = -1;
    if (bn < b_end) {
      pb0 = block_id(bn);
      load(buf0, pb0);
    }
    if (pb1 >= 0)
      consume_block<E, D>(st, buf1, q, b * kBlockTokens, key_end, seq_len, scale_log2, lane);
    if (bn >= b_end) break;
    b = bn;
  }
}

}  // namespace pa
