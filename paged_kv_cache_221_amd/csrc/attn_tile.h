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

// max(v[l], v[l ^ 16]) and max(v[l], v[l ^ 32]) with the gfx950 row swaps
// (VALU only: no LDS traffic, no lgkmcnt wait).
// Maxima of scores use the IEEE-754-2019 maximum (NaN-propagating, one
// v_maximum3_f32): fmaxf would make the compiler quiet both operands of every
// lane exchange first. Scores are finite or -inf (masked).
__device__ inline float fmax2(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ inline float max_xor16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmax2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float max_xor32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmax2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_xor16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float sum_xor32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Buffer resource over one KV block's slice for one head: base address,
// byte range (reads at or past it return zeros), gfx9 data-format word.
using Rsrc = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcFlags = 0x00020000;
// `base` and `range_bytes` must be the same in every lane of the wave (one
// block of one head). Reading them from the first lane puts the resource in
// scalar registers even where the compiler cannot prove that (64-bit index
// math done on the vector unit): a resource in vector registers makes it
// guard every load with a loop over the distinct values in the wave.
__device__ inline Rsrc make_rsrc(const void* base, int range_bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, __builtin_amdgcn_readfirstlane(range_bytes),
                                          kRsrcFlags);
}
// AUX is the load's cache-policy field (bit 1: nt, streaming).
template <int AUX = 0>
__device__ inline u32x4 buf_load16(Rsrc r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
}
template <int AUX = 0>
__device__ inline unsigned buf_load4(Rsrc r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX);
}
template <int AUX = 0>
__device__ inline u32x2 buf_load8(Rsrc r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX);
}
// Cache policy of the decode kernels' KV block loads. A decode call reads
// each KV byte once, so the blocks are loaded as streaming (nt) data: on a
// read of 8,877 random 32 KB K and V blocks (581 MB) the nt hint took a
// loads-only kernel from 97 to 86 us (5.99 -> 6.78 TB/s), whatever the block
// order; a linear read of the same bytes gains the same (94 -> 84 us).
#ifndef PA_KV_LOAD_AUX
#define PA_KV_LOAD_AUX 2
#endif
constexpr int kKvAux = PA_KV_LOAD_AUX;

// ----------------------------------------------------------- element types
struct Bf16 {
  using storage = uint16_t;     // q, outputs
  using kv_storage = uint16_t;  // the KV cache
  // two floats -> packed bf16 pair (round to nearest even), lo in bits 0..15
  __device__ static unsigned pack2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 h = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(unsigned, h);
  }
  __device__ static uint16_t from_float(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);  // round to nearest even
    return (uint16_t)(u >> 16);
  }
  __device__ static float to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
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
  using kv_storage = uint16_t;
  __device__ static unsigned pack2(float lo, float hi) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    f16x2 h = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(unsigned, h);
  }
  __device__ static uint16_t from_float(float f) {
    _Float16 h = (_Float16)f;  // hardware conversion, round to nearest even
    return __builtin_bit_cast(uint16_t, h);
  }
  __device__ static float to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
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
  using kv_storage = float;
};

// An E4M3 KV cache (OCP 8-bit float: 4 exponent bits, bias 7, 3 mantissa
// bits, no infinities) with bf16 queries, outputs and arithmetic. Every E4M3
// value is a bf16 value, so blocks are widened to bf16 MFMA operands exactly
// after loading; the cache's scales are folded into the softmax scale (K)
// and the output normalisation (V) by the caller of the kernels.
struct Fp8 : Bf16 {
  using kv_storage = uint8_t;
};

// E4M3 code of an fp32 value: the nearest of the 8-bit float's values, ties
// to the even code, magnitudes of 448 (the largest finite value) and more
// saturating to 448, NaN kept (0x7f with the sign). Integer operations on the
// fp32 bits: a normal result keeps 3 mantissa bits (a carry moves into the
// exponent); below 2^-6 the values are the multiples of 2^-9.
__device__ inline unsigned e4m3_code(float y) {
  const unsigned u = __float_as_uint(y);
  const unsigned sign = (u >> 24) & 0x80u;
  const unsigned au = u & 0x7fffffffu;
  if (au > 0x7f800000u) return sign | 0x7fu;
  const float ay = __uint_as_float(au);
  if (!(ay < 448.0f)) return sign | 0x7eu;
  if (ay < 0.015625f) return sign | (unsigned)__builtin_rintf(ay * 512.0f);
  const unsigned e = (au >> 23) - 120u;  // biased E4M3 exponent, 1 .. 15
  const unsigned mant = au & 0x7fffffu;
  unsigned r = mant >> 20;
  const unsigned rem = mant & 0xfffffu;
  if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
  return sign | min((e << 3) + r, 0x7eu);
}

// E4M3 codes of 4 bf16 values (two packed words, element 0 in the low half of
// lo) divided by `scale` in fp32, as one word (element k in byte k): the
// cache write's quantisation.
__device__ inline unsigned bf16x4_to_fp8(unsigned lo, unsigned hi, float scale) {
  const unsigned c0 = e4m3_code(__fdiv_rn(__uint_as_float(lo << 16), scale));
  const unsigned c1 = e4m3_code(__fdiv_rn(__uint_as_float(lo & 0xffff0000u), scale));
  const unsigned c2 = e4m3_code(__fdiv_rn(__uint_as_float(hi << 16), scale));
  const unsigned c3 = e4m3_code(__fdiv_rn(__uint_as_float(hi & 0xffff0000u), scale));
  return c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
}

// Four E4M3 codes (byte k of w is element k) -> four bf16, as two packed
// words in the same order. gfx950 converts two codes to two bf16 in one
// instruction; with a scale of 1 that is exact, since every E4M3 value
// (subnormals, signed zeros) is a bf16 value and NaN stays NaN (checked on the
// GPU for all 256 codes). It halves the widening work against converting to
// fp32 and packing to bf16.
__device__ inline void fp8x4_to_bf16(unsigned w, unsigned* lo, unsigned* hi) {
  *lo = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  *hi = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

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

  // Lane-constant byte offsets of this lane's operand pieces inside a block
  // slice (rs = elements between consecutive keys, Hkv * D).
  struct Off {
    int k[kQk];
    int v[4];
  };
  __device__ static Off offsets(int64_t rs, int lane) {
    const int m = lane & 15, grp = lane >> 4;
    Off o;
#pragma unroll
    for (int c = 0; c < kQk; ++c) o.k[c] = (int)((m * rs + 32 * c + 8 * grp) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) o.v[i] = (int)(((4 * grp + i) * rs + kVe * m) * 2);
    return o;
  }
  __device__ static void load(KV& kv, Rsrc kr, Rsrc vr, const Off& o) {
#pragma unroll
    for (int c = 0; c < kQk; ++c) kv.k[c] = buf_load16<kKvAux>(kr, o.k[c]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (kVe == 8) {
        u32x4 t = buf_load16<kKvAux>(vr, o.v[i]);
        kv.v[i].w[0] = t.x; kv.v[i].w[1] = t.y; kv.v[i].w[2] = t.z; kv.v[i].w[3] = t.w;
      } else {
        u32x2 t = buf_load8<kKvAux>(vr, o.v[i]);
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
  // q -> -q (sign bits flipped: exact)
  __device__ static void negate_q(Q& q) {
#pragma unroll
    for (int c = 0; c < kQk; ++c) q.q[c] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  }
  // A new key row and value row (one head, D elements each) in this lane's
  // operand positions: nr.k as if the lane's key row were the new one, and
  // every nr.v[i] the lane's columns of the new value row.
  __device__ static void load_new(KV& nr, const void* k_row, const void* v_row, int lane,
                                  float /*k_scale*/, float /*v_scale*/) {
    const int m = lane & 15, grp = lane >> 4;
    const uint16_t* kr = static_cast<const uint16_t*>(k_row);
    const uint16_t* vr = static_cast<const uint16_t*>(v_row) + kVe * m;
#pragma unroll
    for (int c = 0; c < kQk; ++c) nr.k[c] = *reinterpret_cast<const u32x4*>(kr + 32 * c + 8 * grp);
    VVec v;
    if constexpr (kVe == 8) {
      const u32x4 t = *reinterpret_cast<const u32x4*>(vr);
      v.w[0] = t.x; v.w[1] = t.y; v.w[2] = t.z; v.w[3] = t.w;
    } else {
      const u32x2 t = *reinterpret_cast<const u32x2*>(vr);
      v.w[0] = t.x; v.w[1] = t.y;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) nr.v[i] = v;
  }
  // Replaces key/value row `row` of a loaded block by the new row.
  __device__ static void patch(KV& kv, const KV& nr, int row, int lane) {
    const int m = lane & 15, grp = lane >> 4;
    if (m == row) {
#pragma unroll
      for (int c = 0; c < kQk; ++c) kv.k[c] = nr.k[c];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * grp + i == row) kv.v[i] = nr.v[i];
  }
  // Stores the new rows (as held by load_new) to one head's cache rows.
  __device__ static void store_new(const KV& nr, void* k_dst, void* v_dst, int lane) {
    const int m = lane & 15, grp = lane >> 4;
    if (m == 0) {
#pragma unroll
      for (int c = 0; c < kQk; ++c)
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(k_dst) + 32 * c + 8 * grp) = nr.k[c];
    }
    if (grp == 0) {
      uint16_t* vd = static_cast<uint16_t*>(v_dst) + kVe * m;
      if constexpr (kVe == 8) {
        *reinterpret_cast<u32x4*>(vd) = u32x4{nr.v[0].w[0], nr.v[0].w[1], nr.v[0].w[2], nr.v[0].w[3]};
      } else {
        *reinterpret_cast<u32x2*>(vd) = u32x2{nr.v[0].w[0], nr.v[0].w[1]};
      }
    }
  }
  __device__ static f32x4 scores(const KV& kv, const Q& q) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kQk; ++c) acc = E::mma_qk(kv.k[c], q.q[c], acc);
    return acc;
  }
  __device__ static P pack_p(const float (&p)[4]) {
    P r;
    r.x = E::pack2(p[0], p[1]);
    r.y = E::pack2(p[2], p[3]);
    return r;
  }
  // The PV A operands of a block, one per 16-dim chunk: element c of each of
  // the lane's four key rows (low or high halves of word c/2).
  struct VA {
    u32x2 a[kChunks];
  };
  __device__ static VA build_v(const KV& kv) {
    VA va;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int w = c >> 1;
      const unsigned sel = (c & 1) == 0 ? 0x05040100u : 0x07060302u;
      va.a[c].x = __builtin_amdgcn_perm(kv.v[1].w[w], kv.v[0].w[w], sel);
      va.a[c].y = __builtin_amdgcn_perm(kv.v[3].w[w], kv.v[2].w[w], sel);
    }
    return va;
  }
  __device__ static void pv_with(f32x4 (&o)[kChunks], const VA& va, P p) {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) o[c] = E::mma_pv(va.a[c], p, o[c]);
  }
  __device__ static void pv(f32x4 (&o)[kChunks], const KV& kv, P p) { pv_with(o, build_v(kv), p); }
  __device__ static storage to_storage(float f) { return E::from_float(f); }
};

template <int D>
struct Ops<Bf16, D> : Ops16<Bf16, D> {
  using kv_storage = uint16_t;
};
template <int D>
struct Ops<F16, D> : Ops16<F16, D> {
  using kv_storage = uint16_t;
};

// E4M3 cache: the bf16 tile with half-size loads. The registers keep the raw
// codes until the block is consumed (so loads stay in flight); scores() and
// build_v() widen them to the bf16 operands of Ops16<Bf16, D>.
//
// The QK product sums over head_dim in any order as long as K and Q agree, so
// K is read in 16-byte pieces: lane (m, grp) loads bytes 16*(grp + 4j) .. +15
// of key row m for j < D/64, whose two 8-byte halves are the lane's slots of
// QK chunks 2j and 2j+1. load_q reads q with the same assignment. V keeps the
// bf16 layout (one 128-byte key row per 16 lanes and load).
template <int D>
struct Ops<Fp8, D> : Ops16<Bf16, D> {
  using Base = Ops16<Bf16, D>;
  using kv_storage = uint8_t;
  using typename Base::Q;
  using typename Base::P;
  using typename Base::VA;
  static constexpr int kQk = D / 32;
  static constexpr int kK16 = D / 64;  // 16-byte K loads per lane
  static constexpr int kVe = D / 16;
  struct KV {
    u32x4 k[kK16];
    unsigned v[4][kVe / 4];  // kVe codes of each of the lane's four key rows
  };
  struct Off {
    int k[kK16];
    int v[4];
  };
  // head_dim index of the first of the 8 elements lane group grp holds in QK chunk c
  __device__ static int qk_dim(int c, int grp) { return 16 * (grp + 4 * (c >> 1)) + 8 * (c & 1); }
  __device__ static Off offsets(int64_t rs, int lane) {
    const int m = lane & 15, grp = lane >> 4;
    Off o;
#pragma unroll
    for (int j = 0; j < kK16; ++j) o.k[j] = (int)(m * rs + 16 * (grp + 4 * j));
#pragma unroll
    for (int i = 0; i < 4; ++i) o.v[i] = (int)((4 * grp + i) * rs + kVe * m);
    return o;
  }
  __device__ static void load(KV& kv, Rsrc kr, Rsrc vr, const Off& o) {
#pragma unroll
    for (int j = 0; j < kK16; ++j) kv.k[j] = buf_load16<kKvAux>(kr, o.k[j]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (kVe == 8) {
        const u32x2 t = buf_load8<kKvAux>(vr, o.v[i]);
        kv.v[i][0] = t.x;
        kv.v[i][1] = t.y;
      } else {
        kv.v[i][0] = buf_load4<kKvAux>(vr, o.v[i]);
      }
    }
  }
  __device__ static void load_q(Q& q, const uint16_t* qrow, bool valid, int lane) {
    const int grp = lane >> 4;
#pragma unroll
    for (int c = 0; c < kQk; ++c) {
      q.q[c] = valid ? *reinterpret_cast<const u32x4*>(qrow + qk_dim(c, grp))
                     : u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ static f32x4 scores(const KV& kv, const Q& q) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kQk; ++c) {
      const u32x4& w = kv.k[c >> 1];
      unsigned w0, w1, w2, w3;
      fp8x4_to_bf16((c & 1) ? w.z : w.x, &w0, &w1);
      fp8x4_to_bf16((c & 1) ? w.w : w.y, &w2, &w3);
      acc = Bf16::mma_qk(u32x4{w0, w1, w2, w3}, q.q[c], acc);
    }
    return acc;
  }
  __device__ static VA build_v(const KV& kv) {
    typename Base::KV w;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < kVe / 4; ++j)
        fp8x4_to_bf16(kv.v[i][j], &w.v[i].w[2 * j], &w.v[i].w[2 * j + 1]);
    return Base::build_v(w);
  }
  __device__ static void pv(f32x4 (&o)[Base::kChunks], const KV& kv, P p) {
    Base::pv_with(o, build_v(kv), p);
  }
  // New rows arrive as bf16 and are quantised like the cache write.
  __device__ static void load_new(KV& nr, const void* k_row, const void* v_row, int lane,
                                  float k_scale, float v_scale) {
    const int m = lane & 15, grp = lane >> 4;
    const uint16_t* kr = static_cast<const uint16_t*>(k_row);
    const uint16_t* vr = static_cast<const uint16_t*>(v_row) + kVe * m;
#pragma unroll
    for (int j = 0; j < kK16; ++j) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(kr + 16 * (grp + 4 * j));
      const u32x4 b = *reinterpret_cast<const u32x4*>(kr + 16 * (grp + 4 * j) + 8);
      nr.k[j] = u32x4{bf16x4_to_fp8(a.x, a.y, k_scale), bf16x4_to_fp8(a.z, a.w, k_scale),
                      bf16x4_to_fp8(b.x, b.y, k_scale), bf16x4_to_fp8(b.z, b.w, k_scale)};
    }
    unsigned v[kVe / 4];
    if constexpr (kVe == 8) {
      const u32x4 t = *reinterpret_cast<const u32x4*>(vr);
      v[0] = bf16x4_to_fp8(t.x, t.y, v_scale);
      v[1] = bf16x4_to_fp8(t.z, t.w, v_scale);
    } else {
      const u32x2 t = *reinterpret_cast<const u32x2*>(vr);
      v[0] = bf16x4_to_fp8(t.x, t.y, v_scale);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int w = 0; w < kVe / 4; ++w) nr.v[i][w] = v[w];
  }
  __device__ static void patch(KV& kv, const KV& nr, int row, int lane) {
    const int m = lane & 15, grp = lane >> 4;
    if (m == row) {
#pragma unroll
      for (int j = 0; j < kK16; ++j) kv.k[j] = nr.k[j];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * grp + i == row) {
#pragma unroll
        for (int w = 0; w < kVe / 4; ++w) kv.v[i][w] = nr.v[i][w];
      }
  }
  __device__ static void store_new(const KV& nr, void* k_dst, void* v_dst, int lane) {
    const int m = lane & 15, grp = lane >> 4;
    if (m == 0) {
#pragma unroll
      for (int j = 0; j < kK16; ++j)
        *reinterpret_cast<u32x4*>(static_cast<uint8_t*>(k_dst) + 16 * (grp + 4 * j)) = nr.k[j];
    }
    if (grp == 0) {
      uint8_t* vd = static_cast<uint8_t*>(v_dst) + kVe * m;
      if constexpr (kVe == 8) {
        *reinterpret_cast<u32x2*>(vd) = u32x2{nr.v[0][0], nr.v[0][1]};
      } else {
        *reinterpret_cast<unsigned*>(vd) = nr.v[0][0];
      }
    }
  }
};

// fp32 storage: QK and PV with 16x16x4 (one element per lane per MFMA).
template <int D>
struct Ops<F32, D> {
  static_assert(D == 64 || D == 128, "head_dim");
  using storage = float;
  using kv_storage = float;
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

  struct Off {
    int k[kKv];
    int v[4];
  };
  __device__ static Off offsets(int64_t rs, int lane) {
    const int m = lane & 15, grp = lane >> 4;
    Off o;
#pragma unroll
    for (int j = 0; j < kKv; ++j) o.k[j] = (int)((m * rs + 16 * j + 4 * grp) * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) o.v[i] = (int)(((4 * grp + i) * rs + kVe * m) * 4);
    return o;
  }
  __device__ static void load(KV& kv, Rsrc kr, Rsrc vr, const Off& o) {
#pragma unroll
    for (int j = 0; j < kKv; ++j) kv.k[j] = __builtin_bit_cast(f32x4, buf_load16<kKvAux>(kr, o.k[j]));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int w = 0; w < kVe / 4; ++w) {
        f32x4 t = __builtin_bit_cast(f32x4, buf_load16<kKvAux>(vr, o.v[i] + 16 * w));
        kv.v[i][4 * w + 0] = t.x; kv.v[i][4 * w + 1] = t.y;
        kv.v[i][4 * w + 2] = t.z; kv.v[i][4 * w + 3] = t.w;
      }
  }
  __device__ static void load_lds(KV& kv, const char* kb, const char* vb, int row_bytes,
                                  int lane) {
    const int m = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int j = 0; j < kKv; ++j)
      kv.k[j] = *reinterpret_cast<const f32x4*>(kb + m * row_bytes + (16 * j + 4 * grp) * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int w = 0; w < kVe / 4; ++w) {
        f32x4 t = *reinterpret_cast<const f32x4*>(vb + (4 * grp + i) * row_bytes +
                                                  (kVe * m + 4 * w) * 4);
        kv.v[i][4 * w + 0] = t.x; kv.v[i][4 * w + 1] = t.y;
        kv.v[i][4 * w + 2] = t.z; kv.v[i][4 * w + 3] = t.w;
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
  __device__ static void negate_q(Q& q) {
#pragma unroll
    for (int j = 0; j < kKv; ++j) q.q[j] = -q.q[j];
  }
  __device__ static void load_new(KV& nr, const void* k_row, const void* v_row, int lane,
                                  float /*k_scale*/, float /*v_scale*/) {
    const int m = lane & 15, grp = lane >> 4;
    const float* kr = static_cast<const float*>(k_row);
    const float* vr = static_cast<const float*>(v_row) + kVe * m;
#pragma unroll
    for (int j = 0; j < kKv; ++j) nr.k[j] = *reinterpret_cast<const f32x4*>(kr + 16 * j + 4 * grp);
    float v[kVe];
#pragma unroll
    for (int w = 0; w < kVe / 4; ++w) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(vr + 4 * w);
      v[4 * w] = t.x; v[4 * w + 1] = t.y; v[4 * w + 2] = t.z; v[4 * w + 3] = t.w;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < kVe; ++e) nr.v[i][e] = v[e];
  }
  __device__ static void patch(KV& kv, const KV& nr, int row, int lane) {
    const int m = lane & 15, grp = lane >> 4;
    if (m == row) {
#pragma unroll
      for (int j = 0; j < kKv; ++j) kv.k[j] = nr.k[j];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * grp + i == row) {
#pragma unroll
        for (int e = 0; e < kVe; ++e) kv.v[i][e] = nr.v[i][e];
      }
  }
  __device__ static void store_new(const KV& nr, void* k_dst, void* v_dst, int lane) {
    const int m = lane & 15, grp = lane >> 4;
    if (m == 0) {
#pragma unroll
      for (int j = 0; j < kKv; ++j)
        *reinterpret_cast<f32x4*>(static_cast<float*>(k_dst) + 16 * j + 4 * grp) = nr.k[j];
    }
    if (grp == 0) {
      float* vd = static_cast<float*>(v_dst) + kVe * m;
#pragma unroll
      for (int w = 0; w < kVe / 4; ++w)
        *reinterpret_cast<f32x4*>(vd + 4 * w) =
            f32x4{nr.v[0][4 * w], nr.v[0][4 * w + 1], nr.v[0][4 * w + 2], nr.v[0][4 * w + 3]};
    }
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
  struct VA {
    float v[4][kVe];
  };
  __device__ static VA build_v(const KV& kv) {
    VA va;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < kVe; ++e) va.v[i][e] = kv.v[i][e];
    return va;
  }
  __device__ static void pv_with(f32x4 (&o)[kChunks], const VA& va, const P& p) {
#pragma unroll
    for (int c = 0; c < kChunks; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.v[i][c], p.p[i], o[c], 0, 0, 0);
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

// Stores D/16 consecutive output values of one row in the storage dtype.
template <class E, int D>
__device__ inline void store_chunk(typename Ops<E, D>::storage* dst, const float* v) {
  constexpr int n = D / 16;
  using S = typename Ops<E, D>::storage;
  if constexpr (sizeof(S) == 2) {
    unsigned w[n / 2];
#pragma unroll
    for (int j = 0; j < n / 2; ++j)
      w[j] = (unsigned)Ops<E, D>::to_storage(v[2 * j]) |
             ((unsigned)Ops<E, D>::to_storage(v[2 * j + 1]) << 16);
    if constexpr (n == 8) {
      *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
    } else {
      *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
    }
  } else {
#pragma unroll
    for (int j = 0; j < n / 4; ++j)
      *reinterpret_cast<f32x4*>(dst + 4 * j) = f32x4{v[4 * j], v[4 * j + 1], v[4 * j + 2],
                                                    v[4 * j + 3]};
  }
}

// Partial output rows -- the pieces of cut segments and tiles, merged by
// their LSEs -- are kept in the output's storage type: the merged row is
// rounded to that type anyway, and 16-bit partials halve the bytes written
// and read back. Loads of n (4 or 8) consecutive partial values, widened.
template <class E, int N>
__device__ inline void load_part(const typename E::storage* p, float* v) {
  static_assert(N == 4 || N == 8, "4 or 8 values");
  if constexpr (sizeof(typename E::storage) == 2) {
    if constexpr (N == 8) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = E::to_f32((uint16_t)(w[k] & 0xffffu));
        v[2 * k + 1] = E::to_f32((uint16_t)(w[k] >> 16));
      }
    } else {
      const u32x2 w = *reinterpret_cast<const u32x2*>(p);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        v[2 * k] = E::to_f32((uint16_t)(w[k] & 0xffffu));
        v[2 * k + 1] = E::to_f32((uint16_t)(w[k] >> 16));
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < N; k += 4) {
      const f32x4 w = *reinterpret_cast<const f32x4*>(p + k);
      v[k] = w[0];
      v[k + 1] = w[1];
      v[k + 2] = w[2];
      v[k + 3] = w[3];
    }
  }
}

// KV blocks each wave keeps in flight. fp32 operands are twice the size, so
// they get half the depth to stay within the register budget; E4M3 blocks
// are half the size and get their own.
#ifndef PA_KV_DEPTH
#define PA_KV_DEPTH 4
#endif
#ifndef PA_KV_FP8_DEPTH
#define PA_KV_FP8_DEPTH 4
#endif
template <class E>
constexpr int kv_depth() {
  return sizeof(typename E::kv_storage) == 4   ? 2
         : sizeof(typename E::kv_storage) == 1 ? PA_KV_FP8_DEPTH
                                               : PA_KV_DEPTH;
}

// ------------------------------------------------------------ row tile state
template <int D>
struct RowState {
  float m;  // reference maximum of the row's scores, log2 domain (replicated per row)
  float l;  // this lane's partial sum of exp2(s - m) (summed across lanes at the end)
  f32x4 o[D / 16];
  __device__ void init() {
    m = neg_inf();
    l = 0.f;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
};

// The exponent base of a row. Online softmax only needs o and l to be taken
// against one common reference m; the result sum(p v) / sum(p) does not
// depend on it as long as nothing overflows. So m moves only when a block's
// maximum exceeds it by more than kRescaleLog2: then p = exp2(s - m) stays at
// most 2^kRescaleLog2 (fine for fp32 sums and for bf16/fp16 P operands) and
// most blocks skip the rescale of o altogether. A row that has seen no key yet
// (m = -inf, o = l = 0) takes the first block's maximum without a rescale.
constexpr float kRescaleLog2 = 8.0f;
// Updates m for a block whose row maximum is mx; returns the factor for o
// and l (exactly 1 when m stays).
__device__ inline float advance_max(float& m, float mx) {
  const bool up = mx > m + kRescaleLog2;
  const float alpha = (up && m != neg_inf()) ? fast_exp2(m - mx) : 1.0f;
  m = up ? mx : m;
  return alpha;
}

// Where one wave's KV blocks live.
template <class Storage>
struct KvView {
  const Storage* k;        // k_cache + kv_head * D
  const Storage* v;        // v_cache + kv_head * D
  int64_t rs;              // elements between consecutive keys: Hkv * D
  const int32_t* table;    // this request's block-table row
  int num_blocks;          // pool size in cache blocks, for the out-of-pool guard
  int shift;               // cache blocks hold 16 << shift tokens
};

// The pool's 16-token block holding 16-token block `li` of a request whose
// table entry for it is `e` (cache blocks of 16 << shift tokens), or -1 when
// the entry is outside the pool (checked before the shift can overflow).
__device__ inline int block16(int e, int li, int shift, int num_blocks) {
  return (e >= 0 && e < num_blocks) ? (e << shift) + (li & ((1 << shift) - 1)) : -1;
}

// One block: mask, online softmax update, P.V accumulation. Keys at or past
// seq_len were read as zeros (the buffer range stops there); keys at or past
// key_end are invisible to this lane's row and get probability 0.
template <class E, int D>
__device__ inline void consume_block(RowState<D>& st, const typename Ops<E, D>::KV& kv,
                                     const typename Ops<E, D>::Q& q, int key0, int key_end,
                                     float scale_log2, int lane) {
  using O = Ops<E, D>;
  const int grp = lane >> 4;
  f32x4 acc = O::scores(kv, q);
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = key0 + 4 * grp + i;
    s[i] = key < key_end ? acc[i] * scale_log2 : neg_inf();
  }
  float mx = fmax2(fmax2(s[0], s[1]), fmax2(s[2], s[3]));
  mx = max_xor16(mx);
  mx = max_xor32(mx);
  const float alpha = advance_max(st.m, mx);
  const float m_use = st.m == neg_inf() ? 0.f : st.m;
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = fast_exp2(s[i] - m_use);
  st.l = st.l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
  if (__any(alpha != 1.0f)) {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) st.o[c] *= alpha;
  }
  O::pv(st.o, kv, O::pack_p(p));
}

// One block against RT row tiles that share it (prefill): every tile's
// scores, then every tile's softmax update, one combined rescale test, and
// the block's PV operand built once for all tiles. Straight-line code, so
// the tiles' independent MFMA and VALU chains interleave.
// With MASK false every key of the block is visible to every valid row (the
// caller has checked), the per-key comparison is skipped, and scale_log2
// must be >= 0 (a caller with a negative scale negates q instead).
template <class E, int D, int RT, bool MASK = true>
__device__ inline void consume_block_tiles(RowState<D> (&st)[RT], const typename Ops<E, D>::KV& kv,
                                           const typename Ops<E, D>::Q (&q)[RT], int key0,
                                           const int (&key_end)[RT], float scale_log2, int lane) {
  using O = Ops<E, D>;
  const int grp = lane >> 4;
  f32x4 acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = O::scores(kv, q[t]);
  typename O::P pk[RT];
  float alpha[RT];
  bool moved = false;
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    float p[4];
    if constexpr (MASK) {
      float s[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = key0 + 4 * grp + i;
        s[i] = key < key_end[t] ? acc[t][i] * scale_log2 : neg_inf();
      }
      float mx = fmax2(fmax2(s[0], s[1]), fmax2(s[2], s[3]));
      mx = max_xor16(mx);
      mx = max_xor32(mx);
      alpha[t] = advance_max(st[t].m, mx);
      const float m_use = st[t].m == neg_inf() ? 0.f : st[t].m;
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = fast_exp2(s[i] - m_use);
    } else {
      // every key visible and scale_log2 >= 0: the row maximum of the scaled
      // scores is the scaled maximum of the raw ones (rounding is monotonic),
      // the reference is finite once the block is taken in, and each
      // exponent is one fused multiply-add
      float mx = fmax2(fmax2(acc[t][0], acc[t][1]), fmax2(acc[t][2], acc[t][3]));
      mx = max_xor16(mx);
      mx = max_xor32(mx) * scale_log2;
      alpha[t] = advance_max(st[t].m, mx);
      const float neg_m = -st[t].m;
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = fast_exp2(__builtin_fmaf(acc[t][i], scale_log2, neg_m));
    }
    moved = moved || alpha[t] != 1.0f;
    st[t].l = st[t].l * alpha[t] + ((p[0] + p[1]) + (p[2] + p[3]));
    pk[t] = O::pack_p(p);
  }
  if (__any(moved)) {
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int c = 0; c < D / 16; ++c) st[t].o[c] *= alpha[t];
  }
  const typename O::VA va = O::build_v(kv);
#pragma unroll
  for (int t = 0; t < RT; ++t) O::pv_with(st[t].o, va, pk[t]);
}

// Streams this wave's contiguous run of n blocks, starting at logical block
// b_begin, through one row tile. DEPTH blocks are in flight: while block i is
// consumed, blocks i+1 .. i+DEPTH-1 are loading. Block ids are read with
// scalar loads; each block is read through a buffer resource whose range ends
// at the request's last key, so rows past it, blocks whose id is outside the
// pool and the padding blocks past the run come back as zeros without
// touching memory. Every iteration loads and consumes unconditionally (a
// padding block is consumed with no visible key), which lets the compiler wait
// for exactly the block it consumes instead of draining every load.
//
// With SYNC, the workgroup meets at a barrier once per DEPTH blocks, so that
// waves walking the same blocks (other heads) keep fetching them together;
// every wave of the workgroup must then run the same number of blocks.
// `patch(kv, i)` sees block i of the run after its loads and before it is
// consumed (the fused decode step substitutes the new token's row there).
struct NoPatch {
  template <class KV>
  __device__ void operator()(KV&, int) const {}
};
template <class E, int D, int DEPTH, bool SYNC = false, class Patch = NoPatch>
__device__ inline void stream_blocks(RowState<D>& st, const typename Ops<E, D>::Q& q,
                                     const KvView<typename Ops<E, D>::kv_storage>& kv_view,
                                     int b_begin, int n, int key_end, int seq_len,
                                     float scale_log2, int lane, const Patch& patch = Patch{}) {
  using O = Ops<E, D>;
  using S = typename O::kv_storage;
  using KV = typename O::KV;
  if (n <= 0) return;
  const typename O::Off off = O::offsets(kv_view.rs, lane);
  const int64_t block_elems = (int64_t)kBlockTokens * kv_view.rs;
  const int row_bytes = (int)(kv_view.rs * (int64_t)sizeof(S));
  const __attribute__((address_space(4))) int32_t* tab =
      (const __attribute__((address_space(4))) int32_t*)kv_view.table;

  auto load = [&](KV& kv, int i) {
    const int li = b_begin + min(i, n - 1);
    const int pb = block16(tab[li >> kv_view.shift], li, kv_view.shift, kv_view.num_blocks);
    const bool ok = i < n && pb >= 0;
    const int keys = min(seq_len - (b_begin + i) * kBlockTokens, kBlockTokens);
    const int range = ok ? keys * row_bytes : 0;
    const int64_t base = (int64_t)(ok ? pb : 0) * block_elems;
    O::load(kv, make_rsrc(kv_view.k + base, range), make_rsrc(kv_view.v + base, range), off);
  };
  auto consume = [&](KV& kv, int i) {
    patch(kv, i);
    consume_block<E, D>(st, kv, q, (b_begin + i) * kBlockTokens, i < n ? key_end : 0,
                        scale_log2, lane);
  };

  KV buf[DEPTH];
#pragma unroll
  for (int j = 0; j < DEPTH; ++j) load(buf[j], j);
  for (int i0 = 0; i0 < n; i0 += DEPTH) {
    if constexpr (SYNC) __syncthreads();
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
      consume(buf[j], i0 + j);
      // keep the refill of buf[j] here: the scheduler would otherwise sink
      // it towards its use and collapse the pipeline
      __builtin_amdgcn_sched_barrier(0);
      load(buf[j], i0 + j + DEPTH);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

}  // namespace pa
