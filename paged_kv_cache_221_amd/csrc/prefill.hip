// prefill.hip -- the chunked-prefill rows of a varlen step [P1 §07] on gfx950.
//
// A request whose query rows times the GQA group exceed one 16-row tile is a
// prefill chunk: query row i of it sees keys 0 .. c + i (its cached context c
// plus itself and earlier new tokens [P1 §04 causal mask]). Prefill is a dense
// contraction [P1 §04 table: GEMM, compute-bound], so the work is arranged for
// operand reuse: a workgroup of 8 waves owns a tile of query tokens of one
// (request, KV head); every KV block is fetched once per workgroup into
// double-buffered LDS through a register prefetch ring of PA_PREFILL_RING
// blocks, and each wave reads the block's MFMA operands from LDS once for all
// of its rows. bf16, fp16 and E4M3 caches (the codes widened exactly to bf16
// as they are staged) give each wave 32 rows and consume blocks in pairs on
// 32x32x16 products (pf_piece32); fp32 caches give it one 16-row tile and
// single blocks (pf_piece). Scores and probabilities stay in registers (the
// FlashAttention principle [P3 §3.4]).
//
// A workgroup's time is its tile's key count, which in a causal chunk grows
// with the tile's position and with the request's cached context: one
// workgroup per (tile, request, KV head) leaves most CUs idle while the last
// tiles of the longest request finish (the mixed step's 4k-context chunk
// holds half the work in a quarter of the workgroups). With a workspace, the
// batch's (request, KV head, tile, KV block) items are instead cut into one
// equal contiguous share per resident workgroup, like the balanced decode
// kernel; a tile cut between shares is written as partials (normalised
// output and log-sum-exp per piece) and renormalised by a small merge kernel
// [P1 §07 LSE merge].
#include <algorithm>
#include <type_traits>

#include "attn_tile.h"
#include "pa_launch.h"

#ifndef PA_PREFILL_RT
#define PA_PREFILL_RT 2
#endif
#ifndef PA_PREFILL_RING
#define PA_PREFILL_RING 4
#endif
// Workgroups per CU the prefill kernels are compiled for (with 8 waves: two
// waves per SIMD)
#ifndef PA_PREFILL_OCC
#define PA_PREFILL_OCC 1
#endif
// Fixed cost of a tile in the equal-share prefill, in KV blocks: a piece
// pays its query loads, pipeline fill and stores (a cut tile's fp32 partial
// rows are 64 KB, the bytes of eight of its KV block slices), so shares of
// many short tiles get fewer blocks. On the mixed step's four chunks: 0 ->
// 190 us, 2 -> 177, 4 -> 166, 8 -> 150, 12-16 -> 148-151, 32 -> 157.
#ifndef PA_PREFILL_TILE_COST
#define PA_PREFILL_TILE_COST 8
#endif

namespace pa {
namespace {

// Waves per workgroup; each stages KV blocks for all of them. Eight waves
// (256 query rows of the 32-row tile) use each staged block twice as often
// as four: mixed-step chunks 122 -> 120 us, the mixed step 451 -> 444 us.
#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 8
#endif
constexpr int kPrefillWaves = PA_PREFILL_WAVES;
// Cache policy of the prefill's KV block loads (0: default; 2: nt). Several
// workgroups (the tiles of one request) read the same blocks, so they are
// not marked as streaming data by default.
#ifndef PA_PF_LOAD_AUX
#define PA_PF_LOAD_AUX 0
#endif
constexpr int kPfAux = PA_PF_LOAD_AUX;
constexpr int kPrefillThreads = kPrefillWaves * kWave;
static_assert(PA_PREFILL_RING % 4 == 0, "the ring (halved for fp32) alternates two LDS buffers");

// How one workgroup of the 16-row tile stages a block's head slice (16 keys)
// in LDS, in the cache's storage type.
template <class E, int D>
struct Stage {
  using KS = typename Ops<E, D>::kv_storage;
  static constexpr int kRowBytes = D * (int)sizeof(KS);     // one key's slice
  static constexpr int kLdsRow = kRowBytes + 16;            // padded: no bank conflicts
  static constexpr int kChunksPerRow = kRowBytes / 16;
  static constexpr int kChunks = kBlockTokens * kChunksPerRow;
  static constexpr int kPerThread = (kChunks + kPrefillThreads - 1) / kPrefillThreads;
  struct Regs {
    u32x4 k[kPerThread];
    u32x4 v[kPerThread];
  };
};

// Query rows and keys of one prefill request (cu_seqlens and seq_lens
// clamped to the batch and the block table like the other kernels).
struct PfRequest {
  int q_lo, n, seq_len, ctx;
};
__device__ inline PfRequest pf_request(const AttnArgs& a, int r) {
  int lo = a.cu_seqlens[r], hi = a.cu_seqlens[r + 1];
  lo = min(max(lo, 0), a.num_tokens);
  hi = min(max(hi, lo), a.num_tokens);
  PfRequest q;
  q.q_lo = lo;
  q.n = hi - lo;
  q.seq_len = min(max(a.seq_lens[r], 0), (a.max_blocks * kBlockTokens) << a.block_shift);
  q.ctx = max(q.seq_len - q.n, 0);
  return q;
}
// A request is a prefill chunk when its query rows fill more than one tile.
__device__ inline bool pf_is_prefill(const PfRequest& q, int g) { return q.n * g > kTileRows; }
__device__ inline int pf_tiles(const PfRequest& q, int tile_tokens) {
  return (q.n + tile_tokens - 1) / tile_tokens;
}
// KV blocks tile `tile` reads: keys up to its last row's causal limit.
__device__ inline int pf_tile_blocks(const AttnArgs& a, const PfRequest& q, int tile,
                                     int tile_tokens) {
  const int tile_end = min((tile + 1) * tile_tokens, q.n);
  const int kmax = a.causal ? min(q.ctx + tile_end, q.seq_len) : q.seq_len;
  return (kmax + kBlockTokens - 1) / kBlockTokens;
}

// Double-buffered LDS copies of the KV blocks' head slices (16-row tile).
template <class E, int D>
struct PfLds {
  char k[2][kBlockTokens * Stage<E, D>::kLdsRow];
  char v[2][kBlockTokens * Stage<E, D>::kLdsRow];
};

// One piece: KV blocks [b0, b1) of tile `tile` of request r (rq) for KV
// head kvh, against all the tile's query rows (each wave RT row tiles). With
// slot < 0 the piece is the whole tile and its rows go to the output; else
// its normalised partial rows and log2-domain LSEs go to partial slot `slot`
// (rows in tile order: (wave * RT + rt) * 16 + row). Called by every thread
// of the workgroup; the caller separates consecutive pieces by a barrier.
template <class E, int D, int RT, int RING>
__device__ inline void pf_piece(const AttnArgs& a, PfLds<E, D>& lds, const PfRequest& rq, int r,
                                int kvh, int tile, int b0, int b1, int64_t slot) {
  using O = Ops<E, D>;
  using S = typename O::storage;       // q and outputs
  using KS = typename O::kv_storage;   // the cache
  using St = Stage<E, D>;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = a.group;
  const int tpw = kTileRows / g;                        // tokens per row tile
  const int tok_base = tile * (kPrefillWaves * RT * tpw);
  const int n = rq.n, seq_len = rq.seq_len, ctx = rq.ctx, q_lo = rq.q_lo;

  // this wave's row tiles
  const int row = lane & 15, grp = lane >> 4;
  typename O::Q q[RT];
  RowState<D> st[RT];
  int key_end[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int tok0 = tok_base + (wave * RT + rt) * tpw;
    const int tok = tok0 + row / g, hh = row - (row / g) * g;
    const bool valid = row < tpw * g && tok < n;
    key_end[rt] = !valid ? 0 : (a.causal ? min(ctx + tok + 1, seq_len) : seq_len);
    const S* qrow = static_cast<const S*>(a.q) +
                    ((int64_t)(q_lo + (valid ? tok : 0)) * a.num_heads + kvh * g + hh) * D;
    O::load_q(q[rt], qrow, valid, lane);
    st[rt].init();
  }

  // staging of KV blocks: HBM -> registers (ring) -> LDS (two buffers)
  const int64_t rs = (int64_t)a.num_kv_heads * D;
  const int64_t block_elems = (int64_t)kBlockTokens * rs;
  const int row_bytes_g = (int)(rs * (int64_t)sizeof(KS));
  const KS* k_head = static_cast<const KS*>(a.k_cache) + (int64_t)kvh * D;
  const KS* v_head = static_cast<const KS*>(a.v_cache) + (int64_t)kvh * D;
  const __attribute__((address_space(4))) int32_t* tab =
      (const __attribute__((address_space(4))) int32_t*)(a.block_table + (int64_t)r * a.max_blocks);
  auto issue = [&](typename St::Regs& rg, int i) {
    const int li = min(i, b1 - 1);
    const int pb = block16(tab[li >> a.block_shift], li, a.block_shift, a.num_blocks);
    const bool ok = i < b1 && pb >= 0;
    const int keys = min(seq_len - i * kBlockTokens, kBlockTokens);
    const int range = ok ? keys * row_bytes_g : 0;
    const int64_t base = (int64_t)(ok ? pb : 0) * block_elems;
    const Rsrc rk = make_rsrc(k_head + base, range), rv = make_rsrc(v_head + base, range);
#pragma unroll
    for (int p = 0; p < St::kPerThread; ++p) {
      const int c = tid + p * kPrefillThreads;
      // a thread without a chunk reads past the range: zeros, no memory access
      const int off = c < St::kChunks
                          ? (c / St::kChunksPerRow) * row_bytes_g + (c % St::kChunksPerRow) * 16
                          : 0x7ffffff0;
      rg.k[p] = buf_load16<kPfAux>(rk, off);
      rg.v[p] = buf_load16<kPfAux>(rv, off);
    }
  };
  auto stage = [&](const typename St::Regs& rg, int buf) {
#pragma unroll
    for (int p = 0; p < St::kPerThread; ++p) {
      const int c = tid + p * kPrefillThreads;
      if (c < St::kChunks) {
        const int off = (c / St::kChunksPerRow) * St::kLdsRow + (c % St::kChunksPerRow) * 16;
        *reinterpret_cast<u32x4*>(&lds.k[buf][off]) = rg.k[p];
        *reinterpret_cast<u32x4*>(&lds.v[buf][off]) = rg.v[p];
      }
    }
  };

  // a negative softmax scale is applied as a positive one to -q (exact), as
  // the unmasked blocks need
  const bool neg = a.scale_log2 < 0.f;
  const float scale_log2 = neg ? -a.scale_log2 : a.scale_log2;
  if (neg) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) O::negate_q(q[rt]);
  }

  // keys at or past b1 * 16 belong to the next piece
  int kend[RT];
  int kmin = 0x7fffffff;  // the fewest keys any valid row of this wave sees
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    kend[rt] = min(key_end[rt], b1 * kBlockTokens);
    const int tok = tok_base + (wave * RT + rt) * tpw + row / g;
    if (row < tpw * g && tok < n) kmin = min(kmin, kend[rt]);
  }
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) kmin = min(kmin, __shfl_xor(kmin, m, kWave));
  // blocks before b_full are visible whole to every valid row: no mask
  const int b_full = __builtin_amdgcn_readfirstlane(min(b1, kmin / kBlockTokens));

  typename St::Regs ring[RING];
#pragma unroll
  for (int j = 0; j < RING; ++j) issue(ring[j], b0 + j);
  // One group of RING blocks; the ring slot of block i is (i - b0) % RING.
  // Blocks are consumed unconditionally, like the loads: a padding block at
  // or past b1 was read as zeros and its keys are past every row's limit
  // (kend), so it adds nothing, and the accumulators stay in one set of
  // registers.
  auto group = [&](int i0, auto masked) {
#pragma unroll
    for (int j = 0; j < RING; ++j) {
      const int i = i0 + j;
      const int buf = j & 1;
      stage(ring[j], buf);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      issue(ring[j], i + RING);
      __builtin_amdgcn_sched_barrier(0);
      typename O::KV kv;
      O::load_lds(kv, lds.k[buf], lds.v[buf], St::kLdsRow, lane);
      consume_block_tiles<E, D, RT, decltype(masked)::value>(st, kv, q, i * kBlockTokens, kend,
                                                             scale_log2, lane);
    }
  };
  int i0 = b0;
  for (; i0 + RING <= b_full; i0 += RING) group(i0, std::false_type{});
  for (; i0 < b1; i0 += RING) group(i0, std::true_type{});

  // epilogue: normalise and store every valid row (partials when cut)
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    st[rt].l = sum_xor16(st[rt].l);
    st[rt].l = sum_xor32(st[rt].l);
    const int tok0 = tok_base + (wave * RT + rt) * tpw;
    const int tok = tok0 + row / g, hh = row - (row / g) * g;
    if (row < tpw * g && tok < n) {
      // out_scale: an E4M3 cache's V scale (1 otherwise); partial rows carry
      // it too, and the merge's weighted mean keeps it
      const float inv = (st[rt].l > 0.f ? 1.f / st[rt].l : 0.f) * a.out_scale;
      if (slot < 0) {
        const int64_t orow = (int64_t)(q_lo + tok) * a.num_heads + kvh * g + hh;
        S* dst = static_cast<S*>(a.out) + orow * D + (D / 4) * grp;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v[D / 16];
#pragma unroll
          for (int c = 0; c < D / 16; ++c) v[c] = st[rt].o[c][i] * inv;
          store_chunk<E, D>(dst + (D / 16) * i, v);
        }
      } else {
        const int64_t prow =
            slot * (kPrefillWaves * RT * kTileRows) + (wave * RT + rt) * kTileRows + row;
        S* dst = static_cast<S*>(a.pf_o) + prow * D + (D / 4) * grp;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v[D / 16];
#pragma unroll
          for (int c = 0; c < D / 16; ++c) v[c] = st[rt].o[c][i] * inv;
          store_chunk<E, D>(dst + (D / 16) * i, v);
        }
        if (grp == 0) a.pf_lse[prow] = st[rt].l > 0.f ? st[rt].m + fast_log2(st[rt].l) : neg_inf();
      }
    }
  }
}

// ------------------------------------------------------------ 32-row tiles
// 16-bit operands (16-bit caches, and E4M3 caches widened to bf16 in LDS)
// take 32 query rows per wave and a pair of blocks (32 keys)
// per step on 32x32x16 MFMAs. S^T = K.Q^T leaves each lane 16 scores of one
// query row -- register 4J + I holds key 8J + 4h + I of the pair, h being the
// lane's half of the wave -- so a row's maximum is 15 in-lane maxima and one
// exchange between the halves. P stays in its lane as the B operand of
// O^T += V^T.P^T, one product per block and 32-dim chunk: contraction slot
// 8h + 4J' + I of block b is key 8J' + 4h + I, i.e. registers 8b .. 8b + 7.
// The matching A operand is V at keys {4h + I} and {8 + 4h + I} of the
// block, one dim per lane row: V is staged in LDS transposed by key quads
// (entry (quad, dim) = that dim of four consecutive keys, 8 bytes), so each
// operand is two entries read as they are, with no permutes. Output rows are
// dims (D/32)(8J + 4h + I) + c of chunk c, so each lane stores 4D/32
// consecutive dims per J.
template <class E>
constexpr bool pf32() {
  return sizeof(typename E::storage) == 2;
}
typedef float f32x16 __attribute__((ext_vector_type(16)));
template <class E>
__device__ inline f32x16 mma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (std::is_same<E, F16>::value)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else  // bf16, and E4M3 codes widened to bf16
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <int D>
struct T32 {
  static constexpr int kQc = D / 16;                          // QK products per pair
  static constexpr int kOc = D / 32;                          // 32-dim output chunks
  static constexpr int kKRow = 2 * D + 16;                    // padded K row in LDS (bytes)
  static constexpr int kKPieces = kBlockTokens * (2 * D / 16);  // 16-byte K pieces per block
  static constexpr int kVItems = 4 * (D / 2);                 // (key quad, dim pair) items per block
  static constexpr int kVQuad = 8 * D;                        // bytes of one key quad in LDS
  // LDS slot of dim entry e inside a quad. An operand read takes entry
  // kOc * dslot + c (8 bytes) in lane dslot = 0..31; unswizzled, lanes 4 or 8
  // (D = 128, 64) apart hit the same banks. The entry index within each run
  // of kOc is XORed with bits of dslot chosen so that any 16 lanes cover 32
  // four-byte banks, and any 32 lanes 64 banks, once each.
  __device__ static int vpos(int e) {
    return D == 128 ? e ^ (((e >> 4) ^ (e >> 6)) & 3) : e ^ (((e >> 4) ^ (e >> 5)) & 1);
  }
};
static_assert(kPrefillWaves * kWave >= T32<128>::kKPieces && kPrefillWaves * kWave >= T32<128>::kVItems,
              "one staging item per thread and block");
// Block pairs consumed per barrier by the 32-row tile (1 or 2). Two pairs
// share one row maximum, reference update and rescale test, their score
// products are independent chains, and barriers and block addressing are
// halved: mixed-step chunks 119 -> 113 us (min), at 249 VGPRs and 100 KB of
// LDS per workgroup.
#ifndef PA_PF32_PAIRS
#define PA_PF32_PAIRS 2
#endif
constexpr int kPf32Pairs = PA_PF32_PAIRS;
// Thread groups that share the staging of a step's blocks on a 16-bit cache
// (1: every thread < 2 D stages a piece of every block).
#ifndef PA_PF32_STAGE_GROUPS
#define PA_PF32_STAGE_GROUPS 1
#endif
// Whether a step's blocks are staged in LDS in the middle of the previous
// step (1) or at its own start, right before its barrier (0), for E4M3 and
// for 16-bit caches.
#ifndef PA_PF32_MIDSTAGE_CODES
#define PA_PF32_MIDSTAGE_CODES 1
#endif
#ifndef PA_PF32_MIDSTAGE_16
#define PA_PF32_MIDSTAGE_16 0
#endif
template <int D>
struct PfLds32 {
  char k[2][2 * kPf32Pairs][kBlockTokens * T32<D>::kKRow];  // [buffer][block][key row]
  char v[2][2 * kPf32Pairs][4 * T32<D>::kVQuad];            // [buffer][block][quad][dim][4 keys]
};
// One block's staging registers of a thread: a 16-byte K piece, and one dword
// (two dims, or four E4M3 codes) of each of the four keys of a V quad.
struct Regs32 {
  u32x4 k;
  u32x4 v;
};

// As pf_piece, for 16-bit operands with 32 rows per wave (partial rows in
// tile order: wave * 32 + row). A 16-bit cache is staged as it is; an E4M3
// cache's codes are widened exactly to bf16 on their way into LDS, so the
// LDS layout and everything after it are the bf16 tile's.
template <class E, int D, int RING>
__device__ inline void pf_piece32(const AttnArgs& a, PfLds32<D>& lds, const PfRequest& rq, int r,
                                  int kvh, int tile, int b0, int b1, int64_t slot) {
  using T = T32<D>;
  using S = typename E::storage;
  using KS = typename E::kv_storage;
  static_assert(RING % 4 == 0, "pairs alternate between two LDS pair buffers");
  constexpr bool kCodes = sizeof(KS) == 1;  // an E4M3 cache
  constexpr int kStep = 2 * kPf32Pairs;     // blocks per barrier
  static_assert(RING % kStep == 0, "whole steps per group");
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = a.group;
  const int tpw = 32 / g;  // query tokens per wave
  const int tok_base = tile * (kPrefillWaves * tpw);
  const int n = rq.n, seq_len = rq.seq_len, ctx = rq.ctx, q_lo = rq.q_lo;
  const int j = lane & 31, h = lane >> 5;  // the lane's query row (and key row, dim slot) and half

  // the lane's query row: token tok, head hh of the GQA group
  const int tok = tok_base + wave * tpw + j / g, hh = j - (j / g) * g;
  const bool valid = j < tpw * g && tok < n;
  const int key_end = !valid ? 0 : (a.causal ? min(ctx + tok + 1, seq_len) : seq_len);
  u32x4 q[T::kQc];
  {
    const S* qrow = static_cast<const S*>(a.q) +
                    ((int64_t)(q_lo + (valid ? tok : 0)) * a.num_heads + kvh * g + hh) * D;
#pragma unroll
    for (int c = 0; c < T::kQc; ++c)
      q[c] = valid ? *reinterpret_cast<const u32x4*>(qrow + 16 * c + 8 * h) : u32x4{0u, 0u, 0u, 0u};
  }
  // a negative softmax scale is applied as a positive one to -q (exact)
  const bool neg = a.scale_log2 < 0.f;
  const float scale_log2 = neg ? -a.scale_log2 : a.scale_log2;
  if (neg) {
#pragma unroll
    for (int c = 0; c < T::kQc; ++c) q[c] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  }

  float m = neg_inf(), l = 0.f;
  f32x16 o[T::kOc];
#pragma unroll
  for (int c = 0; c < T::kOc; ++c) o[c] = f32x16{};

  // keys at or past b1 * 16 belong to the next piece; blocks before b_full
  // are visible whole to every valid row of the wave (no mask)
  const int kend = min(key_end, b1 * kBlockTokens);
  int kmin = valid ? kend : 0x7fffffff;
#pragma unroll
  for (int s = 1; s < kWave; s <<= 1) kmin = min(kmin, __shfl_xor(kmin, s, kWave));
  const int b_full = __builtin_amdgcn_readfirstlane(min(b1, kmin / kBlockTokens));

  // staging: HBM -> registers (ring of RING blocks) -> LDS (two pair buffers)
  const int64_t rs = (int64_t)a.num_kv_heads * D;
  const int64_t block_elems = (int64_t)kBlockTokens * rs;
  const int row_bytes_g = (int)(rs * (int64_t)sizeof(KS));
  const KS* k_head = static_cast<const KS*>(a.k_cache) + (int64_t)kvh * D;
  const KS* v_head = static_cast<const KS*>(a.v_cache) + (int64_t)kvh * D;
  const __attribute__((address_space(4))) int32_t* tab =
      (const __attribute__((address_space(4))) int32_t*)(a.block_table + (int64_t)r * a.max_blocks);
  // Staging items: the threads form kGroups groups and group qb stages
  // blocks qb * kPer .. qb * kPer + kPer - 1 of each step, item `it` of each.
  // An item is a 16-byte piece of K (16-bit cache: 8 dims of one key; E4M3:
  // 16 codes, 16 dims) and a dword of each of the four keys of a V quad (2
  // dims, or 4 codes). E4M3 blocks are half the bytes, so every group takes
  // one block per step; 16-bit caches take PA_PF32_STAGE_GROUPS groups.
  constexpr int kGroups = kCodes ? kStep : PA_PF32_STAGE_GROUPS;
  static_assert(kStep % kGroups == 0, "whole blocks per staging group");
  constexpr int kPer = kStep / kGroups;                  // blocks of a step per thread
  constexpr int kGroupThreads = kPrefillThreads / kGroups;
  constexpr int kItems = kCodes ? D : T::kKPieces;       // items per block (K pieces = V items)
  static_assert(kCodes || T::kKPieces == T::kVItems, "one K piece and one V item per staging item");
  static_assert(kGroupThreads >= kItems, "one staging item per thread and block");
  const int qb = kGroups > 1 ? __builtin_amdgcn_readfirstlane(tid / kGroupThreads) : 0;
  const int it = tid - qb * kGroupThreads;
  const bool k_item = it < kItems, v_item = it < kItems;
  constexpr int kPiecesPerRow = D * (int)sizeof(KS) / 16;  // 16-byte pieces of a key's slice
  constexpr int kVDims = 4 / (int)sizeof(KS);              // dims of one V dword
  // a thread without an item reads past every range: zeros, no memory access
  const int k_goff = k_item ? (it / kPiecesPerRow) * row_bytes_g + (it % kPiecesPerRow) * 16
                            : 0x40000000;
  const int k_loff = (it / kPiecesPerRow) * T::kKRow + (it % kPiecesPerRow) * 16 * (int)(2 / sizeof(KS));
  const int vq = it / (D / kVDims), vd = it % (D / kVDims);
  const int v_goff = v_item ? 4 * vq * row_bytes_g + 4 * vd : 0x40000000;
  // entries d and d + 1 (d even) land in one aligned 16-byte slot, swapped
  // when the swizzle flips bit 0; an E4M3 item has two such pairs
  const int vd0 = kVDims * vd;
  const int v_loff = vq * T::kVQuad + 8 * (T::vpos(vd0) & ~1);
  const bool v_swap = (T::vpos(vd0) & 1) != 0;
  const int v_loff2 = vq * T::kVQuad + 8 * (T::vpos(vd0 + 2) & ~1);
  const bool v_swap2 = (T::vpos(vd0 + 2) & 1) != 0;
  // Block ids of the loop's loads are read one group ahead by a vector load
  // (lane k: block first + k) and taken from their lanes when used: scalar
  // loads would share the LDS reads' wait counter, and every wait for an LDS
  // result would then wait for them too.
  const __attribute__((address_space(1))) int32_t* tabv =
      (const __attribute__((address_space(1))) int32_t*)(a.block_table + (int64_t)r * a.max_blocks);
  auto load_ids = [&](int first) {
    const int li = min(first + (lane & (RING - 1)), b1 - 1);
    return block16(tabv[li >> a.block_shift], li, a.block_shift, a.num_blocks);
  };
  // pb: the pool's 16-token block, or -1 (outside the pool)
  auto issue = [&](Regs32& rg, int i, int pb) {
    const bool ok = i < b1 && pb >= 0;
    const int keys = min(seq_len - i * kBlockTokens, kBlockTokens);
    const int range = ok ? keys * row_bytes_g : 0;
    const int64_t base = (int64_t)(ok ? pb : 0) * block_elems;
    const Rsrc rk = make_rsrc(k_head + base, range), rv = make_rsrc(v_head + base, range);
    rg.k = buf_load16<kPfAux>(rk, k_goff);
    rg.v.x = buf_load4<kPfAux>(rv, v_goff);
    rg.v.y = buf_load4<kPfAux>(rv, v_goff + row_bytes_g);
    rg.v.z = buf_load4<kPfAux>(rv, v_goff + 2 * row_bytes_g);
    rg.v.w = buf_load4<kPfAux>(rv, v_goff + 3 * row_bytes_g);
  };
  // x0 .. x3: two dims d, d + 1 (low, high halves) of keys 4vq .. 4vq + 3,
  // as the entries (d: 4 keys) and (d + 1: 4 keys) at loff
  auto put_v_pair = [&](int s, int bsel, unsigned x0, unsigned x1, unsigned x2, unsigned x3,
                        int loff, bool swap) {
    const u32x2 e0 = {__builtin_amdgcn_perm(x1, x0, 0x05040100u),
                      __builtin_amdgcn_perm(x3, x2, 0x05040100u)};
    const u32x2 e1 = {__builtin_amdgcn_perm(x1, x0, 0x07060302u),
                      __builtin_amdgcn_perm(x3, x2, 0x07060302u)};
    const u32x2 first = swap ? e1 : e0, second = swap ? e0 : e1;
    *reinterpret_cast<u32x4*>(&lds.v[s][bsel][loff]) = u32x4{first.x, first.y, second.x, second.y};
  };
  auto stage = [&](const Regs32& rg, int s, int bsel) {
    if constexpr (kCodes) {
      if (it < D) {
        // every E4M3 value is a bf16 value: exact widening
        unsigned w[8];
        fp8x4_to_bf16(rg.k.x, &w[0], &w[1]);
        fp8x4_to_bf16(rg.k.y, &w[2], &w[3]);
        fp8x4_to_bf16(rg.k.z, &w[4], &w[5]);
        fp8x4_to_bf16(rg.k.w, &w[6], &w[7]);
        char* kd = &lds.k[s][bsel][k_loff];
        *reinterpret_cast<u32x4*>(kd) = u32x4{w[0], w[1], w[2], w[3]};
        *reinterpret_cast<u32x4*>(kd + 16) = u32x4{w[4], w[5], w[6], w[7]};
        unsigned lo[4], hi[4];  // key i: dims vd0, vd0 + 1 and vd0 + 2, vd0 + 3
        fp8x4_to_bf16(rg.v.x, &lo[0], &hi[0]);
        fp8x4_to_bf16(rg.v.y, &lo[1], &hi[1]);
        fp8x4_to_bf16(rg.v.z, &lo[2], &hi[2]);
        fp8x4_to_bf16(rg.v.w, &lo[3], &hi[3]);
        put_v_pair(s, bsel, lo[0], lo[1], lo[2], lo[3], v_loff, v_swap);
        put_v_pair(s, bsel, hi[0], hi[1], hi[2], hi[3], v_loff2, v_swap2);
      }
    } else {
      if (k_item) *reinterpret_cast<u32x4*>(&lds.k[s][bsel][k_loff]) = rg.k;
      if (v_item) put_v_pair(s, bsel, rg.v.x, rg.v.y, rg.v.z, rg.v.w, v_loff, v_swap);
    }
  };

  // S^T of pair pp in LDS buffer s (keys x rows, 32 x 32)
  auto qk = [&](int s, int pp) {
    const char* kb = &lds.k[s][2 * pp + (j >> 4)][(j & 15) * T::kKRow + 16 * h];
    u32x4 kk[T::kQc];
#pragma unroll
    for (int c = 0; c < T::kQc; ++c) kk[c] = *reinterpret_cast<const u32x4*>(kb + 32 * c);
    // all of the pair's K reads go out before its first product (left to
    // itself the compiler waits for each read just before its product)
    __builtin_amdgcn_sched_barrier(0);
    f32x16 acc = {};
#pragma unroll
    for (int c = 0; c < T::kQc; ++c) acc = mma32<E>(kk[c], q[c], acc);
    return acc;
  };
  // online softmax of NP pairs' scores (pair pp: keys key0 + 32 pp ..
  // + 31): the probabilities relative to the row's reference m, and the
  // factor for o and l when m moves (one maximum and one reference update
  // for all NP pairs)
  auto softmax = [&](const f32x16 (&acc)[kPf32Pairs], int key0, float (&p)[kPf32Pairs][16],
                     auto masked) {
    float alpha;
    if constexpr (decltype(masked)::value) {
      float sv[kPf32Pairs][16];
      float mx = neg_inf();
#pragma unroll
      for (int pp = 0; pp < kPf32Pairs; ++pp)
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int key = key0 + 32 * pp + 8 * (t >> 2) + 4 * h + (t & 3);
          sv[pp][t] = key < kend ? acc[pp][t] * scale_log2 : neg_inf();
          mx = fmax2(mx, sv[pp][t]);
        }
      mx = max_xor32(mx);
      alpha = advance_max(m, mx);
      const float m_use = m == neg_inf() ? 0.f : m;
#pragma unroll
      for (int pp = 0; pp < kPf32Pairs; ++pp)
#pragma unroll
        for (int t = 0; t < 16; ++t) p[pp][t] = fast_exp2(sv[pp][t] - m_use);
    } else {
      // every key visible and scale_log2 >= 0: the scaled maximum of the raw
      // scores is the maximum of the scaled ones, and each exponent is one
      // fused multiply-add
      float mx = acc[0][0];
#pragma unroll
      for (int pp = 0; pp < kPf32Pairs; ++pp)
#pragma unroll
        for (int t = 0; t < 16; ++t) mx = fmax2(mx, acc[pp][t]);
      mx = max_xor32(mx) * scale_log2;
      alpha = advance_max(m, mx);
      const float neg_m = -m;
#pragma unroll
      for (int pp = 0; pp < kPf32Pairs; ++pp)
#pragma unroll
        for (int t = 0; t < 16; ++t) p[pp][t] = fast_exp2(__builtin_fmaf(acc[pp][t], scale_log2, neg_m));
    }
    return alpha;
  };
  // l and o take the pairs: rescale when the reference moved, then P.V with
  // the values from LDS buffer s
  auto accumulate = [&](const float (&p)[kPf32Pairs][16], float alpha, int s) {
    float ps = 0.f;
#pragma unroll
    for (int pp = 0; pp < kPf32Pairs; ++pp)
#pragma unroll
      for (int t = 0; t < 16; t += 4) ps += (p[pp][t] + p[pp][t + 1]) + (p[pp][t + 2] + p[pp][t + 3]);
    l = l * alpha + ps;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int c = 0; c < T::kOc; ++c) o[c] *= alpha;
    }
#pragma unroll
    for (int b = 0; b < 2 * kPf32Pairs; ++b) {
      const float* pb = &p[b >> 1][8 * (b & 1)];
      const u32x4 pk = {E::pack2(pb[0], pb[1]), E::pack2(pb[2], pb[3]), E::pack2(pb[4], pb[5]),
                        E::pack2(pb[6], pb[7])};
      const char* vb = &lds.v[s][b][0];
#pragma unroll
      for (int c = 0; c < T::kOc; ++c) {
        const int e = 8 * T::vpos(T::kOc * j + c);
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vb + h * T::kVQuad + e);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vb + (h + 2) * T::kVQuad + e);
        o[c] = mma32<E>(u32x4{lo.x, lo.y, hi.x, hi.y}, pk, o[c]);
      }
    }
  };

  // Two stagings. Either each step's blocks are staged right before its
  // barrier (16-bit caches), or step k's blocks (LDS buffer k & 1) are
  // staged in the middle of step k - 1, once its score products are issued
  // (E4M3 caches, whose staging every wave shares): every wave passed step
  // k - 1's barrier after its last reads of that buffer (step k - 2), so it
  // is free, and the LDS writes, which queue behind the other waves' operand
  // reads, have the rest of the step to finish. Either way a step's loads
  // are issued one step ahead of its staging. Measured on the mixed step's
  // chunks: E4M3 mid-step 109-111 us against 112-114; 16-bit caches, whose
  // staging falls on waves 0-3 alone, 119 us against 112-113.
  constexpr bool kMid = kCodes ? PA_PF32_MIDSTAGE_CODES : PA_PF32_MIDSTAGE_16;
  static_assert(!kMid || RING == kStep, "mid-step staging: one step of blocks in flight");
  int nid = load_ids(b0 + RING);  // lane k: the id of the block the group's load k reads
  // the blocks of a group this thread stages: its kPer blocks of each of the
  // group's RING / kStep steps (ring slot (step, bb) = step * kPer + bb)
  constexpr int kMine = RING / kStep * kPer;
  Regs32 ring[kMine];
#pragma unroll
  for (int m = 0; m < kMine; ++m) {
    const int jj = (m / kPer) * kStep + qb * kPer + m % kPer;
    const int li = min(b0 + jj, b1 - 1);
    issue(ring[m], b0 + jj, block16(tab[li >> a.block_shift], li, a.block_shift, a.num_blocks));
  }
  if constexpr (kMid) {
    // step 0 into buffer 0, then step 1's loads
#pragma unroll
    for (int bb = 0; bb < kPer; ++bb) stage(ring[bb], 0, qb * kPer + bb);
#pragma unroll
    for (int bb = 0; bb < kPer; ++bb) {
      const int blk = qb * kPer + bb;  // this thread's block of the step
      issue(ring[bb], b0 + RING + blk, __builtin_amdgcn_readlane(nid, blk));
    }
    nid = load_ids(b0 + 2 * RING);  // ids of step 2
  }
  // take the ids in here (a wait for the one load issued before the ring's):
  // entering the loop with the load still pending makes the compiler wait
  // for nearly every load at the top of each group
  asm volatile("" ::"v"(nid));
  // One group of RING blocks (RING / 2 pairs); the ring slot of block i is
  // (i - b0) % RING. Blocks are consumed unconditionally, like the loads: a
  // padding block at or past b1 was read as zeros and its keys are past
  // every row's limit (kend), so it adds nothing.
  // With kPf32Pairs == 2 a group is one step of 4 blocks and the LDS buffer
  // alternates between groups.
  auto group = [&](int i0, auto masked) {
    if constexpr (kMid) {
      const int s = ((i0 - b0) / kStep) & 1;
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      f32x16 acc[kPf32Pairs];
#pragma unroll
      for (int pp = 0; pp < kPf32Pairs; ++pp) acc[pp] = qk(s, pp);
      __builtin_amdgcn_sched_barrier(0);
      const int nxt = load_ids(i0 + 3 * RING);
#pragma unroll
      for (int bb = 0; bb < kPer; ++bb) stage(ring[bb], s ^ 1, qb * kPer + bb);
#pragma unroll
      for (int bb = 0; bb < kPer; ++bb) {
        const int blk = qb * kPer + bb;
        issue(ring[bb], i0 + 2 * RING + blk, __builtin_amdgcn_readlane(nid, blk));
      }
      __builtin_amdgcn_sched_barrier(0);
      float pr[kPf32Pairs][16];
      const float alpha = softmax(acc, i0 * kBlockTokens, pr, masked);
      accumulate(pr, alpha, s);
      nid = nxt;
    } else {
      const int nxt = load_ids(i0 + 2 * RING);
#pragma unroll
      for (int jj = 0; jj < RING; jj += kStep) {
        const int i = i0 + jj;
        const int s = RING / kStep >= 2 ? (jj / kStep) & 1 : ((i - b0) / kStep) & 1;
#pragma unroll
        for (int bb = 0; bb < kPer; ++bb) stage(ring[jj / kStep * kPer + bb], s, qb * kPer + bb);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int bb = 0; bb < kPer; ++bb) {
          const int blk = qb * kPer + bb;  // this thread's block of the step
          issue(ring[jj / kStep * kPer + bb], i + blk + RING,
                __builtin_amdgcn_readlane(nid, jj + blk));
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x16 acc[kPf32Pairs];
#pragma unroll
        for (int pp = 0; pp < kPf32Pairs; ++pp) acc[pp] = qk(s, pp);
        float pr[kPf32Pairs][16];
        const float alpha = softmax(acc, i * kBlockTokens, pr, masked);
        accumulate(pr, alpha, s);
      }
      nid = nxt;
    }
  };
  int i0 = b0;
  for (; i0 + RING <= b_full; i0 += RING) group(i0, std::false_type{});
  for (; i0 < b1; i0 += RING) group(i0, std::true_type{});

  // epilogue: normalise and store (partials when cut)
  l = sum_xor32(l);
  if (valid) {
    const float inv = (l > 0.f ? 1.f / l : 0.f) * a.out_scale;
    constexpr int kRun = 4 * T::kOc;  // consecutive dims per J
    // the output row, or the piece's partial row (same type)
    const int64_t prow = slot * (kPrefillWaves * 32) + wave * 32 + j;
    S* dst = slot < 0 ? static_cast<S*>(a.out) + ((int64_t)(q_lo + tok) * a.num_heads + kvh * g + hh) * D
                      : static_cast<S*>(a.pf_o) + prow * D;
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      unsigned w[kRun / 2];
#pragma unroll
      for (int x = 0; x < kRun; x += 2) {
        // value x of the run is dim slot 8J + 4h + x / kOc, chunk x % kOc
        w[x / 2] = E::pack2(o[x % T::kOc][4 * J + x / T::kOc] * inv,
                            o[(x + 1) % T::kOc][4 * J + (x + 1) / T::kOc] * inv);
      }
      S* d = dst + T::kOc * (8 * J + 4 * h);
#pragma unroll
      for (int x = 0; x < kRun / 2; x += 4)
        *reinterpret_cast<u32x4*>(d + 2 * x) = u32x4{w[x], w[x + 1], w[x + 2], w[x + 3]};
    }
    if (slot >= 0 && h == 0) a.pf_lse[prow] = l > 0.f ? m + fast_log2(l) : neg_inf();
  }
}

// fp32 operands are twice the size: half the row tiles and half the ring.
template <class E>
constexpr int prefill_rt() {
  return sizeof(typename E::storage) == 4 ? (PA_PREFILL_RT + 1) / 2 : PA_PREFILL_RT;
}
template <class E>
constexpr int prefill_ring() {
  return sizeof(typename E::storage) == 4 ? PA_PREFILL_RING / 2 : PA_PREFILL_RING;
}

// Query rows per wave and query tokens per wave of the prefill tiles.
template <class E>
constexpr int pf_wave_rows() {
  return pf32<E>() ? 32 : kTileRows * prefill_rt<E>();
}
// Rows of one unit of the row layout: a 32-row wave tile, or a 16-row tile.
template <class E>
constexpr int pf_unit_rows() {
  return pf32<E>() ? 32 : kTileRows;
}
template <class E>
__device__ __host__ inline int pf_wave_tokens(int g) {
  return (pf_wave_rows<E>() / pf_unit_rows<E>()) * (pf_unit_rows<E>() / g);
}
template <class E, int D>
using PfLdsOf = typename std::conditional<pf32<E>(), PfLds32<D>, PfLds<E, D>>::type;

template <class E, int D, int RT, int RING>
__device__ inline void pf_run_piece(const AttnArgs& a, PfLdsOf<E, D>& lds, const PfRequest& rq,
                                    int r, int kvh, int tile, int b0, int b1, int64_t slot) {
  if constexpr (pf32<E>())
    pf_piece32<E, D, RING>(a, lds, rq, r, kvh, tile, b0, b1, slot);
  else
    pf_piece<E, D, RT, RING>(a, lds, rq, r, kvh, tile, b0, b1, slot);
}

// One workgroup per (tile, request, KV head), tiles in descending order (the
// tiles that see the most keys start first); every tile written whole.
template <class E, int D, int RT, int RING>
__global__ __launch_bounds__(kPrefillThreads, PA_PREFILL_OCC) void prefill_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) PfLdsOf<E, D> lds;
  int u = blockIdx.x;
  const int kvh = u % a.num_kv_heads;
  u /= a.num_kv_heads;
  const int r = u % a.num_seqs;
  const int tile = a.num_tiles - 1 - u / a.num_seqs;
  const PfRequest rq = pf_request(a, r);
  if (!pf_is_prefill(rq, a.group)) return;  // a single-tile request: the decode kernel's
  const int tile_tokens = kPrefillWaves * pf_wave_tokens<E>(a.group);
  if (tile * tile_tokens >= rq.n) return;
  const int nblk = pf_tile_blocks(a, rq, tile, tile_tokens);
  if (nblk <= 0) return;
  pf_run_piece<E, D, RT, RING>(a, lds, rq, r, kvh, tile, 0, nblk, -1);
}

// Exclusive prefix sum over the workgroup (int64); *total gets the sum.
__device__ inline int64_t pf_exclusive_sum(int64_t v, int64_t* s_tmp, int64_t* total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int64_t x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int64_t y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  if (lane == kWave - 1) s_tmp[wave] = x;
  __syncthreads();
  int64_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kPrefillWaves; ++w) {
    const int64_t t = s_tmp[w];
    off += w < wave ? t : 0;
    tot += t;
  }
  *total = tot;
  return off + x - v;
}

// Share items of a tile: its KV blocks plus the fixed tile cost (0 for a
// tile with no keys, which has nothing to do).
__device__ inline int pf_tile_items(int nblk) { return nblk > 0 ? nblk + PA_PREFILL_TILE_COST : 0; }

// Share items summed over all tiles of a prefill request (one KV head).
__device__ inline int64_t pf_request_items(const AttnArgs& a, const PfRequest& rq,
                                           int tile_tokens) {
  const int tiles = pf_tiles(rq, tile_tokens);
  int64_t sum = 0;
  for (int t = 0; t < tiles; ++t) sum += pf_tile_items(pf_tile_blocks(a, rq, t, tile_tokens));
  return sum;
}

// Writes the merge record of every query token of a tile for one KV head:
// first partial slot, piece count (0: the tile was written whole) and the
// token's first row in the tile's partial slot.
// Rows are laid out in units of `unit` rows (a 16-row tile, or a 32-row
// wave tile), each holding unit / g whole tokens.
template <int UNIT>
__device__ inline void pf_write_records(const AttnArgs& a, const PfRequest& rq, int kvh,
                                        int tile, int tile_tokens, int s0, int cnt) {
  const int g = a.group, tpu = UNIT / g;
  const int t0 = tile * tile_tokens;
  const int nt = min(tile_tokens, rq.n - t0);
  for (int i = threadIdx.x; i < nt; i += kPrefillThreads)
    a.pf_rec[(int64_t)(rq.q_lo + t0 + i) * a.num_kv_heads + kvh] =
        int4{s0, cnt, (i / tpu) * UNIT + (i % tpu) * g, 0};
}

// Equal shares: the W items -- (request, KV head, tile, KV block) in that
// order, prefill requests only, each tile followed by PA_PREFILL_TILE_COST
// items that stand for its fixed cost -- are cut into T = min(pf_shares, W)
// contiguous shares with floor-spaced bounds, one per workgroup (share index
// XCD-major, so neighbouring shares, which mostly read the same request's
// blocks, share an L2). A share walks its pieces; a piece that is a whole
// tile writes the output rows, a cut one its partial slot: 2j for the
// share's first piece, 2j + 1 for its last (only these two can be cut).
// Every piece of a tile writes the records of the tile's tokens (first slot,
// piece count -- 0: written whole -- and row), for the merge; workgroup 0
// writes empty records for the batch's other tokens.
template <class E, int D, int RT, int RING>
__global__ __launch_bounds__(kPrefillThreads, PA_PREFILL_OCC) void prefill_shares_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) PfLdsOf<E, D> lds;
  __shared__ int64_t s_pre[kMaxBalancedSeqs + 1];
  __shared__ int64_t s_tmp[kPrefillWaves];
  const int tid = threadIdx.x;
  const int B = a.num_seqs, hkv = a.num_kv_heads, g = a.group;
  const int tile_tokens = kPrefillWaves * pf_wave_tokens<E>(g);

  // 1. items before each request, in LDS
  const int per = (B + kPrefillThreads - 1) / kPrefillThreads;
  const int c0 = min(tid * per, B), c1 = min(c0 + per, B);
  int64_t chunk = 0;
  for (int i = c0; i < c1; ++i) {
    const PfRequest rq = pf_request(a, i);
    const int64_t items = pf_is_prefill(rq, g) ? hkv * pf_request_items(a, rq, tile_tokens) : 0;
    s_pre[i + 1] = items;
    chunk += items;
    if (blockIdx.x == 0) {
      // tokens no piece covers get an empty record: single-tile requests'
      // tokens and those of tiles without keys
      const bool pre = pf_is_prefill(rq, g);
      for (int t = 0; t < (pre ? pf_tiles(rq, tile_tokens) : 1); ++t) {
        if (pre && pf_tile_blocks(a, rq, t, tile_tokens) > 0) continue;
        const int lo_t = pre ? t * tile_tokens : 0;
        const int hi_t = pre ? min(lo_t + tile_tokens, rq.n) : rq.n;
        for (int tok = lo_t; tok < hi_t; ++tok)
          for (int k = 0; k < hkv; ++k)
            a.pf_rec[(int64_t)(rq.q_lo + tok) * hkv + k] = int4{0, 0, 0, 0};
      }
    }
  }
  int64_t W = 0;
  int64_t run = pf_exclusive_sum(chunk, s_tmp, &W);
  for (int i = c0; i < c1; ++i) {
    run += s_pre[i + 1];
    s_pre[i + 1] = run;
  }
  if (tid == 0) s_pre[0] = 0;
  __syncthreads();

  // 2. this workgroup's share
  const int64_t T = min((int64_t)a.pf_shares, W);
  const int nx = (int)gridDim.x;
  const int64_t j = (nx % 8 == 0) ? (int64_t)(blockIdx.x % 8) * (nx / 8) + blockIdx.x / 8
                                  : (int64_t)blockIdx.x;
  if (j >= T) return;
  auto begin_of = [&](int64_t t) { return t * W / T; };
  auto share_of = [&](int64_t x) { return ((x + 1) * T - 1) / W; };  // share holding item x
  const int64_t lo = begin_of(j), hi = begin_of(j + 1);
  int r_lo = 0, r_hi = B - 1;
  while (r_lo < r_hi) {
    const int mid = (r_lo + r_hi + 1) >> 1;
    if (s_pre[mid] <= lo) r_lo = mid; else r_hi = mid - 1;
  }
  int r = r_lo;
  int64_t x = lo;
  bool first = true;
  while (x < hi) {
    while (r < B - 1 && s_pre[r + 1] <= x) ++r;
    const PfRequest rq = pf_request(a, r);
    const int64_t per_head = (s_pre[r + 1] - s_pre[r]) / hkv;
    const int64_t off = x - s_pre[r];
    const int kvh = (int)(off / per_head);
    int64_t rem = off - (int64_t)kvh * per_head;
    int tile = 0, nblk = pf_tile_blocks(a, rq, 0, tile_tokens), nit = pf_tile_items(nblk);
    while (rem >= nit) {
      rem -= nit;
      ++tile;
      nblk = pf_tile_blocks(a, rq, tile, tile_tokens);
      nit = pf_tile_items(nblk);
    }
    const int b0 = (int)rem;
    const int len = (int)min((int64_t)(nit - b0), hi - x);
    // the piece's KV blocks: items past nblk are the tile's fixed cost
    const int b1 = min(b0 + len, nblk);
    if (b0 < b1) {
      const bool whole = b0 == 0 && b1 == nblk;
      const int64_t slot = whole ? -1 : 2 * j + (x == lo ? 0 : 1);
      if (!first) __syncthreads();  // the previous piece's LDS reads are done
      first = false;
      pf_run_piece<E, D, RT, RING>(a, lds, rq, r, kvh, tile, b0, b1, slot);
      int s0 = 0, cnt = 0;
      if (!whole) {
        // shares holding the tile's first and last KV block
        const int64_t t_begin = x - b0, t_last = t_begin + nblk - 1;
        const int64_t j0 = share_of(t_begin), j1 = share_of(t_last);
        s0 = (int)(2 * j0 + (t_begin == begin_of(j0) ? 0 : 1));
        cnt = (int)(j1 - j0 + 1);
      }
      pf_write_records<pf_unit_rows<E>()>(a, rq, kvh, tile, tile_tokens, s0, cnt);
    }
    x += len;
  }
}

// Renormalises the cut tiles of the equal-share prefill [P1 §07 LSE merge]:
// one wave per (query token, KV head), its g heads side by side (lph lanes
// per head, DPL = D / lph >= 4 dims per lane). The token's record names its
// tile's first partial slot s0 and piece count c (0: nothing to merge); piece
// p > 0 sits at slot 2 (s0 / 2 + p), the first piece of each later share. The
// loads of kPieceBatch pieces are issued together and then folded in with a
// running maximum, so a tile of up to kPieceBatch pieces costs two dependent
// memory round trips (record, then pieces). A record naming slots past the
// workspace is ignored.
constexpr int kPieceBatch = 4;
template <class E, int DPL>
__global__ __launch_bounds__(4 * kWave) void prefill_share_merge_kernel(const AttnArgs a,
                                                                        int pf_rows, int D) {
  using S = typename E::storage;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t unit = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (unit >= (int64_t)a.num_tokens * a.num_kv_heads) return;
  const int4 rec = a.pf_rec[unit];  // unit = token * Hkv + kvh
  const int s0 = rec.x, cnt = rec.y;
  const int64_t slots = 2 * (int64_t)a.pf_shares;
  if (cnt <= 0 || s0 < 0 || s0 >= slots || 2 * ((int64_t)(s0 >> 1) + cnt - 1) >= slots) return;
  const int g = a.group;
  const int lph = D / DPL;  // lanes per head
  const int hh = lane / lph;
  if (hh >= g) return;
  const int d0 = (lane % lph) * DPL;
  const int64_t prow = rec.z + hh;
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
  float m = neg_inf(), l = 0.f;
  for (int p0 = 0; p0 < cnt; p0 += kPieceBatch) {
    float lse[kPieceBatch];
    float v[kPieceBatch][DPL];
#pragma unroll
    for (int k = 0; k < kPieceBatch; ++k) {
      const int p = p0 + k;
      const bool ok = p < cnt;
      const int64_t sr = (p == 0 ? s0 : 2 * ((int64_t)(s0 >> 1) + p)) * pf_rows + prow;
      lse[k] = ok ? a.pf_lse[sr] : neg_inf();
      // a piece past cnt reads slot 0 (in bounds; any bits) and counts as zeros
      const S* o = static_cast<const S*>(a.pf_o) + (ok ? sr : 0) * D + d0;
#pragma unroll
      for (int i = 0; i < DPL; i += 8) {
        if constexpr (DPL >= 8)
          load_part<E, 8>(o + i, &v[k][i]);
        else
          load_part<E, 4>(o + i, &v[k][i]);
      }
#pragma unroll
      for (int i = 0; i < DPL; ++i) v[k][i] = ok ? v[k][i] : 0.f;
    }
    float mn = m;
#pragma unroll
    for (int k = 0; k < kPieceBatch; ++k) mn = fmaxf(mn, lse[k]);
    if (mn == neg_inf()) continue;  // no piece with keys yet
    const float alpha = fast_exp2(m - mn);
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[i] *= alpha;
    l *= alpha;
#pragma unroll
    for (int k = 0; k < kPieceBatch; ++k) {
      const float w = fast_exp2(lse[k] - mn);  // 0 for a piece without keys or past cnt
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc[i] += w * v[k][i];
      l += w;
    }
    m = mn;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int token = (int)(unit / a.num_kv_heads), kvh = (int)(unit - (int64_t)token * a.num_kv_heads);
  S* out = static_cast<S*>(a.out) + ((int64_t)token * a.num_heads + kvh * g + hh) * D + d0;
  // the lane's DPL consecutive outputs in 8- or 16-byte stores
  if constexpr (sizeof(S) == 2) {
    unsigned w[DPL / 2];
#pragma unroll
    for (int i = 0; i < DPL / 2; ++i)
      w[i] = (unsigned)E::from_float(acc[2 * i] * inv) |
             ((unsigned)E::from_float(acc[2 * i + 1] * inv) << 16);
    if constexpr (DPL == 4) {
      *reinterpret_cast<u32x2*>(out) = u32x2{w[0], w[1]};
    } else {
#pragma unroll
      for (int i = 0; i < DPL / 2; i += 4)
        *reinterpret_cast<u32x4*>(out + 2 * i) = u32x4{w[i], w[i + 1], w[i + 2], w[i + 3]};
    }
  } else {
#pragma unroll
    for (int i = 0; i < DPL; i += 4)
      *reinterpret_cast<f32x4*>(out + i) =
          f32x4{acc[i] * inv, acc[i + 1] * inv, acc[i + 2] * inv, acc[i + 3] * inv};
  }
}

template <class E, int D>
hipError_t launch_pf(const AttnArgs& a, int64_t grid, hipStream_t stream) {
  prefill_kernel<E, D, prefill_rt<E>(), prefill_ring<E>()>
      <<<dim3((unsigned)grid), dim3(kPrefillThreads), 0, stream>>>(a);
  return hipGetLastError();
}

template <class E, int D>
hipError_t launch_pf_shares(const AttnArgs& a, hipStream_t stream) {
  prefill_shares_kernel<E, D, prefill_rt<E>(), prefill_ring<E>()>
      <<<dim3((unsigned)a.pf_shares), dim3(kPrefillThreads), 0, stream>>>(a);
  return hipGetLastError();
}

template <class E, int D>
int resident_pf_shares() {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, prefill_shares_kernel<E, D, prefill_rt<E>(), prefill_ring<E>()>,
          kPrefillThreads, 0) != hipSuccess)
    return 0;
  return per_cu * cus;
}

}  // namespace

int prefill_tile_tokens(pa_dtype dtype, int group) {
  switch (dtype) {
    case PA_F32: return kPrefillWaves * pf_wave_tokens<F32>(group);
    case PA_FP8_E4M3: return kPrefillWaves * pf_wave_tokens<Fp8>(group);
    default: return kPrefillWaves * pf_wave_tokens<Bf16>(group);
  }
}

int prefill_rows(pa_dtype dtype) {
  switch (dtype) {
    case PA_F32: return kPrefillWaves * pf_wave_rows<F32>();
    case PA_FP8_E4M3: return kPrefillWaves * pf_wave_rows<Fp8>();
    default: return kPrefillWaves * pf_wave_rows<Bf16>();
  }
}

int prefill_resident_shares(pa_dtype dtype, int head_dim) {
  switch (dtype) {
    case PA_BF16: return head_dim == 128 ? resident_pf_shares<Bf16, 128>() : resident_pf_shares<Bf16, 64>();
    case PA_F16: return head_dim == 128 ? resident_pf_shares<F16, 128>() : resident_pf_shares<F16, 64>();
    case PA_F32: return head_dim == 128 ? resident_pf_shares<F32, 128>() : resident_pf_shares<F32, 64>();
    case PA_FP8_E4M3: return head_dim == 128 ? resident_pf_shares<Fp8, 128>() : resident_pf_shares<Fp8, 64>();
  }
  return 0;
}

hipError_t launch_prefill(const AttnArgs& a, pa_dtype dtype, int head_dim, int64_t grid,
                          hipStream_t stream) {
  if (a.pf_shares > 0) {
    switch (dtype) {
      case PA_BF16: return head_dim == 128 ? launch_pf_shares<Bf16, 128>(a, stream) : launch_pf_shares<Bf16, 64>(a, stream);
      case PA_F16: return head_dim == 128 ? launch_pf_shares<F16, 128>(a, stream) : launch_pf_shares<F16, 64>(a, stream);
      case PA_F32: return head_dim == 128 ? launch_pf_shares<F32, 128>(a, stream) : launch_pf_shares<F32, 64>(a, stream);
      case PA_FP8_E4M3: return head_dim == 128 ? launch_pf_shares<Fp8, 128>(a, stream) : launch_pf_shares<Fp8, 64>(a, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (grid <= 0) return hipSuccess;
  switch (dtype) {
    case PA_BF16: return head_dim == 128 ? launch_pf<Bf16, 128>(a, grid, stream) : launch_pf<Bf16, 64>(a, grid, stream);
    case PA_F16: return head_dim == 128 ? launch_pf<F16, 128>(a, grid, stream) : launch_pf<F16, 64>(a, grid, stream);
    case PA_F32: return head_dim == 128 ? launch_pf<F32, 128>(a, grid, stream) : launch_pf<F32, 64>(a, grid, stream);
    case PA_FP8_E4M3: return head_dim == 128 ? launch_pf<Fp8, 128>(a, grid, stream) : launch_pf<Fp8, 64>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill_merge(const AttnArgs& a, pa_dtype dtype, int head_dim,
                                hipStream_t stream) {
  const int64_t units = (int64_t)a.num_tokens * a.num_kv_heads;
  if (units <= 0 || a.pf_shares <= 0) return hipSuccess;
  const int rows = prefill_rows(dtype);
  int gp = 1;
  while (gp < a.group) gp <<= 1;
  const int dpl = head_dim / std::min(kWave / gp, head_dim / 4);  // 4 .. 32 for group <= 16
  const dim3 grid((unsigned)((units + 3) / 4)), block(4 * kWave);
#define PA_PF_MERGE(E)                                                                             \
  switch (dpl) {                                                                                   \
    case 4: prefill_share_merge_kernel<E, 4><<<grid, block, 0, stream>>>(a, rows, head_dim); break;   \
    case 8: prefill_share_merge_kernel<E, 8><<<grid, block, 0, stream>>>(a, rows, head_dim); break;   \
    case 16: prefill_share_merge_kernel<E, 16><<<grid, block, 0, stream>>>(a, rows, head_dim); break; \
    case 32: prefill_share_merge_kernel<E, 32><<<grid, block, 0, stream>>>(a, rows, head_dim); break; \
    default: return hipErrorInvalidValue;                                                          \
  }
  switch (dtype) {
    case PA_BF16: PA_PF_MERGE(Bf16) break;
    case PA_F16: PA_PF_MERGE(F16) break;
    case PA_F32: PA_PF_MERGE(F32) break;
    case PA_FP8_E4M3: PA_PF_MERGE(Fp8) break;
    default: return hipErrorInvalidValue;
  }
#undef PA_PF_MERGE
  return hipGetLastError();
}

}  // namespace pa
