// prefill.hip -- the chunked-prefill rows of a varlen step [P1 §07] on gfx950.
//
// A request whose query rows times the GQA group exceed one 16-row tile is a
// prefill chunk: query row i of it sees keys 0 .. c + i (its cached context c
// plus itself and earlier new tokens [P1 §04 causal mask]). Prefill is a dense
// contraction [P1 §04 table: GEMM, compute-bound], so the work is arranged for
// operand reuse: a workgroup owns 4 waves x RT row tiles x 16/g query tokens
// of one (request, KV head); every KV block is fetched once per workgroup into
// double-buffered LDS through a register prefetch ring of PA_PREFILL_RING
// blocks, and each wave reads the block's MFMA operands from LDS once and
// applies them to all of its RT row tiles. Scores and probabilities stay in
// registers (the FlashAttention principle [P3 §3.4]).
#include "attn_tile.h"
#include "pa_launch.h"

#ifndef PA_PREFILL_RT
#define PA_PREFILL_RT 2
#endif
#ifndef PA_PREFILL_RING
#define PA_PREFILL_RING 4
#endif
#ifndef PA_PREFILL_OCC
#define PA_PREFILL_OCC 2
#endif
// KV blocks per split of a long prefill tile, and the most splits per tile
// (longer contexts get longer splits). Splits only pay when the prefill
// tiles cannot fill the GPU: on the mixed step (4 chunks of 512 tokens on
// contexts up to 4k, 512 workgroups) 96-block splits made the prefill slower
// (254 -> 280 us), because its workgroups already keep every CU busy.
#ifndef PA_PREFILL_SPLIT_BLOCKS
#define PA_PREFILL_SPLIT_BLOCKS 512
#endif
#ifndef PA_PREFILL_MAX_SPLITS
#define PA_PREFILL_MAX_SPLITS 8
#endif

namespace pa {
namespace {

// Waves per workgroup; each stages KV blocks for all of them.
#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 4
#endif
constexpr int kPrefillWaves = PA_PREFILL_WAVES;
constexpr int kPrefillThreads = kPrefillWaves * kWave;
static_assert(PA_PREFILL_RING % 4 == 0, "the ring (halved for fp32) alternates two LDS buffers");

// How one workgroup stages a block's head slice (16 keys) in LDS.
template <class E, int D>
struct Stage {
  using S = typename Ops<E, D>::storage;
  static constexpr int kRowBytes = D * (int)sizeof(S);      // one key's slice
  static constexpr int kLdsRow = kRowBytes + 16;            // padded: no bank conflicts
  static constexpr int kChunksPerRow = kRowBytes / 16;
  static constexpr int kChunks = kBlockTokens * kChunksPerRow;
  static constexpr int kPerThread = (kChunks + kPrefillThreads - 1) / kPrefillThreads;
  struct Regs {
    u32x4 k[kPerThread];
    u32x4 v[kPerThread];
  };
};

template <class E, int D, int RT, int RING>
__global__ __launch_bounds__(kPrefillThreads, PA_PREFILL_OCC) void prefill_kernel(const AttnArgs a) {
  using O = Ops<E, D>;
  using S = typename O::storage;
  using St = Stage<E, D>;
  __shared__ __attribute__((aligned(16))) char s_k[2][kBlockTokens * St::kLdsRow];
  __shared__ __attribute__((aligned(16))) char s_v[2][kBlockTokens * St::kLdsRow];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  // tiles in descending order: the tiles that see the most keys start first
  int u = blockIdx.x;
  const int kvh = u % a.num_kv_heads;
  u /= a.num_kv_heads;
  const int split = u % a.pf_splits;
  u /= a.pf_splits;
  const int r = u % a.num_seqs;
  const int tile = a.num_tiles - 1 - u / a.num_seqs;

  int lo = a.cu_seqlens[r], hi = a.cu_seqlens[r + 1];
  lo = min(max(lo, 0), a.num_tokens);
  hi = min(max(hi, lo), a.num_tokens);
  const int q_lo = lo, n = hi - lo;
  const int g = a.group;
  if (n * g <= 16) return;  // a single-tile request: handled by the decode kernel
  const int seq_len = min(max(a.seq_lens[r], 0), a.max_blocks * kBlockTokens);
  const int ctx = max(seq_len - n, 0);
  const int tpw = 16 / g;                               // tokens per row tile
  const int tile_tokens = kPrefillWaves * RT * tpw;
  const int tok_base = tile * tile_tokens;
  if (tok_base >= n) return;
  const int tile_end = min(tok_base + tile_tokens, n);
  const int kmax = a.causal ? min(ctx + tile_end, seq_len) : seq_len;
  const int nblk = (kmax + kBlockTokens - 1) / kBlockTokens;
  if (nblk <= 0) return;
  // this workgroup's blocks [b0, b1) of the tile's nblk
  const int nsplit = a.pf_splits > 1 ? (nblk + a.pf_split_blocks - 1) / a.pf_split_blocks : 1;
  if (split >= nsplit) return;
  const int b0 = nsplit > 1 ? split * a.pf_split_blocks : 0;
  const int b1 = nsplit > 1 ? min(b0 + a.pf_split_blocks, nblk) : nblk;

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
  const int row_bytes_g = (int)(rs * (int64_t)sizeof(S));
  const S* k_head = static_cast<const S*>(a.k_cache) + (int64_t)kvh * D;
  const S* v_head = static_cast<const S*>(a.v_cache) + (int64_t)kvh * D;
  const __attribute__((address_space(4))) int32_t* tab =
      (const __attribute__((address_space(4))) int32_t*)(a.block_table + (int64_t)r * a.max_blocks);
  auto issue = [&](typename St::Regs& rg, int i) {
    const int pb = tab[min(i, b1 - 1)];
    const bool ok = i < b1 && pb >= 0 && pb < a.num_blocks;
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
      rg.k[p] = buf_load16(rk, off);
      rg.v[p] = buf_load16(rv, off);
    }
  };
  auto stage = [&](const typename St::Regs& rg, int buf) {
#pragma unroll
    for (int p = 0; p < St::kPerThread; ++p) {
      const int c = tid + p * kPrefillThreads;
      if (c < St::kChunks) {
        const int off = (c / St::kChunksPerRow) * St::kLdsRow + (c % St::kChunksPerRow) * 16;
        *reinterpret_cast<u32x4*>(&s_k[buf][off]) = rg.k[p];
        *reinterpret_cast<u32x4*>(&s_v[buf][off]) = rg.v[p];
      }
    }
  };

  typename St::Regs ring[RING];
#pragma unroll
  for (int j = 0; j < RING; ++j) issue(ring[j], b0 + j);
  for (int i0 = b0; i0 < b1; i0 += RING) {
#pragma unroll
    for (int j = 0; j < RING; ++j) {
      const int i = i0 + j;
      const int buf = j & 1;
      stage(ring[j], buf);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      issue(ring[j], i + RING);
      __builtin_amdgcn_sched_barrier(0);
      // Unconditional, like the loads: a padding block past b1 was read as
      // zeros and is fully masked (b1 < nblk only before the last split,
      // whose keys come after), so it adds nothing, and the accumulators stay
      // in one set of registers.
      typename O::KV kv;
      O::load_lds(kv, s_k[buf], s_v[buf], St::kLdsRow, lane);
      consume_block_tiles<E, D, RT>(st, kv, q, i * kBlockTokens, key_end, a.scale_log2, lane);
    }
  }

  // epilogue: normalise and store every valid row (a split's partial when
  // the tile has several splits)
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    st[rt].l = sum_xor16(st[rt].l);
    st[rt].l = sum_xor32(st[rt].l);
    const int tok0 = tok_base + (wave * RT + rt) * tpw;
    const int tok = tok0 + row / g, hh = row - (row / g) * g;
    if (row < tpw * g && tok < n) {
      const float inv = st[rt].l > 0.f ? 1.f / st[rt].l : 0.f;
      const int64_t orow = (int64_t)(q_lo + tok) * a.num_heads + kvh * g + hh;
      if (nsplit == 1) {
        S* dst = static_cast<S*>(a.out) + orow * D + (D / 4) * grp;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v[D / 16];
#pragma unroll
          for (int c = 0; c < D / 16; ++c) v[c] = st[rt].o[c][i] * inv;
          store_chunk<E, D>(dst + (D / 16) * i, v);
        }
      } else {
        const int64_t prow = orow * a.pf_splits + split;
        float* dst = a.pf_o + prow * D + (D / 4) * grp;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int c = 0; c < D / 16; c += 4)
            *reinterpret_cast<f32x4*>(dst + (D / 16) * i + c) =
                f32x4{st[rt].o[c][i] * inv, st[rt].o[c + 1][i] * inv, st[rt].o[c + 2][i] * inv,
                      st[rt].o[c + 3][i] * inv};
        if (grp == 0) a.pf_lse[prow] = st[rt].l > 0.f ? st[rt].m + fast_log2(st[rt].l) : neg_inf();
      }
    }
  }
}

// Merges the splits of long prefill tiles [P1 §07 LSE merge]: one wave per
// (query token, head). Tokens of single-tile requests and of tiles that had
// one split were written directly and are skipped. The tile's split count is
// recomputed exactly as prefill_kernel derives it; it never exceeds
// pf_splits because keys are clipped to the block table's width, from which
// pf_splits is sized.
template <class E>
__global__ __launch_bounds__(4 * kWave) void prefill_merge_kernel(const AttnArgs a,
                                                                  int tile_tokens, int D) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t unit = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (unit >= (int64_t)a.num_tokens * a.num_heads) return;
  const int token = (int)(unit / a.num_heads);
  // the request holding this token: the largest r with cu[r] <= token
  int lo = 0, hi = a.num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.cu_seqlens[mid] <= token) lo = mid; else hi = mid - 1;
  }
  const int r = lo;
  int q_lo = a.cu_seqlens[r], q_hi = a.cu_seqlens[r + 1];
  q_lo = min(max(q_lo, 0), a.num_tokens);
  q_hi = min(max(q_hi, q_lo), a.num_tokens);
  if (token < q_lo || token >= q_hi) return;
  const int n = q_hi - q_lo, g = a.group;
  if (n * g <= 16) return;
  const int seq_len = min(max(a.seq_lens[r], 0), a.max_blocks * kBlockTokens);
  const int ctx = max(seq_len - n, 0);
  const int tile_end = min(((token - q_lo) / tile_tokens + 1) * tile_tokens, n);
  const int kmax = a.causal ? min(ctx + tile_end, seq_len) : seq_len;
  const int nblk = (kmax + kBlockTokens - 1) / kBlockTokens;
  const int nsplit = (nblk + a.pf_split_blocks - 1) / a.pf_split_blocks;
  if (nsplit <= 1) return;
  const int64_t prow = unit * a.pf_splits;  // unit = token * Hq + head
  const int d0 = lane, d1 = lane + kWave;
  // outputs of every split, loaded together with the LSEs
  float x0[PA_PREFILL_MAX_SPLITS], x1[PA_PREFILL_MAX_SPLITS];
#pragma unroll
  for (int j = 0; j < PA_PREFILL_MAX_SPLITS; ++j) {
    const bool ok = j < nsplit;
    x0[j] = ok && d0 < D ? a.pf_o[(prow + j) * D + d0] : 0.f;
    x1[j] = ok && d1 < D ? a.pf_o[(prow + j) * D + d1] : 0.f;
  }
  const float lse = lane < nsplit ? a.pf_lse[prow + lane] : neg_inf();
  float mx = lse;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, xor_shuffle(mx, m));
  const float mu = mx == neg_inf() ? 0.f : mx;
  const float w = lane < nsplit ? fast_exp2(lse - mu) : 0.f;
  float wsum = w;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) wsum += xor_shuffle(wsum, m);
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int j = 0; j < PA_PREFILL_MAX_SPLITS; ++j) {
    const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
    acc0 += wj * x0[j];  // zero past nsplit (loaded as 0, weight 0)
    acc1 += wj * x1[j];
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  using S = typename E::storage;
  S* out = static_cast<S*>(a.out) + unit * D;
  if constexpr (sizeof(S) == 2) {
    if (d0 < D) out[d0] = E::from_float(acc0 * inv);
    if (d1 < D) out[d1] = E::from_float(acc1 * inv);
  } else {
    if (d0 < D) out[d0] = acc0 * inv;
    if (d1 < D) out[d1] = acc1 * inv;
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

template <class E, int D>
hipError_t launch_pf(const AttnArgs& a, int64_t grid, hipStream_t stream) {
  prefill_kernel<E, D, prefill_rt<E>(), prefill_ring<E>()>
      <<<dim3((unsigned)grid), dim3(kPrefillThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

void prefill_splits(int max_blocks, int* splits, int* split_blocks) {
  int sp = (max_blocks + PA_PREFILL_SPLIT_BLOCKS - 1) / PA_PREFILL_SPLIT_BLOCKS;
  sp = min(max(sp, 1), PA_PREFILL_MAX_SPLITS);
  *splits = sp;
  *split_blocks = max((max_blocks + sp - 1) / sp, 1);
}

hipError_t launch_prefill_merge(const AttnArgs& a, pa_dtype dtype, int head_dim,
                                hipStream_t stream) {
  const int64_t units = (int64_t)a.num_tokens * a.num_heads;
  if (units <= 0 || a.pf_splits <= 1) return hipSuccess;
  const int tt = prefill_tile_tokens(dtype, a.group);
  const dim3 grid((unsigned)((units + 3) / 4)), block(4 * kWave);
  switch (dtype) {
    case PA_BF16: prefill_merge_kernel<Bf16><<<grid, block, 0, stream>>>(a, tt, head_dim); break;
    case PA_F16: prefill_merge_kernel<F16><<<grid, block, 0, stream>>>(a, tt, head_dim); break;
    case PA_F32: prefill_merge_kernel<F32><<<grid, block, 0, stream>>>(a, tt, head_dim); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int prefill_tile_tokens(pa_dtype dtype, int group) {
  const int rt = dtype == PA_F32 ? prefill_rt<F32>() : prefill_rt<Bf16>();
  return kPrefillWaves * rt * (16 / group);
}

hipError_t launch_prefill(const AttnArgs& a, pa_dtype dtype, int head_dim, int64_t grid,
                          hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  switch (dtype) {
    case PA_BF16: return head_dim == 128 ? launch_pf<Bf16, 128>(a, grid, stream) : launch_pf<Bf16, 64>(a, grid, stream);
    case PA_F16: return head_dim == 128 ? launch_pf<F16, 128>(a, grid, stream) : launch_pf<F16, 64>(a, grid, stream);
    case PA_F32: return head_dim == 128 ? launch_pf<F32, 128>(a, grid, stream) : launch_pf<F32, 64>(a, grid, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
