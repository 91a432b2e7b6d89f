// attention.hip -- paged attention kernel for decode, split-K partials and
// varlen mixed steps on gfx950.
//
// One workgroup works on one (query tile, request, KV head, KV split).
// - A request whose query rows times the GQA group fit one 16-row tile
//   (decode, [P1 §04 table]: query_len 1; also short multi-token queries)
//   is a "single-tile" unit: the waves of the workgroup take contiguous runs
//   of the split's KV blocks and their partial softmax states are merged
//   through LDS at the end. Decode streams the whole KV from HBM, so this is the
//   bandwidth-bound path ([P1 §04], [P3 §1.2]).
// - A longer query (chunked prefill, [P1 §07]) is left to prefill.hip.
// Split-K (Flash-Decoding, [P1 §07]) writes each split's normalised output
// and its natural-log LSE; pa_lse_merge renormalises them.
#include "attn_tile.h"
#include "pa_launch.h"


namespace pa {
namespace {

// At least two waves per SIMD: 256 registers per lane.
template <class E, int D, int NW>
__global__ __launch_bounds__(NW * kWave, 2) void paged_attention_kernel(const AttnArgs a) {
  using O = Ops<E, D>;
  using S = typename O::storage;
  constexpr int kComb = NW > 1 ? NW : 1;
  __shared__ float sm_o[kComb][16][NW > 1 ? D : 1];
  __shared__ float sm_m[kComb][16];
  __shared__ float sm_l[kComb][16];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  int u = blockIdx.x;
  const int split = u % a.num_splits;
  u /= a.num_splits;
  const int kvh = u % a.num_kv_heads;
  u /= a.num_kv_heads;
  const int r = u % a.num_seqs;
  const int tile = u / a.num_seqs;

  int q_lo = r, n = 1;
  if (a.cu_seqlens != nullptr) {
    int lo = a.cu_seqlens[r], hi = a.cu_seqlens[r + 1];
    lo = min(max(lo, 0), a.num_tokens);
    hi = min(max(hi, lo), a.num_tokens);
    q_lo = lo;
    n = hi - lo;
  }
  int seq_len = a.seq_lens[r];
  seq_len = min(max(seq_len, 0), (a.max_blocks * kBlockTokens) << a.block_shift);
  const int g = a.group;
  const int ctx = max(seq_len - n, 0);
  const int row = lane & 15;
  const int grp = lane >> 4;

  using KS = typename O::kv_storage;
  KvView<KS> view;
  view.k = static_cast<const KS*>(a.k_cache) + (int64_t)kvh * D;
  view.v = static_cast<const KS*>(a.v_cache) + (int64_t)kvh * D;
  view.rs = (int64_t)a.num_kv_heads * D;
  view.table = a.block_table + (int64_t)r * a.max_blocks;
  view.num_blocks = a.num_blocks;
  view.shift = a.block_shift;

  typename O::Q qop;
  RowState<D> st;
  st.init();

  // A query longer than one 16-row tile is a prefill chunk: prefill.hip.
  if (n * g > 16) return;
  {
    // ---------------------------------------------------- single-tile unit
    if (tile != 0 || n == 0) return;
    const int tok = row / g, hh = row - (row / g) * g;
    const bool valid = row < n * g;
    const int key_end = !valid ? 0 : (a.causal ? min(ctx + tok + 1, seq_len) : seq_len);
    const S* qrow = static_cast<const S*>(a.q) +
                    ((int64_t)(q_lo + (valid ? tok : 0)) * a.num_heads + kvh * g + hh) * D;
    O::load_q(qop, qrow, valid, lane);
    const int nblk = (seq_len + kBlockTokens - 1) / kBlockTokens;
    const int b0 = split * a.split_blocks;
    const int b1 = min(b0 + a.split_blocks, nblk);
    // wave w takes the w-th of NW contiguous, nearly equal runs of [b0, b1)
    const int cnt = max(b1 - b0, 0);
    const int w_lo = b0 + (int)(((int64_t)cnt * wave) / NW);
    const int w_hi = b0 + (int)(((int64_t)cnt * (wave + 1)) / NW);
    stream_blocks<E, D, kv_depth<E>()>(st, qop, view, w_lo, w_hi - w_lo, key_end, seq_len,
                                     a.scale_log2, lane);
    st.l = sum_xor16(st.l);
    st.l = sum_xor32(st.l);

    const int nrows = n * g;
    auto emit = [&](int rr, int d, float acc, float lsum, float mx) {
      const int head = kvh * g + rr % g;
      const float val = (lsum > 0.f ? acc / lsum : 0.f) * a.out_scale;
      if (a.o_part != nullptr) {
        const int64_t unit = (int64_t)r * a.num_heads + head;
        a.o_part[(unit * a.num_splits + split) * D + d] = val;
        if (d == 0)
          a.lse_part[unit * a.num_splits + split] =
              lsum > 0.f ? (mx + fast_log2(lsum)) * kLn2 : neg_inf();
      } else {
        S* dst = static_cast<S*>(a.out) + ((int64_t)(q_lo + rr / g) * a.num_heads + head) * D;
        dst[d] = O::to_storage(val);
      }
    };

    if constexpr (NW > 1) {
      if (lane < 16) {
        sm_m[wave][lane] = st.m;
        sm_l[wave][lane] = st.l;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < D / 16; ++c) sm_o[wave][row][(D / 4) * grp + (D / 16) * i + c] = st.o[c][i];
      __syncthreads();
      for (int it = threadIdx.x; it < nrows * D; it += NW * kWave) {
        const int rr = it / D, d = it - (it / D) * D;
        float mx = neg_inf();
#pragma unroll
        for (int w = 0; w < NW; ++w) mx = fmaxf(mx, sm_m[w][rr]);
        const float mu = mx == neg_inf() ? 0.f : mx;
        float lsum = 0.f, acc = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const float e = fast_exp2(sm_m[w][rr] - mu);
          lsum += e * sm_l[w][rr];
          acc += e * sm_o[w][rr][d];
        }
        emit(rr, d, acc, lsum, mx);
      }
    } else {
      if (row < nrows) {
        if (a.o_part == nullptr) {
          const float inv = (st.l > 0.f ? 1.f / st.l : 0.f) * a.out_scale;
          S* dst = static_cast<S*>(a.out) +
                   ((int64_t)(q_lo + tok) * a.num_heads + kvh * g + hh) * D + (D / 4) * grp;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v[D / 16];
#pragma unroll
            for (int c = 0; c < D / 16; ++c) v[c] = st.o[c][i] * inv;
            store_chunk<E, D>(dst + (D / 16) * i, v);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int c = 0; c < D / 16; ++c)
              emit(row, (D / 4) * grp + (D / 16) * i + c, st.o[c][i], st.l, st.m);
        }
      }
    }
    return;
  }

}

// Split-K partials (and whole-request decode, one split) with the KV heads
// of a group read together: one workgroup per (request, group of NW KV
// heads, split), one wave per head, the waves walking the split's blocks
// side by side and meeting at a barrier every DEPTH blocks. One head's slice
// of a block is a piece of each token row, so the workgroup fetches every
// block whole, at once; one workgroup per head instead reads the slices of a
// block at unrelated times. A wave's 16 rows are its head's GQA group (the
// query rows of one token: decode rows only, no cu_seqlens). Writes the
// split's normalised output and natural-log LSE, or with o_part == nullptr
// the output rows.
#ifndef PA_COAL_OCC
#define PA_COAL_OCC 2
#endif
template <class E, int D, int NW>
__global__ __launch_bounds__(NW * kWave, PA_COAL_OCC) void coalesced_attention_kernel(const AttnArgs a) {
  using O = Ops<E, D>;
  using S = typename O::storage;
  using KS = typename O::kv_storage;
  constexpr int kDepth = sizeof(KS) == 4 ? 1 : 2;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  int u = blockIdx.x;
  const int split = u % a.num_splits;
  u /= a.num_splits;
  const int groups = a.num_kv_heads / NW;
  const int hg = u % groups;
  const int r = u / groups;
  const int kvh = hg * NW + wave;
  const int seq_len = min(max(a.seq_lens[r], 0), (a.max_blocks * kBlockTokens) << a.block_shift);
  const int g = a.group;
  const int row = lane & 15, grp = lane >> 4;
  const bool valid = row < g;
  const int head = kvh * g + (valid ? row : 0);

  KvView<KS> view;
  view.k = static_cast<const KS*>(a.k_cache) + (int64_t)kvh * D;
  view.v = static_cast<const KS*>(a.v_cache) + (int64_t)kvh * D;
  view.rs = (int64_t)a.num_kv_heads * D;
  view.table = a.block_table + (int64_t)r * a.max_blocks;
  view.num_blocks = a.num_blocks;
  view.shift = a.block_shift;

  typename O::Q qop;
  O::load_q(qop, static_cast<const S*>(a.q) + ((int64_t)r * a.num_heads + head) * D, valid, lane);
  const int nblk = (seq_len + kBlockTokens - 1) / kBlockTokens;
  const int b0 = __builtin_amdgcn_readfirstlane(split * a.split_blocks);
  const int n = __builtin_amdgcn_readfirstlane(max(min(a.split_blocks, nblk - b0), 0));
  RowState<D> st;
  st.init();
  // every wave of the workgroup walks the same n blocks: same trip count
  stream_blocks<E, D, kDepth, true>(st, qop, view, b0, n, valid ? seq_len : 0, seq_len,
                                    a.scale_log2, lane);
  st.l = sum_xor16(st.l);
  st.l = sum_xor32(st.l);
  if (!valid) return;
  const float inv = (st.l > 0.f ? 1.f / st.l : 0.f) * a.out_scale;
  const int64_t unit = (int64_t)r * a.num_heads + head;
  if (a.o_part == nullptr) {
    S* dst = static_cast<S*>(a.out) + unit * D + (D / 4) * grp;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v[D / 16];
#pragma unroll
      for (int c = 0; c < D / 16; ++c) v[c] = st.o[c][i] * inv;
      store_chunk<E, D>(dst + (D / 16) * i, v);
    }
    return;
  }
  float* dst = a.o_part + (unit * a.num_splits + split) * D + (D / 4) * grp;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < D / 16; c += 4)
      *reinterpret_cast<f32x4*>(dst + (D / 16) * i + c) =
          f32x4{st.o[c][i] * inv, st.o[c + 1][i] * inv, st.o[c + 2][i] * inv,
                st.o[c + 3][i] * inv};
  if (grp == 0)
    a.lse_part[unit * a.num_splits + split] =
        st.l > 0.f ? (st.m + fast_log2(st.l)) * kLn2 : neg_inf();
}

template <class E, int D>
hipError_t launch_coalesced_d(const AttnArgs& a, int nw, int64_t grid, hipStream_t stream) {
  switch (nw) {
    case 8:
      coalesced_attention_kernel<E, D, 8><<<dim3((unsigned)grid), dim3(8 * kWave), 0, stream>>>(a);
      break;
    case 4:
      coalesced_attention_kernel<E, D, 4><<<dim3((unsigned)grid), dim3(4 * kWave), 0, stream>>>(a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class E, int D>
hipError_t launch_dw(const AttnArgs& a, int waves, int64_t grid, hipStream_t stream) {
  switch (waves) {
    case 1:
      paged_attention_kernel<E, D, 1><<<dim3((unsigned)grid), dim3(kWave), 0, stream>>>(a);
      break;
    case 2:
      paged_attention_kernel<E, D, 2><<<dim3((unsigned)grid), dim3(2 * kWave), 0, stream>>>(a);
      break;
    case 4:
      paged_attention_kernel<E, D, 4><<<dim3((unsigned)grid), dim3(4 * kWave), 0, stream>>>(a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class E>
hipError_t launch_d(const AttnArgs& a, int head_dim, int waves, int64_t grid,
                    hipStream_t stream) {
  if (head_dim == 128) return launch_dw<E, 128>(a, waves, grid, stream);
  if (head_dim == 64) return launch_dw<E, 64>(a, waves, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_coalesced(const AttnArgs& a, pa_dtype dtype, int head_dim, int nw,
                            int64_t grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  const bool d128 = head_dim == 128;
  switch (dtype) {
    case PA_BF16: return d128 ? launch_coalesced_d<Bf16, 128>(a, nw, grid, stream) : launch_coalesced_d<Bf16, 64>(a, nw, grid, stream);
    case PA_F16: return d128 ? launch_coalesced_d<F16, 128>(a, nw, grid, stream) : launch_coalesced_d<F16, 64>(a, nw, grid, stream);
    case PA_F32: return d128 ? launch_coalesced_d<F32, 128>(a, nw, grid, stream) : launch_coalesced_d<F32, 64>(a, nw, grid, stream);
    case PA_FP8_E4M3: return d128 ? launch_coalesced_d<Fp8, 128>(a, nw, grid, stream) : launch_coalesced_d<Fp8, 64>(a, nw, grid, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attention(const AttnArgs& args, pa_dtype dtype, int head_dim, int waves,
                            int64_t grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  switch (dtype) {
    case PA_BF16: return launch_d<Bf16>(args, head_dim, waves, grid, stream);
    case PA_F16: return launch_d<F16>(args, head_dim, waves, grid, stream);
    case PA_F32: return launch_d<F32>(args, head_dim, waves, grid, stream);
    case PA_FP8_E4M3: return launch_d<Fp8>(args, head_dim, waves, grid, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
