// balanced.hip -- paged decode with equal work per workgroup, for ragged batches.
//
// Decode streams every request's whole KV [P1 §04 table; P3 §1.2], so its
// time is the slowest workgroup's share of bytes. With one workgroup per
// (request, KV head) a batch of ragged lengths leaves most of the GPU idle
// while its longest requests finish. Here the batch's work items -- every
// (request, KV-head group, 16-token block), in request-major order -- are cut
// into one contiguous, equal share per resident workgroup (grid sized from
// occupancy, so every workgroup runs at once).
//
// A workgroup has one wave per KV head of a head group (NW = 8 heads when the
// head count allows), and its waves walk the same blocks together, each its
// own head's slice. A block's head slices are 256-byte pieces of each 2 KB
// token row, so this way every block is fetched whole, at once; when
// different waves fetched the slices of one block at different times, the
// same batch read at 4.2 TB/s instead of 5.7 TB/s (loads-only probe).
//
// A workgroup walks its share piece by piece: a piece that is a whole
// (request, head group) segment is written as final output; pieces that cut
// one are written per head as partials (normalised output plus log-sum-exp),
// stored contiguously per (request, KV head) with a record of where they are.
// A second, small kernel renormalises them: the Flash-Decoding merge of
// [P1 §07] with split points chosen for balance instead of a fixed size.
// (Merging inside this kernel would need device-scope fences, which write
// back and invalidate a whole L2 per piece and cost far more than the extra
// launch.)
//
// Given new K/V rows (the fused decode step [P1 §02 slot_mapping write]),
// the piece holding a request's last block also stores the request's new
// rows of its heads to their slot and substitutes them, in registers, for
// key position seq_len - 1, so the write and the read need no ordering.
#include "attn_tile.h"
#include "pa_launch.h"

namespace pa {
namespace {

// Waves per SIMD the kernel is built for and KV blocks each wave keeps in
// flight (compile-time tunables; fp32 operands get half the depth, an E4M3
// cache, whose blocks are half the bytes, its own).
#ifndef PA_BAL_OCC
#define PA_BAL_OCC 2
#endif
#ifndef PA_BAL_DEPTH
#define PA_BAL_DEPTH 2
#endif
#ifndef PA_BAL_FP8_DEPTH
#define PA_BAL_FP8_DEPTH 2
#endif
// Whether the head waves of a workgroup meet at a barrier every DEPTH blocks.
#ifndef PA_BAL_SYNC
#define PA_BAL_SYNC 1
#endif
// Work items charged to each (request, head group) segment beyond its
// blocks: a piece's fixed cost (its query load, the refill of the block
// pipeline before its first block arrives, the final reduction and stores),
// so that a share crossing more segment boundaries gets fewer blocks. On the
// 64-request Llama-3-8B batch 3 and 4 were best (0: +2 us per call, 6: +2 us).
#ifndef PA_BAL_PIECE_COST
#define PA_BAL_PIECE_COST 3
#endif
constexpr int kPieceCost = PA_BAL_PIECE_COST;
template <class E>
constexpr int bal_depth() {
  return sizeof(typename E::kv_storage) == 4   ? (PA_BAL_DEPTH + 1) / 2
         : sizeof(typename E::kv_storage) == 1 ? PA_BAL_FP8_DEPTH
                                               : PA_BAL_DEPTH;
}

// Exclusive prefix sum over the workgroup; *total gets the sum of all v.
template <int NW>
__device__ inline int block_exclusive_sum(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  if (lane == kWave - 1) s_tmp[wave] = x;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = s_tmp[w];
    off += w < wave ? t : 0;
    tot += t;
  }
  *total = tot;
  return off + x - v;
}

// Item range [lo, hi) of share t when W items are cut into T equal shares.
__device__ __host__ inline int64_t share_begin(int64_t t, int64_t W, int64_t T) {
  return t * W / T;
}

// The T workgroup shares of W items, numbered as "ranges" in item order
// without gaps: share t is range t when every share is non-empty (W >= T),
// else (at most one item per share) range share_begin(t), the item index.
struct Shares {
  int64_t W, T;
  __device__ int64_t begin(int64_t t) const { return share_begin(t, W, T); }
  __device__ int64_t range(int64_t t) const { return W >= T ? t : begin(t); }
  // range holding item x: the largest t with begin(t) <= x
  __device__ int64_t range_of(int64_t x) const { return W >= T ? ((x + 1) * T - 1) / W : x; }
};

// Query rows [*lo, *lo + *n) of request i: one row (the request's own) for
// decode, else from cu_seqlens (clamped to the batch like the other kernels).
__device__ inline void request_rows(const BalancedArgs& a, int i, int* lo, int* n) {
  if (a.cu_seqlens == nullptr) {
    *lo = i;
    *n = 1;
    return;
  }
  int l = a.cu_seqlens[i], h = a.cu_seqlens[i + 1];
  l = min(max(l, 0), a.num_tokens);
  h = min(max(h, l), a.num_tokens);
  *lo = l;
  *n = h - l;
}

// Requests whose query rows (tokens x group) fill at most one 16-row tile
// are this kernel's work; longer ones (prefill chunks) are another kernel's.
__device__ inline bool single_tile(int n, int g) { return n >= 1 && n * g <= kTileRows; }

// Slot of range j's piece of head-group segment sg, for one head. Ranges and
// segments both advance with the item index, so j + sg differs for every
// non-empty piece and the pieces of one segment sit at consecutive slots;
// j + sg < T + segments, the per-head slot count.
__device__ inline int64_t piece_slot(int64_t j, int64_t sg) { return j + sg; }

// The fused write of request r's new rows (all KV heads) by one thread, for
// requests without KV blocks, which no piece covers.
template <class E, int D>
__device__ inline void write_new_rows(const BalancedArgs& a, int r) {
  using O = Ops<E, D>;
  using S = typename O::storage;
  using KS = typename O::kv_storage;
  const int64_t slot = a.slot_mapping[r];
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t rs = (int64_t)a.num_kv_heads * D;
  const S* ks = static_cast<const S*>(a.k_new) + (int64_t)r * rs;
  const S* vs = static_cast<const S*>(a.v_new) + (int64_t)r * rs;
  KS* kd = static_cast<KS*>(const_cast<void*>(a.k_cache)) + slot * rs;
  KS* vd = static_cast<KS*>(const_cast<void*>(a.v_cache)) + slot * rs;
  for (int64_t e = 0; e < rs; ++e) {
    if constexpr (sizeof(KS) == 1) {
      kd[e] = (KS)e4m3_code(__fdiv_rn(__uint_as_float((unsigned)ks[e] << 16), a.k_scale));
      vd[e] = (KS)e4m3_code(__fdiv_rn(__uint_as_float((unsigned)vs[e] << 16), a.v_scale));
    } else {
      kd[e] = ks[e];
      vd[e] = vs[e];
    }
  }
}

template <class E, int D, int NW>
__global__ __launch_bounds__(NW * kWave, PA_BAL_OCC) void balanced_decode_kernel(const BalancedArgs a) {
  using O = Ops<E, D>;
  using S = typename O::storage;
  __shared__ int s_prefix[kMaxBalancedSeqs + 1];
  __shared__ int s_tmp[NW];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int B = a.num_seqs;
  const int max_len = (a.max_blocks * kBlockTokens) << a.block_shift;

  // 1. prefix sums of per-request item counts (blocks plus the fixed cost of
  //    a segment, per head group), in LDS
  constexpr int T = NW * kWave;
  const int per = (B + T - 1) / T;
  const int c0 = min(tid * per, B), c1 = min(c0 + per, B);
  int chunk = 0;
  for (int i = c0; i < c1; ++i) {
    int q_lo, n;
    request_rows(a, i, &q_lo, &n);
    const int len = min(max(a.seq_lens[i], 0), max_len);
    const int nb = single_tile(n, a.group) ? (len + kBlockTokens - 1) / kBlockTokens : 0;
    const int items = nb > 0 ? nb + kPieceCost : 0;
    s_prefix[i + 1] = items;
    chunk += items;
  }
  int total_items = 0;
  int run = block_exclusive_sum<NW>(chunk, s_tmp, &total_items);
  total_items = __builtin_amdgcn_readfirstlane(total_items);
  for (int i = c0; i < c1; ++i) {
    run += s_prefix[i + 1];
    s_prefix[i + 1] = run;
  }
  if (tid == 0) s_prefix[0] = 0;
  __syncthreads();
  if (blockIdx.x == 0) {
    // single-tile requests with no KV have no work items: zero output rows,
    // nothing to merge (prefill requests' rows belong to the prefill kernel)
    for (int i = tid; i < B; i += T) {
      if (s_prefix[i + 1] != s_prefix[i]) continue;
      int q_lo, n;
      request_rows(a, i, &q_lo, &n);
      if (!single_tile(n, a.group)) continue;
      S* dst = static_cast<S*>(a.out) + (int64_t)q_lo * a.num_heads * D;
      for (int64_t e = 0; e < (int64_t)n * a.num_heads * D; ++e) dst[e] = S(0);
      for (int k = 0; k < a.num_kv_heads; ++k) a.records[(int64_t)i * a.num_kv_heads + k] = int2{0, 0};
      if (a.k_new != nullptr) write_new_rows<E, D>(a, i);
    }
  }

  // 2. this workgroup's share of the W = HG * total_items items; a segment's
  //    first kPieceCost items stand for its fixed cost and hold no block
  const int hkv = a.num_kv_heads, g = a.group;
  const int HG = hkv / NW;  // head groups
  const int64_t TWG = a.total_waves / NW;
  const Shares sh{(int64_t)HG * total_items, TWG};
  const int64_t head_slots = TWG + (int64_t)B * HG;  // slots per head (wave)
  const int64_t t = blockIdx.x;
  const int64_t lo = sh.begin(t), hi = sh.begin(t + 1), j = sh.range(t);
  if (lo >= hi) return;

  // (values read from LDS are wave-uniform here; readfirstlane tells the
  // compiler so, keeping the addressing below in scalar registers)
  auto prefix = [&](int i) { return __builtin_amdgcn_readfirstlane(s_prefix[i]); };
  // request holding item lo: the largest r with HG * prefix[r] <= lo
  int r_lo = 0, r_hi = B - 1;
  while (r_lo < r_hi) {
    const int mid = (r_lo + r_hi + 1) >> 1;
    if ((int64_t)HG * prefix(mid) <= lo) r_lo = mid; else r_hi = mid - 1;
  }
  int r = r_lo;

  const int row = lane & 15, grp = lane >> 4;
  const int tok = row / g, hh = row - tok * g;  // this lane's query token and head in group
  int64_t x = lo;
  while (x < hi) {
    while (r < B - 1 && (int64_t)HG * prefix(r + 1) <= x) ++r;
    r = __builtin_amdgcn_readfirstlane(r);
    const int p_r = prefix(r);
    const int seg = prefix(r + 1) - p_r;  // items per head group of request r
    const int nb = seg - kPieceCost;      // its blocks
    const int off = __builtin_amdgcn_readfirstlane((int)(x - (int64_t)HG * p_r));
    const int hg = __builtin_amdgcn_readfirstlane(off / seg);
    const int item = __builtin_amdgcn_readfirstlane(off - hg * seg);
    if (item < kPieceCost) {  // the segment's fixed-cost items: no block
      x += min((int64_t)(kPieceCost - item), hi - x);
      continue;
    }
    const int b = item - kPieceCost;
    const int len = __builtin_amdgcn_readfirstlane((int)min((int64_t)(nb - b), hi - x));
    const int seq_len = __builtin_amdgcn_readfirstlane(min(max(a.seq_lens[r], 0), max_len));
    int q_lo, n_r;
    request_rows(a, r, &q_lo, &n_r);
    q_lo = __builtin_amdgcn_readfirstlane(q_lo);
    n_r = __builtin_amdgcn_readfirstlane(n_r);
    const int ctx = max(seq_len - n_r, 0);
    const bool row_valid = tok < n_r;
    // bottom-right causal mask: token i of the request sees keys 0 .. ctx + i
    const int key_end = !row_valid ? 0 : (a.causal ? min(ctx + tok + 1, seq_len) : seq_len);
    const int kvh = hg * NW + wave;

    using KS = typename O::kv_storage;
    KvView<KS> view;
    view.k = static_cast<const KS*>(a.k_cache) + (int64_t)kvh * D;
    view.v = static_cast<const KS*>(a.v_cache) + (int64_t)kvh * D;
    view.rs = (int64_t)hkv * D;
    view.table = a.block_table + (int64_t)r * a.max_blocks;
    view.num_blocks = a.num_blocks;
    view.shift = a.block_shift;

    const int head = kvh * g + (row_valid ? hh : 0);
    const int64_t qrow = (int64_t)q_lo + (row_valid ? tok : 0);
    typename O::Q qop;
    O::load_q(qop, static_cast<const S*>(a.q) + (qrow * a.num_heads + head) * D, row_valid, lane);
    // fused KV write: the piece holding the request's last block writes the
    // new rows of its heads and uses them for that block's last key
    int64_t slot = -1;
    if (a.k_new != nullptr && b + len == nb)
      slot = __builtin_amdgcn_readfirstlane(a.slot_mapping[r]);
    const bool subst = slot >= 0 && slot < a.num_slots;
    typename O::KV nr{};
    if (subst) {
      const int64_t src = ((int64_t)r * hkv + kvh) * D;
      O::load_new(nr, static_cast<const S*>(a.k_new) + src, static_cast<const S*>(a.v_new) + src,
                  lane, a.k_scale, a.v_scale);
    }
    const int new_row = (seq_len - 1) & (kBlockTokens - 1), new_blk = nb - 1 - b;
    auto patch = [&](typename O::KV& kv, int i) {
      if (subst && i == new_blk) O::patch(kv, nr, new_row, lane);
    };
    RowState<D> st;
    st.init();
    // every wave of the workgroup walks the same blocks: same trip count
    stream_blocks<E, D, bal_depth<E>(), PA_BAL_SYNC != 0>(st, qop, view, b, len, key_end,
                                                         seq_len, a.scale_log2, lane, patch);
    if (subst) {
      // stored after the walk, so the new rows' loads are not waited for
      // before the first block; this piece is the only reader of the slot
      // and used the rows from registers
      const int64_t dst = slot * view.rs + (int64_t)kvh * D;
      O::store_new(nr, static_cast<KS*>(const_cast<void*>(a.k_cache)) + dst,
                   static_cast<KS*>(const_cast<void*>(a.v_cache)) + dst, lane);
    }
    st.l = sum_xor16(st.l);
    st.l = sum_xor32(st.l);

    const int64_t sg = (int64_t)r * HG + hg;
    const bool whole = b == 0 && len == nb;
    if (row_valid) {
      const float inv = (st.l > 0.f ? 1.f / st.l : 0.f) * a.out_scale;
      if (whole) {
        S* dst = static_cast<S*>(a.out) + (qrow * a.num_heads + head) * D + (D / 4) * grp;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v[D / 16];
#pragma unroll
          for (int c = 0; c < D / 16; ++c) v[c] = st.o[c][i] * inv;
          store_chunk<E, D>(dst + (D / 16) * i, v);
        }
      } else {
        const int64_t slot = ((int64_t)wave * head_slots + piece_slot(j, sg)) * a.slot_rows + row;
        S* dst = static_cast<S*>(a.part_o) + slot * D + (D / 4) * grp;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v[D / 16];
#pragma unroll
          for (int c = 0; c < D / 16; ++c) v[c] = st.o[c][i] * inv;
          store_chunk<E, D>(dst + (D / 16) * i, v);
        }
        if (grp == 0) a.part_lse[slot] = st.l > 0.f ? st.m + fast_log2(st.l) : neg_inf();
      }
    }
    if (lane == 0) {
      // every piece of a segment writes the same record; a whole one writes 0
      int2 rec{0, 0};
      if (!whole) {
        const int64_t s0 = (int64_t)HG * p_r + (int64_t)hg * seg + kPieceCost;  // block 0's item
        const int64_t first = (int64_t)wave * head_slots + piece_slot(sh.range_of(s0), sg);
        rec = int2{(int)first, (int)(sh.range_of(s0 + nb - 1) - sh.range_of(s0) + 1)};
      }
      a.records[(int64_t)r * hkv + kvh] = rec;
    }
    x += len;
  }
}

// Stores 8 consecutive output values in the storage dtype.
template <class E, int D>
__device__ inline void store8(typename Ops<E, D>::storage* dst, const float* v) {
  using S = typename Ops<E, D>::storage;
  if constexpr (sizeof(S) == 2) {
    unsigned w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (unsigned)Ops<E, D>::to_storage(v[2 * j]) |
             ((unsigned)Ops<E, D>::to_storage(v[2 * j + 1]) << 16);
    *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
  } else {
    *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
}

// Renormalises the pieces of a segment that was cut between workgroups
// [P1 §07: out = sum_j w_j o_j / sum_j w_j, w_j = exp(lse_j - max lse), here
// in log2 units]: merge_waves(slot_rows, D) waves per (request, KV head),
// each taking every such wave's share of 512 values of the flattened rows.
// The record gives the first piece slot and the piece count; each slot holds
// slot_rows x D values, of which the request's n * group rows are valid.
// Lanes take 8 consecutive values and fold kMergeBatch pieces per memory
// round trip with a running maximum, so a segment of up to kMergeBatch
// pieces costs two dependent round trips (record, then pieces).
constexpr int kMergeBatch = 16;
__host__ __device__ inline int merge_waves(int slot_rows, int head_dim) {
  return (slot_rows * head_dim + kWave * 8 - 1) / (kWave * 8);
}
template <class E, int D>
__global__ __launch_bounds__(4 * kWave) void balanced_merge_kernel(const BalancedArgs a) {
  using S = typename Ops<E, D>::storage;
  const int lane = threadIdx.x & (kWave - 1);
  const int mw = merge_waves(a.slot_rows, D);
  const int64_t wid = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  const int64_t unit = wid / mw;
  const int part = (int)(wid - unit * mw);
  if (unit >= (int64_t)a.num_seqs * a.num_kv_heads) return;
  const int r = (int)(unit / a.num_kv_heads);
  const int kvh = (int)(unit - (int64_t)r * a.num_kv_heads);
  const int g = a.group;
  int q_lo, n_r;
  request_rows(a, r, &q_lo, &n_r);
  if (!single_tile(n_r, g)) return;
  const int2 rec = a.records[unit];
  const int np = rec.y;
  if (np <= 0) return;  // written whole by one workgroup, or an empty request
  const int64_t sr = a.slot_rows;
  const S* po = static_cast<const S*>(a.part_o) + (int64_t)rec.x * sr * D;
  const float* pl = a.part_lse + (int64_t)rec.x * sr;
  for (int f = (part * kWave + lane) * 8; f < n_r * g * D; f += mw * kWave * 8) {
    const int row = f / D, dim = f - row * D;
    float m = neg_inf(), wsum = 0.f, acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int k0 = 0; k0 < np; k0 += kMergeBatch) {
      float l[kMergeBatch];
      float v[kMergeBatch][8];
#pragma unroll
      for (int kk = 0; kk < kMergeBatch; ++kk) {
        // past the last piece: reload it (in bounds), weighted 0 below
        const int64_t k = min(k0 + kk, np - 1);
        l[kk] = pl[k * sr + row];
        load_part<E, 8>(po + k * sr * D + f, v[kk]);
      }
      float mb = m;
#pragma unroll
      for (int kk = 0; kk < kMergeBatch; ++kk)
        if (k0 + kk < np) mb = fmaxf(mb, l[kk]);
      const float mu = mb == neg_inf() ? 0.f : mb;
      const float alpha = fast_exp2(m - mu);  // 0 while nothing was folded (m = -inf)
      wsum *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
      for (int kk = 0; kk < kMergeBatch; ++kk) {
        const float w = k0 + kk < np ? fast_exp2(l[kk] - mu) : 0.f;
        wsum += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += w * v[kk][e];
      }
      m = mb;
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
    const int tok = row / g, hh = row - tok * g;
    S* dst = static_cast<S*>(a.out) + (((int64_t)q_lo + tok) * a.num_heads + kvh * g + hh) * D + dim;
    store8<E, D>(dst, acc);
  }
}

template <class E, int D, int NW>
hipError_t launch_bal(const BalancedArgs& a, hipStream_t stream) {
  balanced_decode_kernel<E, D, NW>
      <<<dim3((unsigned)(a.total_waves / NW)), dim3(NW * kWave), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t waves = (int64_t)a.num_seqs * a.num_kv_heads * merge_waves(a.slot_rows, D);
  balanced_merge_kernel<E, D><<<dim3((unsigned)((waves + 3) / 4)), dim3(4 * kWave), 0, stream>>>(a);
  return hipGetLastError();
}

template <class E, int D, int NW>
int occupancy_blocks() {
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &blocks, balanced_decode_kernel<E, D, NW>, NW * kWave, 0) != hipSuccess)
    return 0;
  return blocks;
}

template <class E, int D>
int occupancy_waves(int nw) {
  switch (nw) {
    case 8: return occupancy_blocks<E, D, 8>() * 8;
    case 4: return occupancy_blocks<E, D, 4>() * 4;
    case 2: return occupancy_blocks<E, D, 2>() * 2;
    case 1: return occupancy_blocks<E, D, 1>();
  }
  return 0;
}

template <class E, int D>
hipError_t launch_nw(const BalancedArgs& a, int nw, hipStream_t stream) {
  switch (nw) {
    case 8: return launch_bal<E, D, 8>(a, stream);
    case 4: return launch_bal<E, D, 4>(a, stream);
    case 2: return launch_bal<E, D, 2>(a, stream);
    case 1: return launch_bal<E, D, 1>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int balanced_total_waves(pa_dtype dtype, int head_dim, int num_kv_heads) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  const int nw = balanced_group_waves(num_kv_heads);
  int per_cu = 0;
  switch (dtype) {
    case PA_BF16: per_cu = head_dim == 128 ? occupancy_waves<Bf16, 128>(nw) : occupancy_waves<Bf16, 64>(nw); break;
    case PA_F16: per_cu = head_dim == 128 ? occupancy_waves<F16, 128>(nw) : occupancy_waves<F16, 64>(nw); break;
    case PA_F32: per_cu = head_dim == 128 ? occupancy_waves<F32, 128>(nw) : occupancy_waves<F32, 64>(nw); break;
    case PA_FP8_E4M3: per_cu = head_dim == 128 ? occupancy_waves<Fp8, 128>(nw) : occupancy_waves<Fp8, 64>(nw); break;
  }
  return per_cu * cus;
}

hipError_t launch_balanced(const BalancedArgs& a, pa_dtype dtype, hipStream_t stream) {
  const int nw = balanced_group_waves(a.num_kv_heads);
  if (a.total_waves <= 0 || a.total_waves % nw != 0) return hipErrorInvalidValue;
  const int d = a.head_dim;
  switch (dtype) {
    case PA_BF16: return d == 128 ? launch_nw<Bf16, 128>(a, nw, stream) : launch_nw<Bf16, 64>(a, nw, stream);
    case PA_F16: return d == 128 ? launch_nw<F16, 128>(a, nw, stream) : launch_nw<F16, 64>(a, nw, stream);
    case PA_F32: return d == 128 ? launch_nw<F32, 128>(a, nw, stream) : launch_nw<F32, 64>(a, nw, stream);
    case PA_FP8_E4M3: return d == 128 ? launch_nw<Fp8, 128>(a, nw, stream) : launch_nw<Fp8, 64>(a, nw, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
