// balanced.hip -- paged decode with equal work per wave, for ragged batches.
//
// Decode streams every request's whole KV [P1 §04 table; P3 §1.2], so its
// time is the slowest wave's share of bytes. With one workgroup per
// (request, KV head) a batch of ragged lengths leaves most of the GPU idle
// while its longest requests finish. Here the batch's work items -- every
// (request, KV head, 16-token block), in request-major order -- are cut into
// one contiguous, equal share per resident wave (grid sized from occupancy,
// so every wave runs at once). A wave walks its share piece by piece: a piece
// that is a whole (request, KV head) segment is written as the final output;
// the pieces at the ends of a share that cut a segment are written as
// partials (normalised output plus log-sum-exp), stored contiguously per
// segment with a record of where they are. A second, small kernel
// renormalises them: the Flash-Decoding merge of [P1 §07] with split points
// chosen for balance instead of a fixed size. (Merging inside this kernel
// would need device-scope fences, which write back and invalidate a whole
// L2 per piece and cost far more than the extra launch.)
#include "attn_tile.h"
#include "pa_launch.h"


namespace pa {
namespace {

constexpr int kBalWaves = 4;
// Waves per SIMD the kernel is built for and KV blocks each wave keeps in
// flight (compile-time tunables; fp32 operands get half the depth).
#ifndef PA_BAL_OCC
#define PA_BAL_OCC 2
#endif
#ifndef PA_BAL_DEPTH
#define PA_BAL_DEPTH 4
#endif
template <class E>
constexpr int bal_depth() {
  return sizeof(typename E::storage) == 4 ? (PA_BAL_DEPTH + 1) / 2 : PA_BAL_DEPTH;
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

// Item range [lo, hi) of wave t when W items are cut into TW equal shares.
__device__ __host__ inline int64_t share_begin(int64_t t, int64_t W, int64_t TW) {
  return t * W / TW;
}

// Slot of share t's piece of a segment: shares hold at most one item each
// when W < TW (then the item index is unique), else the share index is; the
// segment index keeps consecutive segments' ranges apart. Pieces of one
// segment therefore sit at consecutive slots.
__device__ inline int64_t piece_slot(int64_t t, int64_t W, int64_t TW, int64_t seg) {
  return (W >= TW ? t : share_begin(t, W, TW)) + seg;
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
  const int max_len = a.max_blocks * kBlockTokens;

  // 1. prefix sums of per-request block counts, in LDS
  constexpr int T = NW * kWave;
  const int per = (B + T - 1) / T;
  const int c0 = min(tid * per, B), c1 = min(c0 + per, B);
  int chunk = 0;
  for (int i = c0; i < c1; ++i) {
    const int len = min(max(a.seq_lens[i], 0), max_len);
    const int nb = (len + kBlockTokens - 1) / kBlockTokens;
    s_prefix[i + 1] = nb;
    chunk += nb;
  }
  int total_blocks = 0;
  int run = block_exclusive_sum<NW>(chunk, s_tmp, &total_blocks);
  total_blocks = __builtin_amdgcn_readfirstlane(total_blocks);
  for (int i = c0; i < c1; ++i) {
    run += s_prefix[i + 1];
    s_prefix[i + 1] = run;
  }
  if (tid == 0) s_prefix[0] = 0;
  __syncthreads();
  if (blockIdx.x == 0) {
    // requests with no KV have no work items: zero output, nothing to merge
    for (int i = tid; i < B; i += T) {
      if (s_prefix[i + 1] != s_prefix[i]) continue;
      S* dst = static_cast<S*>(a.out) + (int64_t)i * a.num_heads * D;
      for (int e = 0; e < a.num_heads * D; ++e) dst[e] = S(0);
      for (int k = 0; k < a.num_kv_heads; ++k) a.records[(int64_t)i * a.num_kv_heads + k] = int2{0, 0};
    }
  }

  // 2. this wave's share of the W = Hkv * total_blocks items
  const int hkv = a.num_kv_heads, g = a.group;
  const int64_t W = (int64_t)hkv * total_blocks;
  const int64_t TW = a.total_waves;
  const int64_t t = (int64_t)blockIdx.x * NW + wave;
  const int64_t lo = share_begin(t, W, TW), hi = share_begin(t + 1, W, TW);
  if (lo >= hi) return;

  // request holding item lo: the largest r with hkv * prefix[r] <= lo
  // (values read from LDS are wave-uniform here; readfirstlane tells the
  // compiler so, keeping the addressing below in scalar registers)
  auto prefix = [&](int i) { return __builtin_amdgcn_readfirstlane(s_prefix[i]); };
  int r_lo = 0, r_hi = B - 1;
  while (r_lo < r_hi) {
    const int mid = (r_lo + r_hi + 1) >> 1;
    if ((int64_t)hkv * prefix(mid) <= lo) r_lo = mid; else r_hi = mid - 1;
  }
  int r = r_lo;

  const int row = lane & 15, grp = lane >> 4;
  const bool row_valid = row < g;
  int64_t x = lo;
  while (x < hi) {
    while (r < B - 1 && (int64_t)hkv * prefix(r + 1) <= x) ++r;
    r = __builtin_amdgcn_readfirstlane(r);
    const int p_r = prefix(r);
    const int nb = prefix(r + 1) - p_r;
    const int off = __builtin_amdgcn_readfirstlane((int)(x - (int64_t)hkv * p_r));
    const int kvh = __builtin_amdgcn_readfirstlane(off / nb);
    const int b = __builtin_amdgcn_readfirstlane(off - kvh * nb);
    const int len = __builtin_amdgcn_readfirstlane((int)min((int64_t)(nb - b), hi - x));
    const int seq_len = __builtin_amdgcn_readfirstlane(min(max(a.seq_lens[r], 0), max_len));

    KvView<S> view;
    view.k = static_cast<const S*>(a.k_cache) + (int64_t)kvh * D;
    view.v = static_cast<const S*>(a.v_cache) + (int64_t)kvh * D;
    view.rs = (int64_t)hkv * D;
    view.table = a.block_table + (int64_t)r * a.max_blocks;
    view.num_blocks = a.num_blocks;

    const int head = kvh * g + (row_valid ? row : 0);
    typename O::Q qop;
    O::load_q(qop, static_cast<const S*>(a.q) + ((int64_t)r * a.num_heads + head) * D, row_valid,
              lane);
    RowState<D> st;
    st.init();
    stream_blocks<E, D, bal_depth<E>()>(st, qop, view, b, len, row_valid ? seq_len : 0, seq_len,
                                     a.scale_log2, lane);
    st.l = sum_xor16(st.l);
    st.l = sum_xor32(st.l);

    const bool whole = b == 0 && len == nb;
    if (row_valid) {
      const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
      if (whole) {
        S* dst = static_cast<S*>(a.out) + ((int64_t)r * a.num_heads + head) * D + (D / 4) * grp;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v[D / 16];
#pragma unroll
          for (int c = 0; c < D / 16; ++c) v[c] = st.o[c][i] * inv;
          store_chunk<E, D>(dst + (D / 16) * i, v);
        }
      } else {
        const int64_t seg = (int64_t)r * hkv + kvh;
        const int64_t slot = piece_slot(t, W, TW, seg) * g + row;
        float* dst = a.part_o + slot * D + (D / 4) * grp;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int c = 0; c < D / 16; c += 4)
            *reinterpret_cast<f32x4*>(dst + (D / 16) * i + c) =
                f32x4{st.o[c][i] * inv, st.o[c + 1][i] * inv, st.o[c + 2][i] * inv,
                      st.o[c + 3][i] * inv};
        if (grp == 0) a.part_lse[slot] = st.l > 0.f ? st.m + fast_log2(st.l) : neg_inf();
      }
    }
    if (lane == 0) {
      // every piece of a segment writes the same record; a whole one writes 0
      const int64_t seg = (int64_t)r * hkv + kvh;
      int2 rec{0, 0};
      if (!whole) {
        const int64_t s0 = (int64_t)hkv * p_r + (int64_t)kvh * nb;
        const int64_t ta = ((s0 + 1) * TW - 1) / W, tb = ((s0 + nb) * TW - 1) / W;
        const int64_t first = piece_slot(ta, W, TW, seg);
        rec = int2{(int)first, (int)(piece_slot(tb, W, TW, seg) - first + 1)};
      }
      a.records[seg] = rec;
    }
    x += len;
  }
}

// One wave per (request, query head): renormalises the pieces of a segment
// that was cut between waves. Lane j reads piece j's LSE; the outputs of all
// pieces are then read with independent loads, lanes over head_dim.
template <class E>
__global__ __launch_bounds__(4 * kWave) void balanced_merge_kernel(const BalancedArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t unit = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (unit >= (int64_t)a.num_seqs * a.num_heads) return;
  const int r = (int)(unit / a.num_heads);
  const int h = (int)(unit - (int64_t)r * a.num_heads);
  const int g = a.group, kvh = h / g, row = h - kvh * g;
  const int D = a.head_dim;
  const int2 rec = a.records[(int64_t)r * a.num_kv_heads + kvh];
  const int np = rec.y;
  if (np <= 0) return;  // written whole by one wave, or an empty request
  float mx = neg_inf();
  for (int j = lane; j < np; j += kWave) mx = fmaxf(mx, a.part_lse[((int64_t)rec.x + j) * g + row]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, xor_shuffle(mx, m));
  const float mu = mx == neg_inf() ? 0.f : mx;
  float acc0 = 0.f, acc1 = 0.f, wsum = 0.f;
  const int d0 = lane, d1 = lane + kWave;
  for (int c = 0; c < np; c += kWave) {
    const int j = c + lane;
    const float w = j < np ? fast_exp2(a.part_lse[((int64_t)rec.x + j) * g + row] - mu) : 0.f;
    wsum += w;
    const int cnt = min(kWave, np - c);
#pragma unroll 8
    for (int k = 0; k < cnt; ++k) {
      const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k));
      const float* src = a.part_o + (((int64_t)rec.x + c + k) * g + row) * D;
      if (d0 < D) acc0 += wk * src[d0];
      if (d1 < D) acc1 += wk * src[d1];
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) wsum += xor_shuffle(wsum, m);
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

template <class E, int D>
hipError_t launch_bal(const BalancedArgs& a, hipStream_t stream) {
  balanced_decode_kernel<E, D, kBalWaves>
      <<<dim3((unsigned)(a.total_waves / kBalWaves)), dim3(kBalWaves * kWave), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t units = (int64_t)a.num_seqs * a.num_heads;
  balanced_merge_kernel<E><<<dim3((unsigned)((units + 3) / 4)), dim3(4 * kWave), 0, stream>>>(a);
  return hipGetLastError();
}

template <class E, int D>
int occupancy_blocks() {
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &blocks, balanced_decode_kernel<E, D, kBalWaves>, kBalWaves * kWave, 0) != hipSuccess)
    return 0;
  return blocks;
}

}  // namespace

int balanced_total_waves(pa_dtype dtype, int head_dim) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  int per_cu = 0;
  switch (dtype) {
    case PA_BF16: per_cu = head_dim == 128 ? occupancy_blocks<Bf16, 128>() : occupancy_blocks<Bf16, 64>(); break;
    case PA_F16: per_cu = head_dim == 128 ? occupancy_blocks<F16, 128>() : occupancy_blocks<F16, 64>(); break;
    case PA_F32: per_cu = head_dim == 128 ? occupancy_blocks<F32, 128>() : occupancy_blocks<F32, 64>(); break;
  }
  return per_cu * cus * kBalWaves;
}

hipError_t launch_balanced(const BalancedArgs& a, pa_dtype dtype, hipStream_t stream) {
  if (a.total_waves <= 0 || a.total_waves % kBalWaves != 0) return hipErrorInvalidValue;
  const int d = a.head_dim;
  switch (dtype) {
    case PA_BF16: return d == 128 ? launch_bal<Bf16, 128>(a, stream) : launch_bal<Bf16, 64>(a, stream);
    case PA_F16: return d == 128 ? launch_bal<F16, 128>(a, stream) : launch_bal<F16, 64>(a, stream);
    case PA_F32: return d == 128 ? launch_bal<F32, 128>(a, stream) : launch_bal<F32, 64>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
