// lse_merge.hip -- log-sum-exp renormalisation of split-K partials [P1 §07].
//
// One wavefront per (request, query head). With M the largest split LSE and
// w_j = exp(lse_j - M): out = sum_j w_j o_j / sum_j w_j, lse = M + log sum_j w_j.
// Only the ceil(seq_len / split_tokens) splits the request has are read.
#include "attn_tile.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kMergeWaves = 4;

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, xor_shuffle(v, m));
  return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += xor_shuffle(v, m);
  return v;
}

template <class E>
__device__ inline void put(void* out, int64_t i, float v) {
  if constexpr (sizeof(typename E::storage) == 2) {
    static_cast<uint16_t*>(out)[i] = E::from_float(v);
  } else {
    static_cast<float*>(out)[i] = v;
  }
}

template <class E>
__global__ __launch_bounds__(kMergeWaves* kWave) void lse_merge_kernel(const MergeArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t unit = (int64_t)blockIdx.x * kMergeWaves + threadIdx.x / kWave;
  if (unit >= (int64_t)a.num_seqs * a.num_heads) return;
  const int r = (int)(unit / a.num_heads);
  const int seq_len = a.seq_lens[r];
  const int ns = seq_len > 0 ? min((seq_len + a.split_tokens - 1) / a.split_tokens, a.num_splits)
                             : 0;
  const float* lse = a.lse_part + unit * a.num_splits;
  const float* op = a.o_part + unit * a.num_splits * a.head_dim;

  // Pass 1: the largest split LSE and the sum of weights; lane s holds split s.
  float mx = neg_inf();
  for (int s = lane; s < ns; s += kWave) mx = fmaxf(mx, lse[s]);
  mx = wave_max(mx);
  const float mu = mx == neg_inf() ? 0.f : mx;
  float tot = 0.f;
  for (int s = lane; s < ns; s += kWave) tot += fast_exp2((lse[s] - mu) * kLog2e);
  tot = wave_sum(tot);
  const float inv = tot > 0.f ? 1.f / tot : 0.f;

  // Pass 2: lanes over head_dim; splits in chunks of 64, the weight of split
  // s0 + j read from lane j (readlane ignores the exec mask).
  for (int d0 = 0; d0 < a.head_dim; d0 += kWave) {
    const int d = d0 + lane;
    const bool live = d < a.head_dim;
    float acc = 0.f;
    for (int s0 = 0; s0 < ns; s0 += kWave) {
      const int sl = s0 + lane;
      const float w = sl < ns ? fast_exp2((lse[sl] - mu) * kLog2e) * inv : 0.f;
      const int cnt = min(kWave, ns - s0);
#pragma unroll 8
      for (int j = 0; j < cnt; ++j) {
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
        if (live) acc += wj * op[(int64_t)(s0 + j) * a.head_dim + d];
      }
    }
    if (live) put<E>(a.out, unit * a.head_dim + d, acc);
  }
  if (a.lse_out != nullptr && lane == 0)
    a.lse_out[unit] = tot > 0.f ? mx + fast_log2(tot) * kLn2 : neg_inf();
}

}  // namespace

hipError_t launch_lse_merge(const MergeArgs& a, pa_dtype out_dtype, hipStream_t stream) {
  const int64_t units = (int64_t)a.num_seqs * a.num_heads;
  if (units <= 0) return hipSuccess;
  const dim3 grid((unsigned)((units + kMergeWaves - 1) / kMergeWaves));
  const dim3 block(kMergeWaves * kWave);
  switch (out_dtype) {
    case PA_BF16: lse_merge_kernel<Bf16><<<grid, block, 0, stream>>>(a); break;
    case PA_F16: lse_merge_kernel<F16><<<grid, block, 0, stream>>>(a); break;
    case PA_F32: lse_merge_kernel<F32><<<grid, block, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
