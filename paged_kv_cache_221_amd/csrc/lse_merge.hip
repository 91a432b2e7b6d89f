// lse_merge.hip -- log-sum-exp renormalisation of split-K partials [P1 §07].
//
// One workgroup per (request, query head) runs the merge of merge_tile.h
// over the ceil(seq_len / split_tokens) splits the request has.
#include "merge_tile.h"
#include "pa_launch.h"

namespace pa {
namespace {

template <class E>
__device__ inline void put(void* out, int64_t i, float v) {
  if constexpr (sizeof(typename E::storage) == 2) {
    static_cast<uint16_t*>(out)[i] = E::from_float(v);
  } else {
    static_cast<float*>(out)[i] = v;
  }
}

// One workgroup per (request, query head); split LSEs are natural-log.
template <class E>
__global__ __launch_bounds__(kMergeThreads) void lse_merge_kernel(const MergeArgs a) {
  __shared__ MergeSmem sm;
  const int64_t unit = blockIdx.x;
  const int r = (int)(unit / a.num_heads);
  const int seq_len = a.seq_lens[r];
  const int ns = seq_len > 0 ? min((seq_len + a.split_tokens - 1) / a.split_tokens, a.num_splits)
                             : 0;
  float o0 = 0.f, o1 = 0.f, lse2 = 0.f;
  merge_pieces(sm, a.lse_part + unit * a.num_splits, 1, kLog2e,
               a.o_part + unit * a.num_splits * a.head_dim, a.head_dim, ns, a.head_dim, &o0, &o1,
               &lse2);
  const int tid = threadIdx.x;
  if (tid < kWave) {
    if (tid < a.head_dim) put<E>(a.out, unit * a.head_dim + tid, o0);
    if (tid + kWave < a.head_dim) put<E>(a.out, unit * a.head_dim + tid + kWave, o1);
  }
  if (a.lse_out != nullptr && tid == 0) a.lse_out[unit] = lse2 == neg_inf() ? lse2 : lse2 * kLn2;
}

}  // namespace

hipError_t launch_lse_merge(const MergeArgs& a, pa_dtype out_dtype, hipStream_t stream) {
  const int64_t units = (int64_t)a.num_seqs * a.num_heads;
  if (units <= 0) return hipSuccess;
  const dim3 grid((unsigned)units);
  const dim3 block(kMergeThreads);
  switch (out_dtype) {
    case PA_BF16: lse_merge_kernel<Bf16><<<grid, block, 0, stream>>>(a); break;
    case PA_F16: lse_merge_kernel<F16><<<grid, block, 0, stream>>>(a); break;
    case PA_F32: lse_merge_kernel<F32><<<grid, block, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
