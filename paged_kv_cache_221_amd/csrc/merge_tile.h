// merge_tile.h -- the log-sum-exp merge of partial attention results [P1 §07],
// one workgroup per (request, query head).
//
// Piece k of a (request, query head) has a log-sum-exp L_k and an output o_k
// already normalised by its own softmax sum. With M = max_k L_k and
// w_k = exp(L_k - M), the merged output is sum_k w_k o_k / sum_k w_k and the
// merged log-sum-exp M + log sum_k w_k. The work is latency-bound (a few KB
// per unit), so it is arranged to need few dependent memory round trips:
// every wave loads the outputs of its first kMergePre pieces before the
// weights are known, the LSEs are reduced through LDS, and the four waves'
// partial sums are combined through LDS.
#pragma once

#include "attn_tile.h"

namespace pa {

constexpr int kMergeWaves = 4;
constexpr int kMergeThreads = kMergeWaves * kWave;
constexpr int kMergePre = 8;

struct MergeSmem {
  float w[kMergeThreads];            // weights of one round of pieces
  float red[kMergeWaves];            // per-wave max, then per-wave sum
  float acc[kMergeWaves][2][kWave];  // per-wave partial outputs, 2 dims per lane
};

// Merges n pieces: piece k's LSE is lse[k * lse_stride] * to_log2 in log2
// units, its output o[k * o_stride + d] for d < D (D <= 2 * kWave). Called by
// all threads of the workgroup. On return, threads of wave 0 hold the merged
// output for dims lane and lane + kWave in *out0 / *out1, and every thread
// holds the merged LSE in log2 units (-inf when no piece has weight).
__device__ inline void merge_pieces(MergeSmem& sm, const float* lse, int64_t lse_stride,
                                    float to_log2, const float* o, int64_t o_stride, int n,
                                    int D, float* out0, float* out1, float* lse2_out) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int d0 = lane, d1 = lane + kWave;

  // outputs of this wave's first pieces (k = wave + kMergeWaves * i), early
  float p0[kMergePre], p1[kMergePre];
#pragma unroll
  for (int i = 0; i < kMergePre; ++i) {
    const int k = wave + kMergeWaves * i;
    const bool ok = k < n;
    p0[i] = ok && d0 < D ? o[(int64_t)k * o_stride + d0] : 0.f;
    p1[i] = ok && d1 < D ? o[(int64_t)k * o_stride + d1] : 0.f;
  }

  // M = max_k L_k over the workgroup
  float mx = neg_inf();
  for (int k = tid; k < n; k += kMergeThreads) mx = fmaxf(mx, lse[(int64_t)k * lse_stride] * to_log2);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, xor_shuffle(mx, m));
  if (lane == 0) sm.red[wave] = mx;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) mx = fmaxf(mx, sm.red[w]);
  const float mu = mx == neg_inf() ? 0.f : mx;
  __syncthreads();  // sm.red is reused below

  float acc0 = 0.f, acc1 = 0.f, wsum = 0.f;
  for (int base = 0; base < n; base += kMergeThreads) {
    // weights of pieces base .. base + kMergeThreads - 1, one per thread
    const int k = base + tid;
    const float wt = k < n ? fast_exp2(lse[(int64_t)k * lse_stride] * to_log2 - mu) : 0.f;
    wsum += wt;
    sm.w[tid] = wt;
    __syncthreads();
    const int cnt = min(kMergeThreads, n - base);
    int i = 0;
    if (base == 0) {
#pragma unroll
      for (int j = 0; j < kMergePre; ++j) {
        const int kk = wave + kMergeWaves * j;
        const float wk = kk < cnt ? sm.w[kk] : 0.f;
        acc0 += wk * p0[j];
        acc1 += wk * p1[j];
      }
      i = kMergePre;
    }
    // the rest of this round, kMergePre pieces per batch
    for (; wave + kMergeWaves * i < cnt; i += kMergePre) {
      float q0[kMergePre], q1[kMergePre];
#pragma unroll
      for (int j = 0; j < kMergePre; ++j) {
        const int kk = wave + kMergeWaves * (i + j);
        const bool ok = kk < cnt;
        q0[j] = ok && d0 < D ? o[(int64_t)(base + kk) * o_stride + d0] : 0.f;
        q1[j] = ok && d1 < D ? o[(int64_t)(base + kk) * o_stride + d1] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < kMergePre; ++j) {
        const int kk = wave + kMergeWaves * (i + j);
        const float wk = kk < cnt ? sm.w[kk] : 0.f;
        acc0 += wk * q0[j];
        acc1 += wk * q1[j];
      }
    }
    __syncthreads();  // sm.w is rewritten by the next round
  }

  // sum of weights and the four waves' outputs
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) wsum += xor_shuffle(wsum, m);
  if (lane == 0) sm.red[wave] = wsum;
  sm.acc[wave][0][lane] = acc0;
  sm.acc[wave][1][lane] = acc1;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) tot += sm.red[w];
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  if (wave == 0) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) {
      s0 += sm.acc[w][0][lane];
      s1 += sm.acc[w][1][lane];
    }
    *out0 = s0 * inv;
    *out1 = s1 * inv;
  }
  *lse2_out = tot > 0.f ? mx + fast_log2(tot) : neg_inf();
}

}  // namespace pa
