// n-way log-sum-exp merge of normalised partial attention outputs.
//
// For items j with normalised outputs A_j and log-sum-exps lse_j of the same
// query row: M = max_j lse_j, w_j = exp(lse_j - M), lse = M + log(sum_j w_j),
// out = sum_j (w_j / sum w) A_j. This is the global aggregation of the Star
// Attention pages (page 1, "assembling the global result"), evaluated with the
// largest term subtracted first as "numerical stability: log-sum-exp" advises;
// items with lse = -inf weigh 0 and a row with no finite item gives out = 0,
// lse = -inf. The same kernel merges split-KV chunks into per-partition
// partials and partitions into the final output.
#include <math.h>

#include "sa_common.h"

namespace sa {

namespace {
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}
}  // namespace

// One wavefront per merged row. Every lane first issues all of its loads (the
// items' LSEs and its head_dim elements of up to kBatch items) so that a
// merge costs one memory round trip; the weights reach every lane by
// readlane. Items beyond kBatch are taken kBatch at a time.
template <typename TO>
__global__ __launch_bounds__(64) void lse_merge_kernel(MergeArgs a) {
  constexpr int kBatch = 32;
  constexpr int kMaxPerLane = 2;   // head_dim <= 128
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t bt = row / a.rows;
  const int64_t r = row % a.rows;
  const float* __restrict__ lse_in = a.lse_in + bt * a.n * a.rows + r;
  const float* __restrict__ o_in = a.o_in + (bt * a.n * a.rows + r) * a.head_dim + lane;
  const int per_lane = a.head_dim / 64;

  float mx = -INFINITY;
  float acc[kMaxPerLane] = {0.f, 0.f};
  float wsum = 0.f;
  for (int64_t j0 = 0; j0 < a.n; j0 += kBatch) {
    const int cnt = (a.n - j0) < kBatch ? (int)(a.n - j0) : kBatch;
    float x[kBatch][kMaxPerLane];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int jj = u < cnt ? u : cnt - 1;
      const float* src = o_in + (j0 + jj) * a.rows * a.head_dim;
#pragma unroll
      for (int e = 0; e < kMaxPerLane; ++e) x[u][e] = e < per_lane ? src[64 * e] : 0.f;
    }
    const float ll = lane < cnt ? lse_in[(j0 + lane) * a.rows] : -INFINITY;
    // Online rescale when a later batch raises the maximum (one batch in practice).
    const float m_new = fmaxf(mx, wave_max(ll));
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float scale = mx == -INFINITY ? 0.f : expf(mx - m_use);
    wsum *= scale;
#pragma unroll
    for (int e = 0; e < kMaxPerLane; ++e) acc[e] *= scale;
    mx = m_new;
    const float wl = expf(ll - m_use);
    wsum += wave_sum(wl);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (u < cnt) {
        const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), u));
#pragma unroll
        for (int e = 0; e < kMaxPerLane; ++e) acc[e] += w > 0.f ? w * x[u][e] : 0.f;
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  TO* out = static_cast<TO*>(a.o_out) + row * a.head_dim + lane;
#pragma unroll
  for (int e = 0; e < kMaxPerLane; ++e)
    if (e < per_lane) out[64 * e] = from_f32<TO>(acc[e] * inv);
  if (a.lse_out && lane == 0) a.lse_out[row] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
}

hipError_t launch_merge(const MergeArgs& a, bool out_bf16, hipStream_t s) {
  const int64_t total = a.rows * a.batch;
  if (total == 0) return hipSuccess;
  if (out_bf16) hipLaunchKernelGGL(lse_merge_kernel<bf16_t>, dim3((unsigned)total), dim3(64), 0, s, a);
  else hipLaunchKernelGGL(lse_merge_kernel<float>, dim3((unsigned)total), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace sa
