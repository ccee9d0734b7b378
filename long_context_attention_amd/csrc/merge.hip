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

// One wavefront per merged row; lanes stride over head_dim.
template <typename TO>
__global__ __launch_bounds__(256) void lse_merge_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows * a.batch) return;
  const int64_t bt = row / a.rows;
  const int64_t r = row % a.rows;
  const float* lse_in = a.lse_in + bt * a.n * a.rows + r;
  const float* o_in = a.o_in + (bt * a.n * a.rows + r) * a.head_dim;

  float mx = -INFINITY;
  for (int64_t j = 0; j < a.n; ++j) mx = fmaxf(mx, lse_in[j * a.rows]);
  const float mref = mx == -INFINITY ? 0.f : mx;
  float wsum = 0.f;
  for (int64_t j = 0; j < a.n; ++j) wsum += expf(lse_in[j * a.rows] - mref);
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;

  TO* out = static_cast<TO*>(a.o_out) + row * a.head_dim;
  for (int d = lane; d < a.head_dim; d += 64) {
    float acc = 0.f;
    for (int64_t j = 0; j < a.n; ++j) {
      const float w = expf(lse_in[j * a.rows] - mref);
      if (w > 0.f) acc = fmaf(w, o_in[j * a.rows * a.head_dim + d], acc);
    }
    out[d] = from_f32<TO>(acc * inv);
  }
  if (a.lse_out && lane == 0) a.lse_out[row] = wsum > 0.f ? mref + logf(wsum) : -INFINITY;
}

hipError_t launch_merge(const MergeArgs& a, bool out_bf16, hipStream_t s) {
  const int64_t total = a.rows * a.batch;
  if (total == 0) return hipSuccess;
  const unsigned grid = (unsigned)((total + 3) / 4);
  if (out_bf16) hipLaunchKernelGGL(lse_merge_kernel<bf16_t>, dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(lse_merge_kernel<float>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace sa
