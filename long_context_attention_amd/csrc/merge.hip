// n-way log-sum-exp merge of normalised partial attention outputs.
//
// For items j with normalised outputs A_j and log-sum-exps lse_j of the same
// query row: M = max_j lse_j, w_j = exp(lse_j - M), lse = M + log(sum_j w_j),
// out = sum_j (w_j / sum w) A_j. This is the global aggregation of the Star
// Attention pages (page 1, "assembling the global result"), evaluated with the
// largest term subtracted first as "numerical stability: log-sum-exp" advises;
// items with lse = -inf weigh 0 and a row with no finite item gives out = 0,
// lse = -inf. lse_merge_kernel (a wavefront per row) merges split-KV chunks
// into per-partition partials and partitions into the final output;
// lse_merge_wide_kernel (a workgroup per row) takes rows of more than 32 items,
// such as every chunk of every partition at once.
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

// Merge of items [j_lo, j_hi) of one row by one wavefront: every lane first
// issues all of its loads (the items' LSEs and its head_dim elements of up to
// kBatch items), so that a batch costs one memory round trip; the weights reach
// every lane by readlane. Leaves the running maximum `mx`, the weight sum
// `wsum` = sum_j exp(lse_j - mx) and this lane's sum_j exp(lse_j - mx) A_j.
constexpr int kBatch = 32;
constexpr int kMaxPerLane = 2;   // head_dim <= 128
__device__ __forceinline__ void merge_items(const float* __restrict__ lse_in, const float* __restrict__ o_in,
                                            int64_t stride_lse, int64_t stride_o, int64_t j_lo, int64_t j_hi,
                                            int lane, int per_lane, float& mx, float& wsum,
                                            float (&acc)[kMaxPerLane]) {
  mx = -INFINITY;
  wsum = 0.f;
  acc[0] = acc[1] = 0.f;
  for (int64_t j0 = j_lo; j0 < j_hi; j0 += kBatch) {
    const int cnt = (j_hi - j0) < kBatch ? (int)(j_hi - j0) : kBatch;
    float x[kBatch][kMaxPerLane];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int jj = u < cnt ? u : cnt - 1;
      const float* src = o_in + (j0 + jj) * stride_o;
#pragma unroll
      for (int e = 0; e < kMaxPerLane; ++e) x[u][e] = e < per_lane ? src[64 * e] : 0.f;
    }
    const float ll = lane < cnt ? lse_in[(j0 + lane) * stride_lse] : -INFINITY;
    // Online rescale when a later batch raises the maximum.
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
}

// One wavefront per merged row (few items per row: the chunk merge and the
// partition merge).
template <typename TO>
__global__ __launch_bounds__(64) void lse_merge_kernel(MergeArgs a) {
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t bt = row / a.rows;
  const int64_t r = row % a.rows;
  const int per_lane = a.head_dim / 64;
  float mx, wsum, acc[kMaxPerLane];
  merge_items(a.lse_in + bt * a.n * a.rows + r, a.o_in + (bt * a.n * a.rows + r) * a.head_dim + lane, a.rows,
              a.rows * a.head_dim, 0, a.n, lane, per_lane, mx, wsum, acc);
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  TO* out = static_cast<TO*>(a.o_out) + row * a.head_dim + lane;
#pragma unroll
  for (int e = 0; e < kMaxPerLane; ++e)
    if (e < per_lane) out[64 * e] = from_f32<TO>(acc[e] * inv);
  if (a.lse_out && lane == 0) a.lse_out[row] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
}

// One workgroup of kWideWaves wavefronts per merged row (many items per row:
// every chunk of every partition at once). Each wavefront merges a contiguous
// share of the items; the shares combine through LDS with the same
// max-subtracted weights.
constexpr int kWideWaves = 8;
template <typename TO>
__device__ __forceinline__ void merge_row_wide(const MergeArgs& a, int64_t r) {
  __shared__ float s_m[kWideWaves], s_w[kWideWaves];
  __shared__ float s_acc[kWideWaves][64 * kMaxPerLane];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int per_lane = a.head_dim / 64;
  const int64_t per = (a.n + kWideWaves - 1) / kWideWaves;
  const int64_t j_lo = wave * per < a.n ? wave * per : a.n;
  const int64_t j_hi = j_lo + per < a.n ? j_lo + per : a.n;
  float mx, wsum, acc[kMaxPerLane];
  merge_items(a.lse_in + r, a.o_in + r * a.head_dim + lane, a.rows, a.rows * a.head_dim, j_lo, j_hi, lane, per_lane,
              mx, wsum, acc);
  if (lane == 0) {
    s_m[wave] = mx;
    s_w[wave] = wsum;
  }
#pragma unroll
  for (int e = 0; e < kMaxPerLane; ++e) s_acc[wave][lane + 64 * e] = acc[e];
  __syncthreads();
  if (wave != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWideWaves; ++w) M = fmaxf(M, s_m[w]);
  const float Mu = M == -INFINITY ? 0.f : M;
  float W = 0.f, o[kMaxPerLane] = {0.f, 0.f};
#pragma unroll
  for (int w = 0; w < kWideWaves; ++w) {
    const float f = s_m[w] == -INFINITY ? 0.f : expf(s_m[w] - Mu);
    W += f * s_w[w];
#pragma unroll
    for (int e = 0; e < kMaxPerLane; ++e) o[e] += f * s_acc[w][lane + 64 * e];
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  TO* out = static_cast<TO*>(a.o_out) + r * a.head_dim + lane;
#pragma unroll
  for (int e = 0; e < kMaxPerLane; ++e)
    if (e < per_lane) out[64 * e] = from_f32<TO>(o[e] * inv);
  if (a.lse_out && lane == 0) a.lse_out[r] = W > 0.f ? Mu + logf(W) : -INFINITY;
}

template <typename TO>
__global__ __launch_bounds__(64 * kWideWaves) void lse_merge_wide_kernel(MergeArgs a) {
  merge_row_wide<TO>(a, blockIdx.x);   // row (one batch)
}

// Several sequences' merges in one grid: workgroup w merges row w - begin[s] of
// sequence s.
template <typename TO>
__global__ __launch_bounds__(64 * kWideWaves) void lse_merge_wide_batch_kernel(MergeBatch b) {
  const int64_t w = blockIdx.x;
  int s = 0;
  while (s + 1 < b.n_seq && w >= b.begin[s + 1]) ++s;
  merge_row_wide<TO>(b.seq[s], w - b.begin[s]);
}

hipError_t launch_merge(const MergeArgs& a, bool out_bf16, hipStream_t s) {
  const int64_t total = a.rows * a.batch;
  if (total == 0) return hipSuccess;
  if (a.batch == 1 && a.n > kBatch) {
    const dim3 block(64 * kWideWaves);
    if (out_bf16) hipLaunchKernelGGL(lse_merge_wide_kernel<bf16_t>, dim3((unsigned)total), block, 0, s, a);
    else hipLaunchKernelGGL(lse_merge_wide_kernel<float>, dim3((unsigned)total), block, 0, s, a);
    return hipGetLastError();
  }
  if (out_bf16) hipLaunchKernelGGL(lse_merge_kernel<bf16_t>, dim3((unsigned)total), dim3(64), 0, s, a);
  else hipLaunchKernelGGL(lse_merge_kernel<float>, dim3((unsigned)total), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_merge_wide_batch(const MergeBatch& b, bool out_bf16, hipStream_t s) {
  const int64_t total = b.begin[b.n_seq];
  if (total == 0) return hipSuccess;
  const dim3 block(64 * kWideWaves);
  if (out_bf16) hipLaunchKernelGGL(lse_merge_wide_batch_kernel<bf16_t>, dim3((unsigned)total), block, 0, s, b);
  else hipLaunchKernelGGL(lse_merge_wide_batch_kernel<float>, dim3((unsigned)total), block, 0, s, b);
  return hipGetLastError();
}

}  // namespace sa
