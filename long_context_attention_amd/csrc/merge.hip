// n-way log-sum-exp merge of normalised partial attention outputs.
//
// For items j with normalised outputs A_j and log-sum-exps lse_j of the same
// query row: M = max_j lse_j, w_j = exp(lse_j - M), lse = M + log(sum_j w_j),
// out = sum_j (w_j / sum w) A_j. This is the global aggregation of the Star
// Attention pages (page 1, "assembling the global result"), evaluated with the
// largest term subtracted first as "numerical stability: log-sum-exp" advises;
// items with lse = -inf weigh 0 (their outputs are never read into the sum)
// and a row with no finite item gives out = 0, lse = -inf.
//
// Layout of the work: a wavefront merges items of one row with 16-byte loads,
// head_dim/4 lanes per item (one float4 each), so one load instruction covers
// 64 / (head_dim/4) items (2 at head_dim 128, 4 at 64). lse_merge_kernel gives
// each row one wavefront (four rows per workgroup): the chunk merge into
// per-partition partials and the partition merge when rows are many and items
// few. lse_merge_wide_kernel serves rows of many items (every chunk of every
// partition at once) and merges of few rows (a decode step's): a workgroup of
// kWideWaves wavefronts per (row, slice of head_dim), each wavefront merging a
// contiguous share of the items, the shares combined through LDS; a step with
// few rows splits head_dim into up to 8 slices (the weights depend on the LSEs
// alone) so that it still spreads over hundreds of workgroups. A lane keeps
// four item loads in flight (loads past the span are masked off, not
// redirected) and folds them into a running maximum, so each batch of loads is
// one round trip to memory. Measured at 128K (kernel trace): against one
// wavefront per row with 4-byte loads, the query step's chunk merge 11.5 -> 8.9
// us and its one-launch merge 25 -> 14 us; with the running maximum instead of
// a first pass over the LSEs, 13.6 -> 12.4 us; with four-wavefront workgroups
// and head_dim slices, 11.4 us, and a decode step's one-launch merge (32 rows,
// 160 items, 8 slices: 256 workgroups instead of 32) 6.2 -> 4.3 us; its chunk
// merge (5 x 32 rows of 32 items, 2 slices) 6.6 -> 4.35 us.
#include <math.h>

#include "sa_common.h"

namespace sa {

constexpr int kRowsPerBlock = 4;   // narrow merge: rows (wavefronts) per workgroup

// One wavefront merges items [j_lo, j_hi) of one row (item j at o_in + j *
// stride_o, its LSE at lse_in + j * stride_lse). Lane = p * LPI + c: c is the
// float4 chunk of the row, p the item slot. Leaves in every lane the row's
// maximum LSE `mx` and the weight sum `wsum` = sum_j exp(lse_j - mx), and in
// lanes p == 0 the chunk c of sum_j exp(lse_j - mx) A_j. One pass: each lane
// loads U items' values and LSEs at once and folds them into a running
// maximum, weight sum and output (scaled when the maximum grows), so a row of
// up to U * 64 / LPI items takes a single round trip to memory; the lane slots
// are then combined with the same max-subtracted weights.
template <int D, int U>
__device__ __forceinline__ void merge_span(const float* __restrict__ lse_in, const float* __restrict__ o_in,
                                           int64_t stride_lse, int64_t stride_o, int64_t j_lo, int64_t j_hi,
                                           int lane, int lpi_log2, int c0, float& mx, float& wsum, f32x4& acc) {
  const int LPI = 1 << lpi_log2;     // lanes per item
  const int IPI = 64 >> lpi_log2;    // items per load instruction
  const int c = lane & (LPI - 1), p = lane >> lpi_log2;
  f32x4 a = {0.f, 0.f, 0.f, 0.f};
  float ws = 0.f;
  float m = -INFINITY;
  for (int64_t j0 = j_lo; j0 < j_hi; j0 += IPI * U) {
    f32x4 x[U];
    float l[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = j0 + p + IPI * u;
      x[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      l[u] = -INFINITY;                          // past the span: weight 0, nothing loaded
      if (j < j_hi) {
        x[u] = *reinterpret_cast<const f32x4*>(o_in + j * stride_o + 4 * (c0 + c));
        l[u] = lse_in[j * stride_lse];
      }
    }
    float mb = m;
#pragma unroll
    for (int u = 0; u < U; ++u) mb = fmaxf(mb, l[u]);
    if (mb == -INFINITY) continue;               // nothing visible yet in this slot
    const float sc = expf(m - mb);               // 0 while m = -inf
    a *= sc;
    ws *= sc;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = expf(l[u] - mb);           // 0 for lse = -inf
      if (w > 0.f) a += w * x[u];
      ws += w;
    }
    m = mb;
  }
  // Combine the item slots p (lanes c, c + LPI, ...) of each chunk c.
  float M = m;
  for (int off = LPI; off < 64; off *= 2) M = fmaxf(M, __shfl_xor(M, off));
  const float f = m == -INFINITY ? 0.f : expf(m - M);
  a *= f;
  ws *= f;
  for (int off = LPI; off < 64; off *= 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] += __shfl_xor(a[e], off);
    ws += __shfl_xor(ws, off);
  }
  mx = M;
  wsum = ws;
  acc = a;
}

template <typename TO>
__device__ __forceinline__ void store4(TO* out, f32x4 v);
template <>
__device__ __forceinline__ void store4<float>(float* out, f32x4 v) {
  *reinterpret_cast<f32x4*>(out) = v;
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* out, f32x4 v) {
  bf16x4 b;
#pragma unroll
  for (int e = 0; e < 4; ++e) b[e] = (bf16_t)v[e];
  *reinterpret_cast<bf16x4*>(out) = b;
}

// One wavefront per merged row, kRowsPerBlock rows per workgroup (few items per
// row: the chunk merge and the partition merge).
template <typename TO, int D>
__global__ __launch_bounds__(64 * kRowsPerBlock) void lse_merge_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= a.rows * a.batch) return;
  const int64_t bt = row / a.rows;
  const int64_t r = row % a.rows;
  float mx, wsum;
  f32x4 acc;
  constexpr int kLpiLog2 = D == 128 ? 5 : 4;   // head_dim/4 lanes per item
  merge_span<D, 4>(a.lse_in + bt * a.n * a.rows + r, a.o_in + (bt * a.n * a.rows + r) * D, a.rows, a.rows * D, 0,
                   a.n, lane, kLpiLog2, 0, mx, wsum, acc);
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  if (lane < D / 4) store4<TO>(static_cast<TO*>(a.o_out) + row * D + 4 * lane, acc * inv);
  if (a.lse_out && lane == 0) a.lse_out[row] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
}

// Rows of many items, or few rows: workgroups of W wavefronts, each wavefront
// merging a contiguous share of one row's items, the shares combined through
// LDS with the same max-subtracted weights. A row's head_dim is split into
// 2^s_log2 slices of head_dim/4 >> s_log2 float4 chunks, one workgroup per
// (row, slice): the weights depend on the LSEs alone, so each slice merges on
// its own, and a step with few rows (a decode step's 32) still spreads over
// hundreds of workgroups with one batch of loads per lane. Row `row` of the
// launch is row row % rows of batch row / rows (items of a batch are n
// consecutive [rows] planes).
template <typename TO, int D, int W, int U>
__device__ __forceinline__ void merge_row_sliced(const MergeArgs& a, int64_t row, int slice, int s_log2) {
  __shared__ float s_m[W], s_w[W];
  __shared__ f32x4 s_acc[W][D / 4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lpi_log2 = (D == 128 ? 5 : 4) - s_log2;
  const int lpi = 1 << lpi_log2;
  const int c0 = slice << lpi_log2;
  // row < 2^32 (a grid index); one batch needs no division
  const uint32_t bt = a.batch == 1 ? 0u : (uint32_t)row / (uint32_t)a.rows;
  const int64_t r = row - (int64_t)bt * a.rows;
  const int64_t per = (a.n + W - 1) / W;
  const int64_t j_lo = wave * per < a.n ? wave * per : a.n;
  const int64_t j_hi = j_lo + per < a.n ? j_lo + per : a.n;
  float mx, wsum;
  f32x4 acc;
  merge_span<D, U>(a.lse_in + bt * a.n * a.rows + r, a.o_in + (bt * a.n * a.rows + r) * D, a.rows, a.rows * D, j_lo,
                   j_hi, lane, lpi_log2, c0, mx, wsum, acc);
  if (lane == 0) {
    s_m[wave] = mx;
    s_w[wave] = wsum;
  }
  if (lane < lpi) s_acc[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < W; ++w) M = fmaxf(M, s_m[w]);
  const float Mu = M == -INFINITY ? 0.f : M;
  float Ws = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const float f = s_m[w] == -INFINITY ? 0.f : expf(s_m[w] - Mu);
    Ws += f * s_w[w];
    if (lane < lpi && f > 0.f) o += f * s_acc[w][lane];
  }
  const float inv = Ws > 0.f ? 1.f / Ws : 0.f;
  if (lane < lpi) store4<TO>(static_cast<TO*>(a.o_out) + row * D + 4 * (c0 + lane), o * inv);
  if (a.lse_out && slice == 0 && lane == 0) a.lse_out[row] = Ws > 0.f ? Mu + logf(Ws) : -INFINITY;
}

constexpr int kWideWaves = 4;
template <typename TO, int D, int U>
__global__ __launch_bounds__(64 * kWideWaves) void lse_merge_wide_kernel(MergeArgs a, int s_log2) {
  merge_row_sliced<TO, D, kWideWaves, U>(a, blockIdx.x >> s_log2, blockIdx.x & ((1 << s_log2) - 1), s_log2);
}

// Several sequences' merges in one grid: workgroup w >> s_log2 merges row
// (w >> s_log2) - begin[s] of sequence s.
template <typename TO, int D>
__global__ __launch_bounds__(64 * kWideWaves) void lse_merge_wide_batch_kernel(MergeBatch b, int s_log2) {
  const int64_t w = blockIdx.x >> s_log2;
  int s = 0;
  while (s + 1 < b.n_seq && w >= b.begin[s + 1]) ++s;
  merge_row_sliced<TO, D, kWideWaves, 4>(b.seq[s], w - b.begin[s], blockIdx.x & ((1 << s_log2) - 1), s_log2);
}

// Slices per row (log2) for `rows` merged rows: enough for about 512
// workgroups, at least 4 lanes (64 bytes) per item slice.
inline int merge_slices_log2(int64_t rows, int head_dim) {
  const int max_log2 = head_dim == 128 ? 3 : 2;
  int s = 0;
  while (s < max_log2 && (rows << (s + 1)) <= 512) ++s;
  return s;
}

namespace {
template <typename TO, int D>
hipError_t launch_merge_t(const MergeArgs& a, hipStream_t s) {
  const int64_t total = a.rows * a.batch;
  // Many items per row, or too few rows to fill the chip with one wavefront
  // each: the sliced kernel (one batch of loads per lane); otherwise one
  // wavefront per row.
  if (a.n > 32 || (a.n > 8 && total < 2048)) {
    const int sl = merge_slices_log2(total, D);
    hipLaunchKernelGGL((lse_merge_wide_kernel<TO, D, 4>), dim3((unsigned)(total << sl)), dim3(64 * kWideWaves), 0, s,
                       a, sl);
  } else {
    const int64_t blocks = (total + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL((lse_merge_kernel<TO, D>), dim3((unsigned)blocks), dim3(64 * kRowsPerBlock), 0, s, a);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_merge(const MergeArgs& a, bool out_bf16, hipStream_t s) {
  if (a.rows * a.batch == 0) return hipSuccess;
  if (a.head_dim == 64) return out_bf16 ? launch_merge_t<bf16_t, 64>(a, s) : launch_merge_t<float, 64>(a, s);
  return out_bf16 ? launch_merge_t<bf16_t, 128>(a, s) : launch_merge_t<float, 128>(a, s);
}

hipError_t launch_merge_wide_batch(const MergeBatch& b, bool out_bf16, hipStream_t s) {
  const int64_t total = b.begin[b.n_seq];
  if (total == 0) return hipSuccess;
  const int d = b.seq[0].head_dim;
  const int sl = merge_slices_log2(total, d);
  const dim3 grid((unsigned)(total << sl)), block(64 * kWideWaves);
  if (d == 64) {
    if (out_bf16) hipLaunchKernelGGL((lse_merge_wide_batch_kernel<bf16_t, 64>), grid, block, 0, s, b, sl);
    else hipLaunchKernelGGL((lse_merge_wide_batch_kernel<float, 64>), grid, block, 0, s, b, sl);
  } else {
    if (out_bf16) hipLaunchKernelGGL((lse_merge_wide_batch_kernel<bf16_t, 128>), grid, block, 0, s, b, sl);
    else hipLaunchKernelGGL((lse_merge_wide_batch_kernel<float, 128>), grid, block, 0, s, b, sl);
  }
  return hipGetLastError();
}

}  // namespace sa
