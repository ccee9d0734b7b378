// RoPE + KV-cache store: K rows are rotated at their positions and written with
// V into a head-major cache [Hkv][rows][d]; optionally the same tokens' queries
// are rotated too, for the query step's attention tile kernel. Used for the Phase-1 cache (only the
// L real context rows; the anchor is never copied per block) and for appending
// query / generated tokens to the query host's tail. A second kernel rotates
// the anchor's keys at other position IDs for each block (the position
// ablation), into a caller's workspace.
#include "sa_common.h"

namespace sa {

// Rotate 8 pairs (d indices 8 grp .. 8 grp + 7 and the same + D/2) of one key
// row at position pos, from ks to kd.
template <typename T>
__device__ __forceinline__ void rope_pairs8(const T* __restrict__ ks, T* __restrict__ kd, int half, int grp,
                                            int64_t pos, const RopeTable& rt) {
  typedef T vec8 __attribute__((ext_vector_type(8)));
  const vec8 x1 = *reinterpret_cast<const vec8*>(ks);
  const vec8 x2 = *reinterpret_cast<const vec8*>(ks + half);
  vec8 y1, y2;
  double f[8];
  rope_freqs8(rt.inv_freq, grp, f);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float c, s;
    if constexpr (sizeof(T) == 2) rope_cos_sin_hw(pos, f[e], &c, &s);   // rounded to bf16 next
    else rope_cos_sin(pos, f[e], &c, &s);
    const float a1 = to_f32(x1[e]), a2 = to_f32(x2[e]);
    y1[e] = from_f32<T>(a1 * c - a2 * s);
    y2[e] = from_f32<T>(a2 * c + a1 * s);
  }
  *reinterpret_cast<vec8*>(kd) = y1;
  *reinterpret_cast<vec8*>(kd + half) = y2;
}

// One thread per (row, KV head, group of 8 rotation pairs): 16-byte accesses
// for bf16, no loop, so even a one-token append is a single short dependency chain.
template <typename T>
__device__ __forceinline__ void rope_store_one(const RopeStoreArgs& a, const RopeTable& rt, int64_t idx) {
  typedef T vec8 __attribute__((ext_vector_type(8)));
  const int D = a.head_dim;
  const int half = D >> 1;
  const int groups = half >> 3;
  if (idx >= a.n_rows * a.n_heads * groups) return;
  const int grp = (int)(idx % groups);
  const int64_t t = idx / groups;
  const int h = (int)(t % a.n_heads);
  const int64_t r = t / a.n_heads;
  const T* __restrict__ ks = static_cast<const T*>(a.k_src) + (r * a.n_heads + h) * D + grp * 8;
  const T* __restrict__ vs = static_cast<const T*>(a.v_src) + (r * a.n_heads + h) * D + grp * 8;
  T* __restrict__ kd = static_cast<T*>(a.k_dst) + ((int64_t)h * a.dst_rows + a.row0 + r) * D + grp * 8;
  T* __restrict__ vd = static_cast<T*>(a.v_dst) + ((int64_t)h * a.dst_rows + a.row0 + r) * D + grp * 8;
  const vec8 v1 = *reinterpret_cast<const vec8*>(vs);
  const vec8 v2 = *reinterpret_cast<const vec8*>(vs + half);
  rope_pairs8<T>(ks, kd, half, grp, a.pos0 + r, rt);
  *reinterpret_cast<vec8*>(vd) = v1;
  *reinterpret_cast<vec8*>(vd + half) = v2;
}

// The anchor's keys at other position IDs: one thread per (anchor of this
// launch, anchor row, KV head, group of 8 rotation pairs).
template <typename T>
__global__ __launch_bounds__(256) void anchor_keys_kernel(AnchorKeysArgs a, RopeTable rt) {
  const int D = a.head_dim;
  const int half = D >> 1;
  const int groups = half >> 3;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)a.count * a.anchor_len * a.n_heads * groups) return;
  const int grp = (int)(idx % groups);
  int64_t t = idx / groups;
  const int h = (int)(t % a.n_heads);
  t /= a.n_heads;
  const int64_t r = t % a.anchor_len;
  const int j = (int)(t / a.anchor_len);
  const T* ks = static_cast<const T*>(a.k_src) + (r * a.n_heads + h) * D + grp * 8;
  T* kd = static_cast<T*>(a.k_dst) + (((int64_t)h * a.n_anchors + a.first + j) * a.anchor_len + r) * D + grp * 8;
  rope_pairs8<T>(ks, kd, half, grp, a.pos[j] + r, rt);
}

// One thread per (row, query head, group of 8 rotation pairs): the rotated
// query scaled by q_scale, rounded once to bf16.
template <typename T>
__device__ __forceinline__ void rope_query_one(const RopeStoreArgs& a, const RopeTable& rt, int64_t idx) {
  typedef T vec8 __attribute__((ext_vector_type(8)));
  const int D = a.head_dim;
  const int half = D >> 1;
  const int groups = half >> 3;
  if (idx >= a.n_rows * a.q_heads * groups) return;
  const int grp = (int)(idx % groups);
  const int64_t t = idx / groups;            // row * q_heads + head
  const T* qs = static_cast<const T*>(a.q_src) + t * D + grp * 8;
  bf16_t* qd = static_cast<bf16_t*>(a.q_dst) + t * D + grp * 8;
  const vec8 x1 = *reinterpret_cast<const vec8*>(qs);
  const vec8 x2 = *reinterpret_cast<const vec8*>(qs + half);
  bf16x8 y1, y2;
  const int64_t pos = a.pos0 + t / a.q_heads;
  double f[8];
  rope_freqs8(rt.inv_freq, grp, f);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float c, s;
    rope_cos_sin_hw(pos, f[e], &c, &s);   // the rotated query is rounded to bf16
    const float a1 = to_f32(x1[e]), a2 = to_f32(x2[e]);
    y1[e] = (bf16_t)((a1 * c - a2 * s) * a.q_scale);
    y2[e] = (bf16_t)((a2 * c + a1 * s) * a.q_scale);
  }
  *reinterpret_cast<bf16x8*>(qd) = y1;
  *reinterpret_cast<bf16x8*>(qd + half) = y2;
}

template <typename T>
__global__ __launch_bounds__(256) void rope_store_kernel(RopeStoreArgs a, RopeTable rt) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t kv_items = a.n_rows * a.n_heads * (a.head_dim / 16);
  if (idx < kv_items) rope_store_one<T>(a, rt, idx);
  else if (a.q_heads > 0) rope_query_one<T>(a, rt, idx - kv_items);
}

hipError_t launch_rope_store(const RopeStoreArgs& a, const RopeTable& rt, bool bf16, hipStream_t s) {
  const int64_t total = a.n_rows * (a.n_heads + a.q_heads) * (a.head_dim / 16);
  if (total == 0) return hipSuccess;
  const unsigned grid = (unsigned)((total + 255) / 256);
  if (bf16)
    hipLaunchKernelGGL(rope_store_kernel<bf16_t>, dim3(grid), dim3(256), 0, s, a, rt);
  else
    hipLaunchKernelGGL(rope_store_kernel<float>, dim3(grid), dim3(256), 0, s, a, rt);
  return hipGetLastError();
}

hipError_t launch_anchor_keys(const AnchorKeysArgs& a, const RopeTable& rt, bool bf16, hipStream_t s) {
  const int64_t total = (int64_t)a.count * a.anchor_len * a.n_heads * (a.head_dim / 16);
  if (total == 0) return hipSuccess;
  const unsigned grid = (unsigned)((total + 255) / 256);
  if (bf16)
    hipLaunchKernelGGL(anchor_keys_kernel<bf16_t>, dim3(grid), dim3(256), 0, s, a, rt);
  else
    hipLaunchKernelGGL(anchor_keys_kernel<float>, dim3(grid), dim3(256), 0, s, a, rt);
  return hipGetLastError();
}

}  // namespace sa
