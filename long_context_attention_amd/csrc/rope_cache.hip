// RoPE + KV-cache store: K rows are rotated at their positions and written with
// V into a head-major cache [Hkv][rows][d]. Used for the Phase-1 cache (only the
// L real context rows; the anchor is never copied per block) and for appending
// query / generated tokens to the query host's tail.
#include "sa_common.h"

namespace sa {

template <typename T>
__global__ __launch_bounds__(256) void rope_store_kernel(RopeStoreArgs a, RopeTable rt) {
  const int D = a.head_dim;
  const int half = D >> 1;
  const int groups = half >> 3;                       // 8 rotation pairs per thread
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = a.n_rows * a.n_heads * groups;
  if (idx >= total) return;
  const int grp = (int)(idx % groups);
  const int64_t t = idx / groups;
  const int h = (int)(t % a.n_heads);
  const int64_t r = t / a.n_heads;

  const T* ks = static_cast<const T*>(a.k_src) + (r * a.n_heads + h) * D;
  const T* vs = static_cast<const T*>(a.v_src) + (r * a.n_heads + h) * D;
  T* kd = static_cast<T*>(a.k_dst) + ((int64_t)h * a.dst_rows + a.row0 + r) * D;
  T* vd = static_cast<T*>(a.v_dst) + ((int64_t)h * a.dst_rows + a.row0 + r) * D;
  const int64_t pos = a.pos0 + r;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int j = grp * 8 + e;
    float c, s;
    rope_cos_sin(pos, rt.inv_freq[j], &c, &s);
    const float x1 = to_f32(ks[j]);
    const float x2 = to_f32(ks[j + half]);
    kd[j] = from_f32<T>(x1 * c - x2 * s);
    kd[j + half] = from_f32<T>(x2 * c + x1 * s);
    vd[j] = vs[j];
    vd[j + half] = vs[j + half];
  }
}

hipError_t launch_rope_store(const RopeStoreArgs& a, const RopeTable& rt, bool bf16, hipStream_t s) {
  const int64_t total = a.n_rows * a.n_heads * (a.head_dim / 16);
  if (total == 0) return hipSuccess;
  const unsigned grid = (unsigned)((total + 255) / 256);
  if (bf16)
    hipLaunchKernelGGL(rope_store_kernel<bf16_t>, dim3(grid), dim3(256), 0, s, a, rt);
  else
    hipLaunchKernelGGL(rope_store_kernel<float>, dim3(grid), dim3(256), 0, s, a, rt);
  return hipGetLastError();
}

}  // namespace sa
