// Float32 (and generic) attention kernels on the vector ALUs.
//
// These carry the float32 workloads, whose tolerance (1e-4) calls for float32
// products; the bf16 workloads run on the MFMA kernels. Both keep an online
// softmax over the keys (running max m and running sum l in base 2, rescaled
// only when m grows). Phase 1: one thread per query row over LDS key tiles.
// Phase 2: one wavefront per query row and chunk, lanes over head_dim.
#include <math.h>

#include "sa_common.h"

namespace sa {

namespace {
constexpr int kP1Rows = 64;   // query rows per workgroup
constexpr int kP1Keys = 32;   // keys per LDS tile

template <typename T, int D>
__device__ __forceinline__ void load_rope_q(const T* qp, int64_t pos, const RopeTable& rt, float scale,
                                            float (&q)[D]) {
#pragma unroll
  for (int j = 0; j < D / 2; ++j) {
    float c, s;
    rope_cos_sin(pos, rt.inv_freq[j], &c, &s);
    const float x1 = to_f32(qp[j]);
    const float x2 = to_f32(qp[j + D / 2]);
    q[j] = (x1 * c - x2 * s) * scale;
    q[j + D / 2] = (x2 * c + x1 * s) * scale;
  }
}
}  // namespace

// Phase 1: grid (row tiles of a block, blocks, query heads).
template <typename T, int D>
__global__ __launch_bounds__(kP1Rows) void phase1_valu_kernel(Phase1Args a, RopeTable rt) {
  __shared__ float ks[kP1Keys][D];
  __shared__ float vs[kP1Keys][D];
  const int tid = threadIdx.x;
  const int64_t b = a.block_len;
  const int64_t r = (int64_t)blockIdx.x * kP1Rows + tid;
  const int64_t blk = blockIdx.y;                      // 0-based block index
  const int h = blockIdx.z;
  const int hk = h / (a.n_q_heads / a.n_kv_heads);
  const bool valid = r < b;
  const int64_t tok = blk * b + (valid ? r : b - 1);   // position == token index

  float q[D], o[D];
  load_rope_q<T, D>(static_cast<const T*>(a.q) + (tok * a.n_q_heads + h) * D, tok, rt, a.qk_scale_log2, q);
#pragma unroll
  for (int d = 0; d < D; ++d) o[d] = 0.f;
  float m = -INFINITY, l = 0.f;

  const T* kc = static_cast<const T*>(a.k_cache) + (int64_t)hk * a.ctx_len * D;
  const T* vc = static_cast<const T*>(a.v_cache) + (int64_t)hk * a.ctx_len * D;
  // Key segments: the anchor (blocks > 1; block 1's or the previous block's
  // first A rows, all before the block and so all visible; its keys rotated
  // for this block from k_anchor when given), then the block's causal prefix.
  const T* seg_k[2];
  const T* seg_v[2];
  int64_t seg_start[2], seg_len[2];
  int nseg = 0;
  if (blk > 0) {
    const int64_t a0 = a.anchor_prev ? (blk - 1) * b : 0;
    const int64_t n_anchors = a.ctx_len / b - 1;
    seg_k[nseg] = a.k_anchor ? static_cast<const T*>(a.k_anchor) + ((int64_t)hk * n_anchors + blk - 1) * a.anchor_len * D
                             : kc + a0 * D;
    seg_v[nseg] = vc + a0 * D;
    seg_start[nseg] = 0;
    seg_len[nseg] = a.anchor_len;
    ++nseg;
  }
  seg_k[nseg] = kc;
  seg_v[nseg] = vc;
  seg_start[nseg] = blk * b;
  seg_len[nseg] = ((int64_t)blockIdx.x + 1) * kP1Rows < b ? ((int64_t)blockIdx.x + 1) * kP1Rows : b;
  ++nseg;

  for (int sg = 0; sg < nseg; ++sg) {
    for (int64_t k0 = 0; k0 < seg_len[sg]; k0 += kP1Keys) {
      __syncthreads();
      for (int e = tid; e < kP1Keys * D; e += kP1Rows) {
        const int kk = e / D, d = e % D;
        const int64_t kr = seg_start[sg] + ((k0 + kk) < seg_len[sg] ? (k0 + kk) : seg_len[sg] - 1);
        ks[kk][d] = to_f32(seg_k[sg][kr * D + d]);
        vs[kk][d] = to_f32(seg_v[sg][kr * D + d]);
      }
      __syncthreads();
      const int nk = (seg_len[sg] - k0) < kP1Keys ? (int)(seg_len[sg] - k0) : kP1Keys;
      for (int kk = 0; kk < nk; ++kk) {
        const int64_t kpos = seg_start[sg] + k0 + kk;   // anchor rows count from 0: all < tok
        if (kpos > tok) continue;
        float sc = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) sc = fmaf(q[d], ks[kk][d], sc);
        if (sc > m) {
          const float al = fast_exp2(m - sc);
          l *= al;
#pragma unroll
          for (int d = 0; d < D; ++d) o[d] *= al;
          m = sc;
        }
        const float p = fast_exp2(sc - m);
        l += p;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = fmaf(p, vs[kk][d], o[d]);
      }
    }
  }
  if (valid) {
    T* op = static_cast<T*>(a.out) + (tok * a.n_q_heads + h) * D;
    const float inv = 1.f / l;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = from_f32<T>(o[d] * inv);
  }
}

// Phase 2 local attention, one chunk of one partition per workgroup:
// grid (chunks, partitions, row groups of 64 (token, head) rows).
// Phase 2 (float32 workloads): one wavefront per (partition chunk, query row).
// Each lane owns head_dim elements lane and lane + 64, so every K and V row is
// read by one coalesced access; the score is a wavefront sum, and the online
// softmax state (m, l) is the same in every lane.
template <typename T, int D>
__global__ __launch_bounds__(64) void phase2_valu_kernel(Phase2Args a, RopeTable rt) {
  constexpr int E = D / 64;   // head_dim elements per lane
  const int lane = threadIdx.x;
  const int64_t rows = a.t_q * a.n_q_heads;
  int64_t job = blockIdx.x;
  const int64_t rr = job % rows;
  job /= rows;
  const int c = (int)(job % a.n_chunks);
  const int p = (int)(job / a.n_chunks);
  const int64_t t = rr / a.n_q_heads;
  const int h = (int)(rr % a.n_q_heads);
  const int hk = h / (a.n_q_heads / a.n_kv_heads);
  const int64_t qpos = a.q_pos0 + t;

  const bool tail = p == a.n_ctx_parts;
  const int64_t len = tail ? a.tail_len : a.block_len;
  const int64_t pos0 = tail ? a.tail_pos0 : (int64_t)p * a.block_len;
  const int64_t head_rows = tail ? a.tail_cap : a.ctx_len;
  const int64_t row0 = tail ? 0 : (int64_t)p * a.block_len;
  const T* kb = static_cast<const T*>(tail ? a.k_tail : a.k_cache) + ((int64_t)hk * head_rows + row0) * D;
  const T* vb = static_cast<const T*>(tail ? a.v_tail : a.v_cache) + ((int64_t)hk * head_rows + row0) * D;

  // This lane's elements of the rotated, scaled query: element d pairs with
  // d +- D/2 (rotate-half).
  const T* qp = static_cast<const T*>(a.q) + (t * a.n_q_heads + h) * D;
  float q[E], o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int d = lane + 64 * e;
    const int j = d % (D / 2);
    float cs, sn;
    rope_cos_sin(qpos, rt.inv_freq[j], &cs, &sn);
    const float x1 = to_f32(qp[j]), x2 = to_f32(qp[j + D / 2]);
    q[e] = (d < D / 2 ? x1 * cs - x2 * sn : x2 * cs + x1 * sn) * a.qk_scale_log2;
    o[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int64_t k_begin = (int64_t)c * a.chunk_len;
  int64_t k_end = (k_begin + a.chunk_len) < len ? (k_begin + a.chunk_len) : len;
  // keys at positions after the query are not visible (positions increase along the partition)
  if (qpos - pos0 + 1 < k_end) k_end = qpos - pos0 + 1 > k_begin ? qpos - pos0 + 1 : k_begin;
  constexpr int U = 4;        // keys in flight
  for (int64_t k0 = k_begin; k0 < k_end; k0 += U) {
    float kv[U][E], vv[U][E], sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = (k0 + u) < k_end ? k0 + u : k_end - 1;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        kv[u][e] = to_f32(kb[k * D + lane + 64 * e]);
        vv[u][e] = to_f32(vb[k * D + lane + 64 * e]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) part = fmaf(q[e], kv[u][e], part);
#pragma unroll
      for (int mk = 32; mk >= 1; mk >>= 1) part += __shfl_xor(part, mk);
      sc[u] = (k0 + u) < k_end ? part : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (sc[u] > m) {
        const float al = fast_exp2(m - sc[u]);
        l *= al;
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] *= al;
        m = sc[u];
      }
      const float pr = sc[u] == -INFINITY ? 0.f : fast_exp2(sc[u] - m);
      l += pr;
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = fmaf(pr, vv[u][e], o[e]);
    }
  }
  const int64_t slot = ((int64_t)p * a.n_chunks + c) * rows + rr;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) a.ws_out[slot * D + lane + 64 * e] = o[e] * inv;
  if (lane == 0) a.ws_lse[slot] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

hipError_t launch_phase1_valu(const Phase1Args& a, const RopeTable& rt, int head_dim, bool bf16, hipStream_t s) {
  const dim3 grid((unsigned)((a.block_len + kP1Rows - 1) / kP1Rows), (unsigned)(a.ctx_len / a.block_len),
                  (unsigned)a.n_q_heads);
  const dim3 block(kP1Rows);
  if (head_dim == 64) {
    if (bf16) hipLaunchKernelGGL((phase1_valu_kernel<bf16_t, 64>), grid, block, 0, s, a, rt);
    else hipLaunchKernelGGL((phase1_valu_kernel<float, 64>), grid, block, 0, s, a, rt);
  } else {
    if (bf16) hipLaunchKernelGGL((phase1_valu_kernel<bf16_t, 128>), grid, block, 0, s, a, rt);
    else hipLaunchKernelGGL((phase1_valu_kernel<float, 128>), grid, block, 0, s, a, rt);
  }
  return hipGetLastError();
}

hipError_t launch_phase2_valu(const Phase2Args& a, const RopeTable& rt, int head_dim, bool bf16, hipStream_t s) {
  const int64_t rows = a.t_q * a.n_q_heads;
  const dim3 grid((unsigned)((int64_t)(a.n_ctx_parts + 1) * a.n_chunks * rows));
  if (head_dim == 64) {
    if (bf16) hipLaunchKernelGGL((phase2_valu_kernel<bf16_t, 64>), grid, dim3(64), 0, s, a, rt);
    else hipLaunchKernelGGL((phase2_valu_kernel<float, 64>), grid, dim3(64), 0, s, a, rt);
  } else {
    if (bf16) hipLaunchKernelGGL((phase2_valu_kernel<bf16_t, 128>), grid, dim3(64), 0, s, a, rt);
    else hipLaunchKernelGGL((phase2_valu_kernel<float, 128>), grid, dim3(64), 0, s, a, rt);
  }
  return hipGetLastError();
}

}  // namespace sa
