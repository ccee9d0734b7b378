// Phase 2 local attention for few query rows (decode steps), bf16 caches.
//
// Star Attention pages, page 1, "Phase 2: local attention and local
// statistics": every partition (context block or the query host's tail)
// returns its normalised local output and log-sum-exp. A decode step has
// R = t_q * (Hq/Hkv) <= 8 query rows per KV head, so the work is a stream over
// the cached K/V with 4-8 FLOP per byte: the kernel is built to keep HBM busy.
//
// One workgroup = one chunk of one partition of one KV head. The tail's
// workgroups come first in the grid (they are short), then the context
// partitions' equal-sized chunks. Its 4 wavefronts each stream a contiguous
// run of keys, KT keys per iteration (32, or 16 with 8 rows), with the next
// iteration's K/V loads in flight (register double buffering):
//   * S = Q K^T on the matrix cores (v_mfma_f32_16x16x32_bf16, rows padded to
//     16). K goes straight from HBM into the B operand: the contraction order
//     over head_dim is permuted (MFMA c, k-group q takes elements 32c+8q..+7)
//     so that the 4 lanes holding one key read 64 contiguous bytes per load
//     instruction (Q uses the same permutation).
//   * online softmax per row (base 2, scale*log2(e) folded into Q), row max by
//     DPP inside each 16-lane row; P goes through LDS to the PV lanes.
//   * O += P V on the vector ALUs: each lane owns a 16-byte slice of head_dim,
//     so every V row is read by one fully coalesced 256-byte access.
// The 4 wavefronts' (m, l, O) are merged in LDS; the chunk's normalised output
// and LSE go to the workspace, where the chunk-merge kernel combines chunks.
#include <math.h>

#include <atomic>

#include "sa_common.h"

namespace sa {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// max / sum over the 16 lanes of a DPP row (result in every lane of the row)
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));    // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp<0x4E>(x));    // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp<0x141>(x));   // row_half_mirror
  x = fmaxf(x, dpp<0x140>(x));   // row_mirror
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}

__device__ __forceinline__ void bf16x8_to_f32(bf16x8 v, float (&f)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (float)v[e];
}

}  // namespace

// KT = keys per wavefront iteration (a multiple of 16): 32 for up to 4 rows per
// KV head, 16 for 8 rows, which keeps two workgroups resident per CU.
template <int D, int RT, int KT>
__device__ __forceinline__ void decode_workgroup(const Phase2Args& a, const RopeTable& rt, int64_t job) {
  constexpr int kKT = KT;
  constexpr int NKG = KT / 16;     // 16-key groups per iteration
  constexpr int NC = D / 32;       // MFMAs per 16 keys
  constexpr int DS = D / 8;        // 16-byte slices of a row (PV lanes)
  constexpr int KG = 64 / DS;      // key groups in the PV layout
  constexpr int KPL = kKT / KG;    // keys per lane per iteration (PV)
  // rows past RT take the stores of the spare threads (straight-line code, so the
  // query loads are not sunk below the first tile's loads)
  constexpr int QIT = (RT * (D / 2) + kThreads - 1) / kThreads;
  __shared__ bf16_t q_lds[QIT * kThreads / (D / 2)][D];
  __shared__ float p_lds[4][kKT][RT];
  __shared__ float red_m[4][RT];
  __shared__ float red_l[4][RT];
  __shared__ float red_o[4][RT][D];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ln16 = lane & 15;
  const int q = lane >> 4;
  const int ds = lane % DS;
  const int kgp = lane / DS;
  const int g = a.n_q_heads / a.n_kv_heads;
  const int R = (int)a.t_q * g;

  const int64_t n_tail_jobs = (int64_t)a.n_kv_heads * a.n_tail_chunks;
  int c, hk, p;
  if (job < n_tail_jobs) {
    c = (int)(job % a.n_tail_chunks);
    hk = (int)(job / a.n_tail_chunks);
    p = a.n_ctx_parts;
  } else {
    job -= n_tail_jobs;
    c = (int)(job % a.n_chunks);
    job /= a.n_chunks;
    hk = (int)(job % a.n_kv_heads);
    p = (int)(job / a.n_kv_heads);
  }

  const bool tail = p == a.n_ctx_parts;
  const int64_t len = tail ? a.tail_len : a.block_len;
  const int64_t pos0 = tail ? a.tail_pos0 : (int64_t)p * a.block_len;
  const int64_t head_rows = tail ? a.tail_cap : a.ctx_len;
  const int64_t row0 = tail ? 0 : (int64_t)p * a.block_len;
  // An empty partition (a tail of length 0, whose buffer may be absent) points its
  // loads at the first context row: the first tile is loaded unconditionally below.
  const bool own = len > 0;
  const int64_t first = ((int64_t)hk * head_rows + row0) * D;
  const bf16_t* kbase = own ? static_cast<const bf16_t*>(tail ? a.k_tail : a.k_cache) + first
                            : static_cast<const bf16_t*>(a.k_cache);
  const bf16_t* vbase = own ? static_cast<const bf16_t*>(tail ? a.v_tail : a.v_cache) + first
                            : static_cast<const bf16_t*>(a.v_cache);

  int64_t ck0 = (int64_t)c * a.chunk_len;
  if (ck0 > len) ck0 = len;
  const int64_t ck1 = (ck0 + a.chunk_len) < len ? ck0 + a.chunk_len : len;
  const int64_t per = (((ck1 - ck0) + 3) / 4 + kKT - 1) / kKT * kKT;
  const int64_t wk0 = (ck0 + wave * per) < ck1 ? ck0 + wave * per : ck1;
  const int64_t wk1 = (wk0 + per) < ck1 ? wk0 + per : ck1;

  // Fused append: the workgroup whose chunk holds new tail rows rotates and
  // writes them before anything reads them (no other workgroup reads those rows).
  if (tail && a.n_new > 0) {
    const int64_t nr0 = a.tail_len - a.n_new;             // first new row
    const int64_t lo = nr0 > ck0 ? nr0 : ck0, hi = a.tail_len < ck1 ? a.tail_len : ck1;
    if (lo < hi) {
      bf16_t* kt_ = static_cast<bf16_t*>(const_cast<void*>(a.k_tail)) + first;
      bf16_t* vt_ = static_cast<bf16_t*>(const_cast<void*>(a.v_tail)) + first;
      const bf16_t* kn = static_cast<const bf16_t*>(a.k_new);
      const bf16_t* vn = static_cast<const bf16_t*>(a.v_new);
      for (int64_t idx = threadIdx.x; idx < (hi - lo) * (D / 2); idx += kThreads) {
        const int64_t r = lo + idx / (D / 2);
        const int f = (int)(idx % (D / 2));
        const int64_t src = ((r - nr0) * a.n_kv_heads + hk) * D;
        float cs, sn;
        rope_cos_sin(a.tail_pos0 + r, rt.inv_freq[f], &cs, &sn);
        const float x1 = (float)kn[src + f], x2 = (float)kn[src + f + D / 2];
        kt_[r * D + f] = (bf16_t)(x1 * cs - x2 * sn);
        kt_[r * D + f + D / 2] = (bf16_t)(x2 * cs + x1 * sn);
        vt_[r * D + f] = vn[src + f];
        vt_[r * D + f + D / 2] = vn[src + f + D / 2];
      }
      __syncthreads();   // the stores are visible to every wavefront's loads below
    }
  }

  // ---- Q rows: the workgroup rotates the R rows once (one rotation pair per
  // thread) into LDS; each lane then takes its A-operand slice: row ln16,
  // head_dim elements 32c + 8q + j. Rows R..15 are zero padding. The query
  // values are loaded first, then the first K/V tile's loads go out, so their
  // latency overlaps the rotation.
  // K/V tile loads: K as MFMA B operands (lane: key ln16, elements 32c+8q..+7),
  // V as 16-byte head_dim slices (lane: slice ds of keys kgp + KG i).
  auto load_k = [&](int64_t kt, bf16x8 (&kb)[NKG][NC]) {
#pragma unroll
    for (int kg = 0; kg < NKG; ++kg) {
      int64_t row = (kt + 16 * kg + ln16) < wk1 ? kt + 16 * kg + ln16 : wk1 - 1;
      row = row < 0 ? 0 : row;   // an empty range still reads a valid row (its values are unused)
      const bf16_t* kp = kbase + row * D + 8 * q;
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) kb[kg][cc] = *reinterpret_cast<const bf16x8*>(kp + 32 * cc);
    }
  };
  auto load_v = [&](int64_t kt, bf16x8 (&vb)[KPL]) {
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      int64_t row = (kt + kgp + KG * i) < wk1 ? kt + kgp + KG * i : wk1 - 1;
      row = row < 0 ? 0 : row;
      vb[i] = *reinterpret_cast<const bf16x8*>(vbase + row * D + 8 * ds);
    }
  };
  bf16_t qx1[QIT], qx2[QIT];
  double qfreq[QIT];
#pragma unroll
  for (int it = 0; it < QIT; ++it) {
    // unconditional loads (padding rows and spare threads read row 0; their
    // values are dropped below), so no use of them comes before the tile loads
    const int idx = threadIdx.x + it * kThreads;
    const int r = idx / (D / 2), f = idx % (D / 2);
    const int rr = r < R ? r : 0;
    const int64_t t = rr / g;
    const int h = hk * g + rr % g;
    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + (t * a.n_q_heads + h) * D;
    qx1[it] = qp[f];
    qx2[it] = qp[f + D / 2];
    qfreq[it] = rt.inv_freq[f];
  }
  bf16x8 kb0[NKG][NC], kb1[NKG][NC];
  bf16x8 vb0[KPL], vb1[KPL];
  __builtin_amdgcn_sched_barrier(0);   // the query loads stay ahead of the tile loads
  load_k(wk0, kb0);   // unconditional, so the waits for the query values can count past these
  load_v(wk0, vb0);
  __builtin_amdgcn_sched_barrier(0);   // keep the uses of the query values below the tile loads
#pragma unroll
  for (int it = 0; it < QIT; ++it) {
    const int idx = threadIdx.x + it * kThreads;
    {
      const int r = idx / (D / 2), f = idx % (D / 2);
      // computed for every row (no branch the loads could sink into); padding rows store 0
      float cs, sn;
      rope_cos_sin(a.q_pos0 + (r < R ? r : 0) / g, qfreq[it], &cs, &sn);
      const float x1 = (float)qx1[it], x2 = (float)qx2[it];
      const float y1 = r < R ? (x1 * cs - x2 * sn) * a.qk_scale_log2 : 0.f;
      const float y2 = r < R ? (x2 * cs + x1 * sn) * a.qk_scale_log2 : 0.f;
      q_lds[r][f] = (bf16_t)y1;
      q_lds[r][f + D / 2] = (bf16_t)y2;
    }
  }
  __syncthreads();
  bf16x8 qa[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc)
    qa[cc] = ln16 < RT ? *reinterpret_cast<const bf16x8*>(&q_lds[ln16][32 * cc + 8 * q]) : bf16x8{};
  // positions of the S-layout rows 4q+i (used by the tail's causal mask)
  int64_t srow_pos[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) srow_pos[i] = a.q_pos0 + (4 * q + i) / g;

  float m_run[4], l_run[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { m_run[i] = -INFINITY; l_run[i] = 0.f; }
  float o[RT][8];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[r][e] = 0.f;

  auto compute = [&](int64_t kt, const bf16x8 (&kb)[NKG][NC], const bf16x8 (&vb)[KPL]) {
    f32x4 s[NKG];
#pragma unroll
    for (int kg = 0; kg < NKG; ++kg) {
      s[kg] = f32x4{};
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) s[kg] = mfma16(qa[cc], kb[kg][cc], s[kg]);
    }
    // Keys past a query's position are masked: in the tail, and in the
    // context wherever a tile reaches past the first query's position (a query
    // inside the context) or past the end of this wavefront's keys.
    if (tail || kt + kKT > wk1 || pos0 + kt + kKT - 1 > a.q_pos0) {
#pragma unroll
      for (int kg = 0; kg < NKG; ++kg)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t key = kt + 16 * kg + ln16;
          const bool vis = key < wk1 && pos0 + key <= srow_pos[i];
          s[kg][i] = vis ? s[kg][i] : -INFINITY;
        }
    }
    float alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mx = s[0][i];
#pragma unroll
      for (int kg = 1; kg < NKG; ++kg) mx = fmaxf(mx, s[kg][i]);
      mx = row16_max(mx);
      const float m_new = fmaxf(m_run[i], mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      alpha[i] = fast_exp2(m_run[i] - m_use);
      m_run[i] = m_new;
      float psum = 0.f;
#pragma unroll
      for (int kg = 0; kg < NKG; ++kg) {
        s[kg][i] = fast_exp2(s[kg][i] - m_use);
        psum += s[kg][i];
      }
      l_run[i] = l_run[i] * alpha[i] + psum;
    }
    if (4 * q < RT) {
#pragma unroll
      for (int kg = 0; kg < NKG; ++kg) *reinterpret_cast<f32x4*>(&p_lds[wave][16 * kg + ln16][4 * q]) = s[kg];
    }
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const float ar = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha[r & 3]),
                                                                           16 * (r >> 2)));
#pragma unroll
      for (int e = 0; e < 8; ++e) o[r][e] *= ar;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int key = kgp + KG * i;
      float pr[RT];
#pragma unroll
      for (int r4 = 0; r4 < RT / 4; ++r4) {
        const f32x4 t4 = *reinterpret_cast<const f32x4*>(&p_lds[wave][key][4 * r4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) pr[4 * r4 + e] = t4[e];
      }
      float v[8];
      bf16x8_to_f32(vb[i], v);
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[r][e] = fmaf(pr[r], v[e], o[r][e]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // Register double buffering: while tile i is reduced, tile i+1's 16 KB of
  // K/V loads are already in flight (issued together, before any use).
  for (int64_t kt = wk0; kt < wk1; kt += 2 * kKT) {
    const int64_t k1 = kt + kKT;
    if (k1 < wk1) {
      load_k(k1, kb1);
      load_v(k1, vb1);
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(kt, kb0, vb0);
    if (k1 < wk1) {
      const int64_t k2 = k1 + kKT;
      if (k2 < wk1) {
        load_k(k2, kb0);
        load_v(k2, vb0);
      }
      __builtin_amdgcn_sched_barrier(0);
      compute(k1, kb1, vb1);
    }
  }

  // ---- wavefront totals: l over the 16 key lanes, O over the key groups.
  float l_tot[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) l_tot[i] = row16_sum(l_run[i]);
#pragma unroll
  for (int step = DS; step < 64; step *= 2)
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[r][e] += __shfl_xor(o[r][e], step);
  if (lane < DS) {
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) red_o[wave][r][8 * lane + e] = o[r][e];
  }
  if (ln16 == 0 && 4 * q < RT) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      red_m[wave][4 * q + i] = m_run[i];
      red_l[wave][4 * q + i] = l_tot[i];
    }
  }
  __syncthreads();

  // ---- merge the 4 wavefronts and write this chunk's partial.
  const int64_t rows_all = a.t_q * a.n_q_heads;
  for (int idx = threadIdx.x; idx < R * D; idx += kThreads) {
    const int r = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red_m[w][r]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = fast_exp2(red_m[w][r] - Mu);
      L += f * red_l[w][r];
      O += f * red_o[w][r][d];
    }
    const int64_t t = r / g;
    const int h = hk * g + r % g;
    const int64_t slot = ((int64_t)p * a.n_chunks + c) * rows_all + t * a.n_q_heads + h;
    a.ws_out[slot * D + d] = L > 0.f ? O / L : 0.f;
    if (d == 0) a.ws_lse[slot] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
  }
  // Tail chunk slots that no workgroup was launched for hold no key: their
  // LSE is -inf, so the chunk merge gives them weight 0 (their outputs are
  // never used).
  if (tail && c == a.n_tail_chunks - 1) {
    const int n_empty = a.n_chunks - 1 - c;
    for (int idx = threadIdx.x; idx < n_empty * R; idx += kThreads) {
      const int ce = c + 1 + idx / R, r = idx % R;
      const int64_t t = r / g;
      const int h = hk * g + r % g;
      a.ws_lse[((int64_t)p * a.n_chunks + ce) * rows_all + t * a.n_q_heads + h] = -INFINITY;
    }
  }
}

template <int D, int RT, int KT>
__global__ __launch_bounds__(kThreads) void phase2_decode_kernel(Phase2Args a, RopeTable rt) {
  decode_workgroup<D, RT, KT>(a, rt, blockIdx.x);
}

// Several sequences' decode steps in one grid (same descriptor and row count).
template <int D, int RT, int KT>
__global__ __launch_bounds__(kThreads) void phase2_decode_batch_kernel(Phase2Batch b, RopeTable rt) {
  const int64_t w = blockIdx.x;
  int s = 0;
  while (s + 1 < b.n_seq && w >= b.begin[s + 1]) ++s;
  decode_workgroup<D, RT, KT>(b.seq[s], rt, w - b.begin[s]);
}

int64_t decode_resident_workgroups(int head_dim, int64_t rows_per_kv) {
  // Cached per device and kernel variant (the answer never changes).
  static std::atomic<int64_t> cache[16][4];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return 0;
  const int var = (head_dim == 64 ? 0 : 2) + (rows_per_kv <= 4 ? 0 : 1);
  const int64_t hit = cache[dev][var].load(std::memory_order_relaxed);
  if (hit > 0) return hit;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  hipError_t e;
  switch (var) {
    case 0: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, phase2_decode_kernel<64, 4, 32>, kThreads, 0); break;
    case 1: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, phase2_decode_kernel<64, 8, 16>, kThreads, 0); break;
    case 2: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, phase2_decode_kernel<128, 4, 32>, kThreads, 0); break;
    default: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, phase2_decode_kernel<128, 8, 16>, kThreads, 0);
  }
  if (e != hipSuccess || per_cu < 1 || cus < 1) return 0;
  const int64_t slots = (int64_t)per_cu * cus;
  cache[dev][var].store(slots, std::memory_order_relaxed);
  return slots;
}

hipError_t launch_phase2_decode(const Phase2Args& a, const RopeTable& rt, int head_dim, hipStream_t s) {
  const int64_t n_jobs = (int64_t)a.n_kv_heads * (a.n_tail_chunks + (int64_t)a.n_ctx_parts * a.n_chunks);
  const int R = (int)a.t_q * (a.n_q_heads / a.n_kv_heads);
  const dim3 grid((unsigned)n_jobs), block(kThreads);
  if (head_dim == 64) {
    if (R <= 4) hipLaunchKernelGGL((phase2_decode_kernel<64, 4, 32>), grid, block, 0, s, a, rt);
    else hipLaunchKernelGGL((phase2_decode_kernel<64, 8, 16>), grid, block, 0, s, a, rt);
  } else {
    if (R <= 4) hipLaunchKernelGGL((phase2_decode_kernel<128, 4, 32>), grid, block, 0, s, a, rt);
    else hipLaunchKernelGGL((phase2_decode_kernel<128, 8, 16>), grid, block, 0, s, a, rt);
  }
  return hipGetLastError();
}

hipError_t launch_phase2_decode_batch(const Phase2Batch& b, const RopeTable& rt, int head_dim, int rows_per_kv,
                                      hipStream_t s) {
  const int64_t n_jobs = b.begin[b.n_seq];
  if (n_jobs == 0) return hipSuccess;
  const dim3 grid((unsigned)n_jobs), block(kThreads);
  if (head_dim == 64) {
    if (rows_per_kv <= 4) hipLaunchKernelGGL((phase2_decode_batch_kernel<64, 4, 32>), grid, block, 0, s, b, rt);
    else hipLaunchKernelGGL((phase2_decode_batch_kernel<64, 8, 16>), grid, block, 0, s, b, rt);
  } else {
    if (rows_per_kv <= 4) hipLaunchKernelGGL((phase2_decode_batch_kernel<128, 4, 32>), grid, block, 0, s, b, rt);
    else hipLaunchKernelGGL((phase2_decode_batch_kernel<128, 8, 16>), grid, block, 0, s, b, rt);
  }
  return hipGetLastError();
}

}  // namespace sa
