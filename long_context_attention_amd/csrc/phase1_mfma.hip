// Phase 1 of Star Attention on CDNA4 matrix cores (bf16 in, fp32 accumulate).
//
// Method (Star Attention pages, page 1, "Phase 1: augmented context" and "local
// attention and KV discard"): block c_i (i > 1) attends to the anchor c_1 and
// causally to itself; block 1 attends causally to itself. The anchor rows of an
// augmented block see only the anchor at the anchor's own positions, so their
// outputs and KV equal block 1's; this kernel never computes them and reads the
// anchor's RoPE'd K/V from block 1's rows of the cache.
//
// Work decomposition: one workgroup = 128 query rows of one query head of one
// block (4 wavefronts x 32 rows). K/V tiles of 64 keys stream through LDS
// (double buffered, one barrier per tile): first the anchor tiles (unmasked),
// then the block's tiles up to the diagonal (masked by position only where a
// tile crosses the wavefront's rows or the end of the segment).
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16): S^T = K Q^T and O^T = V^T P^T, so
// in the accumulators each lane owns one query row (lane % 32) and 16 keys / 16
// head dims. The row max needs one exchange between lanes l and l^32; the
// running sum stays lane-partial until the end; rescaling is a per-lane scalar.
// P^T feeds the second product straight from registers: its key order per lane
// is matched by storing V transposed with keys permuted inside each group of 16
// (bits 2 and 3 of the key index swapped).
#include <math.h>

#include "sa_common.h"

namespace sa {
namespace {

constexpr int kBM = 128;   // query rows per workgroup
constexpr int kBN = 64;    // keys per tile
constexpr int kThreads = 256;
constexpr int kKPad = 8;   // bf16 padding per K row   (row stride 272 B at d = 128)
constexpr int kVPad = 8;   // bf16 padding per V^T row (row stride 144 B)

template <int D>
struct P1Smem {
  bf16_t k[2][kBN][D + kKPad];
  bf16_t vt[2][D][kBN + kVPad];
};

__device__ __forceinline__ int perm16(int x) { return (x & 3) | ((x & 4) << 1) | ((x & 8) >> 1); }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

struct Segment {
  int64_t row0;   // first cache row
  int64_t len;    // rows in the segment
};

}  // namespace

template <int D>
__global__ __launch_bounds__(kThreads, 2) void phase1_mfma_kernel(Phase1Args a, RopeTable rt, int64_t n_qt,
                                                                  int64_t n_jobs) {
  __shared__ P1Smem<D> sm;
  constexpr int NC = D / 16;           // 16-wide d chunks (MFMA K dim of QK^T)
  constexpr int NDB = D / 32;          // 32-wide d blocks (MFMA M dim of PV)
  constexpr int KCH = D / 8;           // 16-byte chunks per row
  constexpr int KPIECES = kBN * KCH / kThreads;    // K loads per thread
  constexpr int VPIECES = (kBN / 4) * KCH;         // (4 keys x 8 dims) V pieces per tile

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane >> 5;            // which half of the wavefront
  const int ln = lane & 31;
  const int g = a.n_q_heads / a.n_kv_heads;

  // Job mapping. Workgroup w runs on XCD w % 8; consecutive slots on one XCD take
  // the g query heads that share a KV head, so its L2 serves their K/V tiles, and
  // the 8 XCDs take neighbouring jobs. Jobs are ordered heaviest (last row tile)
  // first.
  int64_t job = blockIdx.x;
  {
    const int64_t grp = 8LL * g;
    const int64_t n_full = (n_jobs / grp) * grp;
    if (job < n_full) {
      const int64_t x = job & 7, s = job >> 3;
      job = (8 * (s / g) + x) * g + (s % g);
    }
  }
  const int hg = (int)(job % g);
  int64_t rest = job / g;
  const int kvh = (int)(rest % a.n_kv_heads);
  rest /= a.n_kv_heads;
  const int64_t nblk = a.ctx_len / a.block_len;
  const int64_t blk = rest % nblk;
  const int64_t qt = n_qt - 1 - rest / nblk;
  const int h = kvh * g + hg;
  const int64_t b = a.block_len;

  // ---- Q rows: load, RoPE (fp64 angles), fold softmax_scale*log2(e), to bf16.
  const int64_t r_lane = qt * kBM + wave * 32 + ln;
  const int64_t rc = r_lane < b ? r_lane : b - 1;
  const int64_t qpos = blk * b + rc;                    // position == token index
  bf16x8 qf[NC];
  {
    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + (qpos * a.n_q_heads + h) * D + 8 * hl;
    float qv[NC][8];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const bf16x8 raw = *reinterpret_cast<const bf16x8*>(qp + 16 * c);
#pragma unroll
      for (int j = 0; j < 8; ++j) qv[c][j] = (float)raw[j];
    }
#pragma unroll
    for (int c = 0; c < NC / 2; ++c) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float cs, sn;
        rope_cos_sin(qpos, rt.inv_freq[16 * c + 8 * hl + j], &cs, &sn);
        const float x1 = qv[c][j], x2 = qv[c + NC / 2][j];
        qv[c][j] = x1 * cs - x2 * sn;
        qv[c + NC / 2][j] = x2 * cs + x1 * sn;
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[c][j] = (bf16_t)(qv[c][j] * a.qk_scale_log2);
  }
  // Wavefront row range (positions) for mask / skip decisions.
  const int64_t w_r0 = qt * kBM + wave * 32;
  const int64_t w_qpos_lo = blk * b + (w_r0 < b ? w_r0 : b - 1);
  const int64_t w_qpos_hi = blk * b + ((w_r0 + 31) < b ? (w_r0 + 31) : b - 1);

  // ---- Key segments: anchor (blocks > 1), then the block's causal prefix.
  Segment seg[2];
  int nseg = 0;
  int64_t tiles0 = 0;
  if (blk > 0) {
    seg[0] = {0, a.anchor_len};
    tiles0 = (a.anchor_len + kBN - 1) / kBN;
    nseg = 1;
  }
  const int64_t kend = ((qt + 1) * kBM) < b ? (qt + 1) * kBM : b;
  seg[nseg] = {blk * b, kend};
  const int64_t n_tiles = tiles0 + (kend + kBN - 1) / kBN;

  const bf16_t* kc = static_cast<const bf16_t*>(a.k_cache) + (int64_t)kvh * a.ctx_len * D;
  const bf16_t* vc = static_cast<const bf16_t*>(a.v_cache) + (int64_t)kvh * a.ctx_len * D;

  bf16x8 kreg[KPIECES];
  bf16x8 vreg[4];
  auto tile_of = [&](int64_t n, Segment& sg, int64_t& kt0) {
    if (n < tiles0) { sg = seg[0]; kt0 = n * kBN; }
    else { sg = seg[nseg]; kt0 = (n - tiles0) * kBN; }
  };
  auto load_tile = [&](int64_t n) {
    Segment sg; int64_t kt0;
    tile_of(n, sg, kt0);
#pragma unroll
    for (int p = 0; p < KPIECES; ++p) {
      const int idx = p * kThreads + tid;
      const int key = idx / KCH, ch = idx % KCH;
      const int64_t kk = (kt0 + key) < sg.len ? kt0 + key : sg.len - 1;   // clamp: stay inside the cache
      kreg[p] = *reinterpret_cast<const bf16x8*>(kc + (sg.row0 + kk) * D + ch * 8);
    }
    if (tid < VPIECES) {
      const int kq = tid / KCH, dc = tid % KCH;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t kk = (kt0 + 4 * kq + r) < sg.len ? kt0 + 4 * kq + r : sg.len - 1;
        vreg[r] = *reinterpret_cast<const bf16x8*>(vc + (sg.row0 + kk) * D + dc * 8);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int p = 0; p < KPIECES; ++p) {
      const int idx = p * kThreads + tid;
      const int key = idx / KCH, ch = idx % KCH;
      *reinterpret_cast<bf16x8*>(&sm.k[buf][key][ch * 8]) = kreg[p];
    }
    if (tid < VPIECES) {
      const int kq = tid / KCH, dc = tid % KCH;
      const int col = ((4 * kq) & ~15) | perm16((4 * kq) & 15);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16x4 t4 = {vreg[0][e], vreg[1][e], vreg[2][e], vreg[3][e]};
        *reinterpret_cast<bf16x4*>(&sm.vt[buf][dc * 8 + e][col]) = t4;
      }
    }
  };

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int64_t n = 0; n < n_tiles; ++n) {
    const int buf = (int)(n & 1);
    if (n + 1 < n_tiles) load_tile(n + 1);

    Segment sg; int64_t kt0;
    tile_of(n, sg, kt0);
    const int64_t kpos0 = sg.row0 + kt0;                // cache row == position
    const bool all_masked = kpos0 > w_qpos_hi;
    if (!all_masked) {
      const bool need_mask = (kpos0 + kBN - 1 > w_qpos_lo) || (kt0 + kBN > sg.len);
      // S^T = K Q^T for 2 blocks of 32 keys.
      f32x16 s[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        s[sb] = f32x16{};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&sm.k[buf][32 * sb + ln][16 * c + 8 * hl]);
          s[sb] = mfma32(ka, qf[c], s[sb]);
        }
      }
      if (need_mask) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kk = 32 * sb + 8 * (i >> 2) + 4 * hl + (i & 3);
            const bool vis = (kt0 + kk < sg.len) && (kpos0 + kk <= qpos);
            s[sb][i] = vis ? s[sb][i] : -INFINITY;
          }
      }
      // Online softmax (base 2; scores already carry scale*log2(e)).
      float mt = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[sb][i]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = fmaxf(m_run, mt);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      float psum = 0.f;
      bf16x8 pb[2][2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float p = fast_exp2(s[sb][8 * hh + j] - m_use);
            psum += p;
            pb[sb][hh][j] = (bf16_t)p;
          }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
      // O^T += V^T P^T, 16 keys per MFMA.
#pragma unroll
      for (int kc16 = 0; kc16 < 4; ++kc16) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x8 va = *reinterpret_cast<const bf16x8*>(&sm.vt[buf][32 * db + ln][16 * kc16 + 8 * hl]);
          o[db] = mfma32(va, pb[kc16 >> 1][kc16 & 1], o[db]);
        }
      }
    }
    if (n + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- Normalise and store this lane's row.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (r_lane < b) {
    const float inv = 1.f / l_tot;
    bf16_t* op = static_cast<bf16_t*>(a.out) + (qpos * a.n_q_heads + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 t4;
#pragma unroll
        for (int e = 0; e < 4; ++e) t4[e] = (bf16_t)(o[db][4 * i4 + e] * inv);
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * i4 + 4 * hl) = t4;
      }
  }
}

hipError_t launch_phase1_mfma(const Phase1Args& a, const RopeTable& rt, int head_dim, hipStream_t s) {
  const int64_t n_qt = (a.block_len + kBM - 1) / kBM;
  const int64_t n_jobs = n_qt * (a.ctx_len / a.block_len) * a.n_q_heads;
  if (n_jobs == 0) return hipSuccess;
  if (head_dim == 64)
    hipLaunchKernelGGL(phase1_mfma_kernel<64>, dim3((unsigned)n_jobs), dim3(kThreads), 0, s, a, rt, n_qt, n_jobs);
  else
    hipLaunchKernelGGL(phase1_mfma_kernel<128>, dim3((unsigned)n_jobs), dim3(kThreads), 0, s, a, rt, n_qt, n_jobs);
  return hipGetLastError();
}

}  // namespace sa
