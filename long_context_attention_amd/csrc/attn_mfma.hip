// Flash-style attention tiles on CDNA4 matrix cores (bf16 in, fp32 accumulate),
// used for Phase 1 of Star Attention and for the Phase-2 query step.
//
// Phase 1 (mode kPhase1). Method (Star Attention pages, page 1, "Phase 1:
// augmented context" and "local attention and KV discard"): block c_i (i > 1)
// attends to the anchor c_1 and causally to itself; block 1 attends causally to
// itself. The anchor rows of an augmented block see only the anchor at the
// anchor's own positions, so their outputs and KV equal block 1's; this kernel
// never computes them and reads the anchor's RoPE'd K/V from block 1's rows of
// the cache.
//
// Phase-2 query step (mode kQuery; page 1, "Phase 2: local attention and local
// statistics"): the rows are the (token, query head) pairs of one KV head, the
// keys one chunk of one partition; the tile writes the chunk's normalised
// output and LSE, which the chunk-merge kernel combines.
//
// Work decomposition: one workgroup = 256 query rows (8 wavefronts x 32 rows),
// one workgroup per CU. In Phase 1 the rows are 256/gp tokens of gp query heads
// that share one KV head, so every K/V tile staged in LDS serves all of them.
// K/V tiles of 64 keys stream through LDS (double buffered, one barrier per
// tile): first the anchor tiles (unmasked), then the block's tiles up to the
// diagonal (masked by position only where a tile crosses a wavefront's rows or
// the end of the segment).
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16): S^T = K Q^T and O^T = V^T P^T, so
// in the accumulators each lane owns one query row (lane % 32) and 16 keys / 16
// head dims. The row max needs one v_permlane32_swap between the two halves of
// the wavefront; the running sum stays lane-partial until the end. P^T feeds
// the second product straight from registers: its key order per lane is
// matched by storing V transposed with keys permuted inside each group of 16
// (bits 2 and 3 of the key index swapped).
//
// Online softmax with a lazy reference (base 2; softmax_scale*log2(e) is folded
// into Q): scores are computed as S - m_ref by seeding the MFMA accumulator with
// -m_ref, and m_ref moves only when a row's tile maximum exceeds it by more
// than kTau, so the rescale of O (64 multiplies) is skipped on almost every
// tile. Probabilities stay below 2^kTau, well inside fp32/bf16 range, and the
// result is the same softmax up to rounding.
#include <math.h>

#include "sa_common.h"

namespace sa {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;   // query rows per workgroup
constexpr int kBN = 64;            // keys per tile
constexpr int kKPad = 8;           // bf16 padding per K row   (row stride 272 B at d = 128)
constexpr int kVPad = 8;           // bf16 padding per V^T row (row stride 144 B)
constexpr float kTau = 8.f;        // lazy-rescale threshold (log2 units)
constexpr int kBufferFlags = 0x00020000;   // buffer resource word 3: 32-bit data format, raw access

template <int D>
struct TileSmem {
  bf16_t k[2][kBN][D + kKPad];
  bf16_t vt[2][D][kBN + kVPad];
};

__device__ __forceinline__ int perm16(int x) { return (x & 3) | ((x & 4) << 1) | ((x & 8) >> 1); }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// value held by lane l ^ 32, via one v_permlane32_swap
__device__ __forceinline__ float other_half(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v),
                                                  false, false);
  const int lane = threadIdx.x & 63;
  return __builtin_bit_cast(float, lane < 32 ? r[1] : r[0]);
}

__device__ __forceinline__ int64_t wave_min_i64(int64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const int64_t o = __shfl_xor(v, m);
    v = o < v ? o : v;
  }
  return v;
}
__device__ __forceinline__ int64_t wave_max_i64(int64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const int64_t o = __shfl_xor(v, m);
    v = o > v ? o : v;
  }
  return v;
}

// Workgroup w runs on XCD w % 8. Consecutive slots of one XCD take `grp`
// consecutive logical jobs (the jobs that share K/V tiles), so that XCD's L2
// serves them, while the 8 XCDs take neighbouring groups.
__device__ __forceinline__ int64_t xcd_remap(int64_t w, int64_t n_jobs, int64_t grp) {
  const int64_t span = 8 * grp;
  if (w >= (n_jobs / span) * span) return w;
  const int64_t x = w & 7, s = w >> 3;
  return (8 * (s / grp) + x) * grp + (s % grp);
}

struct Segment {
  int64_t row0;   // first cache row
  int64_t len;    // rows in the segment
};

struct TileArgs {
  Phase1Args p1;            // kPhase1
  Phase2Args p2;            // kQuery
  int64_t n_row_tiles;      // kPhase1: row tiles per block; kQuery: row tiles per KV head
  int64_t n_jobs;
  int32_t heads_per_tile;   // kPhase1: query heads packed into one tile (divides 8 and Hq/Hkv)
};

enum { kPhase1 = 0, kQuery = 1 };

}  // namespace

template <int D, int MODE>
__global__ __launch_bounds__(kThreads, 1) void attn_tile_kernel(TileArgs ta, RopeTable rt) {
  __shared__ TileSmem<D> sm;
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
  const int n_q_heads = MODE == kPhase1 ? ta.p1.n_q_heads : ta.p2.n_q_heads;
  const int n_kv_heads = MODE == kPhase1 ? ta.p1.n_kv_heads : ta.p2.n_kv_heads;
  const int g = n_q_heads / n_kv_heads;
  const float qk_scale = MODE == kPhase1 ? ta.p1.qk_scale_log2 : ta.p2.qk_scale_log2;

  // ---- Job decode: this lane's query row (token, head, position) and the key segments.
  int kvh, h;
  int64_t tok, qpos;
  bool row_valid;
  Segment seg_a{0, 0};   // anchor (Phase 1, blocks > 1)
  Segment seg_b{0, 0};   // the block's causal prefix, or the Phase-2 chunk
  int64_t tiles0 = 0;
  const bf16_t* kc;
  const bf16_t* vc;
  int p2_part = 0, p2_chunk = 0;
  int64_t pos_shift = 0;               // key position = cache row + pos_shift
  if constexpr (MODE == kPhase1) {
    const Phase1Args& a = ta.p1;
    const int gp = ta.heads_per_tile;
    const int groups = g / gp;
    const int64_t tpt = kBM / gp;      // tokens per tile
    // jobs ordered heaviest (last row tile) first; head groups of a KV head adjacent
    const int64_t job = xcd_remap(blockIdx.x, ta.n_jobs, groups);
    const int hgrp = (int)(job % groups);
    int64_t rest = job / groups;
    kvh = (int)(rest % n_kv_heads);
    rest /= n_kv_heads;
    const int64_t nblk = a.ctx_len / a.block_len;
    const int64_t blk = rest % nblk;
    const int64_t qt = ta.n_row_tiles - 1 - rest / nblk;
    h = kvh * g + hgrp * gp + wave % gp;
    const int64_t b = a.block_len;
    const int64_t r_lane = qt * tpt + (wave / gp) * 32 + ln;
    row_valid = r_lane < b;
    tok = blk * b + (row_valid ? r_lane : b - 1);
    qpos = tok;
    if (blk > 0) {
      seg_a = {0, a.anchor_len};
      tiles0 = (a.anchor_len + kBN - 1) / kBN;
    }
    const int64_t kend = ((qt + 1) * tpt) < b ? (qt + 1) * tpt : b;
    seg_b = {blk * b, kend};
    kc = static_cast<const bf16_t*>(a.k_cache) + (int64_t)kvh * a.ctx_len * D;
    vc = static_cast<const bf16_t*>(a.v_cache) + (int64_t)kvh * a.ctx_len * D;
  } else {
    const Phase2Args& a = ta.p2;
    // jobs: (partition, KV head, chunk, row tile), row tiles of one chunk adjacent
    const int64_t job = xcd_remap(blockIdx.x, ta.n_jobs, ta.n_row_tiles);
    const int64_t rtile = job % ta.n_row_tiles;
    int64_t rest = job / ta.n_row_tiles;
    p2_chunk = (int)(rest % a.n_chunks);
    rest /= a.n_chunks;
    kvh = (int)(rest % n_kv_heads);
    p2_part = (int)(rest / n_kv_heads);
    const int64_t r = rtile * kBM + wave * 32 + ln;        // row = (head in group) * t_q + token
    row_valid = r < a.t_q * g;
    const int64_t rc = row_valid ? r : 0;
    tok = rc % a.t_q;
    h = kvh * g + (int)(rc / a.t_q);
    qpos = a.q_pos0 + tok;
    const bool tail = p2_part == a.n_ctx_parts;
    const int64_t len = tail ? a.tail_len : a.block_len;
    const int64_t head_rows = tail ? a.tail_cap : a.ctx_len;
    const int64_t part_row0 = tail ? 0 : (int64_t)p2_part * a.block_len;
    int64_t ck0 = (int64_t)p2_chunk * a.chunk_len;
    if (ck0 > len) ck0 = len;
    const int64_t ck1 = (ck0 + a.chunk_len) < len ? ck0 + a.chunk_len : len;
    seg_b = {part_row0 + ck0, ck1 - ck0};
    if (tail) pos_shift = a.tail_pos0;
    kc = static_cast<const bf16_t*>(tail ? a.k_tail : a.k_cache) + (int64_t)kvh * head_rows * D;
    vc = static_cast<const bf16_t*>(tail ? a.v_tail : a.v_cache) + (int64_t)kvh * head_rows * D;
  }

  // ---- Q rows: load, RoPE (fp64 angles), fold softmax_scale*log2(e), to bf16.
  bf16x8 qf[NC];
  {
    const bf16_t* qbase = static_cast<const bf16_t*>(MODE == kPhase1 ? ta.p1.q : ta.p2.q);
    const bf16_t* qp = qbase + (tok * n_q_heads + h) * D + 8 * hl;
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
      for (int j = 0; j < 8; ++j) qf[c][j] = (bf16_t)(qv[c][j] * qk_scale);
  }
  // Wavefront query-position range (valid rows only) for mask / skip decisions.
  const int64_t w_qpos_lo = wave_min_i64(row_valid ? qpos : INT64_MAX);
  const int64_t w_qpos_hi = wave_max_i64(row_valid ? qpos : INT64_MIN);
  const int64_t n_tiles = tiles0 + (seg_b.len + kBN - 1) / kBN;

  bf16x8 kreg[KPIECES];
  bf16x8 vreg[4];
  auto tile_of = [&](int64_t n, Segment& sg, int64_t& kt0) {
    if (n < tiles0) { sg = seg_a; kt0 = n * kBN; }
    else { sg = seg_b; kt0 = (n - tiles0) * kBN; }
  };
  // Tile loads through buffer resources whose base is the tile's first row and
  // whose extent ends at the segment's end: the hardware returns zeros for rows
  // past the end (those keys are masked), the per-lane byte offsets are
  // constants and the tile's position is scalar arithmetic only.
  // K pieces: 16-byte row chunks, a row per 16 lanes (coalesced). V pieces:
  // 4 keys x 8 dims, keys fastest across lanes so the transposed LDS stores of
  // 16 neighbouring lanes fill one 128-byte row span (no bank conflicts).
  auto load_tile = [&](int64_t n) {
    Segment sg; int64_t kt0;
    tile_of(n, sg, kt0);
    const int64_t rows_left = sg.len - kt0;
    const int nbytes = (int)((rows_left < kBN ? rows_left : kBN) * D * 2);
    const int64_t first = (sg.row0 + kt0) * D;
    const auto krs = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(kc + first), 0, nbytes, kBufferFlags);
#pragma unroll
    for (int p = 0; p < KPIECES; ++p)
      kreg[p] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(krs, (p * kThreads + tid) * 16, 0, 0));
    if (tid < VPIECES) {
      const auto vrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(vc + first), 0, nbytes, kBufferFlags);
      const int kq = tid & 15, dc = tid >> 4;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vreg[r] = __builtin_bit_cast(bf16x8,
                                     __builtin_amdgcn_raw_buffer_load_b128(vrs, ((4 * kq + r) * D + dc * 8) * 2, 0, 0));
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
      const int kq = tid & 15, dc = tid >> 4;
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
  float m_use = 0.f;         // reference subtracted from this lane's scores
  bool has_ref = false;      // m_use has been set from a visible score
  f32x16 negm = f32x16{};    // -m_use in every element (accumulator seed)
  float l_run = 0.f;         // lane-partial sum of exp2(s - m_use)
  const bf16x2 ones = {(bf16_t)1.f, (bf16_t)1.f};

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int64_t n = 0; n < n_tiles; ++n) {
    const int buf = (int)(n & 1);
    if (n + 1 < n_tiles) load_tile(n + 1);

    Segment sg; int64_t kt0;
    tile_of(n, sg, kt0);
    const int64_t kpos0 = sg.row0 + kt0 + pos_shift;    // position of the tile's first key
    const bool all_masked = kpos0 > w_qpos_hi;
    if (!all_masked) {
      const bool need_mask = (kpos0 + kBN - 1 > w_qpos_lo) || (kt0 + kBN > sg.len);
      // S^T - m_use for 2 blocks of 32 keys (accumulators seeded with -m_use).
      f32x16 s[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        s[sb] = negm;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&sm.k[buf][32 * sb + ln][16 * c + 8 * hl]);
          s[sb] = mfma32(ka, qf[c], s[sb]);
        }
      }
      if (need_mask) {
        const int lim_len = (int)((sg.len - kt0) < kBN ? sg.len - kt0 : kBN);
        const int64_t dq = qpos - kpos0;                  // keys kk <= dq are visible
        const int lim_pos = dq < 0 ? 0 : (dq >= kBN ? kBN : (int)dq + 1);
        const int lim = lim_len < lim_pos ? lim_len : lim_pos;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kk = 32 * sb + 8 * (i >> 2) + 4 * hl + (i & 3);
            s[sb][i] = kk < lim ? s[sb][i] : -INFINITY;
          }
      }
      float mt = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[sb][i]);
      mt = fmaxf(mt, other_half(mt));
      const bool upd = mt > -INFINITY && (!has_ref || mt > kTau);
      if (__builtin_amdgcn_ballot_w64(upd)) {
        // Rare: move the reference to this tile's maximum for the rows that need it.
        const float delta = upd ? mt : 0.f;
        const float alpha = upd ? (has_ref ? fast_exp2(-delta) : 0.f) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] *= alpha;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) s[sb] -= delta;
        m_use += delta;
        has_ref = has_ref || upd;
#pragma unroll
        for (int i = 0; i < 16; ++i) negm[i] = -m_use;
      }
      bf16x8 pb[2][2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int j = 0; j < 8; ++j) pb[sb][hh][j] = (bf16_t)fast_exp2(s[sb][8 * hh + j]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bf16x2 pr = {pb[sb][hh][2 * j], pb[sb][hh][2 * j + 1]};
            l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run, false);
          }
        }
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
  const float l_tot = l_run + other_half(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if constexpr (MODE == kPhase1) {
    if (row_valid) {
      bf16_t* op = static_cast<bf16_t*>(ta.p1.out) + (tok * n_q_heads + h) * D;
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
  } else {
    if (row_valid) {
      const Phase2Args& a = ta.p2;
      const int64_t slot = (((int64_t)p2_part * a.n_chunks + p2_chunk) * a.t_q + tok) * n_q_heads + h;
      float* op = a.ws_out + slot * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          f32x4 t4;
#pragma unroll
          for (int e = 0; e < 4; ++e) t4[e] = o[db][4 * i4 + e] * inv;
          *reinterpret_cast<f32x4*>(op + 32 * db + 8 * i4 + 4 * hl) = t4;
        }
      if (hl == 0) a.ws_lse[slot] = l_tot > 0.f ? (m_use + log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

namespace {
// Largest power of two that divides the GQA group and 8 (the wavefronts per tile).
int heads_per_tile(int g) {
  int gp = 1;
  while (gp < 8 && g % (gp * 2) == 0) gp *= 2;
  return gp;
}
}  // namespace

hipError_t launch_phase1_mfma(const Phase1Args& a, const RopeTable& rt, int head_dim, hipStream_t s) {
  TileArgs ta{};
  ta.p1 = a;
  ta.heads_per_tile = heads_per_tile(a.n_q_heads / a.n_kv_heads);
  const int64_t tpt = kBM / ta.heads_per_tile;
  ta.n_row_tiles = (a.block_len + tpt - 1) / tpt;
  ta.n_jobs = ta.n_row_tiles * (a.ctx_len / a.block_len) * (a.n_q_heads / ta.heads_per_tile);
  if (ta.n_jobs == 0) return hipSuccess;
  const dim3 grid((unsigned)ta.n_jobs), block(kThreads);
  if (head_dim == 64) hipLaunchKernelGGL((attn_tile_kernel<64, kPhase1>), grid, block, 0, s, ta, rt);
  else hipLaunchKernelGGL((attn_tile_kernel<128, kPhase1>), grid, block, 0, s, ta, rt);
  return hipGetLastError();
}

hipError_t launch_phase2_query(const Phase2Args& a, const RopeTable& rt, int head_dim, hipStream_t s) {
  TileArgs ta{};
  ta.p2 = a;
  ta.heads_per_tile = 1;
  const int64_t rows = a.t_q * (a.n_q_heads / a.n_kv_heads);
  ta.n_row_tiles = (rows + kBM - 1) / kBM;
  ta.n_jobs = ta.n_row_tiles * (int64_t)a.n_chunks * a.n_kv_heads * (a.n_ctx_parts + 1);
  if (ta.n_jobs == 0) return hipSuccess;
  const dim3 grid((unsigned)ta.n_jobs), block(kThreads);
  if (head_dim == 64) hipLaunchKernelGGL((attn_tile_kernel<64, kQuery>), grid, block, 0, s, ta, rt);
  else hipLaunchKernelGGL((attn_tile_kernel<128, kQuery>), grid, block, 0, s, ta, rt);
  return hipGetLastError();
}

}  // namespace sa
