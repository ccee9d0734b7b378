// Flash-style attention tiles on CDNA4 matrix cores (bf16 in, fp32 accumulate),
// used for Phase 1 of Star Attention and for the Phase-2 query step.
//
// Phase 1 (mode kPhase1). Method (Star Attention pages, page 1, "Phase 1:
// augmented context" and "local attention and KV discard"): block c_i (i > 1)
// attends to the anchor c_1 and causally to itself; block 1 attends causally to
// itself. The anchor rows of an augmented block see only the anchor at the
// anchor's own positions, so their outputs and KV equal block 1's; this kernel
// never computes them and reads the anchor's RoPE'd K/V from the anchor block's
// rows of the cache (block 1; block i - 1 for the previous-block anchor, the
// pages' ablation).
//
// Mode kPhase1Ws is Phase 1 with the anchor at other position IDs (the pages'
// position ablation, page 3, section 4.1): its anchor K tiles come from a
// workspace that holds the anchor's keys rotated for each block, its V tiles
// from the cache as before. It is a separate instance so that kPhase1 keeps
// one key base per tile.
//
// Phase-2 query step (mode kQuery; page 1, "Phase 2: local attention and local
// statistics"): the rows are the (token, query head) pairs of one KV head, the
// keys one chunk of one partition; the tile writes the chunk's normalised
// output and LSE, which the chunk-merge kernel combines.
//
// Work decomposition: one workgroup = 256 query rows (8 wavefronts x 32 rows),
// one workgroup per CU. In Phase 1 the rows are 256/gp tokens of gp query heads
// that share one KV head, so every K/V tile staged in LDS serves all of them.
// K/V tiles of 64 keys stream through LDS: first the anchor tiles (unmasked),
// then the block's tiles up to the diagonal (masked by position only where a
// tile crosses a wavefront's rows or the end of the segment).
//
// Phase-1 jobs go out in non-increasing order of work (the dispatcher hands
// workgroups to the CUs in rounds, so a round of unequal jobs leaves CUs idle
// until its longest job ends). With a workspace for its counters, the order is
// taken at run time from one queue per XCD, so that the faster XCDs take over
// the last jobs of the slower ones (see grab_job).
//
// Staging: tiles go from HBM/L2 straight into LDS (buffer_load ... lds, no
// registers) through a ring of five slots (160 KB at head_dim 128), three tiles
// ahead of use, with one barrier per two tiles. Each wavefront's share of a
// tile's loads is issued one instruction at a time between the QK^T MFMAs, so
// the CU's address path drains while the matrix cores work. K and V are stored
// row-major with their 16-byte chunks XOR-swizzled by row, so the operand reads
// below are free of bank conflicts. The loads are issued as statements of
// their own (see load_lds16), so the only waits for them are the tile loop's
// own; the slots are five distinct LDS objects and the tile loop is unrolled by
// ten (two passes over the ring), so every operand address is a constant
// offset from a slot's base.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16): S^T = K Q^T and O^T = V^T P^T, so
// in the accumulators each lane owns one query row (lane % 32) and 16 keys / 16
// head dims. The row max needs one v_permlane32_swap between the two halves of
// the wavefront; the running sum stays lane-partial until the end. P^T feeds
// the second product straight from registers, keys ordered {0-3, 8-11} in the
// low half-wave and {4-7, 12-15} in the high one (the accumulator layout); the
// matching V^T operand comes from row-major V by two transposing reads
// (ds_read_b64_tr_b16), each giving a lane 4 consecutive keys of its column.
// The K operand reads run four ahead of the QK^T MFMAs.
//
// Online softmax with a lazy reference (base 2; softmax_scale*log2(e) is folded
// into Q): scores are computed as S - m_ref by seeding the MFMA accumulator with
// -m_ref, and the probabilities exp2(S - m_ref) are taken against it without a
// row maximum. The reference only has to keep them in range: when a tile's
// probabilities sum past kBig in some lane (a score about 27 above m_ref), and
// on a row's first visible tile, the rare path takes the tile's row maximum,
// moves m_ref there for the rows it exceeds by more than kTau, rescales O (64
// multiplies) and the row sum, and computes the probabilities again. They stay
// below 2^32, well inside fp32/bf16 range (bf16 has fp32's exponent range), and
// the result is the same softmax up to rounding.
//
// Issue order: the hardware issues the oldest ready wavefront first, so of the
// two wavefronts on a SIMD the first one ran ahead and waited at every barrier
// while the second finished alone (18% against 1% of their loop time). The
// second wavefronts (4-7) take the higher priority for the first tile of each
// barrier interval, which evens the two out (Phase 1 about 1.5% faster).
#include <math.h>

#include "sa_common.h"

namespace sa {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;   // query rows per workgroup
constexpr int kBN = 64;            // keys per tile
constexpr float kTau = 8.f;        // lazy-rescale threshold (log2 units)
constexpr float kBig = 4294967296.f;   // 2^32: a tile's lane sum of probabilities past it moves the reference
constexpr int kQkReadDepth = 4;    // K operand reads in flight ahead of the QK^T MFMAs
constexpr int kLoadEvery = 4;      // one direct-to-LDS tile load per this many QK^T MFMAs
constexpr int kBufferFlags = 0x00020000;   // buffer resource word 3: 32-bit data format, raw access

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// One ring slot: a 64-key tile of K and of V, both row-major (key-major) with
// the 16-byte chunks of row r stored at chunk c ^ swz_k(r) / c ^ swz_v(r).
template <int D>
struct TileSlot {
  bf16_t k[kBN * D];
  bf16_t v[kBN * D];
};
// The swizzles make the operand reads conflict-free: for K, the 16 consecutive
// rows read at one logical chunk land in 16 distinct chunk columns; for V, the
// 4 rows x 2 chunks of one transposing read group and the neighbouring group
// two chunks over land in 16 distinct columns.
template <int D> __device__ __forceinline__ int swz_k(int r) { return r % (D / 8); }
template <int D> __device__ __forceinline__ int swz_v(int r) { return (4 * r) % (D / 8); }

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

// Buffer resource of `nbytes` bytes from byte address `a` (both uniform):
// base address, no stride, the extent (reads past it return zeros), 32-bit raw
// access.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t make_rsrc(uint64_t a, int nbytes) {
  return i32x4_t{(int)(unsigned)a, (int)((unsigned)(a >> 32) & 0xffffu), nbytes, kBufferFlags};
}

// A 64-bit value the wavefront holds in every lane, moved to scalar registers.
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// One direct-to-LDS load: 16 bytes per lane from the buffer at byte offset
// `voff`, written to LDS at dst + 16 * lane. Written as a statement of its own
// rather than the compiler's builtin: for the builtin, the compiler's wait
// insertion cannot tell the five ring slots apart inside the unrolled loop and
// waits for every load in flight before each tile's first LDS read, which
// takes the loads of the tiles ahead of use off the wire. The instruction
// writes no register (its data goes to LDS), so nothing the compiler allocates
// is written late; the tile loop orders the LDS writes itself (s_waitcnt
// vmcnt, then a workgroup barrier, before a slot is read; a barrier after the
// last read before a slot is refilled). M0 holds the LDS address. The
// compiler does not look inside the statement for hazards, so it waits itself:
// five wait states between the last vector-ALU write of an SGPR it reads (the
// tile's extent passes through v_readfirstlane, and the compiler may hand such a
// register straight to the load) and the load, as CDNA
// requires for a vector-memory read of such an SGPR (fewer can let the load
// take a stale base or extent). (A helper rather than a call inside the
// kernel's lambdas: there the host-side pass would drop the kernel.)
__device__ __forceinline__ void load_lds16(i32x4_t rs, lds_void* base, int byte_off, int voff) {
  const unsigned lds = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)base + (unsigned)byte_off);
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"{m0}"(lds), "v"(voff), "s"(rs) : "memory");
}

// Wait until at most N of this wavefront's vector-memory operations (the
// direct-to-LDS tile loads) are outstanding. The "memory" clobber keeps LDS
// reads from moving above it.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
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

// Phase-1 jobs handed out at run time: queue x (x = 0..7) holds jobs x, x + 8,
// x + 16, ... in order, the jobs the static mapping gives XCD x (workgroup w
// runs on XCD w % 8), so each XCD keeps the L2 sharing of its super-rounds. A
// workgroup takes the next job of its own XCD's queue; once that queue is
// empty, the next job of the queue with the most jobs left. The XCDs do not run
// equally fast (on MI355X the odd ones are a few percent slower), so with a
// static mapping the kernel ends when the slowest XCD does; the grid carries
// spare workgroups for the faster XCDs, and a workgroup that finds every queue
// empty exits. Only the job index is shared between workgroups (the atomic's
// return value), so no memory fence is needed.
constexpr int kQueues = 8;
__device__ __forceinline__ int grab_job(int* queues, int n_jobs) {
  unsigned xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  const int own = (int)(xcc & (kQueues - 1));
  const int k = atomicAdd(&queues[own], 1);
  if (own + kQueues * (int64_t)k < n_jobs) return own + kQueues * k;
  for (;;) {
    int best = -1, best_left = 0;
    for (int x = 0; x < kQueues; ++x) {
      const int taken = __hip_atomic_load(&queues[x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int left = (n_jobs - x + kQueues - 1) / kQueues - taken;
      if (left > best_left) {
        best_left = left;
        best = x;
      }
    }
    if (best < 0) return -1;
    const int kk = atomicAdd(&queues[best], 1);
    if (best + kQueues * (int64_t)kk < n_jobs) return best + kQueues * kk;
  }
}

__global__ void queue_reset_kernel(int* queues) {
  if (threadIdx.x < kQueues) __hip_atomic_store(&queues[threadIdx.x], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
  int* queues;              // kPhase1 / kPhase1Ws: kQueues job counters (run-time job order), or null (static)
  // kQuery: 1 when no workgroup is launched for the tail partition; the
  // workgroups of chunk fold_chunk of the last context partition take the
  // tail's keys first and write its partial (chunk 0 of the tail; the tail's
  // other chunks get lse = -inf).
  int32_t fold_tail;
  int32_t fold_chunk;
  // kQuery: keys moved from each odd chunk to the even chunk before it (a
  // multiple of the key tile), or 0: chunk c starts at c * chunk_len, plus
  // chunk_skew for odd c.
  int32_t chunk_skew;
};

// kPhase1Ws: Phase 1 with the anchor's keys rotated per block in a workspace
// (Phase1Args::k_anchor), a separate instance so that the plain Phase-1 kernel
// keeps its single key base.
enum { kPhase1 = 0, kQuery = 1, kPhase1Ws = 2 };

}  // namespace

template <int D, int MODE>
__global__ __launch_bounds__(kThreads, 1) void attn_tile_kernel(TileArgs ta, RopeTable rt) {
  // Five distinct objects (not an array): each slot's operand reads are a
  // constant offset from its own base.
  __shared__ TileSlot<D> slot0, slot1, slot2, slot3, slot4;
  constexpr int NC = D / 16;           // 16-wide d chunks (MFMA K dim of QK^T)
  constexpr int NDB = D / 32;          // 32-wide d blocks (MFMA M dim of PV)
  constexpr int ROWS_PER_LOAD = 1024 / (2 * D);                  // rows one wavefront load instruction covers
  constexpr int LOADS_PER_WAVE = kBN / ROWS_PER_LOAD / kWaves;   // per tile, for K and for V
  static_assert(LOADS_PER_WAVE >= 1 && LOADS_PER_WAVE * ROWS_PER_LOAD * kWaves == kBN, "tile split");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane >> 5;            // which half of the wavefront
  const int ln = lane & 31;
  const int n_q_heads = MODE != kQuery ? ta.p1.n_q_heads : ta.p2.n_q_heads;
  const int n_kv_heads = MODE != kQuery ? ta.p1.n_kv_heads : ta.p2.n_kv_heads;
  const int g = n_q_heads / n_kv_heads;
  const float qk_scale = MODE != kQuery ? ta.p1.qk_scale_log2 : ta.p2.qk_scale_log2;

  // ---- Job decode: this lane's query row (token, head, position) and the key segments.
  int kvh, h;
  int64_t tok, qpos;
  bool row_valid;
  Segment seg_a{0, 0};   // anchor (Phase 1, blocks > 1)
  Segment seg_b{0, 0};   // the block's causal prefix, or the Phase-2 chunk
  int64_t tiles0 = 0;
  const bf16_t* kc;
  const bf16_t* vc;
  const bf16_t* kc_a;                  // the anchor segment's rows start here (K; V at vc_a)
  const bf16_t* vc_a;
  int p2_part = 0, p2_chunk = 0;
  int64_t pos_shift = 0;               // key position = cache row + pos_shift
  int64_t a_base = 0;                  // the first anchor-segment row sits at kc_a / vc_a + (row0 - a_base) * D
  bool folded = false;                 // kQuery: this workgroup takes the tail first (TileArgs::fold_tail)
  if constexpr (MODE != kQuery) {
    const Phase1Args& a = ta.p1;
    const int gp = ta.heads_per_tile;
    const int groups = g / gp;
    const int64_t tpt = kBM / gp;      // tokens per tile
    // Jobs in non-increasing order of work, so that every round of workgroups
    // the hardware hands out together runs about equally long: first the row
    // tiles of blocks 2..n (anchor + causal prefix) from the last row tile
    // down, then block 1's. The KV head varies fastest, so workgroup w (which
    // runs on XCD w % 8) keeps to the same KV heads. Blocks 2..n go in
    // super-rounds of 32 row tiles (an XCD's 32 CUs): within one, the row tile
    // varies before the block, so the workgroups an XCD runs together stream
    // the same anchor and block tiles through its L2.
    const int64_t nblk = a.ctx_len / a.block_len;
    const int64_t n_anch = (nblk - 1) * ta.n_row_tiles * groups * n_kv_heads;
    int64_t j = blockIdx.x;
    if (ta.queues) {
      // One lane takes the job; the last ring slot (not loaded before the
      // first barrier of the tile loop) carries it to the other wavefronts.
      int* bcast = reinterpret_cast<int*>(slot4.k);
      if (tid == 0) *bcast = grab_job(ta.queues, (int)ta.n_jobs);
      __syncthreads();
      const int jj = *bcast;
      if (jj < 0) return;   // every job taken (a spare workgroup)
      j = jj;
    }
    int64_t blk, qt;
    int hgrp;
    if (j < n_anch) {
      // super-round of kQS row tiles: KV head, then row tile, then head group
      // and block
      constexpr int64_t kQS = 32;
      const int64_t per_sr = kQS * (nblk - 1) * groups * n_kv_heads;
      const int64_t sr = j / per_sr;
      const int64_t qs = (ta.n_row_tiles - sr * kQS) < kQS ? ta.n_row_tiles - sr * kQS : kQS;
      int64_t r = j - sr * per_sr;
      // the KV head rotates by one per super-round, so that every XCD (which
      // takes one residue of the KV head within a super-round) sees every head
      kvh = (int)((r + sr) % n_kv_heads);
      r /= n_kv_heads;
      const int64_t qo = r % qs;
      r /= qs;
      qt = ta.n_row_tiles - 1 - (sr * kQS + qo);
      hgrp = (int)(r % groups);
      blk = 1 + r / groups;
    } else {
      j -= n_anch;
      const int64_t per_qt = (int64_t)groups * n_kv_heads;
      qt = ta.n_row_tiles - 1 - j / per_qt;
      const int64_t r = j % per_qt;
      kvh = (int)(r % n_kv_heads);
      hgrp = (int)(r / n_kv_heads);
      blk = 0;
    }
    h = kvh * g + hgrp * gp + wave % gp;
    const int64_t b = a.block_len;
    const int64_t r_lane = qt * tpt + (wave / gp) * 32 + ln;
    row_valid = r_lane < b;
    tok = blk * b + (row_valid ? r_lane : b - 1);
    qpos = tok;
    // The anchor: block 1's (or block i - 1's) first A cache rows, every one
    // before the block, so the mask below sees them all. kPhase1Ws reads its
    // keys rotated for this block from the workspace (rows counted from 0).
    const int64_t a_first = a.anchor_prev ? (blk - 1) * b : 0;
    if (blk > 0) {
      seg_a = {MODE == kPhase1Ws ? 0 : a_first, a.anchor_len};
      tiles0 = (a.anchor_len + kBN - 1) / kBN;
    }
    const int64_t kend = ((qt + 1) * tpt) < b ? (qt + 1) * tpt : b;
    seg_b = {blk * b, kend};
    kc = static_cast<const bf16_t*>(a.k_cache) + (int64_t)kvh * a.ctx_len * D;
    vc = static_cast<const bf16_t*>(a.v_cache) + (int64_t)kvh * a.ctx_len * D;
    kc_a = kc;
    vc_a = vc;
    if constexpr (MODE == kPhase1Ws) {
      kc_a = static_cast<const bf16_t*>(a.k_anchor) + ((int64_t)kvh * (nblk - 1) + (blk > 0 ? blk - 1 : 0)) *
                                                          a.anchor_len * D;
      vc_a = vc + a_first * D;
    }
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
    auto chunk_start = [&](int c) {
      const int64_t k0 = (int64_t)c * a.chunk_len + ((c & 1) ? ta.chunk_skew : 0);
      return k0 < len ? k0 : len;
    };
    const int64_t ck0 = chunk_start(p2_chunk);
    const int64_t ck1 = chunk_start(p2_chunk + 1);
    seg_b = {part_row0 + ck0, ck1 - ck0};
    if (tail) pos_shift = a.tail_pos0;
    kc = static_cast<const bf16_t*>(tail ? a.k_tail : a.k_cache) + (int64_t)kvh * head_rows * D;
    vc = static_cast<const bf16_t*>(tail ? a.v_tail : a.v_cache) + (int64_t)kvh * head_rows * D;
    kc_a = kc;
    vc_a = vc;
    folded = ta.fold_tail && p2_part == a.n_ctx_parts - 1 && p2_chunk == ta.fold_chunk;
    if (folded) {
      // The tail's rows come first as the other segment, counted in position
      // space (row = position, so the one positional mask serves both
      // segments: every context key precedes every query).
      seg_a = {a.tail_pos0, a.tail_len};
      tiles0 = (a.tail_len + kBN - 1) / kBN;
      a_base = a.tail_pos0;
      kc_a = static_cast<const bf16_t*>(a.k_tail) + (int64_t)kvh * a.tail_cap * D;
      vc_a = static_cast<const bf16_t*>(a.v_tail) + (int64_t)kvh * a.tail_cap * D;
    }
  }

  bf16x8 qf[NC];   // this lane's Q operands, loaded after the first tiles' loads go out
  // Wavefront query-position range (valid rows only) for mask / skip decisions.
  const int64_t w_qpos_lo = wave_min_i64(row_valid ? qpos : INT64_MAX);
  const int64_t w_qpos_hi = wave_max_i64(row_valid ? qpos : INT64_MIN);
  const int64_t n_tiles = tiles0 + (seg_b.len + kBN - 1) / kBN;

  // Tile bookkeeping in 32-bit cache-row space (rows and positions stay below
  // 2^31): key row r is visible to a query at position p iff r + pos_shift <= p.
  auto clamp32 = [](int64_t v) { return (int)(v < INT32_MIN ? INT32_MIN : (v > INT32_MAX ? INT32_MAX : v)); };
  const int t_a = (int)tiles0;
  const int a_row0 = (int)seg_a.row0, a_len = (int)seg_a.len;
  const int b_row0 = (int)seg_b.row0, b_len = (int)seg_b.len;
  const int w_lo_row = clamp32(w_qpos_lo - pos_shift);
  const int w_hi_row = clamp32(w_qpos_hi - pos_shift);
  const int q_row = clamp32(qpos - pos_shift);
  // Tile n: its first cache row, and the rows left in its segment from there
  // (more than a tile inside the segment, none or fewer past its end). Each is
  // one select and one add from per-segment values held in scalar registers,
  // so the per-tile bookkeeping is a few scalar instructions with no branch.
  const int row0_a = __builtin_amdgcn_readfirstlane(a_row0);
  const int row0_b = __builtin_amdgcn_readfirstlane(b_row0 - t_a * kBN);
  const int rows_a = __builtin_amdgcn_readfirstlane(a_len);
  const int rows_b = __builtin_amdgcn_readfirstlane(b_len + t_a * kBN);
  auto tile_row0 = [&](int n) { return (n < t_a ? row0_a : row0_b) + n * kBN; };
  auto tile_rows = [&](int n) { return (n < t_a ? rows_a : rows_b) - n * kBN; };
  // Tile n goes to slot n % 5 straight from HBM/L2 (buffer_load ... lds, no
  // registers), three tiles ahead of its use. The buffer resource's base is the
  // tile's first row and its extent ends at the segment's end, so rows past the
  // end arrive as zeros (those keys are masked). One wavefront instruction
  // fills 1 KB of LDS, lane i the 16 bytes at 16 i: row i / (D/8) of the
  // piece, stored chunk i % (D/8), which holds logical chunk (stored ^ swizzle).
  // Tile n's first K row sits at byte address seg + n * kTileBytes, where seg
  // is k_seg_a for the anchor segment's tiles (n < t_a) and k_seg_b for the
  // others (each is that segment's first row, less the tiles before it); V
  // likewise. The anchor segment's rows are at kc_a / vc_a + (row - a_base) * D
  // (kPhase1 reads both segments from kc / vc).
  struct TileRsrc { i32x4_t k, v; };
  constexpr uint64_t kTileBytes = (uint64_t)kBN * D * 2;
  const uint64_t a_skip = (uint64_t)(a_row0 - a_base) * D * 2;
  const uint64_t b_skip = (uint64_t)((int64_t)b_row0 * D * 2) - (uint64_t)t_a * kTileBytes;
  const uint64_t k_seg_a = uniform64(reinterpret_cast<uint64_t>(MODE == kPhase1 ? kc : kc_a) + a_skip);
  const uint64_t v_seg_a = uniform64(reinterpret_cast<uint64_t>(MODE == kPhase1 ? vc : vc_a) + a_skip);
  const uint64_t k_seg_b = uniform64(reinterpret_cast<uint64_t>(kc) + b_skip);
  const uint64_t v_seg_b = uniform64(reinterpret_cast<uint64_t>(vc) + b_skip);
  auto tile_rsrc = [&](int n) {
    const bool in_a = n < t_a;
    const int rows = tile_rows(n);
    const int nbytes = __builtin_amdgcn_readfirstlane((rows < 0 ? 0 : (rows < kBN ? rows : kBN)) * D * 2);
    const uint64_t off = (uint64_t)n * kTileBytes;
    return TileRsrc{make_rsrc((in_a ? k_seg_a : k_seg_b) + off, nbytes),
                    make_rsrc((in_a ? v_seg_a : v_seg_b) + off, nbytes)};
  };
  // the wavefront index in a scalar register, so that the LDS address (M0) of
  // every tile load is scalar arithmetic
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  auto load_piece = [&](const TileRsrc& rs, TileSlot<D>& dst, int j) {
    const int piece = wave_s * LOADS_PER_WAVE + j % LOADS_PER_WAVE;
    const int r = piece * ROWS_PER_LOAD + lane / (D / 8);
    const int pc = lane % (D / 8);
    if (j < LOADS_PER_WAVE)
      load_lds16(rs.k, (lds_void*)dst.k, piece * ROWS_PER_LOAD * D * 2, (r * D + 8 * (pc ^ swz_k<D>(r))) * 2);
    else
      load_lds16(rs.v, (lds_void*)dst.v, piece * ROWS_PER_LOAD * D * 2, (r * D + 8 * (pc ^ swz_v<D>(r))) * 2);
  };
  auto issue_tile = [&](int n, TileSlot<D>& dst) {
    const TileRsrc rs = tile_rsrc(n);
#pragma unroll
    for (int j = 0; j < 2 * LOADS_PER_WAVE; ++j) load_piece(rs, dst, j);
  };

  // Per-lane LDS operand offsets (elements). The swizzles depend only on
  // loop-invariant lane bits, so every read is a base plus a constant.
  // K (A of S^T), block sb, chunk c: row 32 sb + ln, logical chunk 2 c + hl,
  // stored at chunk (2 c + hl) ^ (row % (D/8)) = 2 c ^ (hl ^ ln % (D/8)).
  int k_base[NC];
  {
    const int y = hl ^ (ln % (D / 8));
#pragma unroll
    for (int c = 0; c < NC; ++c) k_base[c] = ln * D + 8 * ((2 * c) ^ y);
  }
  // V (A of O^T), transposing read t of d-block db and key chunk kc16: this lane
  // is source lane s = lane % 16 of group gq = lane / 16 and points at row
  // 16 kc16 + 8 t + 4 (gq / 2) + s / 4, column 32 db + 16 (gq % 2) + 4 (s % 4);
  // the row's swizzle reduces to swz_v(s / 4).
  int v_base[NDB];
  {
    const int gq = lane >> 4, sl = lane & 15;
    const int z = 2 * (gq & 1) + ((sl & 3) >> 1);          // column chunk within the d-block
    const int w = swz_v<D>(sl >> 2);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      v_base[db] = (4 * (gq >> 1) + (sl >> 2)) * D + 8 * ((4 * db + z) ^ w) + 4 * (sl & 1);
  }

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  float m_use = 0.f;         // reference subtracted from this lane's scores
  bool has_ref = false;      // m_use has been set from a visible score
  f32x16 negm = f32x16{};    // -m_use in every element (accumulator seed)
  float l_run = 0.f;         // lane-partial sum of exp2(s - m_use)
  const bf16x2 ones = {(bf16_t)1.f, (bf16_t)1.f};

  // One tile. Every second tile (`sync`): wait for this wavefront's loads of
  // tiles n and n + 1 (tile n + 2's may still fly), then a barrier: every
  // wavefront's loads of both tiles landed, and every wavefront is done with
  // tiles n - 2 and n - 1, whose slots take tiles n + 3 and n + 4. Then compute,
  // issuing tile n + 3's loads.
  // kQuery: this lane's normalised row of the partial (part, chunk) and its LSE.
  auto store_partial = [&](int part, int chunk) {
    const float l_tot = l_run + other_half(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (row_valid) {
      const Phase2Args& a = ta.p2;
      const int64_t slot = (((int64_t)part * a.n_chunks + chunk) * a.t_q + tok) * n_q_heads + h;
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
  };
  const int t_split = folded ? t_a : -1;
  const bool late_wave = __builtin_amdgcn_readfirstlane(wave) >= kWaves / 2;   // second wavefront of its SIMD

  auto step = [&](int n, TileSlot<D>& cur, TileSlot<D>& nxt2, bool sync) {
    if constexpr (MODE == kQuery) {
      if (n == t_split) {
        // The tail's keys are done: write its partial (chunk 0; its other
        // chunks hold no key) and start the context chunk afresh: an empty
        // row sum (so a chunk whose tiles are all masked stores an empty
        // partial) and no reference. The rare path then takes the first tile
        // with a visible key: it moves the reference (still the tail's, the
        // one the scores are taken against) to that tile's maximum and
        // multiplies O by 0. Only scalars change here; clearing O and the
        // seed made the compiler carry second copies of them through the loop.
        const Phase2Args& a = ta.p2;
        store_partial(a.n_ctx_parts, 0);
        if (row_valid && hl == 0)
          for (int c = 1; c < a.n_chunks; ++c)
            a.ws_lse[(((int64_t)a.n_ctx_parts * a.n_chunks + c) * a.t_q + tok) * n_q_heads + h] = -INFINITY;
        l_run = 0.f;
        has_ref = false;
      }
    }
    if (sync) {
      wait_vm<2 * LOADS_PER_WAVE>();   // tiles n and n + 1 landed (n + 2 may fly)
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (late_wave) __builtin_amdgcn_s_setprio(1);
    } else {
      if (late_wave) __builtin_amdgcn_s_setprio(0);
    }

    // The tile's first K operand reads go out before its bookkeeping, whose
    // scalar work then covers their latency (the scheduling barrier keeps the
    // compiler from sinking them below it). A tile whose keys are all masked
    // leaves them unused.
    constexpr int NQ = 2 * NC;
    auto kread = [&](int idx) {
      return *reinterpret_cast<const bf16x8*>(&cur.k[k_base[idx / 2] + 32 * (idx % 2) * D]);
    };
    bf16x8 kb[kQkReadDepth];
#pragma unroll
    for (int i = 0; i < kQkReadDepth; ++i) kb[i] = kread(i);
    __builtin_amdgcn_sched_barrier(0);
    const int row0 = tile_row0(n);
    const int rows = tile_rows(n);
    const bool all_masked = row0 > w_hi_row;             // every key in every row's future
    // Tile n + 3's loads; on a computed tile they go out one at a time between
    // the QK^T MFMAs, so the CU's address path drains while the matrix cores work.
    const TileRsrc rs2 = tile_rsrc(n + 3);
    if (all_masked) {
#pragma unroll
      for (int j = 0; j < 2 * LOADS_PER_WAVE; ++j) load_piece(rs2, nxt2, j);
    }
    if (!all_masked) {
      const bool need_mask = (row0 + kBN - 1 > w_lo_row) || (rows < kBN);
      // S^T - m_use for 2 blocks of 32 keys (accumulators seeded with -m_use),
      // the K operand reads kQkReadDepth ahead of their MFMAs. The two blocks'
      // MFMAs alternate, so consecutive ones are independent and one wavefront
      // can issue them back to back.
      f32x16 s[2] = {negm, negm};
#pragma unroll
      for (int idx = 0; idx < NQ; ++idx) {
        const bf16x8 ka = kb[idx % kQkReadDepth];
        if (idx + kQkReadDepth < NQ) kb[idx % kQkReadDepth] = kread(idx + kQkReadDepth);
        s[idx % 2] = mfma32(ka, qf[idx / 2], s[idx % 2]);
        if (idx % kLoadEvery == 1 && idx / kLoadEvery < 2 * LOADS_PER_WAVE) load_piece(rs2, nxt2, idx / kLoadEvery);
      }
      // Schedule: each MFMA followed by the next read, and one tile load after
      // every kLoadEvery-th MFMA (sched_group_barrier masks: 0x100 LDS read,
      // 0x008 MFMA, 0x020 VMEM read).
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + kQkReadDepth < NQ) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (i % kLoadEvery == 1 && i / kLoadEvery < 2 * LOADS_PER_WAVE) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      if (need_mask) {
        const int lim_len = rows < kBN ? rows : kBN;
        const int dq = q_row - row0;                      // keys kk <= dq are visible
        const int lim_pos = dq < 0 ? 0 : (dq >= kBN ? kBN : dq + 1);
        // Element i of block sb holds key 32 sb + 8 (i / 4) + 4 hl + i % 4; the
        // half-wave offset moves to the limit so the other terms stay constants.
        const int lim = (lim_len < lim_pos ? lim_len : lim_pos) - 4 * hl;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kk = 32 * sb + 8 * (i >> 2) + (i & 3);
            s[sb][i] = kk < lim ? s[sb][i] : -INFINITY;
          }
      }
      // Probabilities against the current reference, packed to bf16, and this
      // tile's lane share of the row sum; the rare path (see the file comment)
      // when that share leaves [0, kBig] or the row has no reference yet.
      bf16x8 pb[2][2];
      float l_tile;
      auto probs = [&]() {
        l_tile = 0.f;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
            for (int j = 0; j < 8; ++j) pb[sb][hh][j] = (bf16_t)fast_exp2(s[sb][8 * hh + j]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const bf16x2 pr = {pb[sb][hh][2 * j], pb[sb][hh][2 * j + 1]};
              l_tile = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_tile, false);
            }
          }
      };
      probs();
      if (__builtin_amdgcn_ballot_w64(!has_ref || !(l_tile <= kBig))) {
        float mt = -INFINITY;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[sb][i]);
        mt = fmaxf(mt, other_half(mt));
        const bool upd = mt > -INFINITY && (!has_ref || mt > kTau);
        // Move the reference to this tile's maximum for the rows that need it.
        const float delta = upd ? mt : 0.f;
        // (a row without a reference holds no contribution, or the folded
        // tail's, which the context chunk must not keep)
        const float alpha = !has_ref ? 0.f : (upd ? fast_exp2(-delta) : 1.f);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] *= alpha;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) s[sb] -= delta;
        m_use += delta;
        has_ref = has_ref || upd;
#pragma unroll
        for (int i = 0; i < 16; ++i) negm[i] = -m_use;
        probs();
      }
      l_run += l_tile;
      // O^T += V^T P^T, 16 keys per MFMA. P^T's keys per lane are {0-3, 8-11} in
      // the low half-wave and {4-7, 12-15} in the high one (the accumulator
      // layout); two transposing reads give the matching V^T operand.
#pragma unroll
      for (int kc16 = 0; kc16 < 4; ++kc16) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16_t* v0 = &cur.v[v_base[db] + 16 * kc16 * D];
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_void*)v0);
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_void*)(v0 + 8 * D));
          const i16x4 lohi[2] = {lo, hi};
          o[db] = mfma32(__builtin_bit_cast(bf16x8, lohi), pb[kc16 >> 1][kc16 & 1], o[db]);
        }
      }
    }
  };

  // Tiles 0 and 1 go out first, then the Q rows are loaded (and rotated), then
  // tile 2. The compiler's waits for the Q loads cannot tell the tile loads
  // apart and wait for every load issued before them, so here they cover just
  // the two tiles the first barrier needs. With the Q loads first and all three
  // tiles after them, the compiler placed the rotation behind the tile loads,
  // whose waits then took all three tiles: Phase 1 1.6% slower (same box). The
  // empty asm statements keep the Q work ahead of tile 2's loads.
  issue_tile(0, slot0);
  issue_tile(1, slot1);
  // ---- Q rows: load, RoPE (fp64 angles), fold softmax_scale*log2(e), to bf16
  // (or, in the query step, load the rows the RoPE kernel already rotated).
  if (MODE == kQuery && ta.p2.q_rot != nullptr) {
    const bf16_t* qp = static_cast<const bf16_t*>(ta.p2.q_rot) + (tok * n_q_heads + h) * D + 8 * hl;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qp + 16 * c);
  } else {
    const bf16_t* qbase = static_cast<const bf16_t*>(MODE != kQuery ? ta.p1.q : ta.p2.q);
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
        // both half-waves' frequencies at uniform indices (scalar loads, all
        // in flight together), then a per-lane select
        const double f_lo = rt.inv_freq[16 * c + j], f_hi = rt.inv_freq[16 * c + 8 + j];
        float cs, sn;
        rope_cos_sin_hw(qpos, hl ? f_hi : f_lo, &cs, &sn);
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
#pragma unroll
  for (int c = 0; c < NC; ++c) asm volatile("" : "+v"(qf[c]));
  issue_tile(2, slot2);
  const int nt = (int)n_tiles;
  for (int n = 0; n < nt; n += 10) {
    step(n, slot0, slot3, true);
    if (n + 1 >= nt) break;
    step(n + 1, slot1, slot4, false);
    if (n + 2 >= nt) break;
    step(n + 2, slot2, slot0, true);
    if (n + 3 >= nt) break;
    step(n + 3, slot3, slot1, false);
    if (n + 4 >= nt) break;
    step(n + 4, slot4, slot2, true);
    if (n + 5 >= nt) break;
    step(n + 5, slot0, slot3, false);
    if (n + 6 >= nt) break;
    step(n + 6, slot1, slot4, true);
    if (n + 7 >= nt) break;
    step(n + 7, slot2, slot0, false);
    if (n + 8 >= nt) break;
    step(n + 8, slot3, slot1, true);
    if (n + 9 >= nt) break;
    step(n + 9, slot4, slot2, false);
  }
  wait_vm<0>();   // the last (empty) tile loads still write LDS

  // ---- Normalise and store this lane's row.
  const float l_tot = l_run + other_half(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if constexpr (MODE != kQuery) {
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
    store_partial(p2_part, p2_chunk);
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

hipError_t launch_phase1_mfma(const Phase1Args& a, const RopeTable& rt, int head_dim, void* queues, hipStream_t s) {
  TileArgs ta{};
  ta.p1 = a;
  ta.heads_per_tile = heads_per_tile(a.n_q_heads / a.n_kv_heads);
  const int64_t tpt = kBM / ta.heads_per_tile;
  ta.n_row_tiles = (a.block_len + tpt - 1) / tpt;
  ta.n_jobs = ta.n_row_tiles * (a.ctx_len / a.block_len) * (a.n_q_heads / ta.heads_per_tile);
  if (ta.n_jobs == 0) return hipSuccess;
  ta.queues = static_cast<int*>(queues);
  // spare workgroups for the XCDs that run out of their own jobs first
  const int64_t n_wg = queues ? ta.n_jobs + ta.n_jobs / 16 + 2 * kQueues : ta.n_jobs;
  if (queues) {
    hipLaunchKernelGGL(queue_reset_kernel, dim3(1), dim3(64), 0, s, ta.queues);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)n_wg), block(kThreads);
  if (a.k_anchor != nullptr) {
    if (head_dim == 64) hipLaunchKernelGGL((attn_tile_kernel<64, kPhase1Ws>), grid, block, 0, s, ta, rt);
    else hipLaunchKernelGGL((attn_tile_kernel<128, kPhase1Ws>), grid, block, 0, s, ta, rt);
  } else if (head_dim == 64) {
    hipLaunchKernelGGL((attn_tile_kernel<64, kPhase1>), grid, block, 0, s, ta, rt);
  } else {
    hipLaunchKernelGGL((attn_tile_kernel<128, kPhase1>), grid, block, 0, s, ta, rt);
  }
  return hipGetLastError();
}

hipError_t launch_phase2_query(const Phase2Args& a, const RopeTable& rt, int head_dim, hipStream_t s,
                               int32_t* tail_items) {
  TileArgs ta{};
  ta.p2 = a;
  ta.heads_per_tile = 1;
  const int64_t rows = a.t_q * (a.n_q_heads / a.n_kv_heads);
  ta.n_row_tiles = (rows + kBM - 1) / kBM;
  // A short tail (up to kFoldTiles tiles) rides along with one chunk of the
  // last context partition instead of taking workgroups of its own: the
  // context chunks fill one round of the CUs, and a tail workgroup would start
  // a second round of a Q rotation, one tile and a store. That chunk must hold
  // keys, and tail positions stay below 2^31 (the kernel's 32-bit rows). It is
  // the last but one: with one row tile per KV head, chunk c runs on XCD c, and
  // on MI355X the odd XCDs run a few percent slower, so the extra work goes to
  // an even one.
  constexpr int64_t kFoldTiles = 8;
  // For the same reason, with one row tile per KV head and an even number of
  // chunks of at least 8 tiles, every even chunk takes one key tile from the
  // odd chunk after it.
  ta.chunk_skew = ta.n_row_tiles == 1 && a.n_chunks % 2 == 0 && a.chunk_len >= 8 * kBN ? kBN : 0;
  ta.fold_chunk = a.n_chunks >= 2 ? a.n_chunks - 2 : 0;
  const int64_t fold_chunk0 = (int64_t)ta.fold_chunk * a.chunk_len;   // even: no skew
  ta.fold_tail = a.n_ctx_parts >= 1 && a.tail_len <= kFoldTiles * kBN && fold_chunk0 < a.block_len &&
                 a.tail_pos0 + a.tail_len + kBN < ((int64_t)1 << 31);
  ta.n_jobs = ta.n_row_tiles * (int64_t)a.n_chunks * a.n_kv_heads * (a.n_ctx_parts + (ta.fold_tail ? 0 : 1));
  *tail_items = ta.fold_tail ? 1 : a.n_chunks;   // a folded tail's partial is its chunk 0
  if (ta.n_jobs == 0) return hipSuccess;
  const dim3 grid((unsigned)ta.n_jobs), block(kThreads);
  if (head_dim == 64) hipLaunchKernelGGL((attn_tile_kernel<64, kQuery>), grid, block, 0, s, ta, rt);
  else hipLaunchKernelGGL((attn_tile_kernel<128, kQuery>), grid, block, 0, s, ta, rt);
  return hipGetLastError();
}

}  // namespace sa
